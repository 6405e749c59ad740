// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include "internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SAS_WAVE 64

namespace sas {

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Packs two floats into a bf16x2 word (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(bf16_t* p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 first so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// log g of a selected history block under the gate activation (picx.dev
// summary of SAS, Eq. 4 and 6): 0 softmax, s - LSE(s); 1 sigmoid, log sigmoid(s)
// = -(max(-s, 0) + log1p(exp(-|s|))); 2 raw logit, s.
__device__ __forceinline__ float gate_log(float s, float lse, int act) {
  if (act == 1) return -(fmaxf(-s, 0.0f) + log1pf(expf(-fabsf(s))));
  if (act == 2) return s;
  return s - lse;
}

// History length of selection row t of (batch, KV head) row bk.  Training rows
// (row_offset 0) past the sequence's last block have none; decode rows see the
// sequence's own (L_b - 1) / bs history blocks.
__device__ __forceinline__ int row_history(int t, int row_offset, int C, const RowLens& rl,
                                           size_t bk) {
  const int ct = min(t + row_offset, C);
  if (!rl.lens) return ct;
  const int lb = min(max(rl.lens[bk / rl.hkv], 0), rl.lmax);
  if (row_offset == 0) return t < (lb + rl.bs - 1) / rl.bs ? ct : 0;
  return min(ct, max(lb - 1, 0) / rl.bs);
}

// Inverse of order_key.
__device__ __forceinline__ float from_order_key(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

// Lane exchange x <- x of lane (lane ^ J) within a wave of 64, on cross-lane
// paths that bypass the LDS unit: DPP quad permutes for J = 1, 2; a half-row
// mirror followed by a quad reversal for J = 4 (7 - (i ^ 3) = i ^ 4 within
// eight lanes); a row rotation by 8 for J = 8; gfx950's row-pair swaps for
// J = 16 and 32, whose first result holds the lower row (half) of each pair in
// both, the second the upper, so a lane takes the other side's.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (J == 4) {
    const int m = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    return __builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);               // quad_perm 3,2,1,0
  } else if constexpr (J == 8) {
    return __builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);  // row_ror 8
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

// Sorts a bitonic sequence of 64 keys, one per lane, into descending lane
// order: half-cleaners at distances 32, 16, ..., 1, the larger key kept by the
// lower lane of each pair.
template <int J = 32>
__device__ __forceinline__ uint64_t bitonic_desc64(uint64_t v, int lane) {
  const uint64_t o = ((uint64_t)xor_lane<J>((uint32_t)(v >> 32)) << 32) |
                     xor_lane<J>((uint32_t)v);
  v = ((lane & J) == 0) == (v > o) ? v : o;
  if constexpr (J > 1) return bitonic_desc64<J / 2>(v, lane);
  else return v;
}

// Sorts 64 keys, one per lane, into ascending lane order with the full
// bitonic network: merge stages of width 2, 4, ..., 64, each a run of
// exchanges at distances KK / 2, ..., 1 across lane pairs (the lower lane
// keeps the smaller key when lane & KK is clear, the larger when it is set).
template <int KK = 2, int J = 1>
__device__ __forceinline__ uint64_t bitonic_sort_asc64(uint64_t v, int lane) {
  const uint64_t o = ((uint64_t)xor_lane<J>((uint32_t)(v >> 32)) << 32) |
                     xor_lane<J>((uint32_t)v);
  const bool lower = (lane & J) == 0, up = (lane & KK) == 0 || KK == 64;
  v = (lower == up) ? (v < o ? v : o) : (v < o ? o : v);
  if constexpr (J > 1) return bitonic_sort_asc64<KK, J / 2>(v, lane);
  else if constexpr (KK < 64) return bitonic_sort_asc64<KK * 2, KK>(v, lane);
  else return v;
}

// The same network into descending lane order (the larger key goes where
// the ascending sort puts the smaller).
template <int KK = 2, int J = 1>
__device__ __forceinline__ uint64_t bitonic_sort_desc64(uint64_t v, int lane) {
  const uint64_t o = ((uint64_t)xor_lane<J>((uint32_t)(v >> 32)) << 32) |
                     xor_lane<J>((uint32_t)v);
  const bool lower = (lane & J) == 0, up = (lane & KK) == 0 || KK == 64;
  v = (lower == up) ? (v > o ? v : o) : (v > o ? o : v);
  if constexpr (J > 1) return bitonic_sort_desc64<KK, J / 2>(v, lane);
  else if constexpr (KK < 64) return bitonic_sort_desc64<KK * 2, KK>(v, lane);
  else return v;
}

// Copies n 8-byte keys from global memory to LDS with all of a thread's loads
// (up to PER per pass) issued before its first store, so a pass costs one
// memory round trip instead of one per key; at most one key per thread is
// copied directly (measured: the unrolled pass was slower there).
template <int PER>
__device__ __forceinline__ void copy_keys_to_lds(uint64_t* dst, const uint64_t* __restrict__ src,
                                                 int n, int tid, int nth) {
  if (n <= nth) {
    if (tid < n) dst[tid] = src[tid];
    return;
  }
  for (int base = 0; base < n; base += PER * nth) {
    uint64_t v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + tid + u * nth;
      v[u] = i < n ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + tid + u * nth;
      if (i < n) dst[i] = v[u];
    }
  }
}

// Top K (K <= 64) of nl descending lists of K distinct nonzero keys held in
// LDS, descending.  Two descending lists of 64 (zero-padded) meet by taking
// the larger of a[i] and b[63 - i] lane by lane, which keeps the top 64 of the
// pair as a bitonic sequence, sorted again by bitonic_desc64.  Wave w folds
// lists w, w + NW, ... into its running top list (the next list's LDS read in
// flight during the current fold); wave 0 then folds the other waves' lists
// from `wl` (NW * 64 keys of LDS; one barrier when NW > 1, which every thread
// of the workgroup reaches).  Lane i of wave 0 returns the key of rank i (0
// past the end).
template <int NW>
__device__ __forceinline__ uint64_t merge_top64(const uint64_t* lists, int nl, int K,
                                                uint64_t* wl) {
  const int lane = threadIdx.x & 63, wave = (int)(threadIdx.x >> 6);
  const int rev = 63 - lane;
  uint64_t acc = 0;
  uint64_t nb = wave < nl && rev < K ? lists[wave * K + rev] : 0ull;
  for (int l = wave; l < nl; l += NW) {
    const uint64_t b = nb;
    nb = l + NW < nl && rev < K ? lists[(l + NW) * K + rev] : 0ull;
    acc = bitonic_desc64(acc > b ? acc : b, lane);
  }
  if constexpr (NW > 1) {
    wl[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const uint64_t b = wl[w * 64 + rev];
        acc = bitonic_desc64(acc > b ? acc : b, lane);
      }
    }
  }
  return acc;
}

// Butterfly reductions over the wave (lane distances 32, 16, ..., 1, the
// lane exchanges of xor_lane): every lane ends with the result.
template <int J = 32>
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(xor_lane<J>(__float_as_uint(v))));
  if constexpr (J > 1) return wave_max<J / 2>(v);
  else return v;
}
template <int J = 32>
__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(xor_lane<J>(__float_as_uint(v)));
  if constexpr (J > 1) return wave_sum<J / 2>(v);
  else return v;
}
template <int J = 32>
__device__ __forceinline__ double wave_sum_d(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t o = ((uint64_t)xor_lane<J>((uint32_t)(b >> 32)) << 32) | xor_lane<J>((uint32_t)b);
  v += __longlong_as_double((long long)o);
  if constexpr (J > 1) return wave_sum_d<J / 2>(v);
  else return v;
}

// Inclusive prefix sum across a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Exclusive prefix sum over the whole workgroup (blockDim.x a multiple of 64,
// at most 1024).  `scratch` holds >= 16 ints of LDS.  Returns the exclusive
// prefix; *total receives the workgroup sum.  Contains barriers.
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) scratch[wid] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    int s = scratch[w];
    if (w < wid) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__device__ __forceinline__ float block_sum(float v, float* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  v = wave_sum(v);
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < nw; ++w) r += scratch[w];
  __syncthreads();
  return r;
}

}  // namespace sas
