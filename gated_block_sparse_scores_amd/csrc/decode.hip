// Single-token gated block-sparse decode, split-K with an LSE merge.
//
// picx.dev summary of SAS, 'Key Idea' Eq. 9 (one query row; log-gates on the
// selected history blocks, 0 on the current block) and 'Theoretical
// Foundation' Eq. 2 (the ungated form served at inference, logg == NULL);
// 'Efficiency Benefits': GQA with one selection per KV head group.
//
// Work split: the key list of (b, kv) is [valid selected blocks..., current
// block]; workgroup (b, kv, split) takes `bps` consecutive entries of it and
// serves all G query heads of kv from one read of each K/V row.  The partial
// (max, sum, unnormalised output) of every split goes to the workspace and the
// splits of each (b, h) are merged with log-sum-exp weights.
//  * bf16, head_dim 128, block 64 (decode_block4_kernel): four waves per
//    workgroup, each block shared by two waves (32 keys each) or, on small
//    grids, by four (sixteen keys each); two whole blocks per wave in the paged
//    decode on large grids; MFMA scores; the workgroup folds its waves'
//    partials in LDS into one.
//  * every other shape (decode_split_kernel): each key row is read by 16 lanes
//    with one vector load per lane, dot products reduced with DPP row
//    operations.
// A second kernel (decode_merge_kernel) merges the splits.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace sas {

namespace {

constexpr int kMaxG = 8;
constexpr int kMaxBps = 2;
constexpr int kMaxSplit = 65;  // K + 1 blocks at one block per split

// Valid length of sequence b (its own, clamped, in a ragged batch).
__device__ __forceinline__ int view_len(const KvView& kvv, int b, int L) {
  if (!kvv.seq_lens) return L;
  return min(max(kvv.seq_lens[b], 1), L);
}

// First row of logical block m of (b, kv) in the K or V cache, or nullptr when
// its page number is out of range (the block is then empty).
template <typename T>
__device__ __forceinline__ const T* view_block(const KvView& kvv, const void* base, int b,
                                               int kv, int hkv, int m, int BS, int D) {
  if (kvv.table) {
    const int page = kvv.table[(size_t)b * kvv.bt_ld + m];
    if (page < 0 || page >= kvv.num_pages) return nullptr;
    return (const T*)base + ((size_t)page * hkv + kv) * (size_t)BS * D;
  }
  return (const T*)base + (((size_t)b * hkv + kv) * kvv.cache_len + (size_t)m * BS) * D;
}

template <typename T, int N> struct VecLoad;
template <> struct VecLoad<bf16_t, 8> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct VecLoad<bf16_t, 4> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(u.x << 16);
    o[1] = __uint_as_float(u.x & 0xFFFF0000u);
    o[2] = __uint_as_float(u.y << 16);
    o[3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
};
template <> struct VecLoad<float, 8> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
template <> struct VecLoad<float, 4> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  }
};

// One lane's slice of a K or V row, kept in its storage format until used.
template <typename T, int N> struct RawSlice;
template <int N> struct RawSlice<bf16_t, N> {
  uint32_t w[N / 2];
  __device__ __forceinline__ void load(const bf16_t* p) {
    if constexpr (N == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = u.x; w[1] = u.y;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float get(int e) const {
    return __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
  }
};
template <int N> struct RawSlice<float, N> {
  float f[N];
  __device__ __forceinline__ void load(const float* p) { VecLoad<float, N>::load(p, f); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = 0.0f;
  }
  __device__ __forceinline__ float get(int e) const { return f[e]; }
};

// Sum over the 16 lanes of a DPP row (quad xor 1, quad xor 2, half-row
// mirror, row mirror): every lane of the row ends with the row's total.
__device__ __forceinline__ float row16_sum(float x) {
  auto dpp = [](float v, int ctrl) -> float {
    switch (ctrl) {
      case 0:
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
      case 1:
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
      case 2:
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
      default:
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
    }
  };
  x += dpp(x, 0);
  x += dpp(x, 1);
  x += dpp(x, 2);
  x += dpp(x, 3);
  return x;
}

template <typename T, int D, int BS>
__global__ void __launch_bounds__(256) decode_split_kernel(
    Dims dm, int Lmax, KvView kvv, int bps, int nsplit, const T* __restrict__ q,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, float* __restrict__ part_ml,
    float* __restrict__ part_acc) {
  constexpr int DPL = D / 16;                  // dims per lane (one vector load)
  constexpr int MAXKEYS = kMaxBps * BS;
  constexpr int KPT = MAXKEYS / 16;            // keys per thread (16 key groups)
  __shared__ float sc[kMaxG][MAXKEYS];
  __shared__ __align__(16) float red[4][kMaxG][D];
  __shared__ int blist[kMaxBps];
  __shared__ const T* bk_ptr[kMaxBps];  // first K row of each listed block
  __shared__ const T* bv_ptr[kMaxBps];
  __shared__ float bbias[kMaxBps];  // added to the logits (inner gating)
  __shared__ float bgain[kMaxBps];  // multiplies the values (outer gating)
  __shared__ float mx_sh[kMaxG], l_sh[kMaxG];
  __shared__ int nb_sh;

  const int split = blockIdx.x % nsplit;
  const int bk = blockIdx.x / nsplit;
  const int kv = bk % dm.hkv, b = bk / dm.hkv;
  const int G = dm.g;
  const int L = view_len(kvv, b, Lmax);
  const int c = (L - 1) / BS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid & 15, grp = tid >> 4;

  if (tid == 0) {
    // entries: the valid selected blocks (slot order), then the current block;
    // a block whose page is out of range is left out
    int pos = 0, nb = 0;
    const int first = split * bps, last = first + bps;
    for (int s = 0; s <= dm.K; ++s) {
      const int m = s < dm.K ? idx[(size_t)bk * dm.K + s] : c;
      if (s < dm.K && !(m >= 0 && m < c)) continue;
      const T* kp = view_block<T>(kvv, kvv.k, b, kv, dm.hkv, m, BS, D);
      const T* vp = view_block<T>(kvv, kvv.v, b, kv, dm.hkv, m, BS, D);
      if (!kp || !vp) continue;
      if (pos >= first && pos < last) {
        const float lg = (s < dm.K && logg) ? logg[(size_t)bk * dm.K + s] : 0.0f;
        blist[nb] = m;
        bk_ptr[nb] = kp;
        bv_ptr[nb] = vp;
        bbias[nb] = dm.outer ? 0.0f : lg;
        bgain[nb] = dm.outer ? expf(lg) : 1.0f;
        ++nb;
      }
      ++pos;
    }
    nb_sh = nb;
  }

  float qv[kMaxG][DPL];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      RawSlice<T, DPL> qs;
      qs.load(q + (((size_t)b * dm.hq + kv * G + h) * D) + sub * DPL);
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[h][e] = qs.get(e);
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[h][e] = 0.0f;
    }
  }
  __syncthreads();
  const int nkeys = nb_sh * BS;

  // Issue every K and V row load of this split before any arithmetic.
  RawSlice<T, DPL> kr[KPT], vr[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int kk = grp + 16 * i;
    const int pos = kk < nkeys ? blist[kk / BS] * BS + (kk % BS) : L;
    if (pos < L) {
      kr[i].load(bk_ptr[kk / BS] + (size_t)(kk % BS) * D + sub * DPL);
      vr[i].load(bv_ptr[kk / BS] + (size_t)(kk % BS) * D + sub * DPL);
    } else {
      kr[i].zero();
      vr[i].zero();
    }
  }

  // Phase A: scores of every key of this split for the G heads.
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int kk = grp + 16 * i;
    if (kk >= nkeys) break;  // uniform across each 16-lane row
    const int pos = blist[kk / BS] * BS + (kk % BS);
    const float bias = bbias[kk / BS];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) a += qv[h][e] * kr[i].get(e);
        a = row16_sum(a);
        if (sub == 0) sc[h][kk] = pos < L ? a * dm.scale + bias : -INFINITY;
      }
    }
  }
  __syncthreads();

  // Phase B: per-head max and sum over this split; sc[] becomes exp(z - max).
  for (int h = wave; h < G; h += 4) {
    float mx = -INFINITY;
    for (int kk = lane; kk < nkeys; kk += 64) mx = fmaxf(mx, sc[h][kk]);
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int kk = lane; kk < nkeys; kk += 64) {
      const float z = sc[h][kk];
      const float pz = z == -INFINITY ? 0.0f : expf(z - mx);
      sc[h][kk] = pz;
      sum += pz;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      mx_sh[h] = mx;
      l_sh[h] = sum;
    }
  }
  __syncthreads();

  // Phase C: unnormalised P V.
  float acc[kMaxG][DPL];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.0f;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int kk = grp + 16 * i;
    if (kk < nkeys) {
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
          const float pz = sc[h][kk] * bgain[kk / BS];
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[h][e] += pz * vr[i].get(e);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      if (h < G) {
        float a = acc[h][e];
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        acc[h][e] = a;
      }
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < kMaxG; ++h)
      if (h < G)
#pragma unroll
        for (int e = 0; e < DPL; ++e) red[wave][h][sub * DPL + e] = acc[h][e];
  }
  __syncthreads();
  const size_t prow = (size_t)b * dm.hq + (size_t)kv * G;
  for (int x = tid; x < G * D; x += blockDim.x) {
    const int h = x / D, dd = x % D;
    const float a = red[0][h][dd] + red[1][h][dd] + red[2][h][dd] + red[3][h][dd];
    part_acc[((prow + h) * nsplit + split) * D + dd] = a;
  }
  if (tid < G) {
    part_ml[((prow + tid) * nsplit + split) * 2 + 0] = mx_sh[tid];
    part_ml[((prow + tid) * nsplit + split) * 2 + 1] = l_sh[tid];
  }
}

// Merge, one wave per (b, h): weights w_s = e^{m_s - M} (0 for empty splits),
// o = sum_s w_s acc_s / sum_s w_s l_s, lse = M + log(sum_s w_s l_s).
template <typename T>
__global__ void __launch_bounds__(64) decode_merge_kernel(int nsplit, int D,
                                                          const float* __restrict__ part_ml,
                                                          const float* __restrict__ part_acc,
                                                          T* __restrict__ o,
                                                          float* __restrict__ lse) {
  __shared__ float w[kMaxSplit];
  const size_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const float* ml = part_ml + row * nsplit * 2;
  float M = -INFINITY;
  for (int s = lane; s < nsplit; s += 64) M = fmaxf(M, ml[2 * s]);
  M = wave_max(M);
  float Ls = 0.0f;
  for (int s = lane; s < nsplit; s += 64) {
    const float l = ml[2 * s + 1];
    const float ws = l > 0.0f ? expf(ml[2 * s] - M) : 0.0f;
    w[s] = ws;
    Ls += ws * l;
  }
  Ls = wave_sum(Ls);
  __syncthreads();
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;  // no key at all: o = 0, lse = -inf
  const float* acc = part_acc + row * nsplit * D;
  for (int dd = lane; dd < D; dd += 64) {
    // the splits' loads go out sixteen (then eight) at a time: one memory round
    // trip per batch, the batch's terms spread over independent partial sums
    float a[16] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    int s = 0;
    for (; s + 16 <= nsplit; s += 16) {
#pragma unroll
      for (int u = 0; u < 16; ++u) a[u] += w[s + u] * acc[(size_t)(s + u) * D + dd];
    }
    for (; s + 8 <= nsplit; s += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += w[s + u] * acc[(size_t)(s + u) * D + dd];
    }
    for (; s < nsplit; ++s) a[0] += w[s] * acc[(size_t)s * D + dd];
    const float tot = (((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]))) +
                      (((a[8] + a[9]) + (a[10] + a[11])) + ((a[12] + a[13]) + (a[14] + a[15])));
    Elem<T>::store(o, row * D + dd, tot * inv);
  }
  if (lane == 0) lse[row] = Ls > 0.0f ? M + logf(Ls) : -INFINITY;
}

// ---------------------------------------------------------------- bf16, d 128, block 64
// One wave per selected block (64 keys).  Scores S[h][key] = q_h . k_key come
// from v_mfma_f32_16x16x32_bf16 with A = the G query heads (rows, zero-padded
// to 16) and B = K^T: lane l loads 8 consecutive dims (16 B) of key l % 16 of
// each 16-key tile, so a load instruction covers 64 contiguous bytes of 16
// rows, and the result lands with one key per lane column and four heads per
// lane -- no cross-lane dot-product reductions.  The per-head max and sum over
// the block's 64 keys use DPP within 16-lane rows.  P goes to LDS as
// [key][head]; for P V every lane owns two dims of every V row, so each V row
// is one 256-byte coalesced wave load and no cross-lane reduction is needed.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true)));
  return x;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// kDecWaves waves per workgroup, kBpw selected blocks per wave taken one
// after the other (2 for the paged decode and the fused steps on grids that
// then still fill every CU twice); the workgroup folds its blocks into one
// partial in LDS, so the merge kernel reads a fraction of the partials it would
// read at one block per workgroup.  (Merging in the last
// workgroup to finish would need a device-scope fence per workgroup, which on
// this multi-die part writes back the L2 and costs far more than the second
// launch.)
// With SEL the block list is not read from idx / logg but formed here from the
// long-history selection's chunk candidates (SelectChunks): every workgroup of
// a (b, kv) folds the sorted candidate lists of its row into the top K (the
// wave-level merges the selection merge kernel uses), orders the winners by block
// index and takes the entries it serves; workgroup 0 of each (b, kv) also
// stores idx, logg and lse_s for the caller.
struct SelectChunks {
  const uint64_t* cand;  // [b*hkv][nchunk][K] descending composite keys
  const float2* stats;   // [b*hkv][nchunk] (max, sum of exp) of the chunk's scores
  int nchunk, C, gated, act;
  int32_t* idx_out;  // optional [b*hkv][K]
  float* logg_out;   // optional [b*hkv][K]
  float* lse_out;    // optional [b*hkv]
};

// kKW keys per wave: 64 (a whole block per wave), or fewer with 64 / kKW
// waves of a workgroup sharing one block (wave w takes keys
// (w % (64 / kKW)) kKW .. + kKW - 1), which puts more waves on a small grid
// (their partials are folded in LDS like those of separate blocks).
template <int G, int kDecWaves, bool SEL, int kBpw, int kKW = 64>
__global__ void __launch_bounds__(64 * kDecWaves) decode_block4_kernel(
    Dims dm, int Lmax, KvView kvv, int nsplit, const bf16_t* __restrict__ q,
    const int32_t* __restrict__ idx, const float* __restrict__ logg,
    float* __restrict__ part_ml, float* __restrict__ part_acc, SelectChunks sel) {
  constexpr int D = 128, BS = 64;
  constexpr int GP = G <= 4 ? 4 : 8;          // heads per LDS row (padded)
  constexpr bool kShared = kKW < BS;          // waves share blocks
  constexpr int WPB = BS / kKW;                // waves per block
  static_assert(kKW == BS || (kDecWaves % WPB == 0 && kBpw == 1), "block split over waves");
  constexpr int NKT = kKW / 16;               // 16-key tiles per wave
  __shared__ __align__(16) uint32_t Pb[kDecWaves][kKW / 2][GP];  // bf16 pairs (keys 2i, 2i+1)
  __shared__ __align__(16) float wacc[kDecWaves * kBpw][G][D];  // one partial per block
  __shared__ float wml[kDecWaves * kBpw][G][2];
  __shared__ int sidx[64];
  __shared__ float slg[64];
  const int split = blockIdx.x % nsplit;
  const int bk = blockIdx.x / nsplit;
  const int kv = bk % dm.hkv, b = bk / dm.hkv;
  const int L = view_len(kvv, b, Lmax);
  const int c = (L - 1) / BS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t prow = (size_t)b * dm.hq + (size_t)kv * G;
  const int hbase = (lane >> 4) * 4;

  // Entries: [valid selected blocks (slot order)..., current block].  The
  // workgroup takes kDecWaves * kBpw consecutive entries, wave w the kBpw
  // entries from (split * kDecWaves + w) * kBpw, one after the other; with
  // kShared wave w takes entry split * kDecWaves / WPB + w / WPB.
  int nvalid = 0;  // valid selected blocks of the row (the current block follows)
  int mm = -1;     // given idx: the row's entry `lane`
  unsigned long long bal = 0;
  if constexpr (SEL) {
    extern __shared__ uint64_t lists[];  // nchunk * K keys
    const int K = dm.K, nc = sel.nchunk * K;
    const int tid = threadIdx.x, nth = 64 * kDecWaves;
    const uint64_t* crow = sel.cand + (size_t)bk * nc;
    // Small grids (512K: 992 keys per row) copy with every load of a thread in
    // flight at once; the larger tilings keep the plain loop (measured: the
    // unrolled copy made the 8x64K split kernel 0.5 us slower, 0.4 us faster
    // at 512K).
    if constexpr (kKW == 16) {
      copy_keys_to_lds<8>(lists, crow, nc, tid, nth);
    } else {
      for (int i = tid; i < nc; i += nth) lists[i] = crow[i];
    }
    // lse_s from the chunk statistics (nchunk <= 64: lane i holds chunk i's max
    // and sum of exp), combined by the last wave once its folds are done, while
    // wave 0 folds the waves' lists; the selection merge kernel's arithmetic
    // (fp32 max, fp64 sum of the chunk sums rescaled to it, one fp32 rounding
    // of max + log(sum)).  It reaches wave 0 through LDS at the next barrier.
    __shared__ float lse_sh;
    float2 cst = make_float2(-INFINITY, 0.0f);
    if (wave == kDecWaves - 1 && lane < sel.nchunk)
      cst = sel.stats[(size_t)bk * sel.nchunk + lane];
    __syncthreads();  // lists[] complete
    const int Crow = kvv.seq_lens ? min(sel.C, c) : sel.C;  // this sequence's history
    // wave-level folds of the chunk lists in registers (K <= 64)
    __shared__ uint64_t wl[kDecWaves * 64];
    const uint64_t top = merge_top64<kDecWaves>(lists, sel.nchunk, K, wl);
    if (wave == kDecWaves - 1) {
      const float M = wave_max(cst.x);
      const double S =
          wave_sum_d(cst.y > 0.0f ? (double)cst.y * exp((double)cst.x - (double)M) : 0.0);
      if (lane == 0) lse_sh = Crow > 0 ? (float)((double)M + log(S)) : -INFINITY;
    }
    const int kk = min(K, Crow);
    // wave 0 holds the winners by rank and re-sorts them by block index in
    // registers (key: block index, then the score's order key)
    uint64_t byidx = ~0ull;
    if (wave == 0) {
      if (lane < kk)
        byidx = ((uint64_t)(0xFFFFFFFFu - (uint32_t)(top & 0xFFFFFFFFull)) << 32) | (top >> 32);
      byidx = bitonic_sort_asc64(byidx, lane);
    }
    __syncthreads();  // lse_sh in LDS
    const float lse_s = lse_sh;
    if (wave == 0 && lane < kk) {
      const int mine = (int)(byidx >> 32);
      const float lg = gate_log(from_order_key((uint32_t)byidx), lse_s, sel.act);
      sidx[lane] = mine;
      slg[lane] = lg;
      if (split == 0 && sel.idx_out) {
        sel.idx_out[(size_t)bk * K + lane] = mine;
        sel.logg_out[(size_t)bk * K + lane] = lg;
      }
    }
    if (split == 0 && sel.idx_out) {
      for (int p2 = kk + tid; p2 < K; p2 += nth) {
        sel.idx_out[(size_t)bk * K + p2] = -1;
        sel.logg_out[(size_t)bk * K + p2] = 0.0f;
      }
      if (tid == 0) sel.lse_out[bk] = lse_s;
    }
    __syncthreads();
    nvalid = kk;
  } else {
    mm = lane < dm.K ? idx[(size_t)bk * dm.K + lane] : -1;
    bal = __ballot(mm >= 0 && mm < c);
    nvalid = __popcll(bal);
  }
#pragma unroll 1
  for (int e = 0; e < kBpw; ++e) {
  const int j =
      kShared ? (split * kDecWaves + wave) / WPB : (split * kDecWaves + wave) * kBpw + e;
  int m = -1;
  float bias = 0.0f;
  if (j < nvalid) {
    if constexpr (SEL) {
      m = sidx[j];
      bias = sel.gated ? slg[j] : 0.0f;
    } else {
      const bool ok = mm >= 0 && mm < c;
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      const unsigned long long hit = __ballot(ok && before == j);
      const int src = __ffsll((long long)hit) - 1;
      m = __shfl(mm, src);
      bias = logg ? logg[(size_t)bk * dm.K + src] : 0.0f;
    }
  } else if (j == nvalid) {
    m = c;
  }
  // The block's rows (a block on an out-of-range page is skipped).
  const bf16_t* kblk = nullptr;
  const bf16_t* vblk = nullptr;
  if (m >= 0) {
    kblk = view_block<bf16_t>(kvv, kvv.k, b, kv, dm.hkv, m, BS, D);
    vblk = view_block<bf16_t>(kvv, kvv.v, b, kv, dm.hkv, m, BS, D);
    if (!kblk || !vblk) m = -1;
  }
  // kShared: this wave's keys of the block; all of them past the sequence's end
  // (current block only) leave the wave's entry empty.
  const int koff = kShared ? (wave % WPB) * kKW : 0;
  if (kShared && m >= 0) {
    if (m * BS + koff > L - 1) {
      m = -1;
    } else {
      kblk += (size_t)koff * D;
      vblk += (size_t)koff * D;
    }
  }
  // Outer gating: the logits carry no bias and the block's P V is scaled by g.
  float gain = 1.0f;
  if (dm.outer) {
    gain = expf(bias);
    bias = 0.0f;
  }
  float mh[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float lh[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = 0.0f;
  if (m >= 0) {
    const int pos0 = m * BS + koff;  // position of the wave's first key
    const int last = L - 1;  // rows past it (current block only) are read clamped, then masked

    // Loads: K in MFMA B layout, V one row per wave instruction, q as A operand.
    // With one block per wave the V loads are issued after the score products
    // instead, into the registers K held: 30 fewer registers, and V's latency
    // overlaps the softmax (measured with whole blocks per wave: separate
    // decode 6% faster at 8x64K and 8% at 512K, fused step 2% at 512K).  With
    // two blocks per wave it was slower.
    constexpr bool kLateV = kBpw == 1;
    bf16x8_t kf[NKT][4];
    uint32_t vr[kKW];
    auto load_v = [&]() {
      if (pos0 + kKW <= L) {
        const bf16_t* vrow = vblk + 2 * lane;
#pragma unroll
        for (int r = 0; r < kKW; ++r) vr[r] = *reinterpret_cast<const uint32_t*>(vrow + r * D);
      } else {  // rows past L - 1 are read clamped, then masked
#pragma unroll
        for (int r = 0; r < kKW; ++r)
          vr[r] = *reinterpret_cast<const uint32_t*>(vblk + (size_t)min(r, last - pos0) * D +
                                                     2 * lane);
      }
    };
    if constexpr (kLateV) {
      if (pos0 + kKW <= L) {
        const bf16_t* krow = kblk + (size_t)(lane & 15) * D + (lane >> 4) * 8;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int ch = 0; ch < 4; ++ch)
            kf[kt][ch] = *reinterpret_cast<const bf16x8_t*>(krow + kt * 16 * D + ch * 32);
      } else {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const int rr = min(kt * 16 + (lane & 15), last - pos0);
#pragma unroll
          for (int ch = 0; ch < 4; ++ch)
            kf[kt][ch] = *reinterpret_cast<const bf16x8_t*>(kblk + (size_t)rr * D + ch * 32 +
                                                            (lane >> 4) * 8);
        }
      }
    } else {
      if (pos0 + kKW <= L) {  // full block (every history block): plain offsets
        const bf16_t* krow = kblk + (size_t)(lane & 15) * D + (lane >> 4) * 8;
        const bf16_t* vrow = vblk + 2 * lane;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int ch = 0; ch < 4; ++ch)
            kf[kt][ch] = *reinterpret_cast<const bf16x8_t*>(krow + kt * 16 * D + ch * 32);
#pragma unroll
        for (int r = 0; r < kKW; ++r) vr[r] = *reinterpret_cast<const uint32_t*>(vrow + r * D);
      } else {  // the current block: rows past L - 1 are read clamped, then masked
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const int rr = min(kt * 16 + (lane & 15), last - pos0);
#pragma unroll
          for (int ch = 0; ch < 4; ++ch)
            kf[kt][ch] = *reinterpret_cast<const bf16x8_t*>(kblk + (size_t)rr * D + ch * 32 +
                                                            (lane >> 4) * 8);
        }
#pragma unroll
        for (int r = 0; r < kKW; ++r)
          vr[r] = *reinterpret_cast<const uint32_t*>(vblk + (size_t)min(r, last - pos0) * D +
                                                     2 * lane);
      }
    }
    bf16x8_t qf[4];
    {
      const int h = lane & 15;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        qf[ch] = h < G ? *reinterpret_cast<const bf16x8_t*>(q + (prow + h) * D + ch * 32 +
                                                            (lane >> 4) * 8)
                       : bf16x8_t{};
    }

    // S[h][key]: lane holds key kt*16 + lane%16, heads 4*(lane/16) + r.
    f32x4_t sacc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      sacc[kt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ch], kf[kt][ch], sacc[kt], 0, 0, 0);
    }
    if constexpr (kLateV) {
      __builtin_amdgcn_sched_barrier(0);  // the V loads stay after the score products
      load_v();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const int pos = pos0 + kt * 16 + (lane & 15);
        const float z = pos < L ? sacc[kt][r] * dm.scale + bias : -INFINITY;
        sacc[kt][r] = z;
        mx = fmaxf(mx, z);
      }
      mx = row16_max(mx);
      float sm = 0.0f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const float pz = expf(sacc[kt][r] - mx);  // exp(-inf) = 0 for masked keys
        sacc[kt][r] = pz;
        sm += pz;
      }
      mh[r] = mx;
      lh[r] = row16_sum(sm);
    }
    // P as bf16 pairs of consecutive keys: the even lane of each pair writes.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = hbase + r;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const float mine = sacc[kt][r];
        const float nb = __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(mine), 0xB1, 0xF, 0xF, true));
        if (h < G && (lane & 1) == 0)
          Pb[wave][(kt * 16 + (lane & 15)) >> 1][h] = pack_bf16x2(mine, nb);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's own P is in LDS
#pragma unroll
    for (int kp = 0; kp < kKW / 2; ++kp) {
      const uint32_t v0 = vr[2 * kp], v1 = vr[2 * kp + 1];
      const bf16x2_t vlo =
          __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(v1, v0, 0x05040100u));
      const bf16x2_t vhi =
          __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(v1, v0, 0x07060302u));
      uint32_t pw[GP];
      *reinterpret_cast<uint4*>(&pw[0]) = *reinterpret_cast<const uint4*>(&Pb[wave][kp][0]);
      if constexpr (GP == 8)
        *reinterpret_cast<uint4*>(&pw[4]) = *reinterpret_cast<const uint4*>(&Pb[wave][kp][4]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bf16x2_t ph = __builtin_bit_cast(bf16x2_t, pw[h]);
        acc[h][0] = __builtin_amdgcn_fdot2_f32_bf16(ph, vlo, acc[h][0], false);
        acc[h][1] = __builtin_amdgcn_fdot2_f32_bf16(ph, vhi, acc[h][1], false);
      }
    }
  }
  // The block's partial into LDS (an empty entry contributes max -inf, sum 0).
  const int slot = wave * kBpw + e;
#pragma unroll
  for (int h = 0; h < G; ++h)
    *reinterpret_cast<float2*>(&wacc[slot][h][2 * lane]) =
        make_float2(acc[h][0] * gain, acc[h][1] * gain);
  if ((lane & 15) == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = hbase + r;
      if (h < G) {
        wml[slot][h][0] = mh[r];
        wml[slot][h][1] = lh[r];
      }
    }
  }
  }  // entries of this wave
  __syncthreads();
  constexpr int nslot = kDecWaves * kBpw;

  // Fold the workgroup's blocks: wave w takes heads w, w + kDecWaves, ...;
  // weights e^{m - M}, 0 for empty blocks.
  for (int h = wave; h < G; h += kDecWaves) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < nslot; ++w) M = fmaxf(M, wml[w][h][0]);
    float Ls = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int w = 0; w < nslot; ++w) {
      const float l = wml[w][h][1];
      const float wt = l > 0.0f ? expf(wml[w][h][0] - M) : 0.0f;
      Ls += wt * l;
      const float2 av = *reinterpret_cast<const float2*>(&wacc[w][h][2 * lane]);
      a0 += wt * av.x;
      a1 += wt * av.y;
    }
    const size_t pr = (prow + h) * nsplit + split;
    *reinterpret_cast<float2*>(&part_acc[pr * D + 2 * lane]) = make_float2(a0, a1);
    if (lane == 0) *reinterpret_cast<float2*>(&part_ml[pr * 2]) = make_float2(M, Ls);
  }
}

// bps entries per workgroup of four waves: 8 (two blocks per wave), 2 (two
// blocks, 32 keys per wave) or 1 (one block, sixteen keys per wave).
template <int G, bool SEL>
void launch_decode_block4(const Dims& dm, int L, const KvView& kvv, int nsplit, int bps,
                          const void* q, const int32_t* idx, const float* logg, float* part_ml,
                          float* part_acc, const SelectChunks& sel, hipStream_t st) {
  const size_t wgs = (size_t)dm.b * dm.hkv * nsplit;
  const size_t lds = SEL ? (size_t)sel.nchunk * dm.K * sizeof(uint64_t) : 0;
  if (bps == 8)
    hipLaunchKernelGGL((decode_block4_kernel<G, 4, SEL, 2>), dim3((unsigned)wgs), dim3(256), lds,
                       st, dm, L, kvv, nsplit, (const bf16_t*)q, idx, logg, part_ml, part_acc,
                       sel);
  else if (bps == 2)
    hipLaunchKernelGGL((decode_block4_kernel<G, 4, SEL, 1, 32>), dim3((unsigned)wgs), dim3(256),
                       lds, st, dm, L, kvv, nsplit, (const bf16_t*)q, idx, logg, part_ml,
                       part_acc, sel);
  else
    hipLaunchKernelGGL((decode_block4_kernel<G, 4, SEL, 1, 16>), dim3((unsigned)wgs), dim3(256),
                       lds, st, dm, L, kvv, nsplit, (const bf16_t*)q, idx, logg, part_ml,
                       part_acc, sel);
}

// Workspace: [partials (max, sum) per (b, h, split)][partial outputs per
// (b, h, split, d)].
template <typename T, int D, int BS>
hipError_t decode_typed(const Dims& dm, int L, const KvView& kvv, const void* q,
                        const int32_t* idx, const float* logg, void* o, float* lse, void* ws,
                        hipStream_t st) {
  const int bps = kvv.table && decode_two_per_wave(dm) ? 8 : decode_blocks_per_split(dm);
  const int nsplit = (dm.K + 1 + bps - 1) / bps;
  float* part_ml = (float*)ws;
  float* part_acc = part_ml + (size_t)dm.b * dm.hq * nsplit * 2;
  {
    ProfScope ps("decode_split", st);
    if constexpr (std::is_same<T, bf16_t>::value && D == 128 && BS == 64) {
#define SAS_DEC_G(G_)                                                                     \
  case G_:                                                                                \
    launch_decode_block4<G_, false>(dm, L, kvv, nsplit, bps, q, idx, logg, part_ml,       \
                                    part_acc, SelectChunks{}, st);                        \
    break;
      switch (dm.g) {
        SAS_DEC_G(1) SAS_DEC_G(2) SAS_DEC_G(3) SAS_DEC_G(4)
        SAS_DEC_G(5) SAS_DEC_G(6) SAS_DEC_G(7) SAS_DEC_G(8)
        default: return hipErrorInvalidValue;
      }
#undef SAS_DEC_G
    } else {
      const size_t wgs = (size_t)dm.b * dm.hkv * nsplit;
      hipLaunchKernelGGL((decode_split_kernel<T, D, BS>), dim3((unsigned)wgs), dim3(256), 0, st,
                         dm, L, kvv, bps, nsplit, (const T*)q, idx, logg, part_ml, part_acc);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps("decode_merge", st);
  hipLaunchKernelGGL((decode_merge_kernel<T>), dim3((unsigned)(dm.b * dm.hq)), dim3(64), 0, st,
                     nsplit, D, part_ml, part_acc, (T*)o, lse);
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_path(const Dims& dm) { return dm.bf16 && dm.d == 128 && dm.bs == 64; }

// Four waves of two blocks each per workgroup (MFMA path): when that still
// fills every CU with two workgroups, the grid runs in one round, each wave's
// second block loading after its first is folded.  Measured faster for the
// paged decode and the paged fused step (measured against one block per wave);
// the dense separate decode and the dense fused step share each block between
// two waves, whose V loads wait until after the score products.
bool decode_two_per_wave(const Dims& dm) {
  return decode_mfma_path(dm) && (long)dm.b * dm.hkv * ((dm.K + 8) / 8) >= 512;
}

int decode_blocks_per_split(const Dims& dm) {
  // MFMA path, four waves per workgroup: two blocks, 32 keys per wave, when
  // four blocks per workgroup would still leave two workgroups per CU, else one
  // block of sixteen keys per wave (measured against one block per wave: split
  // kernel 33.5 -> 31.9 us at 8x64K, 10.6 -> 8.8 us at 512K; sixteen keys per
  // wave at 8x64K shortened the split kernel less than the 64 splits lengthened
  // the merge).  The workspace is sized for this split count, which is at least
  // that of two blocks per wave.
  if (decode_mfma_path(dm))
    return (long)dm.b * dm.hkv * ((dm.K + 4) / 4) >= 512 ? 2 : 1;
  const long total = (long)dm.b * dm.hkv * (dm.K + 1);
  return total >= 2048 ? 2 : 1;
}

size_t decode_workspace_bytes(const Dims& dm) {
  const int bps = decode_blocks_per_split(dm);
  const int nsplit = (dm.K + 1 + bps - 1) / bps;
  return (size_t)dm.b * dm.hq * nsplit * (2 + dm.d) * sizeof(float);
}

hipError_t launch_decode(const Dims& dm, int L, const KvView& kvv, const void* q,
                         const int32_t* idx, const float* logg, void* o, float* lse, void* ws,
                         hipStream_t st) {
#define SAS_DEC(T_, D_, BS_)                                                            \
  if ((dm.bf16 == std::is_same<T_, bf16_t>::value) && dm.d == D_ && dm.bs == BS_)    \
    return decode_typed<T_, D_, BS_>(dm, L, kvv, q, idx, logg, o, lse, ws, st);
  SAS_DEC(float, 64, 16) SAS_DEC(float, 64, 32) SAS_DEC(float, 64, 64)
  SAS_DEC(float, 128, 16) SAS_DEC(float, 128, 32) SAS_DEC(float, 128, 64)
  SAS_DEC(bf16_t, 64, 16) SAS_DEC(bf16_t, 64, 32) SAS_DEC(bf16_t, 64, 64)
  SAS_DEC(bf16_t, 128, 16) SAS_DEC(bf16_t, 128, 32) SAS_DEC(bf16_t, 128, 64)
#undef SAS_DEC
  return hipErrorInvalidValue;
}

size_t decode_step_partial_bytes(const Dims& dm) { return decode_workspace_bytes(dm); }

hipError_t launch_decode_step(const Dims& dm, int L, const KvView& kvv, int C, int nchunk,
                              const void* q, const uint64_t* cand, const float2* stats,
                              bool gated, int32_t* idx_out, float* logg_out, float* lse_s_out,
                              void* o, float* lse, void* ws, hipStream_t st) {
  if (!decode_mfma_path(dm)) return hipErrorInvalidValue;
  // Entries split as in the separate decode: every workgroup (four waves)
  // merges the row's chunk candidates first, then serves its entries.  Two
  // waves per block, or four on small grids, put two or four times as many
  // workgroups on the chip as one wave per block (measured: fused split kernel
  // 36.2 -> 34.6 us at 8x64K, 16.5 -> 12.8 us at 512K).
  const int bps = kvv.table && decode_two_per_wave(dm) ? 8 : decode_blocks_per_split(dm);
  const int nsplit = (dm.K + 1 + bps - 1) / bps;
  float* part_ml = (float*)ws;
  float* part_acc = part_ml + (size_t)dm.b * dm.hq * nsplit * 2;
  const SelectChunks sel{cand,         stats,   nchunk,   C,        gated ? 1 : 0,
                         dm.act,       idx_out, logg_out, lse_s_out};
  {
    ProfScope ps("step_decode_split", st);
#define SAS_DEC_G(G_)                                                                          \
  case G_:                                                                                     \
    launch_decode_block4<G_, true>(dm, L, kvv, nsplit, bps, q, nullptr, nullptr, part_ml,      \
                                   part_acc, sel, st);                                         \
    break;
    switch (dm.g) {
      SAS_DEC_G(1) SAS_DEC_G(2) SAS_DEC_G(3) SAS_DEC_G(4)
      SAS_DEC_G(5) SAS_DEC_G(6) SAS_DEC_G(7) SAS_DEC_G(8)
      default: return hipErrorInvalidValue;
    }
#undef SAS_DEC_G
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps("step_decode_merge", st);
  hipLaunchKernelGGL((decode_merge_kernel<bf16_t>), dim3((unsigned)(dm.b * dm.hq)), dim3(64), 0,
                     st, nsplit, 128, part_ml, part_acc, (bf16_t*)o, lse);
  return hipGetLastError();
}

}  // namespace sas
