// Single-token gated block-sparse decode, split-K with an LSE merge.
//
// picx.dev summary of SAS, 'Key Idea' Eq. 9 (one query row; log-gates on the
// selected history blocks, 0 on the current block) and 'Theoretical
// Foundation' Eq. 2 (the ungated form served at inference, logg == NULL);
// 'Efficiency Benefits': GQA with one selection per KV head group.
//
// Work split: the key list of (b, kv) is [valid selected blocks..., current
// block]; workgroup (b, kv, split) takes `bps` consecutive entries of it and
// serves all G query heads of kv from one read of each K/V row.  Each key row
// (head_dim values) is read by 16 lanes with one vector load per lane, so a
// wave reads 4 rows per instruction, fully coalesced.  The partial (max, sum,
// unnormalised output) of every split goes to the workspace; a second kernel
// merges the splits of each (b, h) with log-sum-exp weights.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace sas {

namespace {

constexpr int kMaxG = 8;
constexpr int kMaxBps = 4;

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

template <typename T, int D, int BS>
__global__ void __launch_bounds__(256) decode_split_kernel(
    Dims dm, int L, int cache_len, int bps, int nsplit, const T* __restrict__ q,
    const T* __restrict__ kc, const T* __restrict__ vc, const int32_t* __restrict__ idx,
    const float* __restrict__ logg, float* __restrict__ part_ml, float* __restrict__ part_acc) {
  constexpr int DPL = D / 16;
  constexpr int MAXKEYS = kMaxBps * BS;
  __shared__ float sc[kMaxG][MAXKEYS];
  __shared__ __align__(16) float red[4][kMaxG][D];
  __shared__ int blist[kMaxBps];
  __shared__ float bbias[kMaxBps];
  __shared__ float mx_sh[kMaxG], l_sh[kMaxG];
  __shared__ int nb_sh;

  const int split = blockIdx.x % nsplit;
  const int bk = blockIdx.x / nsplit;
  const int kv = bk % dm.hkv, b = bk / dm.hkv;
  const int G = dm.g;
  const int c = (L - 1) / BS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid & 15, grp = tid >> 4;

  if (tid == 0) {
    int pos = 0, nb = 0;
    const int first = split * bps, last = first + bps;
    for (int s = 0; s < dm.K; ++s) {
      const int m = idx[(size_t)bk * dm.K + s];
      if (m >= 0 && m < c) {
        if (pos >= first && pos < last) {
          blist[nb] = m;
          bbias[nb] = logg ? logg[(size_t)bk * dm.K + s] : 0.0f;
          ++nb;
        }
        ++pos;
      }
    }
    if (pos >= first && pos < last) {
      blist[nb] = c;
      bbias[nb] = 0.0f;
      ++nb;
    }
    nb_sh = nb;
  }

  float qv[kMaxG][DPL];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      const T* qp = q + (((size_t)b * dm.hq + kv * G + h) * D) + sub * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[h][e] = Elem<T>::load(qp, e);
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[h][e] = 0.0f;
    }
  }
  __syncthreads();
  const int nkeys = nb_sh * BS;
  const size_t kvbase = ((size_t)b * dm.hkv + kv) * (size_t)cache_len * D;

  // Phase A: scores of every key of this split for the G heads.
  for (int kk = grp; kk < nkeys; kk += 16) {
    const int bi = kk / BS;
    const int pos = blist[bi] * BS + (kk % BS);
    const bool valid = pos < L;
    float kr[DPL];
    if (valid)
      VecLoad<T, DPL>::load(kc + kvbase + (size_t)pos * D + sub * DPL, kr);
    else
#pragma unroll
      for (int e = 0; e < DPL; ++e) kr[e] = 0.0f;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) a += qv[h][e] * kr[e];
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) a += __shfl_xor(a, o);
      if (sub == 0 && h < G) sc[h][kk] = valid ? a * dm.scale + bbias[bi] : -INFINITY;
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
  for (int kk = grp; kk < nkeys; kk += 16) {
    const int bi = kk / BS;
    const int pos = blist[bi] * BS + (kk % BS);
    if (pos < L) {
      float vr[DPL];
      VecLoad<T, DPL>::load(vc + kvbase + (size_t)pos * D + sub * DPL, vr);
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
          const float pz = sc[h][kk];
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[h][e] += pz * vr[e];
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      float a = acc[h][e];
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[h][e] = a;
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

// Merge: o = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s, lse = M + log(...).
template <typename T>
__global__ void __launch_bounds__(128) decode_merge_kernel(int nsplit, int D,
                                                           const float* __restrict__ part_ml,
                                                           const float* __restrict__ part_acc,
                                                           T* __restrict__ o,
                                                           float* __restrict__ lse) {
  const size_t row = blockIdx.x;
  const float* ml = part_ml + row * nsplit * 2;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float Lsum = 0.0f;
  for (int s = 0; s < nsplit; ++s)
    if (ml[2 * s + 1] > 0.0f) Lsum += ml[2 * s + 1] * expf(ml[2 * s] - M);
  for (int dd = threadIdx.x; dd < D; dd += blockDim.x) {
    float a = 0.0f;
    for (int s = 0; s < nsplit; ++s)
      if (ml[2 * s + 1] > 0.0f) a += part_acc[(row * nsplit + s) * D + dd] * expf(ml[2 * s] - M);
    Elem<T>::store(o, row * D + dd, a / Lsum);
  }
  if (threadIdx.x == 0) lse[row] = M + logf(Lsum);
}

template <typename T, int D, int BS>
hipError_t decode_typed(const Dims& dm, int L, int cache_len, const void* q, const void* kc,
                        const void* vc, const int32_t* idx, const float* logg, void* o,
                        float* lse, void* ws, hipStream_t st) {
  const int bps = decode_blocks_per_split(dm);
  const int nsplit = (dm.K + 1 + bps - 1) / bps;
  float* part_ml = (float*)ws;
  float* part_acc = part_ml + (size_t)dm.b * dm.hq * nsplit * 2;
  {
    ProfScope ps("decode_split", st);
    const size_t wgs = (size_t)dm.b * dm.hkv * nsplit;
    hipLaunchKernelGGL((decode_split_kernel<T, D, BS>), dim3((unsigned)wgs), dim3(256), 0, st,
                       dm, L, cache_len, bps, nsplit, (const T*)q, (const T*)kc, (const T*)vc,
                       idx, logg, part_ml, part_acc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("decode_merge", st);
    hipLaunchKernelGGL((decode_merge_kernel<T>), dim3((unsigned)(dm.b * dm.hq)), dim3(128), 0,
                       st, nsplit, D, part_ml, part_acc, (T*)o, lse);
  }
  return hipGetLastError();
}

}  // namespace

int decode_blocks_per_split(const Dims& dm) {
  const long total = (long)dm.b * dm.hkv * (dm.K + 1);
  return total >= 2048 ? 2 : 1;
}

size_t decode_workspace_bytes(const Dims& dm) {
  const int bps = decode_blocks_per_split(dm);
  const int nsplit = (dm.K + 1 + bps - 1) / bps;
  return (size_t)dm.b * dm.hq * nsplit * (2 + dm.d) * sizeof(float);
}

hipError_t launch_decode(const Dims& dm, int L, int cache_len, const void* q, const void* kc,
                         const void* vc, const int32_t* idx, const float* logg, void* o,
                         float* lse, void* ws, hipStream_t st) {
#define SAS_DEC(T_, D_, BS_)                                                            \
  if ((dm.bf16 == std::is_same<T_, bf16_t>::value) && dm.d == D_ && dm.bs == BS_)    \
    return decode_typed<T_, D_, BS_>(dm, L, cache_len, q, kc, vc, idx, logg, o, lse, ws, st);
  SAS_DEC(float, 64, 16) SAS_DEC(float, 64, 32) SAS_DEC(float, 64, 64)
  SAS_DEC(float, 128, 16) SAS_DEC(float, 128, 32) SAS_DEC(float, 128, 64)
  SAS_DEC(bf16_t, 64, 16) SAS_DEC(bf16_t, 64, 32) SAS_DEC(bf16_t, 64, 64)
  SAS_DEC(bf16_t, 128, 16) SAS_DEC(bf16_t, 128, 32) SAS_DEC(bf16_t, 128, 64)
#undef SAS_DEC
  return hipErrorInvalidValue;
}

}  // namespace sas
