// Gated block-sparse attention, portable kernels with fp32 arithmetic.
//
// These serve every supported shape and dtype (fp32 tensors in particular);
// the bf16 MFMA kernels in attn_mfma_*.hip take over where they apply.
//
// picx.dev summary of SAS, 'Key Idea' Eq. 9: o = softmax(qK_S^T/sqrt(d) +
// log g_S) V_S over the selected history blocks plus the current block (log
// g0 = 0); 'Kernel Design': tile-level logits with the log gates added,
// non-selected blocks skipped, online softmax, no attention matrix stored.
// 'Gradient Analysis' Eq. 5 (inner gating) for the gate gradient and Eq. 6
// for the selector gradient through the gate softmax.
//
// Thread layout (forward and dq pass): P = head_dim / 32 adjacent lanes own
// one query row; lane p holds the float4 groups p, p+P, p+2P, ... of the row
// (32 values).  Dot products are reduced across the P lanes with shuffles.
// K/V tiles are staged in LDS as fp32, KC keys at a time.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace sas {

namespace {

constexpr int kRowsPerWG = 128;  // query rows (all heads) per forward / dq workgroup

__device__ __forceinline__ void decode_tile(int tile, const Dims& dm, int nchunk, int* b,
                                            int* kv, int* t, int* chunk) {
  *chunk = tile % nchunk;
  tile /= nchunk;
  *t = tile % dm.T;
  tile /= dm.T;
  *kv = tile % dm.hkv;
  *b = tile / dm.hkv;
}

// Loads 32 values of row `row` (head_dim D) owned by lane p into r[].
template <typename T, int D>
__device__ __forceinline__ void load_row_slice(const T* __restrict__ base, int p, float* r) {
  constexpr int P = D / 32;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 4 * (p + P * e);
#pragma unroll
    for (int u = 0; u < 4; ++u) r[4 * e + u] = Elem<T>::load(base, c + u);
  }
}

template <typename T, int D>
__device__ __forceinline__ void store_row_slice(T* __restrict__ base, int p, const float* r,
                                                float mul) {
  constexpr int P = D / 32;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 4 * (p + P * e);
#pragma unroll
    for (int u = 0; u < 4; ++u) Elem<T>::store(base, c + u, r[4 * e + u] * mul);
  }
}

template <int D>
__device__ __forceinline__ float dot_slice(const float* r, const float* lds_row, int p) {
  constexpr int P = D / 32;
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float4 x = *reinterpret_cast<const float4*>(lds_row + 4 * (p + P * e));
    acc += r[4 * e] * x.x + r[4 * e + 1] * x.y + r[4 * e + 2] * x.z + r[4 * e + 3] * x.w;
  }
  return acc;
}

template <int D>
__device__ __forceinline__ void axpy_slice(float* acc, float a, const float* lds_row, int p) {
  constexpr int P = D / 32;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float4 x = *reinterpret_cast<const float4*>(lds_row + 4 * (p + P * e));
    acc[4 * e] += a * x.x;
    acc[4 * e + 1] += a * x.y;
    acc[4 * e + 2] += a * x.z;
    acc[4 * e + 3] += a * x.w;
  }
}

template <int D>
__device__ __forceinline__ float reduce_p(float v) {
  constexpr int P = D / 32;
#pragma unroll
  for (int o = 1; o < P; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Copies rows [lo, lo+nk) of a [*, D] tensor (type T) into LDS as fp32.
template <typename T, int D, int KC>
__device__ __forceinline__ void stage_rows(float (*dst)[D], const T* __restrict__ src, int nk) {
  for (int e = threadIdx.x; e < KC * D; e += blockDim.x) {
    const int r = e / D, c = e % D;
    dst[r][c] = r < nk ? Elem<T>::load(src, (size_t)r * D + c) : 0.0f;
  }
}

// Builds the list of key blocks of row (b, kv, t): valid selected blocks in
// slot order (with their slot and log-gate), then the current block t.
__device__ __forceinline__ int build_block_list(const int32_t* __restrict__ idx_row,
                                                const float* __restrict__ logg_row, int K,
                                                int t, int* blist, int* bslot, float* bbias) {
  int cnt = 0;
  for (int s = 0; s < K; ++s) {
    const int m = idx_row[s];
    if (m >= 0 && m < t) {
      blist[cnt] = m;
      bslot[cnt] = s;
      bbias[cnt] = logg_row ? logg_row[s] : 0.0f;
      ++cnt;
    }
  }
  blist[cnt] = t;
  bslot[cnt] = -1;
  bbias[cnt] = 0.0f;
  return cnt + 1;
}

// ---------------------------------------------------------------- forward
template <typename T, int D, int BS>
__global__ void __launch_bounds__(512) fwd_generic_kernel(
    Dims dm, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, T* __restrict__ o,
    float* __restrict__ lse, int hpw, int nchunk) {
  constexpr int P = D / 32;
  constexpr int KC = BS < 32 ? BS : 32;
  __shared__ __align__(16) float Ks[KC][D];
  __shared__ __align__(16) float Vs[KC][D];
  __shared__ int blist[kMaxTrainK + 1], bslot[kMaxTrainK + 1];
  __shared__ float bbias[kMaxTrainK + 1];
  __shared__ int nblk;

  int b, kv, t, chunk;
  decode_tile(blockIdx.x, dm, nchunk, &b, &kv, &t, &chunk);
  const int p = threadIdx.x % P;
  const int rr = threadIdx.x / P;
  const int r = rr % BS, hh = chunk * hpw + rr / BS;
  const int h = kv * dm.g + hh;
  const int i = t * BS + r;
  const bool active = rr / BS < hpw && hh < dm.g && i < dm.n;

  const size_t rowbk = ((size_t)b * dm.hkv + kv) * dm.T + t;
  if (threadIdx.x == 0)
    nblk = build_block_list(idx + rowbk * dm.K, logg ? logg + rowbk * dm.K : nullptr, dm.K, t,
                            blist, bslot, bbias);
  float qv[32], acc[32];
  const size_t qoff = (((size_t)b * dm.hq + h) * dm.n + i) * D;
  if (active)
    load_row_slice<T, D>(q + qoff, p, qv);
  else
#pragma unroll
    for (int e = 0; e < 32; ++e) qv[e] = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  float mrun = -INFINITY, lrun = 0.0f;
  __syncthreads();

  const T* kbase = k + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const T* vbase = v + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const int nb = nblk;
  for (int bi = 0; bi < nb; ++bi) {
    const int m = blist[bi];
    // inner gating adds log g to the logits; outer gating scales P V by g
    const float bias = dm.outer ? 0.0f : bbias[bi];
    const float gain = dm.outer ? expf(bbias[bi]) : 1.0f;
    for (int c0 = 0; c0 < BS; c0 += KC) {
      const int lo = m * BS + c0;
      const int nk = min(KC, dm.n - lo);
      if (nk <= 0) break;
      stage_rows<T, D, KC>(Ks, kbase + (size_t)lo * D, nk);
      stage_rows<T, D, KC>(Vs, vbase + (size_t)lo * D, nk);
      __syncthreads();
      float sc[KC];
      float cmax = -INFINITY;
#pragma unroll 2
      for (int j = 0; j < KC; ++j) {
        const float z = reduce_p<D>(dot_slice<D>(qv, Ks[j], p)) * dm.scale + bias;
        const bool valid = j < nk && (m != t || lo + j <= i);
        sc[j] = valid ? z : -INFINITY;
        cmax = fmaxf(cmax, sc[j]);
      }
      const float mnew = fmaxf(mrun, cmax);
      const float alpha = mrun == -INFINITY ? 0.0f : expf(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] *= alpha;
#pragma unroll 2
      for (int j = 0; j < KC; ++j) {
        const float pj = sc[j] == -INFINITY ? 0.0f : expf(sc[j] - mnew);
        lrun += pj;
        axpy_slice<D>(acc, pj * gain, Vs[j], p);
      }
      mrun = mnew;
      __syncthreads();
    }
  }
  if (active) {
    // ragged batch: rows at or past this sequence's end carry no result
    const bool pad = dm.seq_lens && i >= min(max(dm.seq_lens[b], 0), dm.n);
    store_row_slice<T, D>(o + qoff, p, acc, pad ? 0.0f : 1.0f / lrun);
    if (p == 0) lse[((size_t)b * dm.hq + h) * dm.n + i] = pad ? INFINITY : mrun + logf(lrun);
  }
}

int heads_per_wg(const Dims& dm) {
  int hpw = kRowsPerWG / dm.bs;
  if (hpw > dm.g) hpw = dm.g;
  if (hpw < 1) hpw = 1;
  return hpw;
}

template <typename T, int D, int BS>
hipError_t fwd_generic_typed(const Dims& dm, const void* q, const void* k, const void* v,
                             const int32_t* idx, const float* logg, void* o, float* lse,
                             hipStream_t st) {
  const int hpw = heads_per_wg(dm);
  const int nchunk = (dm.g + hpw - 1) / hpw;
  const int threads = (hpw * BS * (D / 32) + 63) / 64 * 64;
  const size_t tiles = (size_t)dm.b * dm.hkv * dm.T * nchunk;
  ProfScope ps("fwd_generic", st);
  hipLaunchKernelGGL((fwd_generic_kernel<T, D, BS>), dim3((unsigned)tiles), dim3(threads), 0,
                     st, dm, (const T*)q, (const T*)k, (const T*)v, idx, logg, (T*)o, lse,
                     hpw, nchunk);
  return hipGetLastError();
}

// ---------------------------------------------------------------- backward: D and CSR
// D[b, h, i] = dout_i . o_i (fp32), 16 lanes per row.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_dot_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      float* __restrict__ Dv, size_t rows) {
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float acc = 0.0f;
  if (row < rows) {
    for (int e = sub; e < D; e += 16)
      acc += Elem<T>::load(o, row * D + e) * Elem<T>::load(dout, row * D + e);
  }
#pragma unroll
  for (int s = 8; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (row < rows && sub == 0) Dv[row] = acc;
}

// Inverse selection map: slot[b, kv][m][t] = the Top-K slot of block m in
// the selection of query block t (0xFF when t did not select m); the
// key-major kernels read the row of their key block.  One workgroup per
// (b, kv) and kSlotRows rows m: it reads every selection row of (b, kv) (the
// loads of eight passes issued together), marks its kSlotRows x T tile in LDS
// over a 0xFF fill, then writes the tile, which is contiguous in the map, once.
// For T > kSlotMaxT (tiles past 64 KB of LDS) the map is cleared, then marked
// entry by entry.
constexpr int kSlotRows = 16;
constexpr int kSlotMaxT = 4096;

__global__ void __launch_bounds__(256) slotmap_clear_kernel(uint4* __restrict__ sm, size_t n16) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) sm[i] = make_uint4(~0u, ~0u, ~0u, ~0u);
}

__global__ void __launch_bounds__(256) slotmap_mark_kernel(const int32_t* __restrict__ idx,
                                                           int T, int K, size_t entries,
                                                           uint8_t* __restrict__ sm) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= entries) return;
  const size_t row = i / K;  // (bk, t)
  const int t = (int)(row % T);
  const size_t bk = row / T;
  const int m = idx[i];
  if (m >= 0 && m < t) sm[(bk * T + m) * (size_t)T + t] = (uint8_t)(i % K);
}

__global__ void __launch_bounds__(256) slotmap_build_kernel(const int32_t* __restrict__ idx,
                                                            int T, int K,
                                                            uint8_t* __restrict__ sm) {
  extern __shared__ __align__(16) uint32_t tile32[];  // kSlotRows * T bytes
  uint8_t* tile = reinterpret_cast<uint8_t*>(tile32);
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * kSlotRows;
  const size_t bk = blockIdx.y;
  const int rows = min(kSlotRows, T - m0);
  for (int i = tid; i < kSlotRows * T / 4; i += 256) tile32[i] = 0xFFFFFFFFu;
  __syncthreads();
  const int32_t* ib = idx + bk * (size_t)T * K;
  const int n = T * K;
  for (int base = 0; base < n; base += 8 * 256) {
    int mv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = base + u * 256 + tid;
      mv[u] = e < n ? ib[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = base + u * 256 + tid;
      const int m = mv[u];
      if (m >= m0 && m < m0 + rows) {
        const int t = e / K;
        if (m < t) tile[(m - m0) * T + t] = (uint8_t)(e - t * K);
      }
    }
  }
  __syncthreads();
  uint8_t* out = sm + (bk * T + m0) * (size_t)T;
  const int nb = rows * T;
  if ((T & 15) == 0) {  // the tile starts 16-byte aligned
    for (int i = tid; i < nb / 16; i += 256)
      reinterpret_cast<uint4*>(out)[i] = reinterpret_cast<const uint4*>(tile32)[i];
  } else {
    for (int i = tid; i < nb; i += 256) out[i] = tile[i];
  }
}

// ---------------------------------------------------------------- backward: dq + dlogg
template <typename T, int D, int BS>
__global__ void __launch_bounds__(512) bwd_dq_generic_kernel(
    Dims dm, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dv,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, T* __restrict__ dq,
    float* __restrict__ dlogg_part, int hpw, int nchunk) {
  constexpr int P = D / 32;
  constexpr int KC = BS < 32 ? BS : 32;
  __shared__ __align__(16) float Ks[KC][D];
  __shared__ __align__(16) float Vs[KC][D];
  __shared__ int blist[kMaxTrainK + 1], bslot[kMaxTrainK + 1];
  __shared__ float bbias[kMaxTrainK + 1];
  __shared__ float fscr[16];
  __shared__ int nblk;

  int b, kv, t, chunk;
  decode_tile(blockIdx.x, dm, nchunk, &b, &kv, &t, &chunk);
  const int p = threadIdx.x % P;
  const int rr = threadIdx.x / P;
  const int r = rr % BS, hh = chunk * hpw + rr / BS;
  const int h = kv * dm.g + hh;
  const int i = t * BS + r;
  const bool active = rr / BS < hpw && hh < dm.g && i < dm.n;

  const size_t rowbk = ((size_t)b * dm.hkv + kv) * dm.T + t;
  if (threadIdx.x == 0)
    nblk = build_block_list(idx + rowbk * dm.K, logg ? logg + rowbk * dm.K : nullptr, dm.K, t,
                            blist, bslot, bbias);
  float qv[32], dov[32], acc[32];
  const size_t row = ((size_t)b * dm.hq + h) * dm.n + i;
  float lse_i = 0.0f, D_i = 0.0f;
  if (active) {
    load_row_slice<T, D>(q + row * D, p, qv);
    load_row_slice<T, D>(dout + row * D, p, dov);
    lse_i = lse[row];
    D_i = Dv[row];
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) qv[e] = dov[e] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  __syncthreads();

  float* dpart = dlogg_part + (rowbk * nchunk + chunk) * dm.K;
  const T* kbase = k + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const T* vbase = v + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const int nb = nblk;
  // slots without a valid block get 0
  for (int sl = threadIdx.x; sl < dm.K; sl += blockDim.x) {
    bool used = false;
    for (int bi = 0; bi + 1 < nb; ++bi) used |= bslot[bi] == sl;
    if (!used) dpart[sl] = 0.0f;
  }
  for (int bi = 0; bi < nb; ++bi) {
    const int m = blist[bi];
    const float bias = dm.outer ? 0.0f : bbias[bi];
    const float gain = dm.outer ? expf(bbias[bi]) : 1.0f;
    float bsum = 0.0f;
    for (int c0 = 0; c0 < BS; c0 += KC) {
      const int lo = m * BS + c0;
      const int nk = min(KC, dm.n - lo);
      if (nk <= 0) break;
      stage_rows<T, D, KC>(Ks, kbase + (size_t)lo * D, nk);
      stage_rows<T, D, KC>(Vs, vbase + (size_t)lo * D, nk);
      __syncthreads();
#pragma unroll 2
      for (int j = 0; j < KC; ++j) {
        const float z = reduce_p<D>(dot_slice<D>(qv, Ks[j], p)) * dm.scale + bias;
        const float dp = reduce_p<D>(dot_slice<D>(dov, Vs[j], p)) * gain;
        const bool valid = active && j < nk && (m != t || lo + j <= i);
        const float pj = valid ? expf(z - lse_i) : 0.0f;
        const float ds = pj * (dp - D_i);
        axpy_slice<D>(acc, ds, Ks[j], p);
        // dL/dlog g: the block's dS (inner), or its p dP (outer)
        bsum += dm.outer ? pj * dp : ds;
      }
      __syncthreads();
    }
    if (bslot[bi] >= 0) {
      const float tot = block_sum(p == 0 ? bsum : 0.0f, fscr);
      if (threadIdx.x == 0) dpart[bslot[bi]] = tot;
    }
  }
  if (active) store_row_slice<T, D>(dq + row * D, p, acc, dm.scale);
}

// ---------------------------------------------------------------- backward: dk, dv
// One workgroup per key block (b, kv, m); BS keys x P lanes.  Visits the
// diagonal query block t = m, then every query block that selected m, for all
// G heads, staging KC query rows of q and dout at a time.
template <typename T, int D, int BS>
__global__ void __launch_bounds__(256) bwd_dkdv_generic_kernel(
    Dims dm, const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dv,
    const float* __restrict__ logg, const uint8_t* __restrict__ slotmap, T* __restrict__ dk,
    T* __restrict__ dv) {
  constexpr int P = D / 32;
  constexpr int KC = BS < 32 ? BS : 32;
  __shared__ __align__(16) float Qs[KC][D];
  __shared__ __align__(16) float Os[KC][D];
  __shared__ float Ls[KC], Dl[KC];
  __shared__ int lst[256];
  __shared__ int scan_scr[16];
  __shared__ int lst_n;

  const int m = blockIdx.x % dm.T;
  const size_t bk = blockIdx.x / dm.T;
  const int kv = (int)(bk % dm.hkv), b = (int)(bk / dm.hkv);
  const int p = threadIdx.x % P;
  const int jr = threadIdx.x / P;
  const int j = m * BS + jr;
  const bool kact = jr < BS && j < dm.n;

  float kvk[32], kvv[32], adk[32], adv[32];
  const size_t kvrow = ((size_t)b * dm.hkv + kv) * dm.n + j;
  if (kact) {
    load_row_slice<T, D>(k + kvrow * D, p, kvk);
    load_row_slice<T, D>(v + kvrow * D, p, kvv);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) kvk[e] = kvv[e] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) adk[e] = adv[e] = 0.0f;

  const uint8_t* srow = slotmap + (bk * dm.T + m) * (size_t)dm.T;
  // Query blocks attending to block m: t = m (diagonal), then every t > m
  // whose selection holds m, compacted NTH at a time into LDS.
  for (int t0 = m; t0 < dm.T; t0 += blockDim.x) {
    {
      const int tt = t0 + (int)threadIdx.x;
      int sl = 0xFF;
      if (tt == m) sl = 0xFE;
      else if (tt < dm.T) sl = srow[tt];
      const int flag = sl != 0xFF;
      int cnt;
      const int pos = block_excl_scan(flag, scan_scr, &cnt);
      if (flag) lst[pos] = (tt << 8) | sl;
      if (threadIdx.x == 0) lst_n = cnt;
      __syncthreads();
    }
    const int ne = lst_n;
  for (int ei = 0; ei < ne; ++ei) {
    const int t = lst[ei] >> 8;
    const int slot = (lst[ei] & 255) == 0xFE ? -1 : (lst[ei] & 255);
    const float lg = (slot >= 0 && logg) ? logg[(bk * dm.T + t) * (size_t)dm.K + slot] : 0.0f;
    const float bias = dm.outer ? 0.0f : lg;
    const float gain = dm.outer ? expf(lg) : 1.0f;
    for (int hh = 0; hh < dm.g; ++hh) {
      const int h = kv * dm.g + hh;
      const size_t rbase = ((size_t)b * dm.hq + h) * dm.n;
      for (int c0 = 0; c0 < BS; c0 += KC) {
        const int lo = t * BS + c0;
        const int nr = min(KC, dm.n - lo);
        if (nr <= 0) break;
        stage_rows<T, D, KC>(Qs, q + (rbase + lo) * D, nr);
        stage_rows<T, D, KC>(Os, dout + (rbase + lo) * D, nr);
        for (int e = threadIdx.x; e < KC; e += blockDim.x) {
          Ls[e] = e < nr ? lse[rbase + lo + e] : 0.0f;
          Dl[e] = e < nr ? Dv[rbase + lo + e] : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int ii = 0; ii < KC; ++ii) {
          const float z = reduce_p<D>(dot_slice<D>(kvk, Qs[ii], p)) * dm.scale + bias;
          const float dp = reduce_p<D>(dot_slice<D>(kvv, Os[ii], p)) * gain;
          const bool valid = kact && ii < nr && (t != m || j <= lo + ii);
          const float pj = valid ? expf(z - Ls[ii]) : 0.0f;
          const float ds = pj * (dp - Dl[ii]);
          axpy_slice<D>(adv, pj * gain, Os[ii], p);
          axpy_slice<D>(adk, ds, Qs[ii], p);
        }
        __syncthreads();
      }
    }
  }
  }
  if (kact) {
    store_row_slice<T, D>(dk + kvrow * D, p, adk, dm.scale);
    store_row_slice<T, D>(dv + kvrow * D, p, adv, 1.0f);
  }
}

// ---------------------------------------------------------------- backward: ds
// g = phi(s) under the gate activation (0 softmax: exp(s - lse); 1 sigmoid;
// 2 raw logit: exp(s)).
__device__ __forceinline__ float gate_value(float s, float lse, int act) {
  if (act == 1) return 1.0f / (1.0f + expf(-s));
  if (act == 2) return expf(s);
  return expf(s - lse);
}

// Per row (b, kv, t): dlogg = sum of the per-chunk partials (fixed order);
// with ste the forward was hard and dlogg_m is dL/dg_m, so the soft gate's
// Jacobian acts on e_m = g_m dlogg_m, else e_m = dlogg_m.  For m < t:
//   softmax: ds_m = [m in I] e_m - g_m sum(e)   (Eq. 6 differentiated)
//   sigmoid: ds_m = [m in I] e_m (1 - g_m)
//   raw:     ds_m = [m in I] e_m
// and 0 for m >= t.
__global__ void __launch_bounds__(256) bwd_ds_kernel(
    int T, int K, int act, int ste, const int32_t* __restrict__ idx, const float* __restrict__ s,
    const float* __restrict__ lse_s, const float* __restrict__ dlogg_part, int nchunk,
    float* __restrict__ dlogg, float* __restrict__ ds) {
  __shared__ float dl[kMaxTrainK];
  __shared__ int im[kMaxTrainK];
  __shared__ float tot;
  const size_t row = blockIdx.x;
  const int t = (int)(row % T);
  const float ls = lse_s ? lse_s[row] : 0.0f;
  if ((int)threadIdx.x < K) {
    float a = 0.0f;
    for (int c = 0; c < nchunk; ++c) a += dlogg_part[(row * nchunk + c) * K + threadIdx.x];
    const int m = idx[row * K + threadIdx.x];
    const bool ok = m >= 0 && m < t;
    const float e = (ok && ste && s) ? a * gate_value(s[row * T + m], ls, act) : a;
    dl[threadIdx.x] = ok ? e : 0.0f;
    im[threadIdx.x] = ok ? m : -1;
    if (dlogg) dlogg[row * K + threadIdx.x] = ok ? a : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.0f;
    for (int sl = 0; sl < K; ++sl) a += dl[sl];
    tot = a;
  }
  __syncthreads();
  if (!ds) return;
  for (int m = threadIdx.x; m < T; m += blockDim.x) {
    float val = 0.0f;
    if (m < t && ls > -INFINITY) {  // rows without history (or past a sequence's end): 0
      float own = 0.0f;
      for (int sl = 0; sl < K; ++sl)
        if (im[sl] == m) own = dl[sl];
      const float sm = s[row * T + m];
      if (act == 1)
        val = own * (1.0f - gate_value(sm, ls, 1));
      else if (act == 2)
        val = own;
      else
        val = own - expf(sm - ls) * tot;
    }
    ds[row * T + m] = val;
  }
}

template <typename T, int D, int BS>
hipError_t bwd_generic_typed(const Dims& dm, const void* q, const void* k, const void* v,
                             const void* dout, const float* lse, const int32_t* idx,
                             const float* logg, void* dq, void* dk, void* dv,
                             const BwdWorkspace& ws, int* nchunk_out, hipStream_t st) {
  const int hpw = heads_per_wg(dm);
  const int nchunk = (dm.g + hpw - 1) / hpw;
  *nchunk_out = nchunk;
  {
    const int threads = (hpw * BS * (D / 32) + 63) / 64 * 64;
    const size_t tiles = (size_t)dm.b * dm.hkv * dm.T * nchunk;
    ProfScope ps("bwd_dq_generic", st);
    hipLaunchKernelGGL((bwd_dq_generic_kernel<T, D, BS>), dim3((unsigned)tiles), dim3(threads),
                       0, st, dm, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse,
                       ws.D, idx, logg, (T*)dq, ws.dlogg_part, hpw, nchunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const size_t wgs = (size_t)dm.b * dm.hkv * dm.T;
    ProfScope ps("bwd_dkdv_generic", st);
    const int threads = BS * (D / 32) < 64 ? 64 : BS * (D / 32);
    hipLaunchKernelGGL((bwd_dkdv_generic_kernel<T, D, BS>), dim3((unsigned)wgs), dim3(threads),
                       0, st, dm, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse,
                       ws.D, logg, ws.slotmap, (T*)dk, (T*)dv);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_generic(const Dims& dm, const void* q, const void* k, const void* v,
                              const int32_t* idx, const float* logg, void* o, float* lse,
                              hipStream_t st) {
#define SAS_FWD(T_, D_, BS_)                                                         \
  if ((dm.bf16 == std::is_same<T_, bf16_t>::value) && dm.d == D_ && dm.bs == BS_) \
    return fwd_generic_typed<T_, D_, BS_>(dm, q, k, v, idx, logg, o, lse, st);
  SAS_FWD(float, 64, 16) SAS_FWD(float, 64, 32) SAS_FWD(float, 64, 64)
  SAS_FWD(float, 128, 16) SAS_FWD(float, 128, 32) SAS_FWD(float, 128, 64)
  SAS_FWD(bf16_t, 64, 16) SAS_FWD(bf16_t, 64, 32) SAS_FWD(bf16_t, 64, 64)
  SAS_FWD(bf16_t, 128, 16) SAS_FWD(bf16_t, 128, 32) SAS_FWD(bf16_t, 128, 64)
#undef SAS_FWD
  return hipErrorInvalidValue;
}

int bwd_dlogg_chunks(const Dims& dm) {
  const int hpw = heads_per_wg(dm);
  return (dm.g + hpw - 1) / hpw;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdWorkspace bwd_workspace_layout(const Dims& dm, void* base) {
  BwdWorkspace w{};
  char* p = (char*)base;
  size_t off = 0;
  const size_t rows = (size_t)dm.b * dm.hkv * dm.T;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.D = (float*)take((size_t)dm.b * dm.hq * dm.n * sizeof(float));
  w.dlogg_part = (float*)take(rows * (size_t)bwd_dlogg_chunks(dm) * dm.K * sizeof(float));
  w.slotmap_bytes = align256(rows * (size_t)dm.T);
  w.slotmap = (uint8_t*)take(w.slotmap_bytes);
  const int nparts = mfma_bwd_supported(dm) ? dkdv_split_plan(dm).nparts : 0;
  w.dkdv_part =
      nparts ? (float*)take((size_t)nparts * dm.b * dm.hkv * kDkdvPartFloats * sizeof(float))
             : nullptr;
  w.bytes = off;
  return w;
}

hipError_t launch_bwd_prep(const Dims& dm, const void* o, const void* dout, const int32_t* idx,
                           const BwdWorkspace& ws, bool with_d, hipStream_t st) {
  const size_t rows = (size_t)dm.b * dm.hq * dm.n;
  if (with_d) {
    ProfScope ps("bwd_dot", st);
    const unsigned grid = (unsigned)((rows + 15) / 16);
    if (dm.bf16 && dm.d == 128)
      hipLaunchKernelGGL((bwd_dot_kernel<bf16_t, 128>), dim3(grid), dim3(256), 0, st,
                         (const bf16_t*)o, (const bf16_t*)dout, ws.D, rows);
    else if (dm.bf16)
      hipLaunchKernelGGL((bwd_dot_kernel<bf16_t, 64>), dim3(grid), dim3(256), 0, st,
                         (const bf16_t*)o, (const bf16_t*)dout, ws.D, rows);
    else if (dm.d == 128)
      hipLaunchKernelGGL((bwd_dot_kernel<float, 128>), dim3(grid), dim3(256), 0, st,
                         (const float*)o, (const float*)dout, ws.D, rows);
    else
      hipLaunchKernelGGL((bwd_dot_kernel<float, 64>), dim3(grid), dim3(256), 0, st,
                         (const float*)o, (const float*)dout, ws.D, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps("slotmap", st);
  if (dm.T <= kSlotMaxT) {
    const dim3 grid((unsigned)((dm.T + kSlotRows - 1) / kSlotRows), (unsigned)(dm.b * dm.hkv));
    hipLaunchKernelGGL(slotmap_build_kernel, grid, dim3(256), (size_t)kSlotRows * dm.T, st, idx,
                       dm.T, dm.K, ws.slotmap);
  } else {
    const size_t n16 = ws.slotmap_bytes / 16;
    const size_t entries = (size_t)dm.b * dm.hkv * dm.T * dm.K;
    hipLaunchKernelGGL(slotmap_clear_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0,
                       st, (uint4*)ws.slotmap, n16);
    hipLaunchKernelGGL(slotmap_mark_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256),
                       0, st, idx, dm.T, dm.K, entries, ws.slotmap);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_generic(const Dims& dm, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const int32_t* idx,
                              const float* logg, void* dq, void* dk, void* dv,
                              const BwdWorkspace& ws, int* nchunk_out, hipStream_t st) {
#define SAS_BWD(T_, D_, BS_)                                                           \
  if ((dm.bf16 == std::is_same<T_, bf16_t>::value) && dm.d == D_ && dm.bs == BS_)   \
    return bwd_generic_typed<T_, D_, BS_>(dm, q, k, v, dout, lse, idx, logg, dq, dk, dv, ws, \
                                          nchunk_out, st);
  SAS_BWD(float, 64, 16) SAS_BWD(float, 64, 32) SAS_BWD(float, 64, 64)
  SAS_BWD(float, 128, 16) SAS_BWD(float, 128, 32) SAS_BWD(float, 128, 64)
  SAS_BWD(bf16_t, 64, 16) SAS_BWD(bf16_t, 64, 32) SAS_BWD(bf16_t, 64, 64)
  SAS_BWD(bf16_t, 128, 16) SAS_BWD(bf16_t, 128, 32) SAS_BWD(bf16_t, 128, 64)
#undef SAS_BWD
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_ds(const Dims& dm, const int32_t* idx, const float* s, const float* lse_s,
                         const float* dlogg_part, int nchunk, float* dlogg, float* ds,
                         hipStream_t st) {
  const size_t rows = (size_t)dm.b * dm.hkv * dm.T;
  ProfScope ps("bwd_ds", st);
  hipLaunchKernelGGL(bwd_ds_kernel, dim3((unsigned)rows), dim3(256), 0, st, dm.T, dm.K, dm.act,
                     dm.ste ? 1 : 0, idx, s, lse_s, dlogg_part, nchunk, dlogg, ds);
  return hipGetLastError();
}

}  // namespace sas
