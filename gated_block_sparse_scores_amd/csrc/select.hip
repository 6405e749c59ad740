// Block scoring, gate normalisation and hard Top-K for SAS.
//
// picx.dev summary of SAS, 'Theoretical Foundation' Eq. 3 (I = Top-K(s, K))
// and 'Gradient Analysis' Eq. 6 (log g_m = s_m - LSE(s) over the history);
// evolve.pub review FAQ (pooling-based block summaries feed the selector).
#include <math.h>

#include "common.h"
#include "internal.h"

namespace sas {

// ---------------------------------------------------------------- pooling
// One workgroup per (t, output head, batch).  256 threads = (256/d) token
// lanes x d columns; fp64 accumulation, one rounding to fp32 (and optionally
// a second one to bf16).
template <typename Tin>
__global__ void __launch_bounds__(256) pool_kernel(const Tin* __restrict__ x, int heads,
                                                   int group, int n, int d, int bs,
                                                   int out_bf16, void* __restrict__ out) {
  __shared__ double red[256];
  const int t = blockIdx.x, ho = blockIdx.y, b = blockIdx.z;
  const int T = gridDim.x, hout = gridDim.y;
  const int lo = t * bs, hi = min(lo + bs, n);
  const int lanes = blockDim.x / d;
  const int col = threadIdx.x % d, rl = threadIdx.x / d;
  double acc = 0.0;
  if (rl < lanes) {
    for (int hh = 0; hh < group; ++hh) {
      const Tin* base = x + ((size_t)b * heads + (size_t)ho * group + hh) * (size_t)n * d;
      for (int i = lo + rl; i < hi; i += lanes)
        acc += (double)Elem<Tin>::load(base, (size_t)i * d + col);
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  if (rl == 0) {
    double s = 0.0;
    for (int r = 0; r < lanes; ++r) s += red[r * d + col];
    const double mean = s / (double)((hi - lo) * group);
    const float f = (float)mean;
    const size_t o = (((size_t)b * hout + ho) * T + t) * d + col;
    if (out_bf16)
      reinterpret_cast<bf16_t*>(out)[o] = f32_to_bf16(f);
    else
      reinterpret_cast<float*>(out)[o] = f;
  }
}

hipError_t launch_block_pool(const void* x, bool in_bf16, int batch, int heads, int group,
                             int n, int d, int bs, bool out_bf16, void* out, hipStream_t st) {
  const int T = (n + bs - 1) / bs;
  dim3 grid(T, heads / group, batch);
  ProfScope ps("block_pool", st);
  if (in_bf16)
    hipLaunchKernelGGL(pool_kernel<bf16_t>, grid, dim3(256), 0, st,
                       (const bf16_t*)x, heads, group, n, d, bs, (int)out_bf16, out);
  else
    hipLaunchKernelGGL(pool_kernel<float>, grid, dim3(256), 0, st, (const float*)x, heads,
                       group, n, d, bs, (int)out_bf16, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- stand-in scores
// s[r, m] = fp32((qbar[r] . kbar[m]) * scale) with the dot product in fp64.
// Grid (m-chunks, T, b*hkv); 256 threads = 16 groups of 16 lanes, one key
// block summary per group, lanes split head_dim.
constexpr int kScoreChunk = 256;

template <typename Tk>
__global__ void __launch_bounds__(256) standin_score_kernel(
    const float* __restrict__ qbar, const Tk* __restrict__ kbar, int kbar_ld, int T, int C,
    int row_offset, int d, double scale, float* __restrict__ s_out) {
  __shared__ double qs[128];
  const int t = blockIdx.y, bk = blockIdx.z;
  const int ct = min(t + row_offset, C);
  const int m0 = blockIdx.x * kScoreChunk;
  const float* qrow = qbar + ((size_t)bk * T + t) * d;
  for (int e = threadIdx.x; e < d; e += blockDim.x) qs[e] = (double)qrow[e];
  __syncthreads();
  const int sub = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const Tk* kb = kbar + (size_t)bk * kbar_ld * d;
  float* srow = s_out + ((size_t)bk * T + t) * C;
  const int mend = min(m0 + kScoreChunk, C);
  for (int m = m0 + grp; m < mend; m += 16) {
    double acc = 0.0;
    if (m < ct) {
      for (int e = sub; e < d; e += 16)
        acc += qs[e] * (double)Elem<Tk>::load(kb, (size_t)m * d + e);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (sub == 0) srow[m] = (m < ct) ? (float)(acc * scale) : 0.0f;
  }
}

hipError_t launch_standin_scores(const float* qbar, const void* kbar, bool kbar_bf16,
                                 int kbar_ld, int rows_bk, int T, int C, int row_offset,
                                 int d, double scale, float* s_out, hipStream_t st) {
  dim3 grid((C + kScoreChunk - 1) / kScoreChunk, T, rows_bk);
  ProfScope ps("standin_scores", st);
  if (kbar_bf16)
    hipLaunchKernelGGL(standin_score_kernel<bf16_t>, grid, dim3(256), 0, st, qbar,
                       (const bf16_t*)kbar, kbar_ld, T, C, row_offset, d, scale, s_out);
  else
    hipLaunchKernelGGL(standin_score_kernel<float>, grid, dim3(256), 0, st, qbar,
                       (const float*)kbar, kbar_ld, T, C, row_offset, d, scale, s_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gate LSE + Top-K
// One 256-thread workgroup per row.  The valid scores are held in LDS as
// order-preserving uint32 keys.  A 4-pass MSB-first radix select (8 bits per
// pass) finds the K-th largest key v and how many keys equal to v are still
// needed; those are taken in ascending block order, which realises the
// "equal score -> lower block index" rule.  The selection is then compacted in
// ascending block order with two workgroup scans.
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ s, int T, int C,
                                                   int row_offset, int K,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ logg,
                                                   float* __restrict__ lse_s) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[256];
  __shared__ int iscr[16];
  __shared__ float fscr[16];
  __shared__ double dscr[16];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_rem;

  const int tid = threadIdx.x, nth = blockDim.x;
  const size_t row = blockIdx.x;
  const int t = (int)(row % T);
  const int ct = min(t + row_offset, C);
  const float* srow = s + row * (size_t)C;

  float mx = -INFINITY;
  for (int m = tid; m < ct; m += nth) {
    const float f = srow[m];
    keys[m] = order_key(f);
    mx = fmaxf(mx, f);
  }
  mx = block_max(mx, fscr);  // barriers inside; keys[] visible afterwards
  double sum = 0.0;
  for (int m = tid; m < ct; m += nth) sum += (double)expf(srow[m] - mx);
  sum = block_sum_d(sum, dscr);
  const float lse = ct > 0 ? (float)((double)mx + log(sum)) : -INFINITY;

  const int kk = min(K, ct);
  uint32_t thr = 0u;
  int take_eq = 0;
  const bool all = ct <= K;
  if (!all) {
    uint32_t prefix = 0u, mask = 0u;
    int rem = K;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int m = tid; m < ct; m += nth) {
        const uint32_t key = keys[m];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      // bin = 255 - tid; "above" = number of candidates in bins > bin.
      const int bin = 255 - tid;
      const int cnt = hist[bin];
      int total;
      const int above = block_excl_scan(cnt, iscr, &total);
      if (above < rem && rem <= above + cnt) {
        sh_prefix = prefix | ((uint32_t)bin << shift);
        sh_rem = rem - above;
      }
      __syncthreads();
      prefix = sh_prefix;
      rem = sh_rem;
      mask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
    take_eq = rem;
  }

  // Contiguous chunk of block indices per thread, so scans follow index order.
  const int chunk = (ct + nth - 1) / nth;
  const int mb = min(tid * chunk, ct), me = min(mb + chunk, ct);
  int eq_cnt = 0;
  if (!all)
    for (int m = mb; m < me; ++m) eq_cnt += keys[m] == thr;
  int dummy;
  const int eq_before = block_excl_scan(eq_cnt, iscr, &dummy);
  int sel_cnt = 0;
  {
    int e = eq_before;
    for (int m = mb; m < me; ++m) {
      const uint32_t key = keys[m];
      const bool eq = key == thr;
      sel_cnt += all || key > thr || (eq && e < take_eq);
      e += eq;
    }
  }
  const int pos0 = block_excl_scan(sel_cnt, iscr, &dummy);
  int32_t* irow = idx + row * (size_t)K;
  float* lrow = logg + row * (size_t)K;
  {
    int e = eq_before, pos = pos0;
    for (int m = mb; m < me; ++m) {
      const uint32_t key = keys[m];
      const bool eq = key == thr;
      const bool sel = all || key > thr || (eq && e < take_eq);
      e += eq;
      if (sel) {
        irow[pos] = m;
        lrow[pos] = srow[m] - lse;
        ++pos;
      }
    }
  }
  for (int p = kk + tid; p < K; p += nth) {
    irow[p] = -1;
    lrow[p] = 0.0f;
  }
  if (tid == 0) lse_s[row] = lse;
}

hipError_t launch_topk(const float* s, int rows_bk, int T, int C, int row_offset, int K,
                       int32_t* idx, float* logg, float* lse_s, hipStream_t st) {
  const size_t rows = (size_t)rows_bk * T;
  const size_t lds = (size_t)(C > 0 ? C : 1) * sizeof(uint32_t);
  ProfScope ps("topk", st);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(256), lds, st, s, T, C,
                     row_offset, K, idx, logg, lse_s);
  return hipGetLastError();
}

}  // namespace sas
