// Block scoring, gate normalisation and hard Top-K for SAS.
//
// picx.dev summary of SAS, 'Theoretical Foundation' Eq. 3 (I = Top-K(s, K))
// and 'Gradient Analysis' Eq. 6 (log g_m = s_m - LSE(s) over the history);
// evolve.pub review FAQ (pooling-based block summaries feed the selector).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace sas {

// ---------------------------------------------------------------- pooling
// One workgroup per (t, output head, batch).  Each lane reads 16 bytes (8 bf16
// or 4 fp32 values) of a row, LPR = D / 16-byte-chunks lanes cover a row and
// 256 / LPR rows are read per pass, so every load is a full 16-byte vector
// load and all of a block's loads are independent.  fp64 accumulation, the
// per-row-lane sums folded through LDS, one rounding to fp32 (and optionally
// a second one to bf16).
template <typename Tin, int D>
__global__ void __launch_bounds__(256) pool_kernel(const Tin* __restrict__ x, int heads,
                                                   int group, int n, int bs, int out_bf16,
                                                   void* __restrict__ out,
                                                   const int32_t* __restrict__ lens) {
  constexpr int E = 16 / (int)sizeof(Tin);  // values per 16-byte load
  constexpr int LPR = D / E;                // lanes per row
  constexpr int RPP = 256 / LPR;            // rows per pass
  __shared__ double red[RPP][D];
  const int t = blockIdx.x, ho = blockIdx.y, b = blockIdx.z;
  const int T = gridDim.x, hout = gridDim.y;
  const int nb = lens ? min(max(lens[b], 0), n) : n;  // this sequence's tokens
  const int lo = t * bs, hi = min(lo + bs, nb);
  const int li = threadIdx.x % LPR, ri = threadIdx.x / LPR;
  double acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0;
  for (int hh = 0; hh < group; ++hh) {
    const Tin* base = x + ((size_t)b * heads + (size_t)ho * group + hh) * (size_t)n * D + li * E;
#pragma unroll 4
    for (int i = lo + ri; i < hi; i += RPP) {
      float v[E];
      if constexpr (sizeof(Tin) == 2) {
        const uint4 u = *reinterpret_cast<const uint4*>(base + (size_t)i * D);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * k] = __uint_as_float(w[k] << 16);
          v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      } else {
        const float4 f = *reinterpret_cast<const float4*>(base + (size_t)i * D);
        v[0] = f.x;
        v[1] = f.y;
        v[2] = f.z;
        v[3] = f.w;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += (double)v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[ri][li * E + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int col = threadIdx.x;
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < RPP; ++r) sum += red[r][col];
    const double mean = hi > lo ? sum / (double)((hi - lo) * group) : 0.0;
    const float f = (float)mean;
    const size_t o = (((size_t)b * hout + ho) * T + t) * D + col;
    if (out_bf16)
      reinterpret_cast<bf16_t*>(out)[o] = f32_to_bf16(f);
    else
      reinterpret_cast<float*>(out)[o] = f;
  }
}

hipError_t launch_block_pool(const void* x, bool in_bf16, int batch, int heads, int group,
                             int n, int d, int bs, bool out_bf16, void* out, hipStream_t st,
                             const int32_t* lens) {
  const int T = (n + bs - 1) / bs;
  dim3 grid(T, heads / group, batch);
  ProfScope ps("block_pool", st);
#define SAS_POOL(TIN, DD)                                                                 \
  hipLaunchKernelGGL((pool_kernel<TIN, DD>), grid, dim3(256), 0, st, (const TIN*)x, heads, \
                     group, n, bs, (int)out_bf16, out, lens)
  if (in_bf16 && d == 128)
    SAS_POOL(bf16_t, 128);
  else if (in_bf16)
    SAS_POOL(bf16_t, 64);
  else if (d == 128)
    SAS_POOL(float, 128);
  else
    SAS_POOL(float, 64);
#undef SAS_POOL
  return hipGetLastError();
}

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ double row16_sum_d(double x) {
  auto step = [](double v, int ctrl) -> double {
    const long long bits = __double_as_longlong(v);
    int lo = (int)(bits & 0xFFFFFFFFll), hi = (int)(bits >> 32);
    switch (ctrl) {
      case 0:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, true);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, true);
        break;
      case 1:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, true);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, true);
        break;
      case 2:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, true);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, true);
        break;
      default:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, true);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, true);
        break;
    }
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
  };
  x += step(x, 0);
  x += step(x, 1);
  x += step(x, 2);
  x += step(x, 3);
  return x;
}

// Loads 8 consecutive summary values (one lane's slice) widened to double.
template <typename Tk> struct Slice8;
template <> struct Slice8<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ double get(int e) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const uint32_t x = w[e >> 1];
    return (double)__uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
};
template <> struct Slice8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ double get(int e) const {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return (double)v[e];
  }
};

// ---------------------------------------------------------------- gate LSE + Top-K
// Rows of at most kLongHistory history blocks.  One wave selects a row: lane
// l holds blocks l ch .. l ch + ch - 1 (ch = ceil(C_t / 64) <= 8) in
// registers, as order-preserving uint32 keys.  The gate LSE takes wave
// reductions; the K-th largest key v is found bit by bit from the top, each
// step counting the keys at or above the candidate with ballots; keys above v
// and the first (K - #above) keys equal to v in ascending block order (the
// "equal score -> lower block index" rule) are written in ascending block
// order from wave prefix sums.  No workgroup barrier.
// PER >= ceil(C_t / 64) keys per lane (the register arrays and every ballot
// pass are sized by it).
template <int PER>
__device__ __forceinline__ void wave_select_row(const float* src, int ct, int K, int act,
                                                int32_t* __restrict__ irow,
                                                float* __restrict__ lrow, float* lse_out) {
  static_assert(PER * 64 <= kLongHistory, "row longer than the one-wave select");
  const int lane = threadIdx.x & 63;
  const int ch = (ct + 63) >> 6;
  const int mb = lane * ch;
  float f[PER];
  uint32_t key[PER];
  float mxl = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool ok = i < ch && mb + i < ct;
    f[i] = ok ? src[mb + i] : 0.0f;
    key[i] = ok ? order_key(f[i]) : 0u;  // every valid key is above 0
    if (ok) mxl = fmaxf(mxl, f[i]);
  }
  const float mx = wave_max(mxl);
  double sl = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (i < ch && mb + i < ct) sl += (double)expf(f[i] - mx);
  const double sum = wave_sum_d(sl);
  const float lse = ct > 0 ? (float)((double)mx + log(sum)) : -INFINITY;

  const int kk = min(K, ct);
  const bool all = ct <= K;
  uint32_t thr = 0u;
  int take_eq = 0;
  if (!all) {
    // the largest thr with at least K keys >= thr is the K-th largest key
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) cnt += __popcll(__ballot(key[i] >= cand));
      if (cnt >= K) thr = cand;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) gt += __popcll(__ballot(key[i] > thr));
    take_eq = K - gt;
  }
  int eq_cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) eq_cnt += (!all && key[i] == thr) ? 1 : 0;
  const int eq_before = wave_incl_scan(eq_cnt) - eq_cnt;
  bool sel[PER];
  int sel_cnt = 0;
  {
    int e = eq_before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool ok = i < ch && mb + i < ct;
      const bool eq = !all && key[i] == thr;
      sel[i] = ok && (all || key[i] > thr || (eq && e < take_eq));
      e += eq ? 1 : 0;
      sel_cnt += sel[i] ? 1 : 0;
    }
  }
  const int pos0 = wave_incl_scan(sel_cnt) - sel_cnt;
  {
    int pos = pos0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (sel[i]) {
        irow[pos] = mb + i;
        lrow[pos] = gate_log(f[i], lse, act);
        ++pos;
      }
  }
  for (int p = kk + lane; p < K; p += 64) {
    irow[p] = -1;
    lrow[p] = 0.0f;
  }
  if (lane == 0) *lse_out = lse;
}

// Given scores: one wave per row, four rows per workgroup.
template <int PER>
__global__ void __launch_bounds__(256) topk_given_kernel(const float* __restrict__ s,
                                                         size_t rows, int T, int C,
                                                         int row_offset, int K, int act,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ logg,
                                                         float* __restrict__ lse_s, RowLens rl) {
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // the whole wave
  const int ct = row_history((int)(row % T), row_offset, C, rl, row / T);
  wave_select_row<PER>(s + row * (size_t)C, ct, K, act, idx + row * (size_t)K,
                       logg + row * (size_t)K, lse_s + row);
}

// Stand-in scores: one 256-thread workgroup per row forms
// s[m] = fp32((qbar . kbar[m]) * scale), the dot product in fp64 with 16 lanes
// per key-block summary (8 consecutive dims each, reduced with DPP), into LDS
// and s_out (0 past the row's history); then wave 0 selects.
template <typename Tk, int PER>
__global__ void __launch_bounds__(256) topk_standin_kernel(
    const float* __restrict__ qbar, const Tk* __restrict__ kbar, int kbar_ld, int d,
    double scale, float* __restrict__ s_out, int T, int C, int row_offset, int K, int act,
    int32_t* __restrict__ idx, float* __restrict__ logg, float* __restrict__ lse_s,
    RowLens rl) {
  __shared__ float sv[kLongHistory];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const int ct = row_history((int)(row % T), row_offset, C, rl, row / T);
  const int sub = tid & 15, grp = tid >> 4;
  const bool lane_on = sub * 8 < d;
  double qv[8];
  {
    const float* qrow = qbar + row * (size_t)d + (lane_on ? sub * 8 : 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = (double)qrow[e];
  }
  const Tk* kb = kbar + (row / T) * (size_t)kbar_ld * d + (lane_on ? sub * 8 : 0);
  float* orow = s_out + row * (size_t)C;
  // sixteen blocks per round (one per 16-lane group), the loads of RB rounds
  // issued before their products (the DPP reductions keep the compiler from
  // unrolling a loop with a run-time trip count itself); rows of at most 128
  // blocks issue all their loads at once
  constexpr int RB = PER <= 2 ? 8 : 4;
  for (int m0 = 0; m0 < C; m0 += 16 * RB) {
    Slice8<Tk> ks[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int m = m0 + 16 * u + grp;
      if (m < ct && lane_on) ks[u].load(kb + (size_t)m * d);
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int m = m0 + 16 * u + grp;
      double acc = 0.0;
      if (m < ct && lane_on) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += qv[e] * ks[u].get(e);
      }
      acc = row16_sum_d(acc);
      const float v = m < ct ? (float)(acc * scale) : 0.0f;
      if (sub == 0 && m < C) {
        sv[m] = v;
        orow[m] = v;
      }
    }
  }
  __syncthreads();
  if (tid < 64)
    wave_select_row<PER>(sv, ct, K, act, idx + row * (size_t)K, logg + row * (size_t)K,
                         lse_s + row);
}

// ---------------------------------------------------------------- long histories: two stages
// For rows with many history blocks (decode over long contexts) one workgroup
// per row leaves the chip idle and serialises the radix histograms.  Stage 1:
// one workgroup per (row, chunk of 256 history blocks) forms the scores (given,
// or the stand-in score with fp64 dot products read by 16 lanes per summary row
// and reduced with DPP), records the chunk's max and sum of exp, and ranks its
// 256 composite keys (order-preserving score bits, then the complemented block
// index, so equal scores rank the lower block first; all keys are distinct):
// each wave sorts its 64 keys in registers, and a key's rank adds, for every
// other wave, the count of that wave's sorted keys above it; keys of rank < K
// are written in rank order as the chunk's candidates.  Every block of the
// row's Top-K is among its chunk's first K.  Stage 2 (K <= 64) folds the sorted
// chunk lists into one top-K list with wave-level bitonic merges, combines the
// chunk statistics into lse_s, and
// emits the K winners in ascending block order.
constexpr int kChunk = 256;

template <typename Tk>
__global__ void __launch_bounds__(256) select_chunk_kernel(
    const float* __restrict__ s, const float* __restrict__ qbar, const bf16_t* __restrict__ qraw,
    int qgroup, const Tk* __restrict__ kbar, int kbar_ld, int d, double scale, int T, int C,
    int row_offset, int K, int nchunk, float* __restrict__ s_out, uint64_t* __restrict__ cand,
    float2* __restrict__ stats, RowLens rl) {
  __shared__ uint64_t srt[kChunk / 64][64];  // each wave's keys, sorted descending
  __shared__ float sval[kChunk];
  __shared__ float fscr[16];
  __shared__ double dscr[16];
  const int chunk = blockIdx.x;
  const size_t row = blockIdx.y;
  const int t = (int)(row % T);
  const size_t bk = row / T;
  const int ct = row_history(t, row_offset, C, rl, bk);
  const int m0 = chunk * kChunk;
  const int tid = threadIdx.x;
  const int m = m0 + tid;
  const bool valid = m < ct;

  float f = 0.0f;
  if (s) {
    f = valid ? s[row * C + m] : 0.0f;
  } else {
    // 16 groups of 16 lanes; group grp scores blocks m0 + grp + 16 i.
    const int sub = tid & 15, grp = tid >> 4;
    const int nsl = d / 8;  // lanes carrying 8 dims each (16 for d = 128, 8 for d = 64)
    // The summary rows' loads go out first: nothing in their addresses waits on
    // the query, so their latency overlaps the query's.
    // Rows past the history and lanes past d read an in-bounds row (clamped)
    // and weight it 0 (or discard it), so no row needs a branch and the rows'
    // products interleave.
    const int cmax = max(ct - 1, 0), subc = sub < nsl ? sub : 0;
    Slice8<Tk> sl[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mm = min(m0 + grp + 16 * i, cmax);
      sl[i].load(kbar + (bk * kbar_ld + mm) * (size_t)d + subc * 8);
    }
    double qd[8];
    if (qraw) {
      // decode (T = 1): the pooled query is the mean of the qgroup heads of this
      // KV head, formed here exactly as the pooling kernel forms it (the sum of
      // bf16 values in fp64 is exact), rounded once to fp32.  Heads are read
      // eight at a time, every load of a batch issued before the first add (a
      // head index past the group re-reads the last head).
      const bf16_t* qh = qraw + row * (size_t)qgroup * d + (sub < nsl ? sub * 8 : 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) qd[e] = 0.0;
      for (int h0 = 0; h0 < qgroup; h0 += 8) {
        uint4 u[8];
#pragma unroll
        for (int h = 0; h < 8; ++h)
          u[h] = *reinterpret_cast<const uint4*>(qh + (size_t)min(h0 + h, qgroup - 1) * d);
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          // a head past the group adds +0.0, which leaves every sum unchanged
          const bool in = h0 + h < qgroup;
          const uint32_t w[4] = {u[h].x, u[h].y, u[h].z, u[h].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            qd[2 * k] += in ? (double)__uint_as_float(w[k] << 16) : 0.0;
            qd[2 * k + 1] += in ? (double)__uint_as_float(w[k] & 0xFFFF0000u) : 0.0;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qd[e] = sub < nsl ? (double)(float)(qd[e] / qgroup) : 0.0;
    } else {
      const float* qr = qbar + row * (size_t)d;
#pragma unroll
      for (int e = 0; e < 8; ++e) qd[e] = sub < nsl ? (double)qr[sub * 8 + e] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mm = m0 + grp + 16 * i;
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) a += qd[e] * sl[i].get(e);  // qd = 0 past d
      a = row16_sum_d(a);
      if (sub == 0) sval[grp + 16 * i] = mm < ct ? (float)(a * scale) : 0.0f;
    }
    __syncthreads();
    f = sval[tid];
    if (s_out && m < C) s_out[row * C + m] = valid ? f : 0.0f;
  }
  // Invalid entries get keys below every valid one (high word 0), still distinct.
  const uint64_t mykey = ((valid ? (uint64_t)order_key(f) : 0ull) << 32) |
                         (uint64_t)(0xFFFFFFFFu - (uint32_t)m);
  // Rank of every key in the chunk (keys are distinct): each wave sorts its 64
  // keys descending with a bitonic network in registers; a key's rank is its
  // position in its wave plus, for each other wave, how many of that wave's
  // sorted keys exceed it (binary search in LDS).
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t v = bitonic_sort_desc64(mykey, lane);  // lane exchanges by DPP / row swaps
  srt[wave][lane] = v;
  // Chunk statistics: one barrier publishes the sorted lists and the wave
  // maxima together; the waves' fp64 sums of exp are combined, in wave order,
  // after the last barrier below.
  {
    const float wmx = wave_max(valid ? f : -INFINITY);
    if (lane == 0) fscr[wave] = wmx;
  }
  __syncthreads();
  float mx = fscr[0];
#pragma unroll
  for (int w2 = 1; w2 < kChunk / 64; ++w2) mx = fmaxf(mx, fscr[w2]);
  {
    const double wse = wave_sum_d(valid ? (double)expf(f - mx) : 0.0);
    if (lane == 0) dscr[wave] = wse;
  }
  // The count of keys above v in a descending list of 64 is found in six fixed
  // halving steps (exact for counts up to 63), with the last entry checked
  // apart for a count of 64.  The waves' searches are independent, so their LDS
  // reads interleave.  A wave's own list counts its lane index instead.
  int cnt[kChunk / 64];
  bool all_above[kChunk / 64];
#pragma unroll
  for (int w2 = 0; w2 < kChunk / 64; ++w2) {
    cnt[w2] = 0;
    all_above[w2] = srt[w2][63] > v;
  }
#pragma unroll
  for (int step = 32; step > 0; step >>= 1) {
#pragma unroll
    for (int w2 = 0; w2 < kChunk / 64; ++w2)
      if (srt[w2][cnt[w2] + step - 1] > v) cnt[w2] += step;
  }
  int rank = 0;
#pragma unroll
  for (int w2 = 0; w2 < kChunk / 64; ++w2)
    rank += w2 == wave ? lane : all_above[w2] ? 64 : cnt[w2];
  const size_t cbase = (row * nchunk + chunk) * (size_t)K;
  if (rank < K) cand[cbase + rank] = v;
  __syncthreads();
  if (tid == 0) {
    double se = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < kChunk / 64; ++w2) se += dscr[w2];
    stats[row * nchunk + chunk] = make_float2(mx, (float)se);
  }
}

__global__ void __launch_bounds__(256) select_merge_kernel(
    const uint64_t* __restrict__ cand, const float2* __restrict__ stats, int T, int C,
    int row_offset, int K, int nchunk, int act, int32_t* __restrict__ idx,
    float* __restrict__ logg, float* __restrict__ lse_s, RowLens rl) {
  extern __shared__ uint64_t lists[];  // nchunk * K keys
  const size_t row = blockIdx.x;
  const int t = (int)(row % T);
  const int ct = row_history(t, row_offset, C, rl, row / T);
  const int nc = nchunk * K;
  const uint64_t* crow = cand + row * (size_t)nc;
  copy_keys_to_lds<16>(lists, crow, nc, (int)threadIdx.x, (int)blockDim.x);
  // The chunks' (max, sum of exp) are combined by the last wave (nchunk <= 64,
  // lane i holds chunk i) while wave 0 folds the waves' lists: fp32 max, fp64
  // sum of the chunk sums rescaled to it, one fp32 rounding of max + log(sum).
  const int lane = threadIdx.x & 63, wave = (int)(threadIdx.x >> 6);
  __shared__ float lse_sh;
  float2 st = make_float2(-INFINITY, 0.0f);
  if (wave == 3 && lane < nchunk) st = stats[row * nchunk + lane];
  __syncthreads();  // lists[] complete
  // Each wave folds a share of the lists into its top list in registers, then
  // wave 0 folds the waves' lists (the two-stage path runs with K <= 64 only).
  __shared__ uint64_t wl[4 * 64];
  const uint64_t top = merge_top64<4>(lists, nchunk, K, wl);
  if (wave == 3) {
    const float M = wave_max(st.x);
    const double S =
        wave_sum_d(st.y > 0.0f ? (double)st.y * exp((double)st.x - (double)M) : 0.0);
    if (lane == 0) lse_sh = ct > 0 ? (float)((double)M + log(S)) : -INFINITY;
  }
  const int kk = min(K, ct);
  // Wave 0 holds the winners by rank; it re-sorts them by block index in
  // registers (key: block index, then the score's order key) while the last
  // wave combines the statistics.
  uint64_t byidx = ~0ull;
  if (wave == 0) {
    if (lane < kk)
      byidx = ((uint64_t)(0xFFFFFFFFu - (uint32_t)(top & 0xFFFFFFFFull)) << 32) | (top >> 32);
    byidx = bitonic_sort_asc64(byidx, lane);
  }
  __syncthreads();  // lse_sh in LDS
  const float lse = lse_sh;
  int32_t* irow = idx + row * (size_t)K;
  float* lrow = logg + row * (size_t)K;
  if (wave == 0 && lane < kk) {
    irow[lane] = (int)(byidx >> 32);
    lrow[lane] = gate_log(from_order_key((uint32_t)byidx), lse, act);
  }
  for (int p = kk + threadIdx.x; p < K; p += blockDim.x) {
    irow[p] = -1;
    lrow[p] = 0.0f;
  }
  if (threadIdx.x == 0) lse_s[row] = lse;
}

size_t select_workspace_bytes(int rows_bk, int T, int C, int K) {
  if (C <= kLongHistory) return 0;
  const size_t rows = (size_t)rows_bk * T;
  const size_t nchunk = (size_t)(C + kChunk - 1) / kChunk;
  const size_t cand = rows * nchunk * K * sizeof(uint64_t);
  return ((cand + 255) & ~(size_t)255) + rows * nchunk * sizeof(float2);
}

hipError_t launch_select_long(const float* s, const float* qbar, const void* kbar,
                              bool kbar_bf16, int kbar_ld, int d, double scale, int rows_bk,
                              int T, int C, int row_offset, int K, int act, float* s_out,
                              int32_t* idx, float* logg, float* lse_s, void* ws,
                              hipStream_t st, const RowLens& rl) {
  const size_t rows = (size_t)rows_bk * T;
  const int nchunk = (C + kChunk - 1) / kChunk;
  uint64_t* cand = (uint64_t*)ws;
  const size_t cand_bytes = rows * nchunk * K * sizeof(uint64_t);
  float2* stats = (float2*)((char*)ws + ((cand_bytes + 255) & ~(size_t)255));
  {
    ProfScope ps("select_chunk", st);
    dim3 grid(nchunk, (unsigned)rows);
    if (kbar_bf16)
      hipLaunchKernelGGL(select_chunk_kernel<bf16_t>, grid, dim3(256), 0, st, s, qbar,
                         (const bf16_t*)nullptr, 0, (const bf16_t*)kbar, kbar_ld, d, scale, T, C,
                         row_offset, K, nchunk, s_out, cand, stats, rl);
    else
      hipLaunchKernelGGL(select_chunk_kernel<float>, grid, dim3(256), 0, st, s, qbar,
                         (const bf16_t*)nullptr, 0, (const float*)kbar, kbar_ld, d, scale, T, C,
                         row_offset, K, nchunk, s_out, cand, stats, rl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("select_merge", st);
    hipLaunchKernelGGL(select_merge_kernel, dim3((unsigned)rows), dim3(256),
                       (size_t)nchunk * K * sizeof(uint64_t), st, cand, stats, T, C, row_offset,
                       K, nchunk, act, idx, logg, lse_s, rl);
  }
  return hipGetLastError();
}

hipError_t launch_select_chunks_rawq(const bf16_t* q, int qgroup, const void* kbar,
                                     bool kbar_bf16, int kbar_ld, int d, double scale, int rows,
                                     int C, int K, const RowLens& rl, uint64_t* cand,
                                     float2* stats, hipStream_t st) {
  const int nchunk = (C + kChunk - 1) / kChunk;
  if (nchunk == 0) return hipSuccess;
  ProfScope ps("step_select_chunk", st);
  dim3 grid(nchunk, (unsigned)rows);
  if (kbar_bf16)
    hipLaunchKernelGGL(select_chunk_kernel<bf16_t>, grid, dim3(256), 0, st, (const float*)nullptr,
                       (const float*)nullptr, q, qgroup, (const bf16_t*)kbar, kbar_ld, d, scale,
                       1, C, C, K, nchunk, (float*)nullptr, cand, stats, rl);
  else
    hipLaunchKernelGGL(select_chunk_kernel<float>, grid, dim3(256), 0, st, (const float*)nullptr,
                       (const float*)nullptr, q, qgroup, (const float*)kbar, kbar_ld, d, scale, 1,
                       C, C, K, nchunk, (float*)nullptr, cand, stats, rl);
  return hipGetLastError();
}

hipError_t launch_topk(const float* s, const float* qbar, const void* kbar, bool kbar_bf16,
                       int kbar_ld, int d, double scale, float* s_out, int rows_bk, int T, int C,
                       int row_offset, int K, int act, int32_t* idx, float* logg,
                       float* lse_s, hipStream_t st, const RowLens& rl) {
  const size_t rows = (size_t)rows_bk * T;
  ProfScope ps("topk", st);
  // keys per lane sized to the longest row (C <= kLongHistory here)
  auto go = [&](auto per) {
    constexpr int PER = decltype(per)::value;
    if (s)
      hipLaunchKernelGGL((topk_given_kernel<PER>), dim3((unsigned)((rows + 3) / 4)), dim3(256),
                         0, st, s, rows, T, C, row_offset, K, act, idx, logg, lse_s, rl);
    else if (kbar_bf16)
      hipLaunchKernelGGL((topk_standin_kernel<bf16_t, PER>), dim3((unsigned)rows), dim3(256), 0,
                         st, qbar, (const bf16_t*)kbar, kbar_ld, d, scale, s_out, T, C,
                         row_offset, K, act, idx, logg, lse_s, rl);
    else
      hipLaunchKernelGGL((topk_standin_kernel<float, PER>), dim3((unsigned)rows), dim3(256), 0,
                         st, qbar, (const float*)kbar, kbar_ld, d, scale, s_out, T, C,
                         row_offset, K, act, idx, logg, lse_s, rl);
  };
  if (C <= 128)
    go(std::integral_constant<int, 2>());
  else if (C <= 256)
    go(std::integral_constant<int, 4>());
  else
    go(std::integral_constant<int, kLongHistory / 64>());
  return hipGetLastError();
}

}  // namespace sas
