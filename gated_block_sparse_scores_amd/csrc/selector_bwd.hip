// Backward of the stand-in selector: dL/ds to the pooled block summaries, and
// through the mean pools to q and k.
//
// picx.dev summary of SAS, 'Key Idea: Differentiable Continuous Gating' (the
// selector is trained through the gates) and 'Theoretical Foundation' (the hard
// Top-K passes no gradient); evolve.pub review FAQ (pooling-based block
// summaries feed the selector).  With s[t][m] = scale * qbar[t] . kbar[m] on the
// history m < t of a training row,
//   dqbar[t] = scale * sum_{m < t} ds[t][m] kbar[m]
//   dkbar[m] = scale * sum_{t > m} ds[t][m] qbar[t]
// and the pools spread them back over what they averaged:
//   dq[h][i] += dqbar[t(i)] / (G n_t),  dk[j] += dkbar[m(j)] / n_m.
#include "common.h"
#include "internal.h"

namespace sas {

constexpr int kSbRows = 16;   // output rows per workgroup
constexpr int kSbChunk = 32;  // inner rows staged in LDS per pass

// Grid (ceil(T / 16), hkv, 2 b): z & 1 picks the output (0: dqbar, 1: dkbar).
// Each pass stages a 16 x 32 tile of the triangular weights (ds, or its
// transpose for dkbar) and the 32 matching summary rows in LDS; a thread owns
// one column of RPT output rows.  fp32 accumulation in ascending inner order.
template <int D>
__global__ void __launch_bounds__(256) selector_bwd_kernel(const float* __restrict__ ds,
                                                           const float* __restrict__ qbar,
                                                           const float* __restrict__ kbar,
                                                           int T, float scale,
                                                           float* __restrict__ dqbar,
                                                           float* __restrict__ dkbar) {
  constexpr int RSTEP = 256 / D;          // thread-row stride
  constexpr int RPT = kSbRows / RSTEP;    // output rows per thread
  __shared__ float W[kSbRows][kSbChunk + 1];
  __shared__ __align__(16) float X[kSbChunk][D];
  const int r0 = blockIdx.x * kSbRows;
  const int kv = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  const size_t head = (size_t)b * gridDim.y + kv;
  const float* dsh = ds + head * (size_t)T * T;
  const float* src = (which ? qbar : kbar) + head * (size_t)T * D;
  float* dst = (which ? dkbar : dqbar) + head * (size_t)T * D;
  const int col = threadIdx.x % D, rt = threadIdx.x / D;
  const int rend = min(r0 + kSbRows, T);
  // inner rows: u < r for dqbar, u > r for dkbar
  const int u_lo = which ? r0 + 1 : 0;
  const int u_hi = which ? T : rend - 1;
  float acc[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) acc[k] = 0.0f;
  for (int u0 = u_lo; u0 < u_hi; u0 += kSbChunk) {
#pragma unroll
    for (int e0 = 0; e0 < kSbRows * kSbChunk; e0 += 256) {
      const int e = e0 + (int)threadIdx.x;
      // consecutive threads read consecutive addresses of ds in both cases
      const int i = which ? e % kSbRows : e / kSbChunk;
      const int j = which ? e / kSbRows : e % kSbChunk;
      const int r = r0 + i, u = u0 + j;
      float wv = 0.0f;
      if (r < T && u < T && (which ? u > r : u < r))
        wv = which ? dsh[(size_t)u * T + r] : dsh[(size_t)r * T + u];
      W[i][j] = wv;
    }
#pragma unroll
    for (int e0 = 0; e0 < kSbChunk * D / 4; e0 += 256) {
      const int e = e0 + (int)threadIdx.x;
      const int j = e / (D / 4), c4 = e % (D / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (u0 + j < T) v = *reinterpret_cast<const float4*>(src + (size_t)(u0 + j) * D + c4 * 4);
      *reinterpret_cast<float4*>(&X[j][c4 * 4]) = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int j = 0; j < kSbChunk; ++j) {
      const float x = X[j][col];
#pragma unroll
      for (int k = 0; k < RPT; ++k) acc[k] = fmaf(W[rt + k * RSTEP][j], x, acc[k]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int r = r0 + rt + k * RSTEP;
    if (r < T) dst[(size_t)r * D + col] = acc[k] * scale;
  }
}

// x[b][h][i][c] += xbar[b][h / group][i / bs][c] / (group * n_t), for dq
// (its b * hq planes) and dk (b * hkv planes) in one launch.  Grid
// (ceil(n d / (8 * 256 * kSpreadVec)), planes): a workgroup covers a span of
// one (b, h) plane, each lane kSpreadVec 8-value vectors (16 bytes of bf16, 32
// of fp32) 2048 values apart, all loads issued before the arithmetic; the
// division is one reciprocal per vector (exact for the power-of-two counts of
// whole blocks).
constexpr int kSpreadVec = 4;

template <typename Tx>
__device__ __forceinline__ void load8(const Tx* p, float (&v)[8]) {
  if constexpr (sizeof(Tx) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename Tx>
__device__ __forceinline__ void store8(Tx* p, const float (&v)[8]) {
  if constexpr (sizeof(Tx) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <typename Tx>
struct SpreadPlanes {
  Tx* x[2];              // dq, dk (either may be absent: then it has no planes)
  const float* xbar[2];  // dqbar, dkbar
  int heads[2], group[2];
  int planes0;           // planes of the first tensor (b * heads[0], or 0)
};

template <typename Tx, int D>
__global__ void __launch_bounds__(256) pool_spread_kernel(SpreadPlanes<Tx> sp, int n, int bs,
                                                          const int32_t* __restrict__ lens) {
  constexpr int VPR = D / 8;  // vectors per row
  const int which = (int)blockIdx.y >= sp.planes0 ? 1 : 0;
  const int bh = (int)blockIdx.y - (which ? sp.planes0 : 0);
  const int heads = sp.heads[which], group = sp.group[which];
  const int h = bh % heads, b = bh / heads;
  const int T = (n + bs - 1) / bs;
  // ragged batch: only this sequence's own rows, n_t counted within them
  const int nlen = lens ? min(max(lens[b], 0), n) : n;
  const int nvec = nlen * VPR;
  Tx* plane = sp.x[which] + (size_t)bh * n * D;
  const float* sbase =
      sp.xbar[which] + ((size_t)b * (heads / group) + h / group) * (size_t)T * D;
  float v[kSpreadVec][8], a[kSpreadVec][8];
  int ev[kSpreadVec];
#pragma unroll
  for (int k = 0; k < kSpreadVec; ++k) {
    const int e = (blockIdx.x * kSpreadVec + k) * 256 + (int)threadIdx.x;
    ev[k] = e;
    if (e < nvec) {
      const int i = e / VPR, c = (e % VPR) * 8;
      const int t = i / bs;
      load8(plane + (size_t)i * D + c, v[k]);
      const float4 s0 = *reinterpret_cast<const float4*>(sbase + (size_t)t * D + c);
      const float4 s1 = *reinterpret_cast<const float4*>(sbase + (size_t)t * D + c + 4);
      a[k][0] = s0.x; a[k][1] = s0.y; a[k][2] = s0.z; a[k][3] = s0.w;
      a[k][4] = s1.x; a[k][5] = s1.y; a[k][6] = s1.z; a[k][7] = s1.w;
    }
  }
#pragma unroll
  for (int k = 0; k < kSpreadVec; ++k) {
    const int e = ev[k];
    if (e < nvec) {
      const int i = e / VPR, c = (e % VPR) * 8;
      const int t = i / bs;
      const float rden = 1.0f / (float)(group * min(bs, nlen - t * bs));
#pragma unroll
      for (int q = 0; q < 8; ++q) v[k][q] += a[k][q] * rden;
      store8(plane + (size_t)i * D + c, v[k]);
    }
  }
}

hipError_t launch_selector_bwd(const Dims& dm, const float* ds, const float* qbar,
                               const float* kbar, float* dqbar, float* dkbar, void* dq, void* dk,
                               hipStream_t st) {
  {
    ProfScope ps("selector_bwd", st);
    dim3 grid((dm.T + kSbRows - 1) / kSbRows, dm.hkv, 2 * dm.b);
    if (dm.d == 128)
      hipLaunchKernelGGL(selector_bwd_kernel<128>, grid, dim3(256), 0, st, ds, qbar, kbar, dm.T,
                         dm.scale, dqbar, dkbar);
    else
      hipLaunchKernelGGL(selector_bwd_kernel<64>, grid, dim3(256), 0, st, ds, qbar, kbar, dm.T,
                         dm.scale, dqbar, dkbar);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long nvec = (long)dm.n * dm.d / 8;
  const int pq = dq ? dm.b * dm.hq : 0, pk = dk ? dm.b * dm.hkv : 0;
  if (nvec == 0 || pq + pk == 0) return hipSuccess;
  ProfScope ps("pool_spread", st);
  const dim3 grid((unsigned)((nvec + 256 * kSpreadVec - 1) / (256 * kSpreadVec)),
                  (unsigned)(pq + pk));
#define SAS_SPREAD(TX, DD)                                                                    \
  {                                                                                           \
    SpreadPlanes<TX> sp;                                                                      \
    sp.x[0] = dq ? (TX*)dq : (TX*)dk;                                                         \
    sp.xbar[0] = dq ? dqbar : dkbar;                                                          \
    sp.heads[0] = dq ? dm.hq : dm.hkv;                                                        \
    sp.group[0] = dq ? dm.g : 1;                                                              \
    sp.x[1] = (TX*)dk;                                                                        \
    sp.xbar[1] = dkbar;                                                                       \
    sp.heads[1] = dm.hkv;                                                                     \
    sp.group[1] = 1;                                                                          \
    sp.planes0 = dq ? pq : pk;                                                                \
    hipLaunchKernelGGL((pool_spread_kernel<TX, DD>), grid, dim3(256), 0, st, sp, dm.n, dm.bs, \
                       dm.seq_lens);                                                          \
  }
  if (dm.bf16 && dm.d == 128)
    SAS_SPREAD(bf16_t, 128)
  else if (dm.bf16)
    SAS_SPREAD(bf16_t, 64)
  else if (dm.d == 128)
    SAS_SPREAD(float, 128)
  else
    SAS_SPREAD(float, 64)
#undef SAS_SPREAD
  return hipGetLastError();
}

}  // namespace sas
