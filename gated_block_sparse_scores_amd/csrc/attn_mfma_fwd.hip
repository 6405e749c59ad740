// Fused gated block-sparse forward with bf16 MFMA (gfx950): head_dim 128,
// block 64, bf16 tensors, N a multiple of 64, G = hq / hkv a multiple of 4.
//
// picx.dev summary of SAS, 'Key Idea' Eq. 9 and 'Kernel Design': logits of
// the selected blocks get their normalised log gate, the current block gets 0
// (g0 = 1), unselected blocks are never loaded, the softmax is online and no
// attention matrix is stored.
//
// Work unit: one (batch, KV head, query block, 4-head chunk) tile = 4 heads x
// 64 query rows; every K/V block it needs is gathered once into LDS and serves
// the 4 heads (one selection per KV head).  Wave w owns head kv*G + 4*chunk + w
// and its 64 rows.
//   S^T = K Q^T   (32x32x16 MFMA; A = K rows from LDS, B = Q rows held in
//                  registers), so each lane holds one query column and the
//                  softmax max/sum over keys stays inside the lane (plus one
//                  exchange with lane l^32);
//   O^T += V^T P^T (A = V^T from a transposed LDS copy of V, B = P^T straight
//                  from the S^T accumulators, converted to bf16).
// The bias (log-gate) is added before the running max, in log2 units.
// Workgroups are issued longest-row-first (query block descending), KV head
// fastest, so consecutive workgroups (spread over the 8 XCDs) share K/V.
#include <math.h>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {

namespace {

constexpr int D = 128;
constexpr int BS = 64;
constexpr int KLD = D + 8;   // K row stride in LDS (bf16 elements): 272 B
constexpr int VLD = BS + 4;  // V^T row stride in LDS (bf16 elements): 136 B
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

constexpr int HPW = 4;  // heads (waves) per workgroup

struct Stage {
  static constexpr int NT = 64 * HPW;
  static constexpr int KCH = (BS * D / 8) / NT;   // 16-byte K chunks per thread
  static constexpr int VUN = (BS / 2) * (D / 8) / NT;  // (key pair, 8 dims) units per thread
  uint4 kreg[KCH];
  uint4 vreg[VUN][2];

  __device__ __forceinline__ void load(const bf16_t* __restrict__ kblk,
                                       const bf16_t* __restrict__ vblk) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int u = tid + i * NT;
      kreg[i] = *reinterpret_cast<const uint4*>(kblk + (size_t)(u >> 4) * D + (u & 15) * 8);
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + i * NT;
      const int dg = u & 15, kp = u >> 4;
      vreg[i][0] = *reinterpret_cast<const uint4*>(vblk + (size_t)(2 * kp) * D + dg * 8);
      vreg[i][1] = *reinterpret_cast<const uint4*>(vblk + (size_t)(2 * kp + 1) * D + dg * 8);
    }
  }

  __device__ __forceinline__ void store(bf16_t* Ks, bf16_t* Vt) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int u = tid + i * NT;
      *reinterpret_cast<uint4*>(Ks + (u >> 4) * KLD + (u & 15) * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + i * NT;
      const int dg = u & 15, kp = u >> 4;
      const uint32_t a[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
      const uint32_t b[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims dg*8 + 2w (low halves) and dg*8 + 2w + 1 (high halves)
        const uint32_t lo = (a[w] & 0xFFFFu) | (b[w] << 16);
        const uint32_t hi = (a[w] >> 16) | (b[w] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(Vt + (dg * 8 + 2 * w) * VLD + 2 * kp) = lo;
        *reinterpret_cast<uint32_t*>(Vt + (dg * 8 + 2 * w + 1) * VLD + 2 * kp) = hi;
      }
    }
  }
};

__global__ void __launch_bounds__(64 * HPW) fwd_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const float* __restrict__ logg, bf16_t* __restrict__ o, float* __restrict__ lse) {
  __shared__ __align__(16) bf16_t Ks[BS * KLD];
  __shared__ __align__(16) bf16_t Vt[D * VLD];
  __shared__ int blist[65];
  __shared__ float bbias[65];
  __shared__ int nblk;

  const int nchunk = dm.g / HPW;
  int tile = blockIdx.x;
  const int kv = tile % dm.hkv;
  tile /= dm.hkv;
  const int chunk = tile % nchunk;
  tile /= nchunk;
  const int b = tile % dm.b;
  const int t = dm.T - 1 - tile / dm.b;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, c = lane & 31;
  const int h = kv * dm.g + chunk * HPW + wave;

  const size_t rowbk = ((size_t)b * dm.hkv + kv) * dm.T + t;
  if (threadIdx.x == 0) {
    int cnt = 0;
    const int32_t* ir = idx + rowbk * dm.K;
    for (int s = 0; s < dm.K; ++s) {
      const int m = ir[s];
      if (m >= 0 && m < t) {
        blist[cnt] = m;
        bbias[cnt] = logg ? logg[rowbk * dm.K + s] * LOG2E : 0.0f;
        ++cnt;
      }
    }
    blist[cnt] = t;
    bbias[cnt] = 0.0f;
    nblk = cnt + 1;
  }

  // Q^T fragments (B operand): query qt*32 + c, dims kc*16 + g*8 .. +8.
  const bf16_t* qrow = q + (((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS) * D;
  bf16x8 qf[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      qf[qt][kc] = *reinterpret_cast<const bf16x8*>(qrow + (size_t)(qt * 32 + c) * D + kc * 16 +
                                                    g * 8);

  f32x16 oacc[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][qt][r] = 0.0f;
  float mrun[2] = {-INFINITY, -INFINITY};
  float lrun[2] = {0.0f, 0.0f};
  const float sc2 = dm.scale * LOG2E;

  __syncthreads();
  const int nb = nblk;
  const bf16_t* kbase = k + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const bf16_t* vbase = v + ((size_t)b * dm.hkv + kv) * dm.n * D;
  Stage st;
  st.load(kbase + (size_t)blist[0] * BS * D, vbase + (size_t)blist[0] * BS * D);

  for (int bi = 0; bi < nb; ++bi) {
    __syncthreads();
    st.store(Ks, Vt);
    __syncthreads();
    const int m = blist[bi];
    const float bias2 = bbias[bi];
    const bool diag = m == t;
    if (bi + 1 < nb)
      st.load(kbase + (size_t)blist[bi + 1] * BS * D, vbase + (size_t)blist[bi + 1] * BS * D);

    // S^T[key][query] for the 64 keys of this block and the wave's 64 queries.
    f32x16 sacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][qt][r] = 0.0f;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(Ks + (kt * 32 + c) * KLD + kc * 16 + g * 8);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) sacc[kt][qt] = mfma32(a, qf[qt][kc], sacc[kt][qt]);
      }
    }

    // Online softmax, per query column (log2 domain).
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float z = fmaf(sacc[kt][qt][r], sc2, bias2);
          if (diag && (kt * 32 + acc_row(r, g)) > (qt * 32 + c)) z = -INFINITY;
          sacc[kt][qt][r] = z;
          mx = fmaxf(mx, z);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[qt], mx);
      const float alpha = fast_exp2(mrun[qt] - mnew);
      mrun[qt] = mnew;
      float ls = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[kt][qt][r] - mnew);
          sacc[kt][qt][r] = p;
          ls += p;
        }
      lrun[qt] = lrun[qt] * alpha + ls;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][qt][r] *= alpha;
    }

    // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int kt = ch >> 1, half = ch & 1;
      bf16x8 pf[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) pf[qt] = pack8(sacc[kt][qt], half * 8);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16_t* vr = Vt + (dt * 32 + c) * VLD + ch * 16 + g * 4;
        const bf16x8 a = cat4(*reinterpret_cast<const bf16x4*>(vr),
                              *reinterpret_cast<const bf16x4*>(vr + 8));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) oacc[dt][qt] = mfma32(a, pf[qt], oacc[dt][qt]);
      }
    }
  }

  // Normalise and store o (bf16) and LSE (natural log).
  bf16_t* orow = o + (((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS) * D;
  float* lrow = lse + ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float ltot = lrun[qt] + __shfl_xor(lrun[qt], 32);
    const float inv = 1.0f / ltot;
    if (g == 0) lrow[qt * 32 + c] = (mrun[qt] + log2f(ltot)) * LN2;
    bf16_t* op = orow + (size_t)(qt * 32 + c) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dd = dt * 32 + r4 * 8 + g * 4;
        uint2 w;
        w.x = pack_bf16x2(oacc[dt][qt][r4 * 4 + 0] * inv, oacc[dt][qt][r4 * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[dt][qt][r4 * 4 + 2] * inv, oacc[dt][qt][r4 * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + dd) = w;
      }
  }
}

}  // namespace

bool mfma_fwd_supported(const Dims& dm) {
  return dm.bf16 && dm.d == D && dm.bs == BS && dm.n % BS == 0 && dm.g % HPW == 0;
}

hipError_t launch_fwd_mfma(const Dims& dm, const void* q, const void* k, const void* v,
                           const int32_t* idx, const float* logg, void* o, float* lse,
                           hipStream_t st) {
  const size_t tiles = (size_t)dm.b * dm.hkv * dm.T * (dm.g / HPW);
  ProfScope ps("fwd_mfma", st);
  hipLaunchKernelGGL(fwd_mfma_kernel, dim3((unsigned)tiles), dim3(64 * HPW), 0, st, dm,
                     (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, idx, logg,
                     (bf16_t*)o, lse);
  return hipGetLastError();
}

}  // namespace sas
