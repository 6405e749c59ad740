// Fused gated block-sparse backward with bf16 MFMA (gfx950): head_dim 128,
// block 64, bf16 tensors, N a multiple of 64, G = hq / hkv a multiple of 4.
//
// picx.dev summary of SAS, 'Gradient Analysis' Eq. 5 (inner gating): the
// gradient of a block's log gate is the sum of dS over that block's keys
// (dS_ij = P_ij (dO_i . v_j - D_i), D_i = dO_i . o_i); the forward's P is
// recomputed from the saved LSE instead of being stored ('Kernel Design').
//
// Two kernels, no floating-point atomics (results are bitwise reproducible):
//  * dK/dV (key-major): one workgroup of two waves per (batch, KV head, key
//    block m); wave w owns keys 32w..32w+31 of the block with K, V held in
//    registers and dK^T, dV^T accumulated in registers.  It visits the
//    diagonal query block t = m and then every query block that selected m
//    (inverse selection list, ascending t), for each of the G heads, staging
//    that head's 64 rows of q and dout in LDS twice: row-major (A operand of
//    S = Q K^T and dP = dO V^T) and transposed (A operand of dK^T = Q^T dS and
//    dV^T = dO^T P).  Since block m is the only owner of the (t, slot) pairs
//    that selected it, it also writes dlogg[t][slot] (sum over G heads, 64
//    rows and 64 keys) directly.
//  * dQ (query-major): the forward's tiling (4 heads x 64 rows per
//    workgroup), recomputing S^T = K Q^T and dP^T = V dO^T per selected block
//    and accumulating dQ^T += K^T dS^T, with K staged row-major and
//    transposed and V row-major in LDS.
#include <math.h>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {

namespace {

constexpr int D = 128;
constexpr int BS = 64;
constexpr int RLD = D + 8;   // row-major tile stride (bf16 elements): 272 B
constexpr int TLD = BS + 4;  // transposed tile stride (bf16 elements): 136 B
constexpr float LOG2E = 1.4426950408889634f;

// Stages 64 rows x 128 dims of a bf16 tensor (row stride D) into LDS twice:
// row-major (stride RLD) and transposed (stride TLD).  NT threads.
template <int NT>
__device__ __forceinline__ void stage_both(const bf16_t* __restrict__ src, bf16_t* rowm,
                                           bf16_t* trans) {
  constexpr int UN = (BS / 2) * (D / 8) / NT;  // (row pair, 8 dims) units per thread
  uint4 ra[UN], rb[UN];
#pragma unroll
  for (int i = 0; i < UN; ++i) {
    const int u = threadIdx.x + i * NT;
    const int dg = u & 15, rp = u >> 4;
    ra[i] = *reinterpret_cast<const uint4*>(src + (size_t)(2 * rp) * D + dg * 8);
    rb[i] = *reinterpret_cast<const uint4*>(src + (size_t)(2 * rp + 1) * D + dg * 8);
  }
#pragma unroll
  for (int i = 0; i < UN; ++i) {
    const int u = threadIdx.x + i * NT;
    const int dg = u & 15, rp = u >> 4;
    *reinterpret_cast<uint4*>(rowm + (2 * rp) * RLD + dg * 8) = ra[i];
    *reinterpret_cast<uint4*>(rowm + (2 * rp + 1) * RLD + dg * 8) = rb[i];
    const uint32_t a[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
    const uint32_t b[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (a[w] & 0xFFFFu) | (b[w] << 16);
      const uint32_t hi = (a[w] >> 16) | (b[w] & 0xFFFF0000u);
      *reinterpret_cast<uint32_t*>(trans + (dg * 8 + 2 * w) * TLD + 2 * rp) = lo;
      *reinterpret_cast<uint32_t*>(trans + (dg * 8 + 2 * w + 1) * TLD + 2 * rp) = hi;
    }
  }
}

// Row-major only.
template <int NT>
__device__ __forceinline__ void stage_rows(const bf16_t* __restrict__ src, bf16_t* rowm) {
  constexpr int UN = BS * (D / 8) / NT;
  uint4 r[UN];
#pragma unroll
  for (int i = 0; i < UN; ++i) {
    const int u = threadIdx.x + i * NT;
    r[i] = *reinterpret_cast<const uint4*>(src + (size_t)(u >> 4) * D + (u & 15) * 8);
  }
#pragma unroll
  for (int i = 0; i < UN; ++i) {
    const int u = threadIdx.x + i * NT;
    *reinterpret_cast<uint4*>(rowm + (u >> 4) * RLD + (u & 15) * 8) = r[i];
  }
}

__device__ __forceinline__ bf16x8 lds8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// A operand from a transposed tile: row `row`, k-values for 16-column chunk
// `ch` in the accumulator-row order of lane group g.
__device__ __forceinline__ bf16x8 trans_frag(const bf16_t* tile, int row, int ch, int g) {
  const bf16_t* p = tile + row * TLD + ch * 16 + g * 4;
  return cat4(*reinterpret_cast<const bf16x4*>(p), *reinterpret_cast<const bf16x4*>(p + 8));
}

// ---------------------------------------------------------------- dK / dV
constexpr int DKV_NT = 128;

__global__ void __launch_bounds__(DKV_NT) bwd_dkdv_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ Dv,
    const float* __restrict__ logg, const int* __restrict__ csr_count,
    const int* __restrict__ csr_off, const int* __restrict__ csr_list,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ dlogg) {
  __shared__ __align__(16) bf16_t Qs[BS * RLD];
  __shared__ __align__(16) bf16_t Os[BS * RLD];
  __shared__ __align__(16) bf16_t Qt[D * TLD];
  __shared__ __align__(16) bf16_t Ot[D * TLD];
  __shared__ float Ls[BS], Dl[BS];
  __shared__ float red[2];

  // key blocks ascending (low blocks are selected by the most query blocks, so
  // the longest inverse lists go first), KV head fastest
  int tile = blockIdx.x;
  const int kv = tile % dm.hkv;
  tile /= dm.hkv;
  const int b = tile % dm.b;
  const int m = tile / dm.b;
  const size_t bk = (size_t)b * dm.hkv + kv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, c = lane & 31;
  const int key = wave * 32 + c;  // key within the block owned by this lane's column

  // K, V of the wave's 32 keys as B operands (column = key, k = dims).
  const size_t kvrow = (bk * dm.n + (size_t)m * BS + key) * D;
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    kf[kc] = *reinterpret_cast<const bf16x8*>(k + kvrow + kc * 16 + g * 8);
    vf[kc] = *reinterpret_cast<const bf16x8*>(v + kvrow + kc * 16 + g * 8);
  }
  f32x16 dka[4], dva[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[dt][r] = dva[dt][r] = 0.0f;

  const float sc2 = dm.scale * LOG2E;
  const int ncsr = csr_count[bk * dm.T + m];
  const int off = csr_off[bk * dm.T + m];
  for (int ei = -1; ei < ncsr; ++ei) {
    int t, slot;
    if (ei < 0) {
      t = m;
      slot = -1;
    } else {
      const int e = csr_list[off + ei];
      t = e >> 8;
      slot = e & 255;
    }
    const bool diag = slot < 0;
    const float bias2 = (!diag && logg) ? logg[(bk * dm.T + t) * (size_t)dm.K + slot] * LOG2E
                                        : 0.0f;
    float dlsum = 0.0f;
    for (int hh = 0; hh < dm.g; ++hh) {
      const int h = kv * dm.g + hh;
      const size_t rbase = ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS;
      __syncthreads();
      stage_both<DKV_NT>(q + rbase * D, Qs, Qt);
      stage_both<DKV_NT>(dout + rbase * D, Os, Ot);
      if (threadIdx.x < BS) {
        Ls[threadIdx.x] = lse[rbase + threadIdx.x] * LOG2E;
        Dl[threadIdx.x] = Dv[rbase + threadIdx.x];
      }
      __syncthreads();

      // S[q][key] and dP[q][key] for the 64 query rows (two 32-row tiles).
      f32x16 sa[2], pa[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[qt][r] = pa[qt][r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const bf16x8 aq = lds8(Qs + (qt * 32 + c) * RLD + kc * 16 + g * 8);
          const bf16x8 ao = lds8(Os + (qt * 32 + c) * RLD + kc * 16 + g * 8);
          sa[qt] = mfma32(aq, kf[kc], sa[qt]);
          pa[qt] = mfma32(ao, vf[kc], pa[qt]);
        }
      }
      // P and dS in place: sa <- P, pa <- dS.
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qt * 32 + acc_row(r, g);
          float p = fast_exp2(fmaf(sa[qt][r], sc2, bias2) - Ls[qi]);
          if (diag && key > qi) p = 0.0f;
          const float ds = p * (pa[qt][r] - Dl[qi]);
          sa[qt][r] = p;
          pa[qt][r] = ds;
          dlsum += ds;
        }
      // dV^T += dO^T P, dK^T += Q^T dS over four 16-query chunks.
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const int qt = ch >> 1, half = ch & 1;
        const bf16x8 pb = pack8(sa[qt], half * 8);
        const bf16x8 db = pack8(pa[qt], half * 8);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          dva[dt] = mfma32(trans_frag(Ot, dt * 32 + c, ch, g), pb, dva[dt]);
          dka[dt] = mfma32(trans_frag(Qt, dt * 32 + c, ch, g), db, dka[dt]);
        }
      }
    }
    if (!diag && dlogg) {
      // sum over the workgroup (2 waves) in a fixed order
      const float ws = wave_sum(dlsum);
      if (lane == 0) red[wave] = ws;
      __syncthreads();
      if (threadIdx.x == 0) dlogg[(bk * dm.T + t) * (size_t)dm.K + slot] = red[0] + red[1];
    }
  }

  // dK = scale * dK^T^T, dV: lane holds key `key`, dims dt*32 + acc_row(r, g).
  bf16_t* dkp = dk + kvrow;
  bf16_t* dvp = dv + kvrow;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dd = dt * 32 + r4 * 8 + g * 4;
      uint2 wk, wv;
      wk.x = pack_bf16x2(dka[dt][r4 * 4] * dm.scale, dka[dt][r4 * 4 + 1] * dm.scale);
      wk.y = pack_bf16x2(dka[dt][r4 * 4 + 2] * dm.scale, dka[dt][r4 * 4 + 3] * dm.scale);
      wv.x = pack_bf16x2(dva[dt][r4 * 4], dva[dt][r4 * 4 + 1]);
      wv.y = pack_bf16x2(dva[dt][r4 * 4 + 2], dva[dt][r4 * 4 + 3]);
      *reinterpret_cast<uint2*>(dkp + dd) = wk;
      *reinterpret_cast<uint2*>(dvp + dd) = wv;
    }
}

// ---------------------------------------------------------------- dQ
constexpr int HPW = 4;
constexpr int DQ_NT = 64 * HPW;

__global__ void __launch_bounds__(DQ_NT) bwd_dq_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ Dv,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, bf16_t* __restrict__ dq) {
  __shared__ __align__(16) bf16_t Ks[BS * RLD];
  __shared__ __align__(16) bf16_t Vs[BS * RLD];
  __shared__ __align__(16) bf16_t Kt[D * TLD];
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
      const int mm = ir[s];
      if (mm >= 0 && mm < t) {
        blist[cnt] = mm;
        bbias[cnt] = logg ? logg[rowbk * dm.K + s] * LOG2E : 0.0f;
        ++cnt;
      }
    }
    blist[cnt] = t;
    bbias[cnt] = 0.0f;
    nblk = cnt + 1;
  }

  const size_t rbase = ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS;
  bf16x8 qf[2][8], of[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const size_t o = (rbase + qt * 32 + c) * D + kc * 16 + g * 8;
      qf[qt][kc] = *reinterpret_cast<const bf16x8*>(q + o);
      of[qt][kc] = *reinterpret_cast<const bf16x8*>(dout + o);
    }
  float l2[2], dd_[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    l2[qt] = lse[rbase + qt * 32 + c] * LOG2E;
    dd_[qt] = Dv[rbase + qt * 32 + c];
  }
  f32x16 dqa[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqa[dt][qt][r] = 0.0f;
  const float sc2 = dm.scale * LOG2E;

  __syncthreads();
  const int nb = nblk;
  const bf16_t* kbase = k + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const bf16_t* vbase = v + ((size_t)b * dm.hkv + kv) * dm.n * D;
  for (int bi = 0; bi < nb; ++bi) {
    const int m = blist[bi];
    const float bias2 = bbias[bi];
    const bool diag = m == t;
    __syncthreads();
    stage_both<DQ_NT>(kbase + (size_t)m * BS * D, Ks, Kt);
    stage_rows<DQ_NT>(vbase + (size_t)m * BS * D, Vs);
    __syncthreads();

    // S^T[key][query], dP^T[key][query]
    f32x16 sa[2][2], pa[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[kt][qt][r] = pa[kt][qt][r] = 0.0f;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 ak = lds8(Ks + (kt * 32 + c) * RLD + kc * 16 + g * 8);
        const bf16x8 av = lds8(Vs + (kt * 32 + c) * RLD + kc * 16 + g * 8);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          sa[kt][qt] = mfma32(ak, qf[qt][kc], sa[kt][qt]);
          pa[kt][qt] = mfma32(av, of[qt][kc], pa[kt][qt]);
        }
      }
    }
    // dS^T (in pa)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kt * 32 + acc_row(r, g);
          float p = fast_exp2(fmaf(sa[kt][qt][r], sc2, bias2) - l2[qt]);
          if (diag && kk > qt * 32 + c) p = 0.0f;
          pa[kt][qt][r] = p * (pa[kt][qt][r] - dd_[qt]);
        }
    // dQ^T += K^T dS^T over four 16-key chunks
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int kt = ch >> 1, half = ch & 1;
      bf16x8 db[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) db[qt] = pack8(pa[kt][qt], half * 8);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 a = trans_frag(Kt, dt * 32 + c, ch, g);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) dqa[dt][qt] = mfma32(a, db[qt], dqa[dt][qt]);
      }
    }
  }

  // dQ = scale * (dQ^T)^T: lane holds query qt*32 + c, dims dt*32 + acc_row(r, g).
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    bf16_t* op = dq + (rbase + qt * 32 + c) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dd = dt * 32 + r4 * 8 + g * 4;
        uint2 w;
        w.x = pack_bf16x2(dqa[dt][qt][r4 * 4] * dm.scale, dqa[dt][qt][r4 * 4 + 1] * dm.scale);
        w.y = pack_bf16x2(dqa[dt][qt][r4 * 4 + 2] * dm.scale, dqa[dt][qt][r4 * 4 + 3] * dm.scale);
        *reinterpret_cast<uint2*>(op + dd) = w;
      }
  }
}

}  // namespace

bool mfma_bwd_supported(const Dims& dm) {
  return dm.bf16 && dm.d == D && dm.bs == BS && dm.n % BS == 0 && dm.g % HPW == 0;
}

hipError_t launch_bwd_mfma(const Dims& dm, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse, const int32_t* idx,
                           const float* logg, void* dq, void* dk, void* dv,
                           const BwdWorkspace& ws, int* nchunk_out, hipStream_t st) {
  // dlogg is written whole by the dK/dV kernel (one partial per row).
  *nchunk_out = 1;
  {
    const size_t wgs = (size_t)dm.b * dm.hkv * dm.T;
    ProfScope ps("bwd_dkdv_mfma", st);
    hipLaunchKernelGGL(bwd_dkdv_mfma_kernel, dim3((unsigned)wgs), dim3(DKV_NT), 0, st, dm,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                       (const bf16_t*)dout, lse, ws.D, logg, ws.csr_count, ws.csr_off,
                       ws.csr_list, (bf16_t*)dk, (bf16_t*)dv, ws.dlogg_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const size_t tiles = (size_t)dm.b * dm.hkv * dm.T * (dm.g / HPW);
    ProfScope ps("bwd_dq_mfma", st);
    hipLaunchKernelGGL(bwd_dq_mfma_kernel, dim3((unsigned)tiles), dim3(DQ_NT), 0, st, dm,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                       (const bf16_t*)dout, lse, ws.D, idx, logg, (bf16_t*)dq);
  }
  return hipGetLastError();
}

}  // namespace sas
