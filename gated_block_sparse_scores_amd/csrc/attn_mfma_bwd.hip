// Fused gated block-sparse backward with bf16 MFMA (gfx950): head_dim 128,
// block 64, bf16 tensors, N a multiple of 64, G = hq / hkv a multiple of 4.
//
// picx.dev summary of SAS, 'Gradient Analysis' Eq. 5 (inner gating): the
// gradient of a block's log gate is the sum of dS over that block's keys
// (dS_ij = P_ij (dO_i . v_j - D_i), D_i = dO_i . o_i); the forward's P is
// recomputed from the saved LSE instead of being stored ('Kernel Design').
//
// Two kernels, no floating-point atomics (results are bitwise reproducible):
//  * dK/dV (key-major): one workgroup of four waves per (batch, KV head, key
//    block m).  Wave w owns keys 32*(w%2)..+32 of the block (K, V fragments in
//    registers) and query rows 32*(w/2)..+32 of every visited query tile; its
//    partial dK^T, dV^T stay in registers and the two query halves are summed
//    through LDS at the end.  The workgroup visits the diagonal query block
//    t = m and every later query block whose selection holds m (read from the
//    slot map, compacted 256 at a time), for each of the G heads, staging that
//    head's 64 rows of q and dout in LDS row-major: rows are the A operand of
//    S = Q K^T and dP = dO V^T, and the transposing LDS read
//    (ds_read_b64_tr_b16) gives the A operand of dK^T = Q^T dS, dV^T = dO^T P.
//    Block m is the only owner of the (t, slot) pairs that selected it, so it
//    also writes dlogg[t][slot] (sum over G heads, 64 rows, 64 keys) directly.
//  All tiles are copied global -> LDS with the direct-to-LDS load into double
//  buffers (the next tile streams in while the current one is computed) and
//  laid out swizzled so that row fragments and transposed reads are both free
//  of bank conflicts.
//  * dQ (query-major): the forward's tiling (2 heads x 64 rows per workgroup,
//    four waves of 32 rows), recomputing S^T = K Q^T and dP^T = V dO^T per
//    selected block and accumulating dQ^T += K^T dS^T, with K and V staged
//    row-major in LDS (K^T read with ds_read_b64_tr_b16).
#include <math.h>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {

namespace {

constexpr int D = 128;
constexpr int BS = 64;
// q / dout / K / V tiles: 64 x 128 bf16, swizzled (see mfma.h)
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- dK / dV
constexpr int DKV_NT = 256;
constexpr int DKV_MAXT = 4096;  // longest inverse list (query blocks) held in LDS
constexpr int TILE_BYTES_R = BS * TILE_LD * 2;   // one 64 x 128 tile
constexpr int DKV_SMEM = 4 * TILE_BYTES_R;       // q and dout, double buffered (also the
                                                 // 64 KB of the final half-sum)

// One item's q and dout rows (two 64 x 128 tiles) plus its 64 LSE and D
// values, held in registers between the global load and the LDS store:
// thread i holds the 16-byte chunks j = i + 256 u (u = 0..3) of each tile, so
// consecutive threads read consecutive 16 bytes.
// Ordinary loads are used here rather than the direct-to-LDS copy because the
// compiler makes every transposing LDS read wait for all direct-to-LDS copies
// in flight, which would serialise the prefetch with the compute.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct DkvStage {
  u32x4 q0, q1, q2, q3, o0, o1, o2, o3;
  float ld;
};

__device__ __forceinline__ void dkv_stage_load(DkvStage& st, const bf16_t* __restrict__ q,
                                               const bf16_t* __restrict__ dout,
                                               const float* __restrict__ lse,
                                               const float* __restrict__ Dv, size_t rb) {
  const int tid = threadIdx.x;
  constexpr int U = DKV_NT * 8;  // elements between a thread's chunks
  const u32x4* qs = reinterpret_cast<const u32x4*>(q + rb * D + tid * 8);
  const u32x4* os = reinterpret_cast<const u32x4*>(dout + rb * D + tid * 8);
  st.q0 = qs[0];
  st.o0 = os[0];
  st.q1 = qs[U / 8];
  st.o1 = os[U / 8];
  st.q2 = qs[2 * U / 8];
  st.o2 = os[2 * U / 8];
  st.q3 = qs[3 * U / 8];
  st.o3 = os[3 * U / 8];
  // every thread loads (threads past 128 re-read a D value) so the load is
  // unconditional and its register is never written on another path
  st.ld = (tid < BS ? lse : Dv)[rb + (tid & (BS - 1))];
}

// Chunk j = tid + 256 u sits in row j / 16 = tid / 16 + 16 u at chunk tid % 16;
// the swizzle depends on row % 16 only, so the four rows share one pattern.
__device__ __forceinline__ void dkv_stage_store(const DkvStage& st, bf16_t* Qb, bf16_t* Ob,
                                                float* Lb, float* Db) {
  const int tid = threadIdx.x;
  const int o = swz(tid >> 4, (tid & 15) * 8);
  constexpr int U = 16 * TILE_LD;
  *reinterpret_cast<u32x4*>(Qb + o) = st.q0;
  *reinterpret_cast<u32x4*>(Ob + o) = st.o0;
  *reinterpret_cast<u32x4*>(Qb + o + U) = st.q1;
  *reinterpret_cast<u32x4*>(Ob + o + U) = st.o1;
  *reinterpret_cast<u32x4*>(Qb + o + 2 * U) = st.q2;
  *reinterpret_cast<u32x4*>(Ob + o + 2 * U) = st.o2;
  *reinterpret_cast<u32x4*>(Qb + o + 3 * U) = st.q3;
  *reinterpret_cast<u32x4*>(Ob + o + 3 * U) = st.o3;
  if (tid < BS)
    Lb[tid] = st.ld;
  else if (tid < 2 * BS)
    Db[tid - BS] = st.ld;
}

__global__ void __launch_bounds__(DKV_NT) bwd_dkdv_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ Dv,
    const float* __restrict__ logg, const uint8_t* __restrict__ slotmap,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ dlogg) {
  __shared__ __align__(16) unsigned char smem[DKV_SMEM];
  __shared__ float Ls[2][BS], Dl[2][BS];
  __shared__ float red[4];
  // Query blocks t attending to block m (ascending), with the slot of m in
  // t's selection (0xFF on the diagonal) and its log gate (x log2 e).
  __shared__ uint16_t lst[DKV_MAXT];
  __shared__ uint8_t lslot[DKV_MAXT];
  __shared__ float lbias[DKV_MAXT];
  __shared__ int scan_scr[16];

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
  const int kt = wave & 1, qh = wave >> 1;
  const int key = kt * 32 + c;  // key within the block (this lane's column)

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
  // Query blocks attending to block m, in ascending t: the diagonal t = m,
  // then every t > m whose selection holds m (slot map row, compacted into
  // LDS 256 entries per pass).
  const uint8_t* srow = slotmap + (bk * dm.T + m) * (size_t)dm.T;
  int ne = 0;
  for (int t0 = m; t0 < dm.T; t0 += DKV_NT) {
    const int tt = t0 + (int)threadIdx.x;
    const int sl = (tt < dm.T && tt != m) ? srow[tt] : 0xFF;
    const int flag = tt == m || sl != 0xFF;
    int cnt;
    const int pos = block_excl_scan(flag, scan_scr, &cnt);
    if (flag) {
      lst[ne + pos] = (uint16_t)tt;
      lslot[ne + pos] = (uint8_t)sl;
      lbias[ne + pos] =
          (sl != 0xFF && logg) ? logg[(bk * dm.T + tt) * (size_t)dm.K + sl] * LOG2E : 0.0f;
    }
    ne += cnt;
  }
  // K / V fragments in place before the loop, so that the only loads in
  // flight inside it are the staged rows.
  wait_all_loads();
  __syncthreads();

  // Flat loop over (entry, head).  The q / dout rows, LSE and D of items
  // it + 2 and it + 3 are in flight (two register stages, used alternately)
  // while item it is computed; item it + 1 is already in the other LDS buffer.
  const int items = ne * dm.g;
  auto tile_base = [&](int it) {
    const int t = lst[it / dm.g];
    const int h = kv * dm.g + it % dm.g;
    return ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS;
  };
  auto qbuf = [&](int buf) { return reinterpret_cast<bf16_t*>(smem + (2 * buf) * TILE_BYTES_R); };
  auto obuf = [&](int buf) {
    return reinterpret_cast<bf16_t*>(smem + (2 * buf + 1) * TILE_BYTES_R);
  };
  DkvStage sa_st, sb_st;
  if (items > 0) {
    dkv_stage_load(sa_st, q, dout, lse, Dv, tile_base(0));
    dkv_stage_store(sa_st, qbuf(0), obuf(0), Ls[0], Dl[0]);
  }
  if (items > 1) dkv_stage_load(sa_st, q, dout, lse, Dv, tile_base(1));
  if (items > 2) dkv_stage_load(sb_st, q, dout, lse, Dv, tile_base(2));
  __syncthreads();
  float dlsum = 0.0f;
  // One item: compute from buffer it % 2, then move `st` (item it + 1) into
  // the other buffer and start loading item it + 3 into it.
  auto item = [&](int it, DkvStage& st) {
    const int cur = it & 1;
    const int e = it / dm.g;
    const bool diag = lst[e] == m;
    const int slot = lslot[e];
    const float bias2 = lbias[e];
    const int t = lst[e];
    const bf16_t* Qs = qbuf(cur);
    const bf16_t* Os = obuf(cur);
    const float* Lc = Ls[cur];
    const float* Dc = Dl[cur];
    // S[q][key], dP[q][key] for this wave's 32 query rows and 32 keys.
    f32x16 sa, pa;
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = pa[r] = 0.0f;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      sa = mfma32(row_frag(Qs, qh * 32 + c, kc * 16 + g * 8), kf[kc], sa);
      pa = mfma32(row_frag(Os, qh * 32 + c, kc * 16 + g * 8), vf[kc], pa);
    }
    // P and dS in place: sa <- P, pa <- dS.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = qh * 32 + acc_row(r, g);
      float p = fast_exp2(fmaf(sa[r], sc2, bias2) - Lc[qi] * LOG2E);
      if (diag && key > qi) p = 0.0f;
      const float ds = p * (pa[r] - Dc[qi]);
      sa[r] = p;
      pa[r] = ds;
      dlsum += ds;
    }
    // dV^T += dO^T P, dK^T += Q^T dS over this half's two 16-row chunks.
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const bf16x8 pb = pack8(sa, ch * 8);
      const bf16x8 db = pack8(pa, ch * 8);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        dva[dt] = mfma32(tr_frag(Os, qh * 32 + ch * 16, dt * 32), pb, dva[dt]);
        dka[dt] = mfma32(tr_frag(Qs, qh * 32 + ch * 16, dt * 32), db, dka[dt]);
      }
    }
    if (it % dm.g == dm.g - 1) {
      if (!diag && dlogg) {
        // sum over the workgroup in a fixed order
        const float ws = wave_sum(dlsum);
        if (lane == 0) red[wave] = ws;
        __syncthreads();
        if (threadIdx.x == 0)
          dlogg[(bk * dm.T + t) * (size_t)dm.K + slot] = (red[0] + red[1]) + (red[2] + red[3]);
      }
      dlsum = 0.0f;
    }
    if (it + 1 < items)
      dkv_stage_store(st, qbuf(cur ^ 1), obuf(cur ^ 1), Ls[cur ^ 1], Dl[cur ^ 1]);
    if (it + 3 < items) dkv_stage_load(st, q, dout, lse, Dv, tile_base(it + 3));
    __syncthreads();    // item it + 1 stored; everyone is done with `cur`
  };
  for (int it = 0; it < items; it += 2) {
    item(it, sa_st);
    if (it + 1 < items) item(it + 1, sb_st);
  }

  // Sum the two query halves through LDS: partial [kt][dk|dv][dt*16 + r][lane].
  float* part = reinterpret_cast<float*>(smem);
  __syncthreads();
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        part[((kt * 2 + 0) * 64 + dt * 16 + r) * 64 + lane] = dka[dt][r];
        part[((kt * 2 + 1) * 64 + dt * 16 + r) * 64 + lane] = dva[dt][r];
      }
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dka[dt][r] += part[((kt * 2 + 0) * 64 + dt * 16 + r) * 64 + lane];
        dva[dt][r] += part[((kt * 2 + 1) * 64 + dt * 16 + r) * 64 + lane];
      }
    // dK = scale * (dK^T)^T, dV: lane holds key `key`, dims dt*32 + acc_row(r, g).
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
}

// ---------------------------------------------------------------- dQ
constexpr int HPW = 2;   // heads per dQ workgroup
constexpr int DQ_NW = 4;  // waves: two 32-row halves per head
constexpr int DQ_NT = 64 * DQ_NW;

__global__ void __launch_bounds__(DQ_NT, 2) bwd_dq_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ Dv,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, bf16_t* __restrict__ dq) {
  __shared__ __align__(16) bf16_t Ks[2][BS * TILE_LD];
  __shared__ __align__(16) bf16_t Vs[2][BS * TILE_LD];
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
  const int h = kv * dm.g + chunk * HPW + (wave >> 1);
  const int qt = wave & 1;
  const int qi = qt * 32 + c;

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

  const size_t row = ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS + qi;
  bf16x8 qf[8], of[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    qf[kc] = *reinterpret_cast<const bf16x8*>(q + row * D + kc * 16 + g * 8);
    of[kc] = *reinterpret_cast<const bf16x8*>(dout + row * D + kc * 16 + g * 8);
  }
  const float l2 = lse[row] * LOG2E;
  const float dval = Dv[row];
  f32x16 dqa[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[dt][r] = 0.0f;
  const float sc2 = dm.scale * LOG2E;

  __syncthreads();
  const int nb = nblk;
  const bf16_t* kbase = k + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const bf16_t* vbase = v + ((size_t)b * dm.hkv + kv) * dm.n * D;
  tile_load_lds<DQ_NW>(Ks[0], kbase + (size_t)blist[0] * BS * D);
  tile_load_lds<DQ_NW>(Vs[0], vbase + (size_t)blist[0] * BS * D);
  wait_all_loads();
  __syncthreads();
  for (int bi = 0; bi < nb; ++bi) {
    const int cur = bi & 1;
    const int m = blist[bi];
    const float off2 = bbias[bi] - l2;
    const bool diag = m == t;
    if (bi + 1 < nb) {
      tile_load_lds<DQ_NW>(Ks[cur ^ 1], kbase + (size_t)blist[bi + 1] * BS * D);
      tile_load_lds<DQ_NW>(Vs[cur ^ 1], vbase + (size_t)blist[bi + 1] * BS * D);
    }
    const bf16_t* Kc = Ks[cur];
    const bf16_t* Vc = Vs[cur];

    // Per 32-key tile: S^T, dP^T (keys x this wave's 32 queries), then dS^T
    // packed to bf16 as the B operand of the dQ^T update.
    bf16x8 db[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 sa, pa;
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[r] = pa[r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        sa = mfma32(row_frag(Kc, kt * 32 + c, kc * 16 + g * 8), qf[kc], sa);
        pa = mfma32(row_frag(Vc, kt * 32 + c, kc * 16 + g * 8), of[kc], pa);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(sa[r], sc2, off2));
        if (diag && kt * 32 + acc_row(r, g) > qi) p = 0.0f;
        pa[r] = p * (pa[r] - dval);
      }
      db[2 * kt] = pack8(pa, 0);
      db[2 * kt + 1] = pack8(pa, 8);
    }
    // dQ^T += K^T dS^T over four 16-key chunks
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        dqa[dt] = mfma32(tr_frag(Kc, ch * 16, dt * 32), db[ch], dqa[dt]);
    wait_all_loads();
    __syncthreads();
  }

  // dQ = scale * (dQ^T)^T: lane holds query qi, dims dt*32 + acc_row(r, g).
  bf16_t* op = dq + row * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dd = dt * 32 + r4 * 8 + g * 4;
      uint2 w;
      w.x = pack_bf16x2(dqa[dt][r4 * 4] * dm.scale, dqa[dt][r4 * 4 + 1] * dm.scale);
      w.y = pack_bf16x2(dqa[dt][r4 * 4 + 2] * dm.scale, dqa[dt][r4 * 4 + 3] * dm.scale);
      *reinterpret_cast<uint2*>(op + dd) = w;
    }
}

}  // namespace

bool mfma_bwd_supported(const Dims& dm) {
  return dm.bf16 && dm.d == D && dm.bs == BS && dm.n % BS == 0 && dm.g % HPW == 0 &&
         dm.T <= DKV_MAXT;
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
                       (const bf16_t*)dout, lse, ws.D, logg, ws.slotmap, (bf16_t*)dk,
                       (bf16_t*)dv, ws.dlogg_part);
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
