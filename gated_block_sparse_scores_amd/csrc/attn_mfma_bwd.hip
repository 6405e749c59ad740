// Fused gated block-sparse backward with bf16 MFMA (gfx950): head_dim 128,
// block 64, bf16 tensors, N a multiple of 64, G = hq / hkv even.
//
// picx.dev summary of SAS, 'Gradient Analysis' Eq. 5 (inner gating): the
// gradient of a block's log gate is the sum of dS over that block's keys
// (dS_ij = P_ij (dO_i . v_j - D_i), D_i = dO_i . o_i); the forward's P is
// recomputed from the saved LSE instead of being stored ('Kernel Design').
//
// Two kernels, no floating-point atomics (results are bitwise reproducible):
//  * dK/dV (key-major): one workgroup of four waves per (batch, KV head, key
//    block m), two workgroups per CU.  Wave w computes S and dP for keys
//    32*(w%2)..+32 of the block (K, V fragments in registers) and query rows
//    32*(w/2)..+32 of every visited query tile, and accumulates dK^T, dV^T for
//    those keys and head dims 64*(w/2)..+64 over all 64 rows, taking the P / dS
//    fragments of the other 32 rows from its partner wave (w ^ 2) through LDS;
//    each wave owns its part of dK and dV, with no reduction at the end.  The
//    workgroup visits the diagonal query block t = m and every later query
//    block whose selection holds m (read from the slot map, compacted 256 at a
//    time), for each of the G heads, staging that head's 64 rows of q and dout
//    in LDS row-major: rows are the A operand of S = Q K^T and dP = dO V^T, and
//    the transposing LDS read (ds_read_b64_tr_b16) gives the A operand of
//    dK^T = Q^T dS, dV^T = dO^T P.  Block m is the only owner of the (t, slot)
//    pairs that selected it, so it also writes dlogg[t][slot] (sum over G
//    heads, 64 rows, 64 keys) directly.  The q / dout tiles are single-buffered:
//    the next item is copied (direct-to-LDS loads) after every wave is done
//    with the current one, and the second workgroup on the CU computes
//    meanwhile.  When the grid is small enough that the longest lists (the
//    lowest key blocks) would outlast the rest, those blocks are split: several
//    workgroups take contiguous shares of one list and store fp32 partials,
//    which a small kernel sums in share order (the sums stay repeatable).
//  * dQ (query-major): the forward's tiling (2 heads x 64 rows per workgroup,
//    four waves of 32 rows), recomputing S^T = K Q^T and dP^T = V dO^T per
//    selected block and accumulating dQ^T += K^T dS^T, with K and V staged
//    row-major in LDS (K^T read with ds_read_b64_tr_b16), double-buffered.
//  All tiles are laid out swizzled so that row fragments and transposed reads
//  are both free of bank conflicts.
// With OUTER (gates applied after the softmax, the right-hand gradient of
// Eq. 5) the logits carry no bias, dP = g dO . v, dV takes g P, and the gate
// gradient of a block is the sum of P dP instead of dS.
#include <math.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {

namespace {

template <bool B> struct DiagTag { static constexpr bool value = B; };

constexpr int D = 128;
constexpr int BS = 64;
// q / dout / K / V tiles: 64 x 128 bf16, swizzled (see mfma.h)
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- dK / dV
constexpr int DKV_NT = 256;
constexpr int DKV_MAXT = 4096;  // longest inverse list (query blocks) held in LDS

// Two workgroups share a CU (at most 256 registers per lane and 64.6 KB of LDS
// each), so one workgroup's MFMA work overlaps the other's softmax, barriers
// and tile copies.  Wave w computes S and dP for keys 32 (w % 2) .. +32 and
// query rows 32 (w / 2) .. +32, but accumulates dK^T, dV^T for the same keys
// and head dims 64 (w / 2) .. +64 over all 64 rows: it takes the partner wave's
// (w ^ 2) P and dS fragments for the other 32 rows from LDS.  Each wave then
// owns its part of dK and dV outright, with no reduction at the end.  The next
// item's q / dout rows, LSE, D and log gate are copied global -> LDS (direct-to-
// LDS loads) once every wave is done with the current tiles.
template <bool OUTER>
__global__ void __launch_bounds__(DKV_NT, 2) bwd_dkdv_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ Dv,
    const float* __restrict__ logg, const uint8_t* __restrict__ slotmap,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ dlogg,
    const DkdvSplit sp, float* __restrict__ part) {
  // q and dout tiles in one array: they are only read after every copy into
  // them has landed, and one base register with constant offsets addresses both
  __shared__ __align__(16) bf16_t QO[2 * BS * TILE_LD];
  bf16_t* const Qs = QO;
  bf16_t* const Os = QO + BS * TILE_LD;
  __shared__ __align__(16) bf16x8 xch[4][4][64];  // [wave][P0, P1, dS0, dS1][lane]
  __shared__ float Ls[BS], Dl[BS];
  __shared__ float cur_bias;
  __shared__ float red[4];
  // Query blocks t attending to block m (ascending): t | slot << 16, where slot
  // is m's position in t's selection (0xFF on the diagonal).
  __shared__ uint32_t lst[DKV_MAXT];
  __shared__ int scan_scr[16];

  // The parts of the split key blocks first, then the other key blocks
  // ascending (low blocks are selected by the most query blocks, so the longest
  // inverse lists go first); KV head fastest.  A part's partial sums go to slot
  // blockIdx.x of `part`.
  const int kv = blockIdx.x % dm.hkv;
  const int b = (blockIdx.x / dm.hkv) % dm.b;
  const int j = blockIdx.x / (dm.hkv * dm.b);
  const bool split = j < sp.nparts;
  const int m = split ? sp.part_m[j] : sp.nsplit + (j - sp.nparts);
  const int share = split ? sp.part_p[j] : 0;
  const int nshares = split ? sp.first[m + 1] - sp.first[m] : 1;
  float* const partp = split ? part + (size_t)blockIdx.x * kDkdvPartFloats : nullptr;
  const size_t bk = (size_t)b * dm.hkv + kv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, c = lane & 31;
  const int kt = wave & 1, qh = wave >> 1;  // qh also selects the head-dim half
  const int key = kt * 32 + c;  // key within the block (this lane's column)
  const size_t kvrow = (bk * dm.n + (size_t)m * BS + key) * D;
  // ragged batch: a key block past the sequence's end is selected by no row and
  // its diagonal rows are padding, so dK = dV = 0 (uniform over the workgroup)
  if (dm.seq_lens && m * BS >= min(max(dm.seq_lens[b], 0), dm.n)) {
    if (split) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *reinterpret_cast<float4*>(partp + (i * DKV_NT + threadIdx.x) * 4) =
            make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      return;
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dd = qh * 64 + dt * 32 + r4 * 8 + g * 4;
        *reinterpret_cast<uint2*>(dk + kvrow + dd) = make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(dv + kvrow + dd) = make_uint2(0u, 0u);
      }
    return;
  }

  // K, V of the wave's 32 keys as B operands (column = key, k = dims).
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    kf[kc] = *reinterpret_cast<const bf16x8*>(k + kvrow + kc * 16 + g * 8);
    vf[kc] = *reinterpret_cast<const bf16x8*>(v + kvrow + kc * 16 + g * 8);
  }
  f32x16 dka[2], dva[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
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
    if (flag) lst[ne + pos] = (uint32_t)tt | ((uint32_t)sl << 16);
    ne += cnt;
  }
  __syncthreads();

  // this workgroup's share of the list: entries [elo, ehi), G items each
  const int elo = ne * share / nshares, ehi = ne * (share + 1) / nshares;
  const int ilo = elo * dm.g, ihi = ehi * dm.g;
  typedef __attribute__((address_space(3))) void lds_void;
  // Copies item `it` into the tiles: q and dout rows by all waves, LSE and D
  // by wave 0, the log gate by lane 0 of wave 1 (or a 0 when ungated).
  auto fetch = [&](int it) {
    const uint32_t ent = lst[it / dm.g];
    const int t = (int)(ent & 0xFFFF), sl = (int)(ent >> 16);
    const int h = kv * dm.g + it % dm.g;
    const size_t rb = ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS;
    tile_load_lds<4>(Qs, q + rb * D);
    tile_load_lds<4>(Os, dout + rb * D);
    if (wave == 0) {
      __builtin_amdgcn_global_load_lds((const void*)(lse + rb + lane), (lds_void*)Ls, 4, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(Dv + rb + lane), (lds_void*)Dl, 4, 0, 0);
    } else if (wave == 1) {
      if (logg && sl != 0xFF) {
        if (lane == 0)
          __builtin_amdgcn_global_load_lds(
              (const void*)(logg + (bk * dm.T + t) * (size_t)dm.K + sl), (lds_void*)&cur_bias,
              4, 0, 0);
      } else if (lane == 0) {
        cur_bias = 0.0f;
      }
    }
  };
  if (ilo < ihi) fetch(ilo);
  wait_all_loads();
  __syncthreads();
  float dlsum = 0.0f;
  // The list opens with the diagonal block (t = m, one item per head): those
  // items mask the keys past each row; the loop over the rest has no mask.
  auto item = [&](int it, auto diagc) __attribute__((always_inline)) {
    const int e = it / dm.g;
    const uint32_t ent = lst[e];
    const int t = (int)(ent & 0xFFFF);
    const int slot = (int)(ent >> 16);
    constexpr bool diag = decltype(diagc)::value;
    const float bias2 = OUTER ? 0.0f : cur_bias * LOG2E;
    const float gain = OUTER ? expf(cur_bias) : 1.0f;

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
      float p = fast_exp2(fmaf(sa[r], sc2, bias2) - Ls[qi] * LOG2E);
      if (diag && key > qi) p = 0.0f;
      const float dp = OUTER ? pa[r] * gain : pa[r];
      const float ds = p * (dp - Dl[qi]);
      sa[r] = OUTER ? p * gain : p;
      pa[r] = ds;
      dlsum += OUTER ? p * dp : ds;
    }
    const bf16x8 p0 = pack8(sa, 0), p1 = pack8(sa, 8);
    const bf16x8 d0 = pack8(pa, 0), d1 = pack8(pa, 8);
    xch[wave][0][lane] = p0;
    xch[wave][1][lane] = p1;
    xch[wave][2][lane] = d0;
    xch[wave][3][lane] = d1;
    // dV^T += dO^T P, dK^T += Q^T dS for head dims 64 qh .. +64, first over this
    // wave's own 32 rows (P, dS still in registers) ...
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const int col = qh * 64 + dt * 32;
      dva[dt] = mfma32(tr_frag(Os, qh * 32, col), p0, dva[dt]);
      dka[dt] = mfma32(tr_frag(Qs, qh * 32, col), d0, dka[dt]);
      dva[dt] = mfma32(tr_frag(Os, qh * 32 + 16, col), p1, dva[dt]);
      dka[dt] = mfma32(tr_frag(Qs, qh * 32 + 16, col), d1, dka[dt]);
    }
    const bool last_head = it % dm.g == dm.g - 1;
    if (last_head) {
      const float ws = wave_sum(dlsum);
      if (lane == 0) red[wave] = ws;
      dlsum = 0.0f;
    }
    __syncthreads();  // partner fragments and the dlogg partials are in LDS
    if (last_head && !diag && dlogg && threadIdx.x == 0)
      dlogg[(bk * dm.T + t) * (size_t)dm.K + slot] = (red[0] + red[1]) + (red[2] + red[3]);

    // ... then over the partner wave's 32 rows (P, dS from LDS).
    const int pw = wave ^ 2;
    const int prow = (qh ^ 1) * 32;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 xp = xch[pw][hh][lane], xd = xch[pw][2 + hh][lane];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int col = qh * 64 + dt * 32;
        dva[dt] = mfma32(tr_frag(Os, prow + 16 * hh, col), xp, dva[dt]);
        dka[dt] = mfma32(tr_frag(Qs, prow + 16 * hh, col), xd, dka[dt]);
      }
    }
    __syncthreads();  // everyone is done with the tiles and the exchange
    if (it + 1 < ihi) fetch(it + 1);
    wait_all_loads();
    __syncthreads();  // item it + 1 is in the tiles
  };
  // the diagonal's items exist in the first share only
  const int idiag = elo == 0 ? min(dm.g, ihi) : ilo;
  for (int it = ilo; it < idiag; ++it) item(it, DiagTag<true>());
  for (int it = idiag; it < ihi; ++it) item(it, DiagTag<false>());

  if (split) {
    // fp32 partials, float4 i of thread x at (i * 256 + x) * 4: dK^T (unscaled)
    // then dV^T, in the order of the stores below
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<float4*>(partp + ((dt * 4 + r4) * DKV_NT + threadIdx.x) * 4) =
            make_float4(dka[dt][r4 * 4], dka[dt][r4 * 4 + 1], dka[dt][r4 * 4 + 2],
                        dka[dt][r4 * 4 + 3]);
        *reinterpret_cast<float4*>(partp + ((8 + dt * 4 + r4) * DKV_NT + threadIdx.x) * 4) =
            make_float4(dva[dt][r4 * 4], dva[dt][r4 * 4 + 1], dva[dt][r4 * 4 + 2],
                        dva[dt][r4 * 4 + 3]);
      }
    return;
  }

  // dK = scale * (dK^T)^T, dV: lane holds key `key`, dims 64 qh + 32 dt + acc_row(r, g).
  bf16_t* dkp = dk + kvrow;
  bf16_t* dvp = dv + kvrow;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dd = qh * 64 + dt * 32 + r4 * 8 + g * 4;
      uint2 wk, wv;
      wk.x = pack_bf16x2(dka[dt][r4 * 4] * dm.scale, dka[dt][r4 * 4 + 1] * dm.scale);
      wk.y = pack_bf16x2(dka[dt][r4 * 4 + 2] * dm.scale, dka[dt][r4 * 4 + 3] * dm.scale);
      wv.x = pack_bf16x2(dva[dt][r4 * 4], dva[dt][r4 * 4 + 1]);
      wv.y = pack_bf16x2(dva[dt][r4 * 4 + 2], dva[dt][r4 * 4 + 3]);
      *reinterpret_cast<uint2*>(dkp + dd) = wk;
      *reinterpret_cast<uint2*>(dvp + dd) = wv;
    }
}

// Sums the parts of every split key block, in part order, and stores dK
// (scaled) and dV in bf16, each thread the values the dK/dV kernel's own
// epilogue would store.  One workgroup per (split key block, batch, KV head).
__global__ void __launch_bounds__(DKV_NT) bwd_dkdv_combine_kernel(
    Dims dm, const DkdvSplit sp, const float* __restrict__ part, bf16_t* __restrict__ dk,
    bf16_t* __restrict__ dv) {
  const int kv = blockIdx.x % dm.hkv;
  const int b = (blockIdx.x / dm.hkv) % dm.b;
  const int m = blockIdx.x / (dm.hkv * dm.b);
  const size_t bk = (size_t)b * dm.hkv + kv;
  const size_t rows = (size_t)dm.b * dm.hkv;
  const int j0 = sp.first[m], j1 = sp.first[m + 1];
  float4 acc[16];
  {
    const float4* src = reinterpret_cast<const float4*>(part + (j0 * rows + bk) * kDkdvPartFloats);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = src[i * DKV_NT + threadIdx.x];
  }
  for (int j = j0 + 1; j < j1; ++j) {
    const float4* src = reinterpret_cast<const float4*>(part + (j * rows + bk) * kDkdvPartFloats);
    float4 x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = src[i * DKV_NT + threadIdx.x];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i].x += x[i].x;
      acc[i].y += x[i].y;
      acc[i].z += x[i].z;
      acc[i].w += x[i].w;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, kt = wave & 1, qh = wave >> 1;
  const size_t kvrow = (bk * dm.n + (size_t)m * BS + kt * 32 + (lane & 31)) * D;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dd = qh * 64 + dt * 32 + r4 * 8 + g * 4;
      const float4 a = acc[dt * 4 + r4], c = acc[8 + dt * 4 + r4];
      uint2 wk, wv;
      wk.x = pack_bf16x2(a.x * dm.scale, a.y * dm.scale);
      wk.y = pack_bf16x2(a.z * dm.scale, a.w * dm.scale);
      wv.x = pack_bf16x2(c.x, c.y);
      wv.y = pack_bf16x2(c.z, c.w);
      *reinterpret_cast<uint2*>(dk + kvrow + dd) = wk;
      *reinterpret_cast<uint2*>(dv + kvrow + dd) = wv;
    }
}

// ---------------------------------------------------------------- dQ
constexpr int HPW = 2;   // heads per dQ workgroup
constexpr int DQ_NW = 4;  // waves: two 32-row halves per head
constexpr int DQ_NT = 64 * DQ_NW;

template <bool OUTER>
__global__ void __launch_bounds__(DQ_NT, 2) bwd_dq_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ Dv, const float* __restrict__ Dsrc,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, bf16_t* __restrict__ dq) {
  // Two K/V tile buffers as four separate arrays (see the forward kernel: the
  // loop is unrolled by two so that copies and transposed reads of different
  // buffers are known not to alias).
  __shared__ __align__(16) bf16_t K0[BS * TILE_LD];
  __shared__ __align__(16) bf16_t V0[BS * TILE_LD];
  __shared__ __align__(16) bf16_t K1[BS * TILE_LD];
  __shared__ __align__(16) bf16_t V1[BS * TILE_LD];
  __shared__ int blist[kMaxTrainK + 1];
  __shared__ float bbias[kMaxTrainK + 1];
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
  // ragged batch: a query tile past the sequence's end has P = 0 everywhere,
  // so dQ = 0 and D = 0 (uniform over the workgroup)
  if (dm.seq_lens && t * BS >= min(max(dm.seq_lens[b], 0), dm.n)) {
    const size_t prow = ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS + qi;
    if (g == 0 && Dv) Dv[prow] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<uint2*>(dq + prow * D + dt * 32 + r4 * 8 + g * 4) = make_uint2(0u, 0u);
    return;
  }

  const size_t rowbk = ((size_t)b * dm.hkv + kv) * dm.T + t;
  if (wave == 0) wave_block_list<OUTER>(idx, logg, rowbk, dm.K, t, lane, blist, bbias, &nblk);

  const size_t row = ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS + qi;
  bf16x8 qf[8], of[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    qf[kc] = *reinterpret_cast<const bf16x8*>(q + row * D + kc * 16 + g * 8);
    of[kc] = *reinterpret_cast<const bf16x8*>(dout + row * D + kc * 16 + g * 8);
  }
  const float l2 = lse[row] * LOG2E;
  float dval;
  if (Dsrc) {
    dval = Dsrc[row];  // formed by bwd_dval_kernel with the same sums as below
  } else {
    // D = dO . o for this lane's row: 64 dims per lane half, then the halves;
    // also stored for the dK / dV kernel, which runs after this one.
    // D as a fixed tree over the 16 chunk partials p(kc, g) (8 dims each):
    // pairs in kc, then quads, then the two halves (bwd_dval_kernel sums alike)
    float pd[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(o + row * D + kc * 16 + g * 8);
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf((float)of[kc][e], (float)ov[e], a);
      pd[kc] = a;
    }
    dval = ((pd[0] + pd[1]) + (pd[2] + pd[3])) + ((pd[4] + pd[5]) + (pd[6] + pd[7]));
    dval += __shfl_xor(dval, 32);
    if (g == 0 && Dv) Dv[row] = dval;
  }
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
  const TileOffsets<DQ_NW> toff;
  {
    const int m0 = __builtin_amdgcn_readfirstlane(blist[0]);
    tile_copy_lds<DQ_NW>(K0, kbase + (size_t)m0 * BS * D, toff);
    tile_copy_lds<DQ_NW>(V0, vbase + (size_t)m0 * BS * D, toff);
  }
  wait_all_loads();
  __syncthreads();
  // Block bi from (Kc, Vc) while block bi + 1 is copied into (Kn, Vn).
  auto step = [&](int bi, const bf16_t* Kc, const bf16_t* Vc, bf16_t* Kn, bf16_t* Vn) {
    const int m = blist[bi];
    const float off2 = (OUTER ? 0.0f : bbias[bi]) - l2;
    const float gain = OUTER ? bbias[bi] : 1.0f;
    const bool diag = m == t;
    if (bi + 1 < nb) {
      const int mn = __builtin_amdgcn_readfirstlane(blist[bi + 1]);
      tile_copy_lds<DQ_NW>(Kn, kbase + (size_t)mn * BS * D, toff);
      tile_copy_lds<DQ_NW>(Vn, vbase + (size_t)mn * BS * D, toff);
    }

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
      // the diagonal block's keys past the row: logit -inf, so P = 0 (a
      // uniform branch, taken for one block of the row)
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + acc_row(r, g) > qi) sa[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sa[r], sc2, off2));
        pa[r] = p * ((OUTER ? pa[r] * gain : pa[r]) - dval);
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
  };
  for (int bi = 0; bi < nb; bi += 2) {
    step(bi, K0, V0, K1, V1);
    if (bi + 1 < nb) step(bi + 1, K1, V1, K0, V0);
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

// D = dO . o per query row, summed exactly as the dQ kernel's prologue sums it,
// so both kernels see the same D: 16 lanes per row, lane 2 kc + g forms the
// partial of dims kc * 16 + g * 8 .. +8, then the tree over kc (lane xor 2, 4,
// 8) and the two halves (xor 1).
__global__ void __launch_bounds__(256) bwd_dval_kernel(const bf16_t* __restrict__ o,
                                                     const bf16_t* __restrict__ dout,
                                                     float* __restrict__ Dv, size_t rows) {
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int kc = sub >> 1, g = sub & 1;
  float a = 0.0f;
  if (row < rows) {
    const bf16x8 of = *reinterpret_cast<const bf16x8*>(dout + row * D + kc * 16 + g * 8);
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(o + row * D + kc * 16 + g * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf((float)of[e], (float)ov[e], a);
  }
  a += __shfl_xor(a, 2);
  a += __shfl_xor(a, 4);
  a += __shfl_xor(a, 8);
  a += __shfl_xor(a, 1);
  if (row < rows && sub == 0) Dv[row] = a;
}

// The dQ kernel's second stream and its fork / join events, one set per
// device for the whole process (created on first use, default priority, never
// destroyed).  Callers on different threads share it: a backward holds `mu`
// while it enqueues its fork, its kernels and its join, so the events
// always order the right pair of streams; the dQ kernels of concurrent
// backwards then run one after another on the side stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int cus = 0;
  bool ready = false;
  std::mutex mu;
};

SideStream* side_stream() {
  constexpr int kMaxDev = 64;
  static SideStream per_dev[kMaxDev];
  static std::mutex create_mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  SideStream& ss = per_dev[dev];
  std::lock_guard<std::mutex> lk(create_mu);
  if (!ss.ready) {
    // published only when every part exists (else the caller runs serially)
    int cus = 0;
    hipEvent_t fork = nullptr, join = nullptr;
    hipStream_t s = nullptr;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return nullptr;
    if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess) {
      (void)hipEventDestroy(fork);  // clean-up on the failure path; its own status is moot
      return nullptr;
    }
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
      (void)hipEventDestroy(fork);
      (void)hipEventDestroy(join);
      return nullptr;
    }
    ss.s = s;
    ss.fork = fork;
    ss.join = join;
    ss.cus = cus;
    ss.ready = true;
  }
  return &ss;
}

// Dv: where dQ stores the D it forms; Dsrc: D formed beforehand (then o is not read).
void launch_dq(const Dims& dm, const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, float* Dv, const float* Dsrc,
               const int32_t* idx, const float* logg, void* dq, hipStream_t st) {
  const size_t tiles = (size_t)dm.b * dm.hkv * dm.T * (dm.g / HPW);
  ProfScope ps("bwd_dq_mfma", st);
  auto kern = dm.outer ? bwd_dq_mfma_kernel<true> : bwd_dq_mfma_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(DQ_NT), 0, st, dm, (const bf16_t*)q,
                     (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)o, (const bf16_t*)dout,
                     lse, Dv, Dsrc, idx, logg, (bf16_t*)dq);
}

void launch_dkdv(const Dims& dm, const void* q, const void* k, const void* v, const void* dout,
                 const float* lse, const float* logg, const BwdWorkspace& ws, void* dk,
                 void* dv, hipStream_t st) {
  const DkdvSplit sp = dkdv_split_plan(dm);
  const size_t rows = (size_t)dm.b * dm.hkv;
  const size_t wgs = rows * (sp.nparts + dm.T - sp.nsplit);
  // one timing scope over both kernels: the dK/dV work includes the sums
  ProfScope ps("bwd_dkdv_mfma", st);
  auto kern = dm.outer ? bwd_dkdv_mfma_kernel<true> : bwd_dkdv_mfma_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(DKV_NT), 0, st, dm, (const bf16_t*)q,
                     (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)dout, lse, ws.D, logg,
                     ws.slotmap, (bf16_t*)dk, (bf16_t*)dv, ws.dlogg_part, sp, ws.dkdv_part);
  if (sp.nparts > 0)
    hipLaunchKernelGGL(bwd_dkdv_combine_kernel, dim3((unsigned)(rows * sp.nsplit)),
                       dim3(DKV_NT), 0, st, dm, sp, (const float*)ws.dkdv_part, (bf16_t*)dk,
                       (bf16_t*)dv);
}

}  // namespace

DkdvSplit dkdv_split_plan(const Dims& dm) {
  DkdvSplit sp{};
  const int T = dm.T;
  if (T < 2 || dm.K <= 0) return sp;
  int cus = 256, dev = 0, c = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      c > 0)
    cus = c;
  // Expected list length of key block m when every query block t selects K of
  // its t history blocks evenly: the diagonal plus the sum over t > m of
  // min(1, K / t).  Non-increasing in m, so the split blocks are a prefix.
  std::vector<double> e(T);
  double tail = 0.0, total = 0.0;
  for (int m = T - 1; m >= 0; --m) {
    e[m] = 1.0 + tail;
    total += e[m];
    tail += std::min(1.0, (double)dm.K / std::max(m, 1));
  }
  // a part's share: at most an even share of all lists over the grid's
  // workgroup slots (two per CU)
  const double cap = total * dm.b * dm.hkv / (2.0 * cus);
  int parts = 0, m = 0;
  for (; m < T && m < kDkdvMaxSplit; ++m) {
    const int P = (int)std::min((double)kDkdvMaxPartsPerBlock, std::ceil(e[m] / cap));
    if (P < 2 || parts + P > kDkdvMaxParts) break;
    sp.first[m] = (uint16_t)parts;
    for (int p = 0; p < P; ++p) {
      sp.part_m[parts + p] = (uint8_t)m;
      sp.part_p[parts + p] = (uint8_t)p;
    }
    parts += P;
  }
  sp.first[m] = (uint16_t)parts;
  sp.nsplit = m;
  sp.nparts = parts;
  return sp;
}

// Inner and outer gating (templated kernels).
bool mfma_bwd_supported(const Dims& dm) {
  return dm.bf16 && dm.d == D && dm.bs == BS && dm.n % BS == 0 && dm.g % HPW == 0 &&
         dm.T <= DKV_MAXT;
}

hipError_t launch_bwd_mfma(const Dims& dm, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           const int32_t* idx, const float* logg, void* dq, void* dk, void* dv,
                           const BwdWorkspace& ws, const std::function<hipError_t()>& tail,
                           hipStream_t st) {
  // When the dK/dV grid is at most two rounds of its two-per-CU occupancy, its
  // last workgroups (the longest inverse lists) leave CUs idle: dQ then runs
  // beside dK/dV on a second stream.  Larger grids have no such tail and run
  // dQ (which forms D) first.
  SideStream* ss = nullptr;
  const size_t dkdv_wgs = (size_t)dm.b * dm.hkv * dm.T;
  if (!dm.seq_lens) {
    ss = side_stream();
    if (ss && dkdv_wgs > (size_t)4 * ss->cus) ss = nullptr;
  }
  hipError_t e;
  if (!ss) {
    if ((e = launch_bwd_prep(dm, o, dout, idx, ws, false, st)) != hipSuccess) return e;
    launch_dq(dm, q, k, v, o, dout, lse, ws.D, nullptr, idx, logg, dq, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    launch_dkdv(dm, q, k, v, dout, lse, logg, ws, dk, dv, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return tail();
  }
  const size_t rows = (size_t)dm.b * dm.hq * dm.n;
  // The side stream forks before anything of the backward: dQ needs none of
  // its intermediates (it forms D from o with the same sums as bwd_dval_kernel
  // and stores none), so it starts at once while the slot map, D and dK/dV
  // follow on st.  The selector gradient needs only dK/dV's dlogg and runs on
  // st before the join; dQ is the longer of the two, so the join comes last.
  // (Measured at 8K against forking after D and joining before the selector
  // gradient: 1.170 against 1.187 ms per training step, bitwise the same.)
  std::lock_guard<std::mutex> lk(ss->mu);
  if ((e = hipEventRecord(ss->fork, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess) return e;
  launch_dq(dm, q, k, v, o, dout, lse, nullptr, nullptr, idx, logg, dq, ss->s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess) return e;
  if ((e = launch_bwd_prep(dm, o, dout, idx, ws, false, st)) != hipSuccess) return e;
  {
    ProfScope ps("bwd_dot", st);
    hipLaunchKernelGGL(bwd_dval_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st,
                       (const bf16_t*)o, (const bf16_t*)dout, ws.D, rows);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  launch_dkdv(dm, q, k, v, dout, lse, logg, ws, dk, dv, st);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tail()) != hipSuccess) return e;
  return hipStreamWaitEvent(st, ss->join, 0);
}

}  // namespace sas
