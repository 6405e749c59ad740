// Fused gated block-sparse forward with bf16 MFMA (gfx950): head_dim 128,
// block 64, bf16 tensors, N a multiple of 64, G = hq / hkv even.
//
// picx.dev summary of SAS, 'Key Idea' Eq. 9 and 'Kernel Design': logits of
// the selected blocks get their normalised log gate, the current block gets 0
// (g0 = 1), unselected blocks are never loaded, the softmax is online and no
// attention matrix is stored.
//
// Work unit: one (batch, KV head, query block, 2-head chunk) tile = 2 heads x
// 64 query rows; every K/V block it needs is gathered into LDS and serves both
// heads (one selection per KV head).  Four waves: wave w owns 32 rows (half
// w % 2 of the block) of head kv*G + 2*chunk + w / 2, which keeps each wave's
// working set (Q fragments, S^T, O^T) inside 256 VGPRs and lets two workgroups
// share a CU.  K/V blocks are copied global -> LDS with the direct-to-LDS load
// into a double buffer: the next block's copy is in flight while the current
// one is computed, with one barrier per block.
//   S^T = K Q^T   (32x32x16 MFMA; A = K rows from LDS, B = Q rows held in
//                  registers), so each lane holds one query column and the
//                  softmax max/sum over keys stays inside the lane (plus one
//                  exchange with lane l^32);
//   O^T += V^T P^T (A = V^T read from the row-major V tile with the
//                  transposing LDS read ds_read_b64_tr_b16, B = P^T straight
//                  from the S^T accumulators, converted to bf16).
// The bias (log-gate) is added before the running max, in log2 units.  The
// running max is a reference that is only moved (and O, l rescaled) when a
// block's max exceeds it by more than 2^8; the final normalisation uses the
// same reference, so the result is unchanged.
// With OUTER (gates applied after the softmax) the logits carry no bias and P
// is scaled by the block's gate g after the row sum, before the P V product.
// Workgroups are issued longest-row-first (query block descending), KV head
// fastest, so consecutive workgroups (spread over the 8 XCDs) share K/V.
#include <math.h>

#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {

namespace {

template <bool B> struct DiagTag { static constexpr bool value = B; };

constexpr int D = 128;
constexpr int BS = 64;
// K and V tiles: 64 x 128 bf16 each, swizzled (see mfma.h)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

constexpr int HPW = 2;   // heads per workgroup
constexpr int NW = 4;    // waves per workgroup (two 32-row halves per head)
constexpr float RESCALE_SLACK = 8.0f;  // log2 units

// oacc[dt] += V^T(rows 16 ch .. +16, dims 32 dt .. +32) P^T[ch] over the four
// 16-key chunks ch of a gathered V tile (V^T read with ds_read_b64_tr_b16).
// The fragments of chunk ch + 1 are read while chunk ch's four MFMAs run: the
// issue order is pinned (one MFMA, then two of the next chunk's reads), so a
// chunk waits once for its reads instead of once per MFMA.
__device__ __forceinline__ void pv_chunks(const bf16_t* Vc, const bf16x8 (&pf)[4],
                                          f32x16 (&oacc)[4]) {
  bf16x8 fr[2][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) fr[0][dt] = tr_frag(Vc, 0, dt * 32);
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    if (ch < 3) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) fr[(ch + 1) & 1][dt] = tr_frag(Vc, (ch + 1) * 16, dt * 32);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = mfma32(fr[ch & 1][dt], pf[ch], oacc[dt]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // chunk 0's reads
#pragma unroll
  for (int ch = 0; ch < 3; ++ch)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA of chunk ch
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two reads of chunk ch + 1
    }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

template <bool OUTER>
__global__ void __launch_bounds__(64 * NW, 2) fwd_mfma_kernel(
    Dims dm, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const float* __restrict__ logg, bf16_t* __restrict__ o, float* __restrict__ lse) {
  // Two K/V tile buffers as four separate arrays: the loop below is unrolled
  // by two so that each use names its buffer statically, which lets the
  // compiler see that the copies into one buffer never alias the transposed
  // reads of the other (it would otherwise wait for every copy in flight).
  __shared__ __align__(16) bf16_t K0[BS * TILE_LD];
  __shared__ __align__(16) bf16_t V0[BS * TILE_LD];
  __shared__ __align__(16) bf16_t K1[BS * TILE_LD];
  __shared__ __align__(16) bf16_t V1[BS * TILE_LD];
  __shared__ int blist[kMaxTrainK + 1];
  __shared__ float bbias[kMaxTrainK + 1];  // log2 gate (inner) or gate (OUTER)
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
  const int qt = wave & 1;  // which 32-row half of the query block
  const int qi = qt * 32 + c;  // query row within the block
  // ragged batch: rows at or past this sequence's end carry no result
  const int nlen = dm.seq_lens ? min(max(dm.seq_lens[b], 0), dm.n) : dm.n;
  const size_t row = ((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS + qi;
  if (t * BS >= nlen) {  // the whole tile (uniform over the workgroup)
    if (g == 0) lse[row] = INFINITY;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<uint2*>(o + row * D + dt * 32 + r4 * 8 + g * 4) = make_uint2(0u, 0u);
    return;
  }

  const size_t rowbk = ((size_t)b * dm.hkv + kv) * dm.T + t;
  if (wave == 0) wave_block_list<OUTER>(idx, logg, rowbk, dm.K, t, lane, blist, bbias, &nblk);

  // Q^T fragments (B operand): query qt*32 + c, dims kc*16 + g*8 .. +8.
  const bf16_t* qrow = q + (((size_t)b * dm.hq + h) * dm.n + (size_t)t * BS + qt * 32) * D;
  bf16x8 qf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    qf[kc] = *reinterpret_cast<const bf16x8*>(qrow + (size_t)c * D + kc * 16 + g * 8);

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  float mref = -INFINITY;  // reference max (log2 units) of this lane's query
  float lsum = 0.0f;       // sum of 2^(z - mref) over this lane's keys
  const float sc2 = dm.scale * LOG2E;

  __syncthreads();
  const int nb = nblk;
  const bf16_t* kbase = k + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const bf16_t* vbase = v + ((size_t)b * dm.hkv + kv) * dm.n * D;
  const TileOffsets<NW> toff;
  {
    const int m0 = __builtin_amdgcn_readfirstlane(blist[0]);
    tile_copy_lds<NW>(K0, kbase + (size_t)m0 * BS * D, toff);
    tile_copy_lds<NW>(V0, vbase + (size_t)m0 * BS * D, toff);
  }
  wait_all_loads();
  __syncthreads();

  // Block bi from (Kc, Vc) while block bi + 1 is copied into (Kn, Vn).
  auto step = [&](int bi, const bf16_t* Kc, const bf16_t* Vc, bf16_t* Kn, bf16_t* Vn,
                  auto diagc) __attribute__((always_inline)) {
    const float bias2 = OUTER ? 0.0f : bbias[bi];
    constexpr bool diag = decltype(diagc)::value;  // the last block is the diagonal one
    if (bi + 1 < nb) {
      const int mn = __builtin_amdgcn_readfirstlane(blist[bi + 1]);
      tile_copy_lds<NW>(Kn, kbase + (size_t)mn * BS * D, toff);
      tile_copy_lds<NW>(Vn, vbase + (size_t)mn * BS * D, toff);
    }

    // S^T[key][query]: 64 keys x the wave's 32 queries.
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.0f;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sacc[kt] = mfma32(row_frag(Kc, kt * 32 + c, kc * 16 + g * 8), qf[kc], sacc[kt]);
      }

    // Max of the raw logits (scale > 0, bias uniform over the block).
    float smax = -INFINITY;
    if (diag) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + acc_row(r, g) > qi) sacc[kt][r] = -INFINITY;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[kt][r]);
    float mx = fmaf(smax, sc2, bias2);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (mx > mref + RESCALE_SLACK) {
      const float alpha = fast_exp2(mref - mx);
      mref = mx;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    const float off2 = bias2 - mref;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[kt][r], sc2, off2));
        sacc[kt][r] = OUTER ? p * bbias[bi] : p;
        lsum += p;
      }

    // O^T += V^T P^T over four 16-key chunks.
    {
      bf16x8 pf[4];
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) pf[ch] = pack8(sacc[ch >> 1], (ch & 1) * 8);
      pv_chunks(Vc, pf, oacc);
    }
    wait_all_loads();   // this wave's copies of the next block
    __syncthreads();    // everyone's copies landed; everyone is done with (Kc, Vc)
  };
  // history blocks in pairs (the tiles alternate), then the diagonal block
  // last, the only one that masks keys past its rows
  int bi = 0;
  for (; bi + 2 < nb; bi += 2) {
    step(bi, K0, V0, K1, V1, DiagTag<false>());
    step(bi + 1, K1, V1, K0, V0, DiagTag<false>());
  }
  if (bi + 1 < nb) {
    step(bi, K0, V0, K1, V1, DiagTag<false>());
    step(bi + 1, K1, V1, K0, V0, DiagTag<true>());
  } else {
    step(bi, K0, V0, K1, V1, DiagTag<true>());
  }

  // Normalise and store o (bf16) and LSE (natural log); padding rows: 0, +inf.
  const bool pad = t * BS + qi >= nlen;
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = pad ? 0.0f : 1.0f / ltot;
  if (g == 0) lse[row] = pad ? INFINITY : (mref + log2f(ltot)) * LN2;
  bf16_t* op = o + row * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dd = dt * 32 + r4 * 8 + g * 4;
      uint2 w;
      w.x = pack_bf16x2(oacc[dt][r4 * 4 + 0] * inv, oacc[dt][r4 * 4 + 1] * inv);
      w.y = pack_bf16x2(oacc[dt][r4 * 4 + 2] * inv, oacc[dt][r4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + dd) = w;
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
  if (dm.outer)
    hipLaunchKernelGGL(fwd_mfma_kernel<true>, dim3((unsigned)tiles), dim3(64 * NW), 0, st, dm,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, idx, logg,
                       (bf16_t*)o, lse);
  else
    hipLaunchKernelGGL(fwd_mfma_kernel<false>, dim3((unsigned)tiles), dim3(64 * NW), 0, st, dm,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, idx, logg,
                       (bf16_t*)o, lse);
  return hipGetLastError();
}

}  // namespace sas
