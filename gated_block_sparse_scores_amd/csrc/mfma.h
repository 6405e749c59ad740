// gfx950 bf16 MFMA helpers (wave64).
//
// v_mfma_f32_32x32x16_bf16, as used here (the attention parity tests depend on
// every part of this layout):
//   A (32 x 16): lane l supplies row l % 32, eight k-values of k-group l / 32;
//   B (16 x 32): lane l supplies column l % 32, the same eight k-values;
//   D (32 x 32): lane l holds column l % 32, rows
//                (r / 4) * 8 + (l / 32) * 4 + (r % 4) for r = 0..15.
// The contraction only needs A's and B's k-values paired by (k-group, element),
// so any consistent assignment of actual k indices to (group, element) works.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace sas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within a 32-row tile) of accumulator register r for lane group g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return (r >> 2) * 8 + g * 4 + (r & 3);
}

__device__ __forceinline__ bf16x8 cat4(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Packs eight accumulator values (registers r0 .. r0+7) to bf16 (RNE).
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int r0) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = (__bf16)x[r0 + j];
  return o;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short short4_t __attribute__((ext_vector_type(4)));

// Swizzled LDS tiles of 64 rows x 128 bf16 (256-byte rows, no padding): the
// 16-byte chunk c of row r lives at chunk position c ^ f(r),
// f(r) = ((r & 3) << 2) | ((r >> 2) & 3).  Sixteen consecutive rows then map a
// fixed chunk to sixteen distinct positions (row-fragment reads, 16 B per lane,
// are conflict-free), and four consecutive rows of a 16-row-aligned group map
// four adjacent chunks to sixteen distinct positions (transposed reads, 8 B per
// lane, are conflict-free too).
constexpr int TILE_LD = 128;
__device__ __forceinline__ int swz(int row, int col) {
  const int f = ((row & 3) << 2) | ((row >> 2) & 3);
  return row * TILE_LD + ((((col >> 3) ^ f)) << 3) + (col & 7);
}

// Eight consecutive elements (one 16-byte chunk) of a swizzled tile row.
__device__ __forceinline__ bf16x8 row_frag(const bf16_t* X, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(X + swz(row, col));
}

// A operand (32 x 16) read transposed from a swizzled bf16 LDS tile X with
// ds_read_b64_tr_b16: lane l = 32 g + c gets
//   X[kbase + (j / 4) * 8 + g * 4 + (j % 4)][col0 + c],  j = 0..7,
// i.e. A row c is tile column col0 + c and its k-values are tile rows in the
// order the 32x32 accumulator rows of lane group g take (acc_row), so the B
// operand can come straight from an accumulator.  kbase is a multiple of 16.
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 4-element rows addressed by lanes (i / 4) + 4 j, j = 0..3.
// Lane a therefore addresses row kbase + g*4 + a/4, columns
// col0 + 16*(group % 2) + 4*(a % 4) .. +3, and receives column
// col0 + 16*(group % 2) + a of rows kbase + g*4 + 0..3 (second read: +8).
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* X, int kbase, int col0) {
  const int l = threadIdx.x & 63;
  const int g = l >> 5, half = (l >> 4) & 1, a = l & 15;
  const int row = kbase + g * 4 + (a >> 2), col = col0 + 16 * half + 4 * (a & 3);
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  const short4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(X + swz(row, col)));
  const short4_t r1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(X + swz(row + 8, col)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Global -> LDS copy of one 64 x 128 bf16 block (global row stride 128) into a
// swizzled tile, with the direct-to-LDS 16-byte load: a wave instruction fills
// one 1 KB group of four rows, lane l writing slot l of the group, so lane l
// fetches the chunk (l % 16) ^ f(row) of row 4 * group + l / 16.  NW waves share
// the 16 groups.  Completion is awaited with s_waitcnt (vmcnt) + a barrier.
template <int NW>
__device__ __forceinline__ void tile_load_lds(bf16_t* tile, const bf16_t* __restrict__ src) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i) {
    const int grp = wave + i * NW;
    const int row = grp * 4 + (lane >> 4);
    const int f = ((row & 3) << 2) | ((row >> 2) & 3);
    const int chunk = (lane & 15) ^ f;
    __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)row * TILE_LD + chunk * 8),
                                     (lds_void*)(tile + grp * 4 * TILE_LD), 16, 0, 0);
  }
}

// The same copy with the lanes' byte offsets formed once: they depend only on
// the lane and the wave, so a copy then takes a wave-uniform block address (a
// scalar base) plus a precomputed 32-bit offset per load, with no per-copy
// address arithmetic.
template <int NW>
struct TileOffsets {
  uint32_t off[16 / NW];
  __device__ __forceinline__ TileOffsets() {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < 16 / NW; ++i) {
      const int row = (wave + i * NW) * 4 + (lane >> 4);
      const int f = ((row & 3) << 2) | ((row >> 2) & 3);
      off[i] = (uint32_t)((row * TILE_LD + (((lane & 15) ^ f) << 3)) * sizeof(bf16_t));
    }
  }
};

// src must be uniform over the wave (a block's first row).
template <int NW>
__device__ __forceinline__ void tile_copy_lds(bf16_t* tile, const bf16_t* __restrict__ src,
                                              const TileOffsets<NW>& to) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i)
    __builtin_amdgcn_global_load_lds((const void*)((const char*)src + to.off[i]),
                                     (lds_void*)(tile + (wave + i * NW) * 4 * TILE_LD), 16, 0,
                                     0);
}

__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

// The attended blocks of query block t of selection row `rowbk`: the valid
// history blocks of its selection (0 <= m < t) in slot order, then t itself,
// each with its bias, the log2 gate (inner gating) or the gate (OUTER).  Called
// by one whole wave: lane s takes slot s0 + s of each pass of 64 slots, and the
// valid entries are placed with a ballot's prefix counts (all of a pass's
// loads in flight at once, instead of one thread reading the slots in turn).
template <bool OUTER>
__device__ __forceinline__ void wave_block_list(const int32_t* __restrict__ idx,
                                                const float* __restrict__ logg, size_t rowbk,
                                                int K, int t, int lane, int* blist, float* bbias,
                                                int* nblk) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int32_t* ir = idx + rowbk * K;
  int cnt = 0;
  for (int s0 = 0; s0 < K; s0 += 64) {
    const int s = s0 + lane;
    const int m = s < K ? ir[s] : -1;
    const bool ok = m >= 0 && m < t;
    const float lg = (ok && logg) ? logg[rowbk * K + s] : 0.0f;
    const unsigned long long bal = __ballot(ok);
    if (ok) {
      const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
      blist[pos] = m;
      bbias[pos] = OUTER ? expf(lg) : lg * kLog2e;
    }
    cnt += __popcll(bal);
  }
  if (lane == 0) {
    blist[cnt] = t;
    bbias[cnt] = OUTER ? 1.0f : 0.0f;
    *nblk = cnt + 1;
  }
}

}  // namespace sas
