// Internal launch interface between the C ABI (sas_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sas {

// Brackets one kernel launch with timing events when the profiler is on.
struct ProfScope {
  ProfScope(const char* name, hipStream_t stream);
  ~ProfScope();
  int slot;
  hipStream_t stream;
};

// Where a decode reads its K / V cache.  Dense: [b, hkv, cache_len, d] per
// tensor.  Paged (table != nullptr): pages [num_pages, hkv, bs, d], logical
// block m of sequence b in page table[b * bt_ld + m]; a page number outside
// [0, num_pages) makes that block empty.  seq_lens (optional, device) gives each
// sequence its own valid length, clamped to [1, L] (L = the call's seqlen).
struct KvView {
  const void* k;
  const void* v;
  int cache_len;
  const int32_t* table;
  int bt_ld, num_pages;
  const int32_t* seq_lens;
};

// Per-sequence lengths of a ragged batch for the selection kernels: (batch,
// KV head) row bk belongs to sequence bk / hkv.
struct RowLens {
  const int32_t* lens;  // nullptr: every sequence is full
  int lmax, bs, hkv;
};

struct Dims {
  int b, hq, hkv, g, n, d, bs, T, K;
  float scale;
  bool bf16;
  int act;     // gate activation: 0 softmax, 1 sigmoid, 2 raw logit
  bool outer;  // gates applied after the softmax
  bool ste;    // hard forward, straight-through backward
  const int32_t* seq_lens;  // ragged batch: per-sequence lengths (device), or nullptr
};

// ---- selection (select.hip)
// lens (optional): sequence b pools only its first lens[b] tokens (blocks past
// them are 0).
hipError_t launch_block_pool(const void* x, bool in_bf16, int batch, int heads, int group,
                             int n, int d, int bs, bool out_bf16, void* out, hipStream_t st,
                             const int32_t* lens = nullptr);
// Gate LSE + Top-K per row; with s == NULL the stand-in scores are formed
// from qbar / kbar first (written to s_out).
hipError_t launch_topk(const float* s, const float* qbar, const void* kbar, bool kbar_bf16,
                       int kbar_ld, int d, double scale, float* s_out, int rows_bk, int T, int C,
                       int row_offset, int K, int act, int32_t* idx, float* logg, float* lse_s,
                       hipStream_t st, const RowLens& rl = RowLens{});
// Largest Top-K of the training path (selection with C <= kLongHistory, forward,
// backward): slots are stored as uint8 in the inverse map, 0xFE and 0xFF being
// markers.  Decode and the two-stage selection take K <= 64.
constexpr int kMaxTrainK = 254;
// Rows with more than kLongHistory history blocks use the two-stage path.
constexpr int kLongHistory = 512;
size_t select_workspace_bytes(int rows_bk, int T, int C, int K);
hipError_t launch_select_long(const float* s, const float* qbar, const void* kbar,
                              bool kbar_bf16, int kbar_ld, int d, double scale, int rows_bk,
                              int T, int C, int row_offset, int K, int act, float* s_out,
                              int32_t* idx, float* logg, float* lse_s, void* ws, hipStream_t st,
                              const RowLens& rl = RowLens{});

// ---- attention, portable fp32-arithmetic kernels (attn_generic.hip)
hipError_t launch_fwd_generic(const Dims& dm, const void* q, const void* k, const void* v,
                              const int32_t* idx, const float* logg, void* o, float* lse,
                              hipStream_t st);
// Work split of the MFMA dK/dV kernel (attn_mfma_bwd.hip).  Key block m is
// visited by the query blocks whose selection holds it, so low blocks have the
// longest lists; when one such list alone outlasts an even share of the grid's
// work, the key blocks m < nsplit are each taken by several workgroups
// ("parts", contiguous shares of the list), which store fp32 partial dK, dV
// that a small kernel sums in part order.  The plan depends only on the shape,
// K and the device's CU count.
constexpr int kDkdvMaxSplit = 64;   // split key blocks
constexpr int kDkdvMaxParts = 256;  // their parts, summed (per (batch, KV head))
constexpr int kDkdvMaxPartsPerBlock = 4;
struct DkdvSplit {
  int nsplit;                         // key blocks m < nsplit are split
  int nparts;                         // parts over them
  uint16_t first[kDkdvMaxSplit + 1];  // block m's parts are first[m] .. first[m + 1] - 1
  uint8_t part_m[kDkdvMaxParts];      // part j covers block part_m[j] ...
  uint8_t part_p[kDkdvMaxParts];      // ... as its share part_p[j]
};
bool mfma_bwd_supported(const Dims& dm);
DkdvSplit dkdv_split_plan(const Dims& dm);
// fp32 per part: 64 keys x 128 dims for dK and for dV
constexpr size_t kDkdvPartFloats = 2 * 64 * 128;

// Workspace layout helpers for the backward.
struct BwdWorkspace {
  float* D;            // [b, hq, n]          dout . o per query row
  float* dlogg_part;   // [b*hkv*T, nchunk, K] per-chunk gate-gradient partials
  uint8_t* slotmap;    // [b*hkv, T (m), T (t)] Top-K slot of block m in row t, 0xFF = none
  float* dkdv_part;    // [nparts, b, hkv, kDkdvPartFloats] split dK/dV partials (MFMA path)
  size_t slotmap_bytes;
  size_t bytes;
};
BwdWorkspace bwd_workspace_layout(const Dims& dm, void* base);
// D = rowsum(dO o) (when with_d; the MFMA backward forms it in its dQ kernel)
// and the slot map.
hipError_t launch_bwd_prep(const Dims& dm, const void* o, const void* dout, const int32_t* idx,
                           const BwdWorkspace& ws, bool with_d, hipStream_t st);
hipError_t launch_bwd_generic(const Dims& dm, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const int32_t* idx,
                              const float* logg, void* dq, void* dk, void* dv,
                              const BwdWorkspace& ws, int* nchunk_out, hipStream_t st);
hipError_t launch_bwd_ds(const Dims& dm, const int32_t* idx, const float* s, const float* lse_s,
                         const float* dlogg_part, int nchunk, float* dlogg, float* ds,
                         hipStream_t st);
int bwd_dlogg_chunks(const Dims& dm);

// ---- decode (decode.hip)
int decode_blocks_per_split(const Dims& dm);
bool decode_two_per_wave(const Dims& dm);
size_t decode_workspace_bytes(const Dims& dm);
// Fused decode step (bf16, d 128, block 64): chunk selection over the pooled-key
// cache with the query pooled in-kernel, then the decode kernel merging the
// chunk candidates itself, then the LSE merge.
constexpr int kSelectChunk = 256;  // history blocks per selection chunk
// Decode rows (T = 1, row offset C); with rl.lens each sequence ranks its own
// (L_b - 1) / bs history blocks.
hipError_t launch_select_chunks_rawq(const uint16_t* q, int qgroup, const void* kbar,
                                     bool kbar_bf16, int kbar_ld, int d, double scale, int rows,
                                     int C, int K, const RowLens& rl, uint64_t* cand,
                                     float2* stats, hipStream_t st);
bool decode_mfma_path(const Dims& dm);
hipError_t launch_decode_step(const Dims& dm, int L, const KvView& kvv, int C, int nchunk,
                              const void* q, const uint64_t* cand, const float2* stats,
                              bool gated, int32_t* idx_out, float* logg_out, float* lse_s_out,
                              void* o, float* lse, void* ws, hipStream_t st);
hipError_t launch_decode(const Dims& dm, int L, const KvView& kvv, const void* q,
                         const int32_t* idx, const float* logg, void* o, float* lse, void* ws,
                         hipStream_t st);

// ---- selector backward for the stand-in scores (selector_bwd.hip)
hipError_t launch_selector_bwd(const Dims& dm, const float* ds, const float* qbar,
                               const float* kbar, float* dqbar, float* dkbar, void* dq, void* dk,
                               hipStream_t st);

}  // namespace sas
