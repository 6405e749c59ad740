// C ABI of the SAS gated block-sparse attention library: argument checks on
// the host, workspace layout, kernel dispatch and the optional kernel timer.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sas.h"
#include "internal.h"

namespace sas {
// MFMA paths (attn_mfma_fwd.hip / attn_mfma_bwd.hip); return false when the
// shape is not one they handle.
bool mfma_fwd_supported(const Dims& dm);
hipError_t launch_fwd_mfma(const Dims& dm, const void* q, const void* k, const void* v,
                           const int32_t* idx, const float* logg, void* o, float* lse,
                           hipStream_t st);
// Slot map, D, dQ and dK/dV; `tail` enqueues the work that needs only dK/dV's
// outputs (the selector gradient) on st before the backward joins its streams.
hipError_t launch_bwd_mfma(const Dims& dm, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           const int32_t* idx, const float* logg, void* dq, void* dk, void* dv,
                           const BwdWorkspace& ws, const std::function<hipError_t()>& tail,
                           hipStream_t st);
}  // namespace sas

namespace {

// ------------------------------------------------------------------ profiler
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};

struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<ProfRecord> pending;
  std::map<std::string, std::pair<long long, double>> totals;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void drain() {
    for (auto& r : pending) {
      float ms = 0.0f;
      if (hipEventSynchronize(r.stop) == hipSuccess &&
          hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
        auto& t = totals[r.name];
        t.first += 1;
        t.second += ms;
      }
      pool.push_back(r.start);
      pool.push_back(r.stop);
    }
    pending.clear();
  }
};

Profiler& prof() {
  static Profiler p;
  return p;
}

thread_local std::vector<ProfRecord> open_records;

}  // namespace

namespace sas {

ProfScope::ProfScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on) return;
  ProfRecord r{name, p.take(), p.take()};
  if (!r.start || !r.stop) {  // event creation failed: this launch goes untimed
    if (r.start) p.pool.push_back(r.start);
    if (r.stop) p.pool.push_back(r.stop);
    return;
  }
  (void)hipEventRecord(r.start, s);
  open_records.push_back(r);
  slot = (int)open_records.size() - 1;
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  ProfRecord r = open_records[slot];
  open_records.pop_back();
  (void)hipEventRecord(r.stop, stream);
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.pending.push_back(r);
}

}  // namespace sas

using sas::Dims;

namespace {

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

sas_status check_shape(const sas_shape* s, bool need_seq = true) {
  if (!s) return SAS_ERR_INVALID_ARG;
  if (s->batch <= 0 || s->hq <= 0 || s->hkv <= 0 || s->head_dim <= 0 || s->block <= 0)
    return SAS_ERR_INVALID_ARG;
  if (need_seq && s->seqlen <= 0) return SAS_ERR_INVALID_ARG;
  if (s->hq % s->hkv != 0) return SAS_ERR_INVALID_ARG;
  if (s->dtype != SAS_DTYPE_F32 && s->dtype != SAS_DTYPE_BF16) return SAS_ERR_INVALID_ARG;
  if (!(s->scale >= 0.0f) || isinf(s->scale)) return SAS_ERR_INVALID_ARG;
  if ((s->gate & ~(SAS_GATE_ACTIVATION_MASK | SAS_GATE_OUTER | SAS_GATE_STE)) != 0 ||
      (s->gate & SAS_GATE_ACTIVATION_MASK) > SAS_GATE_RAW)
    return SAS_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return SAS_ERR_UNSUPPORTED;
  if (s->block != 16 && s->block != 32 && s->block != 64) return SAS_ERR_UNSUPPORTED;
  return SAS_OK;
}

Dims make_dims(const sas_shape* s, int K) {
  Dims d{};
  d.b = s->batch;
  d.hq = s->hq;
  d.hkv = s->hkv;
  d.g = s->hq / s->hkv;
  d.n = s->seqlen;
  d.d = s->head_dim;
  d.bs = s->block;
  d.T = (s->seqlen + s->block - 1) / s->block;
  d.K = K;
  d.scale = s->scale > 0.0f ? s->scale : (float)(1.0 / sqrt((double)s->head_dim));
  d.bf16 = s->dtype == SAS_DTYPE_BF16;
  d.act = s->gate & SAS_GATE_ACTIVATION_MASK;
  d.outer = (s->gate & SAS_GATE_OUTER) != 0;
  d.ste = (s->gate & SAS_GATE_STE) != 0;
  d.seq_lens = s->seq_lens;
  return d;
}

sas_status launch_status(hipError_t e) { return e == hipSuccess ? SAS_OK : SAS_ERR_LAUNCH; }

#define SAS_TRY(expr)                       \
  do {                                      \
    sas_status st_ = (expr);                \
    if (st_ != SAS_OK) return st_;          \
  } while (0)

#define SAS_LAUNCH(expr)                                \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return SAS_ERR_LAUNCH;        \
  } while (0)

}  // namespace

extern "C" {

const char* sas_status_string(sas_status status) {
  switch (status) {
    case SAS_OK: return "ok";
    case SAS_ERR_INVALID_ARG: return "invalid argument";
    case SAS_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SAS_ERR_WORKSPACE: return "workspace missing or too small";
    case SAS_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int sas_version(void) { return 100; }

sas_status sas_block_pool(const sas_shape* shape, const void* x, int heads, int group,
                          sas_dtype out_dtype, void* out, void* stream) {
  if (!shape) return SAS_ERR_INVALID_ARG;
  if (shape->batch <= 0 || shape->seqlen <= 0 || shape->head_dim <= 0 || shape->block <= 0)
    return SAS_ERR_INVALID_ARG;
  if (heads <= 0 || group <= 0 || heads % group != 0) return SAS_ERR_INVALID_ARG;
  if (!x || !out) return SAS_ERR_INVALID_ARG;
  if (shape->dtype != SAS_DTYPE_F32 && shape->dtype != SAS_DTYPE_BF16) return SAS_ERR_INVALID_ARG;
  if (out_dtype != SAS_DTYPE_F32 && out_dtype != SAS_DTYPE_BF16) return SAS_ERR_INVALID_ARG;
  if (shape->head_dim != 64 && shape->head_dim != 128) return SAS_ERR_UNSUPPORTED;
  if (shape->block > 4096) return SAS_ERR_UNSUPPORTED;
  if (!aligned16(x)) return SAS_ERR_INVALID_ARG;  // 16-byte vector loads
  return launch_status(sas::launch_block_pool(
      x, shape->dtype == SAS_DTYPE_BF16, shape->batch, heads, group, shape->seqlen,
      shape->head_dim, shape->block, out_dtype == SAS_DTYPE_BF16, out, (hipStream_t)stream,
      shape->seq_lens));
}

size_t sas_select_topk_workspace_size(const sas_shape* shape, int T, int C, int K) {
  if (!shape || shape->batch <= 0 || shape->hkv <= 0 || T <= 0 || C < 0 || K <= 0 ||
      K > sas::kMaxTrainK || C > 16384 || (C > sas::kLongHistory && K > 64))
    return 0;
  return sas::select_workspace_bytes(shape->batch * shape->hkv, T, C, K);
}

sas_status sas_select_topk(const sas_shape* shape, int T, int C, int row_offset, int K,
                           const float* s, const float* qbar, const void* kbar,
                           sas_dtype kbar_dtype, int kbar_ld, float* s_out, int32_t* idx,
                           float* logg, float* lse_s, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (!shape || shape->batch <= 0 || shape->hkv <= 0) return SAS_ERR_INVALID_ARG;
  if (T <= 0 || C < 0 || row_offset < 0 || K <= 0) return SAS_ERR_INVALID_ARG;
  if (!idx || !logg || !lse_s) return SAS_ERR_INVALID_ARG;
  if (K > sas::kMaxTrainK || C > 16384 || (C > sas::kLongHistory && K > 64))
    return SAS_ERR_UNSUPPORTED;
  if ((shape->gate & SAS_GATE_ACTIVATION_MASK) > SAS_GATE_RAW) return SAS_ERR_INVALID_ARG;
  const int act = shape->gate & SAS_GATE_ACTIVATION_MASK;
  const hipStream_t st = (hipStream_t)stream;
  const int rows_bk = shape->batch * shape->hkv;
  double scale = 0.0;
  if (!s) {
    if (!qbar || !kbar || !s_out) return SAS_ERR_INVALID_ARG;
    if (kbar_dtype != SAS_DTYPE_F32 && kbar_dtype != SAS_DTYPE_BF16) return SAS_ERR_INVALID_ARG;
    if (kbar_ld < C) return SAS_ERR_INVALID_ARG;
    if (shape->head_dim <= 0) return SAS_ERR_INVALID_ARG;
    if (shape->head_dim != 64 && shape->head_dim != 128) return SAS_ERR_UNSUPPORTED;
    if (!(shape->scale >= 0.0f)) return SAS_ERR_INVALID_ARG;
    if (!aligned16(qbar) || !aligned16(kbar)) return SAS_ERR_INVALID_ARG;
    scale = shape->scale > 0.0f ? (double)shape->scale : 1.0 / sqrt((double)shape->head_dim);
  }
  sas::RowLens rl{};
  if (shape->seq_lens) {  // ragged batch: shape->seqlen and ->block describe the tokens
    if (shape->seqlen <= 0 || shape->block <= 0) return SAS_ERR_INVALID_ARG;
    rl = sas::RowLens{shape->seq_lens, shape->seqlen, shape->block, shape->hkv};
  }
  const size_t need = sas::select_workspace_bytes(rows_bk, T, C, K);
  if (need > 0 && (!workspace || ws_bytes < need)) return SAS_ERR_WORKSPACE;
  if (C > sas::kLongHistory)
    return launch_status(sas::launch_select_long(
        s, qbar, kbar, kbar_dtype == SAS_DTYPE_BF16, kbar_ld, shape->head_dim, scale, rows_bk, T,
        C, row_offset, K, act, s_out, idx, logg, lse_s, workspace, st, rl));
  return launch_status(sas::launch_topk(s, qbar, kbar, kbar_dtype == SAS_DTYPE_BF16, kbar_ld,
                                        shape->head_dim, scale, s_out, rows_bk, T, C,
                                        row_offset, K, act, idx, logg, lse_s, st, rl));
}

size_t sas_attn_fwd_workspace_size(const sas_shape* shape, int K) {
  (void)shape;
  (void)K;
  return 0;
}

sas_status sas_attn_fwd(const sas_shape* shape, int K, const void* q, const void* k,
                        const void* v, const int32_t* idx, const float* logg, void* o,
                        float* lse, void* workspace, size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  SAS_TRY(check_shape(shape));
  if (K <= 0) return SAS_ERR_INVALID_ARG;
  if (K > sas::kMaxTrainK) return SAS_ERR_UNSUPPORTED;
  if (!q || !k || !v || !idx || !o || !lse) return SAS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return SAS_ERR_INVALID_ARG;
  const Dims dm = make_dims(shape, K);
  const hipStream_t st = (hipStream_t)stream;
  const float* lg = dm.ste ? nullptr : logg;  // hard gating: the forward is ungated
  if (sas::mfma_fwd_supported(dm))
    return launch_status(sas::launch_fwd_mfma(dm, q, k, v, idx, lg, o, lse, st));
  return launch_status(sas::launch_fwd_generic(dm, q, k, v, idx, lg, o, lse, st));
}

size_t sas_attn_bwd_workspace_size(const sas_shape* shape, int K) {
  if (check_shape(shape) != SAS_OK || K <= 0 || K > sas::kMaxTrainK) return 0;
  const Dims dm = make_dims(shape, K);
  return sas::bwd_workspace_layout(dm, nullptr).bytes;
}

sas_status sas_attn_bwd(const sas_shape* shape, int K, const void* q, const void* k,
                        const void* v, const void* o, const void* dout, const float* lse,
                        const int32_t* idx, const float* logg, const float* s,
                        const float* lse_s, void* dq, void* dk, void* dv, float* dlogg,
                        float* ds, void* workspace, size_t ws_bytes, void* stream) {
  SAS_TRY(check_shape(shape));
  if (K <= 0) return SAS_ERR_INVALID_ARG;
  if (K > sas::kMaxTrainK) return SAS_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !dout || !lse || !idx || !dq || !dk || !dv)
    return SAS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return SAS_ERR_INVALID_ARG;
  const Dims dm = make_dims(shape, K);
  // selector outputs need the gates (soft) or at least the selection (ste)
  if (!logg && !dm.ste && (dlogg || ds || s || lse_s)) return SAS_ERR_INVALID_ARG;
  if (ds && (!s || (!lse_s && dm.act == SAS_GATE_SOFTMAX))) return SAS_ERR_INVALID_ARG;
  const sas::BwdWorkspace ws = sas::bwd_workspace_layout(dm, workspace);
  if (!workspace || ws_bytes < ws.bytes) return SAS_ERR_WORKSPACE;
  const hipStream_t st = (hipStream_t)stream;
  const bool mfma = sas::mfma_bwd_supported(dm);
  const float* lg = dm.ste ? nullptr : logg;  // hard gating: the attention is ungated
  if (mfma) {
    // dlogg is written whole by the dK/dV kernel (one partial per row)
    const auto tail = [&]() -> hipError_t {
      if (!dlogg && !ds) return hipSuccess;
      return sas::launch_bwd_ds(dm, idx, s, lse_s, ws.dlogg_part, 1, dlogg, ds, st);
    };
    SAS_LAUNCH(
        sas::launch_bwd_mfma(dm, q, k, v, o, dout, lse, idx, lg, dq, dk, dv, ws, tail, st));
    return SAS_OK;
  }
  SAS_LAUNCH(sas::launch_bwd_prep(dm, o, dout, idx, ws, true, st));
  int nchunk = 0;
  SAS_LAUNCH(sas::launch_bwd_generic(dm, q, k, v, dout, lse, idx, lg, dq, dk, dv, ws, &nchunk,
                                     st));
  if (dlogg || ds)
    SAS_LAUNCH(sas::launch_bwd_ds(dm, idx, s, lse_s, ws.dlogg_part, nchunk, dlogg, ds, st));
  return SAS_OK;
}

size_t sas_decode_workspace_size(const sas_shape* shape, int K) {
  if (check_shape(shape) != SAS_OK || K <= 0 || K > 64) return 0;
  return sas::decode_workspace_bytes(make_dims(shape, K));
}

sas_status sas_decode(const sas_shape* shape, int cache_len, int K, const void* q,
                      const void* kcache, const void* vcache, const int32_t* idx,
                      const float* logg, void* o, float* lse, void* workspace,
                      size_t ws_bytes, void* stream) {
  SAS_TRY(check_shape(shape));
  if (K <= 0 || cache_len < 0) return SAS_ERR_INVALID_ARG;
  if (K > 64) return SAS_ERR_UNSUPPORTED;
  const int L = shape->seqlen;
  const int cl = cache_len == 0 ? L : cache_len;
  if (cl < L) return SAS_ERR_INVALID_ARG;
  if (!q || !kcache || !vcache || !idx || !o || !lse) return SAS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o))
    return SAS_ERR_INVALID_ARG;
  if (shape->hq / shape->hkv > 8) return SAS_ERR_UNSUPPORTED;
  const Dims dm = make_dims(shape, K);
  const size_t need = sas::decode_workspace_bytes(dm);
  if (!workspace || ws_bytes < need) return SAS_ERR_WORKSPACE;
  const sas::KvView kvv{kcache, vcache, cl, nullptr, 0, 0, shape->seq_lens};
  return launch_status(sas::launch_decode(dm, L, kvv, q, idx, dm.ste ? nullptr : logg, o, lse,
                                          workspace, (hipStream_t)stream));
}

// ---- fused decode step
namespace {

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct StepLayout {
  bool fused;
  int C, nchunk;
  size_t cand, stats, part;            // fused: offsets of the three regions
  size_t qbar, idx, logg, lse_s, sel;  // composed: pooled q, selection outputs, select workspace
  size_t dec;                          // decode partials
  size_t bytes;
};

StepLayout step_layout(const sas_shape* shape, int K) {
  StepLayout l{};
  const Dims dm = make_dims(shape, K);
  const size_t rows = (size_t)shape->batch * shape->hkv;
  l.C = (shape->seqlen - 1) / shape->block;
  l.nchunk = (l.C + sas::kSelectChunk - 1) / sas::kSelectChunk;
  l.fused = sas::decode_mfma_path(dm) && (size_t)l.nchunk * K <= 2048;
  if (l.fused) {
    l.cand = 0;
    l.stats = align256(rows * l.nchunk * K * sizeof(uint64_t));
    l.part = l.stats + align256(rows * l.nchunk * sizeof(float2));
    l.bytes = l.part + align256(sas::decode_workspace_bytes(dm));
  } else {
    l.qbar = 0;
    l.idx = align256(rows * shape->head_dim * sizeof(float));
    l.logg = l.idx + align256(rows * K * sizeof(int32_t));
    l.lse_s = l.logg + align256(rows * K * sizeof(float));
    l.sel = l.lse_s + align256(rows * sizeof(float));
    // scores (s_out) first, then the long-history candidates
    const size_t s_bytes = align256(rows * (size_t)(l.C > 0 ? l.C : 1) * sizeof(float));
    l.dec = l.sel + s_bytes + align256(sas::select_workspace_bytes((int)rows, 1, l.C, K));
    l.bytes = l.dec + align256(sas::decode_workspace_bytes(dm));
  }
  return l;
}

}  // namespace

size_t sas_decode_step_workspace_size(const sas_shape* shape, int K) {
  if (check_shape(shape) != SAS_OK || K <= 0 || K > 64) return 0;
  return step_layout(shape, K).bytes;
}

namespace {

// One decode step (pool + stand-in select + decode) over a dense or paged view
// of the cache.  Ragged (seq_lens) views take the fused path only.
sas_status decode_step_impl(const sas_shape* shape, int K, const void* q, const void* kbar,
                            sas_dtype kbar_dtype, int kbar_ld, const sas::KvView& kvv,
                            int gated, void* o, float* lse, int32_t* idx, float* logg,
                            float* lse_s, void* workspace, size_t ws_bytes, void* stream) {
  const int L = shape->seqlen;
  if (!q || !kbar || !o || !lse) return SAS_ERR_INVALID_ARG;
  if ((idx == nullptr) != (logg == nullptr) || (idx == nullptr) != (lse_s == nullptr))
    return SAS_ERR_INVALID_ARG;
  if (kbar_dtype != SAS_DTYPE_F32 && kbar_dtype != SAS_DTYPE_BF16) return SAS_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kbar) || !aligned16(o)) return SAS_ERR_INVALID_ARG;
  if (shape->hq / shape->hkv > 8) return SAS_ERR_UNSUPPORTED;
  const StepLayout lay = step_layout(shape, K);
  if (kbar_ld < lay.C) return SAS_ERR_INVALID_ARG;
  if (lay.C > 16384) return SAS_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < lay.bytes) return SAS_ERR_WORKSPACE;
  const Dims dm = make_dims(shape, K);
  const hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const double scale =
      shape->scale > 0.0f ? (double)shape->scale : 1.0 / sqrt((double)shape->head_dim);
  const int rows = shape->batch * shape->hkv;
  const int G = shape->hq / shape->hkv;
  const sas::RowLens rl{kvv.seq_lens, L, shape->block, shape->hkv};
  if (lay.fused) {
    uint64_t* cand = (uint64_t*)(ws + lay.cand);
    float2* stats = (float2*)(ws + lay.stats);
    SAS_LAUNCH(sas::launch_select_chunks_rawq(
        (const uint16_t*)q, G, kbar, kbar_dtype == SAS_DTYPE_BF16, kbar_ld, shape->head_dim,
        scale, rows, lay.C, K, rl, cand, stats, st));
    return launch_status(sas::launch_decode_step(dm, L, kvv, lay.C, lay.nchunk, q, cand, stats,
                                                 gated && !dm.ste, idx, logg, lse_s, o, lse,
                                                 ws + lay.part, st));
  }
  // Every other shape: the same three stages through the separate calls' kernels.
  float* qbar = (float*)(ws + lay.qbar);
  int32_t* idx_w = idx ? idx : (int32_t*)(ws + lay.idx);
  float* logg_w = logg ? logg : (float*)(ws + lay.logg);
  float* lse_s_w = lse_s ? lse_s : (float*)(ws + lay.lse_s);
  float* s_out = (float*)(ws + lay.sel);
  const size_t s_bytes = align256((size_t)rows * (lay.C > 0 ? lay.C : 1) * sizeof(float));
  SAS_LAUNCH(sas::launch_block_pool(q, shape->dtype == SAS_DTYPE_BF16, shape->batch, shape->hq,
                                    G, 1, shape->head_dim, shape->block, false, qbar, st));
  if (lay.C > sas::kLongHistory)
    SAS_LAUNCH(sas::launch_select_long(nullptr, qbar, kbar, kbar_dtype == SAS_DTYPE_BF16, kbar_ld,
                                       shape->head_dim, scale, rows, 1, lay.C, lay.C, K, dm.act,
                                       s_out, idx_w, logg_w, lse_s_w, ws + lay.sel + s_bytes,
                                       st, rl));
  else
    SAS_LAUNCH(sas::launch_topk(nullptr, qbar, kbar, kbar_dtype == SAS_DTYPE_BF16, kbar_ld,
                                shape->head_dim, scale, s_out, rows, 1, lay.C, lay.C, K, dm.act,
                                idx_w, logg_w, lse_s_w, st, rl));
  return launch_status(sas::launch_decode(dm, L, kvv, q, idx_w,
                                          (gated && !dm.ste) ? logg_w : nullptr, o, lse,
                                          ws + lay.dec, st));
}

// Checks of a paged view: pages, table and lengths present and the table wide
// enough for seqlen tokens.
sas_status check_paged(const sas_shape* shape, const void* kpages, const void* vpages,
                       int num_pages, const int32_t* block_table, int bt_ld,
                       const int32_t* seq_lens) {
  if (!kpages || !vpages || !block_table || !seq_lens || num_pages <= 0) return SAS_ERR_INVALID_ARG;
  if (!aligned16(kpages) || !aligned16(vpages)) return SAS_ERR_INVALID_ARG;
  const int need = (shape->seqlen + shape->block - 1) / shape->block;
  if (bt_ld < need) return SAS_ERR_INVALID_ARG;
  return SAS_OK;
}

}  // namespace

sas_status sas_decode_step(const sas_shape* shape, int cache_len, int K, const void* q,
                           const void* kbar, sas_dtype kbar_dtype, int kbar_ld,
                           const void* kcache, const void* vcache, int gated, void* o,
                           float* lse, int32_t* idx, float* logg, float* lse_s,
                           void* workspace, size_t ws_bytes, void* stream) {
  SAS_TRY(check_shape(shape));
  if (K <= 0 || cache_len < 0) return SAS_ERR_INVALID_ARG;
  if (K > 64) return SAS_ERR_UNSUPPORTED;
  const int L = shape->seqlen;
  const int cl = cache_len == 0 ? L : cache_len;
  if (cl < L) return SAS_ERR_INVALID_ARG;
  if (!kcache || !vcache || !aligned16(kcache) || !aligned16(vcache)) return SAS_ERR_INVALID_ARG;
  const sas::KvView kvv{kcache, vcache, cl, nullptr, 0, 0, shape->seq_lens};
  return decode_step_impl(shape, K, q, kbar, kbar_dtype, kbar_ld, kvv, gated, o, lse, idx, logg,
                          lse_s, workspace, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of sas_decode_step_noalloc: one copy per GPU, held until the process
// ends.  Host code never passes `scratch` itself (on the host it names a stand-in,
// not device memory): each device's address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept in scratch_table.
static __device__ __align__(256) unsigned char scratch[SAS_STATIC_SCRATCH_BYTES];

struct ScratchTable {
  std::mutex mu;
  void* ptr[64] = {};
};

ScratchTable& scratch_table() {
  static ScratchTable t;
  return t;
}

// The current device's copy of `scratch`, or nullptr when it cannot be found.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  ScratchTable& t = scratch_table();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    t.ptr[dev] = p;
  }
  return t.ptr[dev];
}

}  // namespace

extern "C" {

sas_status sas_decode_step_noalloc(const sas_shape* shape, int cache_len, int K, const void* q,
                                   const void* kbar, sas_dtype kbar_dtype, int kbar_ld,
                                   const void* kcache, const void* vcache, int gated, void* o,
                                   float* lse, int32_t* idx, float* logg, float* lse_s,
                                   void* stream) {
  SAS_TRY(check_shape(shape));
  if (K <= 0 || cache_len < 0) return SAS_ERR_INVALID_ARG;
  if (K > 64) return SAS_ERR_UNSUPPORTED;
  // the size check is host arithmetic only: no device call before it
  if (step_layout(shape, K).bytes > (size_t)SAS_STATIC_SCRATCH_BYTES) return SAS_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return SAS_ERR_LAUNCH;
  return sas_decode_step(shape, cache_len, K, q, kbar, kbar_dtype, kbar_ld, kcache, vcache,
                         gated, o, lse, idx, logg, lse_s, ws, (size_t)SAS_STATIC_SCRATCH_BYTES,
                         stream);
}

sas_status sas_decode_paged(const sas_shape* shape, int K, const void* q, const void* kpages,
                            const void* vpages, int num_pages, const int32_t* block_table,
                            int bt_ld, const int32_t* seq_lens, const int32_t* idx,
                            const float* logg, void* o, float* lse, void* workspace,
                            size_t ws_bytes, void* stream) {
  SAS_TRY(check_shape(shape));
  if (K <= 0) return SAS_ERR_INVALID_ARG;
  if (K > 64) return SAS_ERR_UNSUPPORTED;
  SAS_TRY(check_paged(shape, kpages, vpages, num_pages, block_table, bt_ld, seq_lens));
  if (!q || !idx || !o || !lse || !aligned16(q) || !aligned16(o)) return SAS_ERR_INVALID_ARG;
  if (shape->hq / shape->hkv > 8) return SAS_ERR_UNSUPPORTED;
  const Dims dm = make_dims(shape, K);
  if (!workspace || ws_bytes < sas::decode_workspace_bytes(dm)) return SAS_ERR_WORKSPACE;
  const sas::KvView kvv{kpages, vpages, 0, block_table, bt_ld, num_pages, seq_lens};
  return launch_status(sas::launch_decode(dm, shape->seqlen, kvv, q, idx,
                                          dm.ste ? nullptr : logg, o, lse, workspace,
                                          (hipStream_t)stream));
}

sas_status sas_decode_step_paged(const sas_shape* shape, int K, const void* q,
                                 const void* kbar, sas_dtype kbar_dtype, int kbar_ld,
                                 const void* kpages, const void* vpages, int num_pages,
                                 const int32_t* block_table, int bt_ld, const int32_t* seq_lens,
                                 int gated, void* o, float* lse, int32_t* idx, float* logg,
                                 float* lse_s, void* workspace, size_t ws_bytes, void* stream) {
  SAS_TRY(check_shape(shape));
  if (K <= 0) return SAS_ERR_INVALID_ARG;
  if (K > 64) return SAS_ERR_UNSUPPORTED;
  SAS_TRY(check_paged(shape, kpages, vpages, num_pages, block_table, bt_ld, seq_lens));
  const sas::KvView kvv{kpages, vpages, 0, block_table, bt_ld, num_pages, seq_lens};
  return decode_step_impl(shape, K, q, kbar, kbar_dtype, kbar_ld, kvv, gated, o, lse, idx, logg,
                          lse_s, workspace, ws_bytes, stream);
}

sas_status sas_selector_bwd(const sas_shape* shape, const float* ds, const float* qbar,
                            const float* kbar, float* dqbar, float* dkbar, void* dq, void* dk,
                            void* stream) {
  SAS_TRY(check_shape(shape));
  if (!ds || !qbar || !kbar || !dqbar || !dkbar) return SAS_ERR_INVALID_ARG;
  if (!aligned16(qbar) || !aligned16(kbar) || !aligned16(dqbar) || !aligned16(dkbar) ||
      (dq && !aligned16(dq)) || (dk && !aligned16(dk)))
    return SAS_ERR_INVALID_ARG;
  if ((long)shape->batch * shape->hq > 65535) return SAS_ERR_UNSUPPORTED;  // grid y / z
  const Dims dm = make_dims(shape, 1);
  if (dm.n == 0) return SAS_OK;
  return launch_status(sas::launch_selector_bwd(dm, ds, qbar, kbar, dqbar, dkbar, dq, dk,
                                                (hipStream_t)stream));
}

void sas_profiler_enable(int on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
}

void sas_profiler_reset(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.drain();
  p.totals.clear();
}

int sas_profiler_read(sas_kernel_time* out, int max_entries) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.drain();
  int i = 0;
  for (auto& kvp : p.totals) {
    if (out && i < max_entries) {
      memset(out[i].name, 0, sizeof(out[i].name));
      strncpy(out[i].name, kvp.first.c_str(), sizeof(out[i].name) - 1);
      out[i].launches = kvp.second.first;
      out[i].total_ms = kvp.second.second;
    }
    ++i;
  }
  return i;
}

}  // extern "C"
