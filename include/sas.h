/*
 * sas.h -- C ABI of the MI355X (gfx950) library for SAS gated block-sparse
 * causal attention.
 *
 * The method (page titles of the sources, then section / equation):
 *   picx.dev summary of "SAS: Simple Attention Sparsification":
 *     'Theoretical Foundation' Eq. 2-3 (block-sparse attention over a Top-K set
 *     of history blocks), 'Key Idea: Differentiable Continuous Gating' Eq. 4
 *     (positive gates, g0 = 1 on the always-kept current block) and Eq. 9 (log
 *     gates added inside the attention softmax), 'Gradient Analysis' Eq. 5
 *     (inner-gate gradient) and Eq. 6 (softmax gates: log g_m = s_m - LSE(s)),
 *     'Kernel Design' (fused flash-style kernel, no attention matrix).
 *   "SAS: End-to-end learning of sparse attention rankings from language-model
 *     loss" (reproduction README): 'Core equations' (the 1/sqrt(d) scale and
 *     g = softmax(s) over the history blocks before Top-K).
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains them; scratch comes from a caller
 *     workspace whose size the matching *_workspace_size call returns.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream) and returns without waiting.
 *   - Argument errors (null pointers, bad sizes, unsupported shapes, short
 *     workspace) are detected on the host before anything is launched and
 *     returned synchronously; nothing is enqueued then.  SAS_ERR_LAUNCH
 *     reports a failed enqueue (hipGetLastError after the launch).
 *   - Layouts are dense row-major with head_dim innermost:
 *       q, o, dout, dq      [batch, hq,  seqlen, head_dim]
 *       k, v, dk, dv        [batch, hkv, seqlen, head_dim]
 *       scores s, ds        [batch, hkv, T, C]        fp32
 *       idx, logg           [batch, hkv, T, K]        int32 / fp32
 *     with T = ceil(seqlen / block) query blocks.  Query head h reads KV head
 *     h / (hq / hkv); all query heads of one KV head share one selection.
 *   - Block B_m holds tokens [m*block, min((m+1)*block, seqlen)); the query
 *     block of row i is B_t, t = i / block.  Row i attends to the tokens of
 *     the selected history blocks (fully) and to tokens j <= i of B_t.
 *   - idx entries are ascending block indices, -1 for unused slots.  Entries
 *     outside [0, t) of their row are ignored by the attention kernels (they
 *     can never make a kernel read outside the tensors).
 *   - Supported: head_dim in {64, 128}; block in {16, 32, 64}; dtype fp32
 *     (all tensors fp32) or bf16 (q, k, v, o, dout, dq, dk, dv bf16; scores,
 *     gates, LSE, ds fp32); hq a multiple of hkv; 1 <= K <= 254 for the
 *     training calls (sas_select_topk with C <= 512, sas_attn_fwd,
 *     sas_attn_bwd), so that K >= C_t -- every history block selected and
 *     gated, the dense scope of the pages' ablations -- is expressible for
 *     up to 255 blocks; 1 <= K <= 64 for sas_select_topk with C > 512 and the
 *     decode calls.  Anything else returns SAS_ERR_UNSUPPORTED.
 *   - Calls are thread-safe.  Calls that share output buffers must not
 *     overlap.  Every call is ordered on the caller's stream; sas_attn_bwd may
 *     fork part of its work onto a second stream of the library's own (one per
 *     device for the whole process, default priority, created on first use,
 *     shared by threads under a lock held while a call enqueues its fork,
 *     kernels and join) and joins it back to the caller's stream with events
 *     before returning.
 *   - No call allocates device memory, records a memset or synchronises, so
 *     every call can be captured in a HIP graph on a capturing stream (make
 *     one eager sas_attn_bwd call first, so that its second stream exists
 *     before the capture begins).
 */
#ifndef SAS_H
#define SAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAS_OK = 0,
  SAS_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, inconsistent shape */
  SAS_ERR_UNSUPPORTED = 2,  /* valid, but outside the supported shapes above */
  SAS_ERR_WORKSPACE = 3,    /* workspace pointer NULL or smaller than required */
  SAS_ERR_LAUNCH = 4        /* the HIP runtime refused a launch */
} sas_status;

typedef enum { SAS_DTYPE_F32 = 0, SAS_DTYPE_BF16 = 1 } sas_dtype;

/* Gate variants, the ablation axes the pages report (the 'Gradient Analysis'
 * and Eq. 4 of the picx.dev summary; Table 1 of the alanhou.org and cctest.ai
 * pages).  sas_shape.gate = one activation | optional flags; 0 is SAS itself
 * (softmax activation, inner gating, soft gates).
 *   activation phi of Eq. 4, the log gate of a selected history block m:
 *     SAS_GATE_SOFTMAX  log g_m = s_m - LSE(s) over the row's history (Eq. 6)
 *     SAS_GATE_SIGMOID  log g_m = log sigmoid(s_m)
 *     SAS_GATE_RAW      log g_m = s_m (the raw selector logit)
 *   SAS_GATE_OUTER  gates applied after the softmax: o = sum_j p_j g_m(j) v_j
 *                   with p the ungated softmax (the right-hand gradient of Eq. 5);
 *                   dlogg_m = g_m dL/dg_m = sum over block m of p dO . (g v)
 *   SAS_GATE_STE    hard gating with a straight-through backward: the attention
 *                   ignores logg (g = 1 on the selected blocks), dlogg is
 *                   dL/dg there, and ds applies the soft phi's Jacobian to it.
 * sas_select_topk reads the activation (logg); sas_attn_fwd / sas_decode read
 * OUTER and STE; sas_attn_bwd reads all three; sas_decode_step reads the
 * activation and OUTER.  Every kernel (bf16 MFMA and portable) runs both
 * inner and outer gating. */
typedef enum {
  SAS_GATE_SOFTMAX = 0,
  SAS_GATE_SIGMOID = 1,
  SAS_GATE_RAW = 2,
  SAS_GATE_ACTIVATION_MASK = 3,
  SAS_GATE_OUTER = 4,
  SAS_GATE_STE = 8
} sas_gate;

typedef struct {
  int batch;
  int hq;        /* query heads */
  int hkv;       /* key/value heads; hq % hkv == 0, G = hq / hkv */
  int seqlen;    /* training: N tokens; decode: valid cache length L (incl. new token) */
  int head_dim;  /* d */
  int block;     /* tokens per block */
  sas_dtype dtype;
  float scale;   /* logit scale; 0 selects 1/sqrt(head_dim) */
  int gate;      /* sas_gate bits; 0 = SAS (softmax, inner, soft) */
  /* Ragged batch (optional, device int32 [batch]; NULL: every sequence has
   * length seqlen).  Training calls: sequence b is its first seq_lens[b]
   * tokens of the padded [.., seqlen, d] tensors (clamped to [0, seqlen]) and
   * is computed exactly as if alone; rows past its end are padding, which must
   * hold finite values and carry no result (o = 0, lse = +inf, gradients 0;
   * selection rows past its last block: idx -1, logg 0, lse_s -inf, ds 0).
   * Decode calls: the valid cache length of sequence b (clamped to
   * [1, seqlen]), its new token at seq_lens[b] - 1. */
  const int32_t* seq_lens;
} sas_shape;

/* Human-readable name of a status code (static string). */
const char* sas_status_string(sas_status status);

/* Library ABI version (major * 100 + minor). */
int sas_version(void);

/* ------------------------------------------------------------------------
 * Block summaries for the stand-in selector (evolve.pub review of SAS, FAQ:
 * pooling-based block summaries).
 *
 * out[b, h / group, t, :] = mean of x[b, h', i, :] over the `group` heads
 * h' of that group and the valid tokens i of block B_t, accumulated in fp64
 * and rounded to fp32 (out_dtype F32) or, for out_dtype BF16, rounded to fp32
 * and then to bf16 (both round-to-nearest-even).
 *   x   : [batch, heads, seqlen, head_dim] in shape->dtype, 16-byte aligned
 *   out : [batch, heads / group, ceil(seqlen / block), head_dim] in out_dtype
 * Uses shape->batch, seqlen, head_dim, block, dtype.  heads % group == 0.
 * ---------------------------------------------------------------------- */
sas_status sas_block_pool(const sas_shape* shape, const void* x, int heads, int group,
                          sas_dtype out_dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * Gate normalisation and hard Top-K (picx Eq. 3, Eq. 4, Eq. 6).
 *
 * Rows r = (b, kv, t), t < T.  Row t ranks the history blocks m < C_t with
 *   C_t = min(t + row_offset, C)
 * (training: T = C = number of blocks, row_offset = 0; decode: T = 1,
 * C = (L - 1) / block, row_offset = C).
 *
 * Scores: either s != NULL (fp32 [b, hkv, T, C]; only m < C_t is read, and
 * those entries must be finite), or s == NULL and the stand-in score
 *   s[r, m] = fp32( (qbar[r] . kbar[b, kv, m]) * scale )
 * is formed from qbar (fp32 [b, hkv, T, head_dim]) and kbar ([b, hkv,
 * kbar_ld, head_dim] in kbar_dtype, kbar_ld >= C), the dot product and the
 * scaling in fp64 (scale = shape->scale, 0 -> 1/sqrt(head_dim)).  The scores
 * are then written to s_out (fp32 [b, hkv, T, C]; 0 for m >= C_t).
 *
 * Outputs, per row:
 *   lse_s[r]  = log sum_{m < C_t} exp(s_m)             (-inf when C_t = 0)
 *   idx[r, :] = the min(K, C_t) blocks of largest s, equal scores resolved
 *               to the lower block index (-0.0 equals +0.0), ascending,
 *               -1 padded
 *   logg[r,:] = log g of those blocks under the gate activation
 *               (shape->gate: s_idx - lse_s for softmax; fp32; 0 on padded
 *               slots)
 * Uses shape->batch, hkv, head_dim, scale, gate.  C <= 16384.
 * Ragged batch (shape->seq_lens): shape->seqlen and ->block then give the
 * tokens and block size; training rows (row_offset 0) at or past a sequence's
 * last block have no history (C_t = 0), decode rows rank the sequence's own
 * (seq_lens[b] - 1) / block blocks.
 *
 * Rows with more than 512 history blocks are served by two kernels (chunked
 * candidates, then a per-row merge) whose candidates live in the workspace:
 * sas_select_topk_workspace_size bytes (0 when C <= 512).
 * ---------------------------------------------------------------------- */
size_t sas_select_topk_workspace_size(const sas_shape* shape, int T, int C, int K);
sas_status sas_select_topk(const sas_shape* shape, int T, int C, int row_offset, int K,
                           const float* s, const float* qbar, const void* kbar,
                           sas_dtype kbar_dtype, int kbar_ld, float* s_out,
                           int32_t* idx, float* logg, float* lse_s, void* workspace,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Fused gated block-sparse forward (picx Eq. 9, 'Kernel Design'):
 *   o_i = sum_j softmax_j( q_i . k_j * scale + bias_j ) v_j,
 *   lse[b, h, i] = log sum_j exp( q_i . k_j * scale + bias_j ),
 * over the keys j of the selected history blocks (bias = logg of the block's
 * slot) and the causal prefix of the current block (bias 0 = log g0).
 * logg == NULL computes the ungated form (picx Eq. 2).
 *   q [b,hq,N,d], k/v [b,hkv,N,d] (shape->dtype); idx/logg [b,hkv,T,K];
 *   o [b,hq,N,d] (shape->dtype); lse fp32 [b,hq,N].
 * ---------------------------------------------------------------------- */
size_t sas_attn_fwd_workspace_size(const sas_shape* shape, int K);
sas_status sas_attn_fwd(const sas_shape* shape, int K, const void* q, const void* k,
                        const void* v, const int32_t* idx, const float* logg, void* o,
                        float* lse, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of L = sum dout . o (picx Eq. 5 inner gating; Eq. 6 for ds).
 *   dq, dk, dv      : gradients of q, k, v (shape->dtype; fp32 accumulation)
 *   dlogg (optional): fp32 [b,hkv,T,K], sum over the block's keys, all rows of
 *                     the query block and all G heads of dS_ij; 0 on pads
 *   ds (optional)   : fp32 [b,hkv,T,T], the selector gradient through the
 *                     gate softmax over ALL history blocks of the row,
 *                     ds_m = [m in I] dlogg_m - g_m * sum_{m' in I} dlogg_m',
 *                     g_m = exp(s_m - lse_s); 0 for m >= t.
 *                     Needs s [b,hkv,T,T] and lse_s [b,hkv,T] from
 *                     sas_select_topk.
 * o and lse are the forward's outputs.  With logg == NULL (ungated) dlogg,
 * ds, s and lse_s must be NULL.  dq/dk/dv are overwritten.
 * The workspace size depends on the shape, K and the CU count of the current
 * device (small grids split the longest dK/dV lists and keep fp32 partials
 * there): query it with the device that runs the call current.
 * ---------------------------------------------------------------------- */
size_t sas_attn_bwd_workspace_size(const sas_shape* shape, int K);
sas_status sas_attn_bwd(const sas_shape* shape, int K, const void* q, const void* k,
                        const void* v, const void* o, const void* dout, const float* lse,
                        const int32_t* idx, const float* logg, const float* s,
                        const float* lse_s, void* dq, void* dk, void* dv, float* dlogg,
                        float* ds, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Single-token decode (picx Eq. 9 with one query; Eq. 2 when logg == NULL,
 * the deployed form without gates, evolve.pub review 'Summary').
 * The new token sits at position L - 1 = shape->seqlen - 1; its current block
 * is c = (L - 1) / block and the history blocks are m < c.
 *   q      [b, hq, d]                       (shape->dtype)
 *   kcache [b, hkv, cache_len, d], vcache the same; cache_len >= L
 *          (cache_len = 0 means L)
 *   idx    [b, hkv, K] int32 (ascending, -1 padded, entries >= c ignored)
 *   logg   [b, hkv, K] fp32 or NULL
 *   o      [b, hq, d] (shape->dtype);  lse fp32 [b, hq]
 * Split-K over the selected blocks with an LSE merge; the partials live in
 * the workspace (no initial contents needed).  Calls that share a workspace
 * must not run concurrently.
 * ---------------------------------------------------------------------- */
size_t sas_decode_workspace_size(const sas_shape* shape, int K);
sas_status sas_decode(const sas_shape* shape, int cache_len, int K, const void* q,
                      const void* kcache, const void* vcache, const int32_t* idx,
                      const float* logg, void* o, float* lse, void* workspace,
                      size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * One decode step with the stand-in selector, fused (picx 'Decode Efficiency'
 * (Figure 7): at long contexts the block selection dominates the decode step).
 * Computes what sas_block_pool (q over the G heads of each KV head, one token)
 * + sas_select_topk (T = 1, C = row_offset = (L - 1) / block, scores from the
 * pooled query and kbar) + sas_decode produce, with the same rounding and the
 * same results, in three kernels for bf16 / head_dim 128 / block 64 (the
 * chunked scores + Top-K candidates, then the decode, which merges the
 * candidates itself, then the LSE merge), and through those calls' kernels for
 * every other supported shape.
 *   q      [b, hq, d] (shape->dtype); L = shape->seqlen (the new token at L - 1)
 *   kbar   pooled-key cache [b, hkv, kbar_ld, d] in kbar_dtype (block means of
 *          kcache, e.g. from sas_block_pool), kbar_ld >= C
 *   kcache, vcache, cache_len: as for sas_decode
 *   gated  1: the selected blocks carry their log gates (Eq. 9); 0: ungated
 *          (Eq. 2), the selection unchanged
 *   o, lse as for sas_decode
 *   idx, logg, lse_s: optional ([b,hkv,K] int32, [b,hkv,K] fp32, [b,hkv] fp32;
 *          all three or none), the selection as sas_select_topk returns it
 * Needs C <= 16384.  The workspace holds the selection candidates and the
 * decode partials (no initial contents needed).
 * ---------------------------------------------------------------------- */
size_t sas_decode_step_workspace_size(const sas_shape* shape, int K);
sas_status sas_decode_step(const sas_shape* shape, int cache_len, int K, const void* q,
                           const void* kbar, sas_dtype kbar_dtype, int kbar_ld,
                           const void* kcache, const void* vcache, int gated, void* o,
                           float* lse, int32_t* idx, float* logg, float* lse_s,
                           void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * sas_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks and results as
 * sas_decode_step; the candidates and decode partials live in a static
 * SAS_STATIC_SCRATCH_BYTES device array that the library holds on every GPU it
 * runs on until the process ends (its address is looked up once per device).
 * Nothing is allocated and nothing needs clearing: the step writes every
 * scratch byte it reads.  Returns SAS_ERR_WORKSPACE, before any device call,
 * when the step needs more scratch than that (sas_decode_step_workspace_size
 * gives the need; e.g. batch 8 x 64K tokens, 32/8 heads, K 63: 4.4 MB).  All
 * calls on one GPU share its array: calls that overlap on one GPU (two streams,
 * two threads) race and must be serialised by the caller.
 * ---------------------------------------------------------------------- */
#define SAS_STATIC_SCRATCH_BYTES (16u << 20)
sas_status sas_decode_step_noalloc(const sas_shape* shape, int cache_len, int K, const void* q,
                                   const void* kbar, sas_dtype kbar_dtype, int kbar_ld,
                                   const void* kcache, const void* vcache, int gated, void* o,
                                   float* lse, int32_t* idx, float* logg, float* lse_s,
                                   void* stream);

/* ------------------------------------------------------------------------
 * Paged cache, ragged batch: the serving setting of the pages' decode
 * measurements (picx 'Decode Efficiency (Figure 7)': batch 8 at 64K, batch 1
 * up to 512K).  Sequence b has its own valid length L_b = seq_lens[b] (its new
 * token at L_b - 1, current block c_b = (L_b - 1) / block, history blocks
 * m < c_b), and its K / V rows live in pages of one block each:
 *   kpages, vpages  [num_pages, hkv, block, d] (shape->dtype); page p holds
 *                   the `block` consecutive tokens of one logical block for
 *                   every KV head
 *   block_table     int32 [b, bt_ld] (device): logical block m of sequence b
 *                   is page block_table[b * bt_ld + m]; bt_ld >= ceil(seqlen /
 *                   block).  A page number outside [0, num_pages) makes that
 *                   block empty (nothing is read from it).
 *   seq_lens        int32 [b] (device); entries are clamped to [1, seqlen],
 *                   shape->seqlen being the longest sequence of the batch
 * sas_decode_paged: as sas_decode with the selection given (idx, logg
 *   [b, hkv, K]; entries outside [0, c_b) ignored); workspace size as
 *   sas_decode_workspace_size.
 * sas_decode_step_paged: as sas_decode_step (kbar [b, hkv, kbar_ld, d] stays a
 *   dense per-sequence cache, rows m < C_b read); each sequence ranks its own
 *   C_b history blocks; workspace size as sas_decode_step_workspace_size.
 * ---------------------------------------------------------------------- */
sas_status sas_decode_paged(const sas_shape* shape, int K, const void* q, const void* kpages,
                            const void* vpages, int num_pages, const int32_t* block_table,
                            int bt_ld, const int32_t* seq_lens, const int32_t* idx,
                            const float* logg, void* o, float* lse, void* workspace,
                            size_t ws_bytes, void* stream);
sas_status sas_decode_step_paged(const sas_shape* shape, int K, const void* q,
                                 const void* kbar, sas_dtype kbar_dtype, int kbar_ld,
                                 const void* kpages, const void* vpages, int num_pages,
                                 const int32_t* block_table, int bt_ld, const int32_t* seq_lens,
                                 int gated, void* o, float* lse, int32_t* idx, float* logg,
                                 float* lse_s, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Selector backward for the stand-in scores of training rows (picx 'Key Idea:
 * Differentiable Continuous Gating': the selector learns through the gates,
 * the hard Top-K carrying no gradient ('Theoretical Foundation'); evolve.pub
 * review FAQ for the pooled block summaries).  With
 * s[t][m] = scale * qbar[t] . kbar[m] on the history m < t:
 *   dqbar[t] = scale * sum_{m<t} ds[t][m] kbar[m]
 *   dkbar[m] = scale * sum_{t>m} ds[t][m] qbar[t]
 * and, when dq / dk are given, the mean pools' adjoints are added to them in
 * place (dq[h][i] += dqbar[t(i)] / (G n_t); dk[j] += dkbar[m(j)] / n_m, n_t the
 * valid tokens of block t), one rounding to shape->dtype per element.
 *   T = ceil(seqlen / block); scale = shape->scale or 1/sqrt(head_dim)
 *   ds           fp32 [b, hkv, T, T] (as sas_attn_bwd returns it; entries
 *                m >= t are not read)
 *   qbar, kbar   fp32 [b, hkv, T, d] (the pooled summaries the scores used)
 *   dqbar, dkbar fp32 [b, hkv, T, d] outputs (caller-allocated)
 *   dq [b, hq, seqlen, d], dk [b, hkv, seqlen, d] (shape->dtype): optional,
 *                accumulated into; 16-byte aligned like qbar..dkbar
 * No workspace.
 * ---------------------------------------------------------------------- */
sas_status sas_selector_bwd(const sas_shape* shape, const float* ds, const float* qbar,
                            const float* kbar, float* dqbar, float* dkbar, void* dq, void* dk,
                            void* stream);

/* ------------------------------------------------------------------------
 * Kernel timing (not part of the method).  When enabled, every kernel the
 * library enqueues is bracketed by a pair of HIP events recorded on the same
 * stream; sas_profiler_read synchronises those events and returns, per kernel
 * name, the launch count and the summed duration.  Process-global state.
 * ---------------------------------------------------------------------- */
typedef struct {
  char name[48];
  long long launches;
  double total_ms;
} sas_kernel_time;

void sas_profiler_enable(int on);
void sas_profiler_reset(void);
/* Writes up to max_entries entries, returns the number of distinct kernels. */
int sas_profiler_read(sas_kernel_time* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* SAS_H */
