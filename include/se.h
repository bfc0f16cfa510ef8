/* se.h -- C ABI of the MI355X (gfx950) sparse-decode library (libse.so).
 *
 * Decode-time sparse attention over a KV cache whose kept positions each
 * method chooses.  The SparseEngine pages describe the contract this follows:
 *   - tokendh.com news f00df0ef4a (SparseEngine explainer), section
 *     "把边界划在'生命周期'上": each method owns a cache manager that creates,
 *     updates and frees its own KV representation at lifecycle hooks, and an
 *     AttentionView turns whatever the method keeps into the one format the
 *     attention computation reads;
 *   - ai-feeds.com digest "SparseEngine：稀疏优先推理引擎", section 方法 /
 *     关键模块: the view exposes the selected positions uniformly so that the
 *     attention kernel does not change per method.
 * Here the cache manager's state is caller-owned device buffers, the update /
 * evict hooks are se_page_meta_update, se_snapkv_score_compact and
 * se_h2o_accumulate_evict, the view producers are se_quest_select and
 * se_omnikv_topk, and the attention backend is se_sparse_decode_attn.
 *
 * Conventions shared by every call
 *   - Every pointer argument except the se_cache descriptor is DEVICE memory
 *     owned by the caller.  The library never allocates or frees memory and
 *     never synchronizes: all work is enqueued on `stream` (a hipStream_t; 0
 *     is the null stream).
 *   - Workspaces (`ws`, se_workspace_bytes() bytes) are caller-owned scratch.
 *     Their leading bytes hold completion counters that let the last block of
 *     a split computation finish it inside the same launch: a workspace must
 *     be zero-filled once before its first use (se_workspace_init) and every
 *     call leaves those counters zero again, so one workspace serves any
 *     sequence of calls, including graph replays.  Calls that share a
 *     workspace must not run concurrently.
 *   - Arguments are validated on the host before anything is enqueued.  On an
 *     error the call returns a negative se_status, nothing is enqueued and the
 *     outputs are untouched.  SE_ERR_HIP reports a failed kernel launch.
 *   - Layouts are row-major and dense.  A "unit" is one (batch row, KV head).
 *     q is [B][Hq][d_k]; K is [B][Hkv][capacity][d_k]; V is
 *     [B][Hkv][capacity][d_v]; query head h reads KV head h / (Hq / Hkv).
 *     For a latent (MLA) cache Hkv = 1 and V is not a separate buffer: the
 *     value of a slot is the first d_v elements of its K row.
 *   - seq_len is int32 [B]: slots [0, seq_len[b]) of every unit of batch row b
 *     are valid.
 *   - Device-side conditions that depend on data (a view longer than the
 *     candidates, an append past capacity) are clamped, not reported.
 *   - NaN or Inf inputs are undefined behaviour (not checked).
 *   - Calls are reentrant; calls that write the same buffers must be ordered
 *     by the caller (same stream or events).
 */
#ifndef SE_H
#define SE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SE_ABI_VERSION 4

typedef enum {
  SE_OK = 0,
  SE_ERR_NULL = -1,        /* a required pointer is NULL */
  SE_ERR_SHAPE = -2,       /* inconsistent or unsupported sizes */
  SE_ERR_DTYPE = -3,       /* unsupported element type */
  SE_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
  SE_ERR_BUDGET = -5,      /* a budget / window / k argument out of range */
  SE_ERR_WORKSPACE = -6,   /* workspace missing or smaller than se_workspace_bytes() */
  SE_ERR_UNSUPPORTED = -7, /* valid but not implemented combination */
  SE_ERR_HIP = -8          /* a HIP launch failed */
} se_status;

typedef enum { SE_F32 = 0, SE_BF16 = 1 } se_dtype;

/* Host-side description of one layer's cache.  Element type `dtype` applies to
 * q, K, V, new rows and page metadata; scores, outputs and logits are float. */
typedef struct {
  int32_t batch;        /* B */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads, Hq / Hkv <= 64 */
  int32_t n_kv_heads;   /* Hkv (1 for a latent cache) */
  int32_t d_k;          /* key width: 64, 128 or 576 */
  int32_t d_v;          /* value width: equals d_k, or 512 for a latent cache */
  int32_t capacity;     /* slots per unit */
  int32_t dtype;        /* se_dtype */
  int32_t latent;       /* nonzero: V is K[..., :d_v] (MLA-style latent cache) */
} se_cache;

/* Operation ids for se_workspace_bytes. */
typedef enum {
  SE_OP_QUEST = 1,      /* a0 = page_size, a1 = top_pages */
  SE_OP_ATTN = 2,       /* a0 = view_cap * granularity (slots per unit), a1 = num_splits (0 = auto) */
  SE_OP_SNAPKV = 3,     /* a0 = prompt_len, a1 = window */
  SE_OP_OMNIKV = 4,     /* a0 = logit_cap, a1 = top_k */
  SE_OP_QUEST_APPEND = 5, /* a0 = page_size (a1 unused) */
  SE_OP_H2O_PREFILL = 6,  /* a0 = prompt_len, a1 = recent_window */
  SE_OP_APPEND_ATTN = 7,  /* a0 = view_cap * granularity (slots per unit), a1 = num_splits (0 = auto) */
  SE_OP_QUEST_STEP = 8,   /* a0 = page_size, a1 = top_pages */
  SE_OP_H2O_STEP = 9      /* a0, a1 unused */
} se_op;

/* Append one decode token's K/V row to every unit (helper of the hooks: the
 * step loop needs no framework compute kernel).
 *   k_new [B][Hkv][d_k], v_new [B][Hkv][d_v] (ignored for a latent cache).
 *   slot: NULL, or int32 [B][Hkv].  Where slot is NULL or slot[b][0] < 0 the
 *   row goes to slot seq_len[b] and seq_len[b] is incremented; otherwise row
 *   (b, h) is written into slot[b][h] and seq_len is unchanged (a slot freed
 *   by eviction).  A write at or past capacity is dropped. */
se_status se_kv_append(const se_cache* c, void* k, void* v, const void* k_new, const void* v_new,
                       const int32_t* slot, int32_t* seq_len, hipStream_t stream);

/* Quest summary index.  tokendh.com explainer, section "历史太长,会撑爆什么":
 * dynamic-sparse methods keep the full history plus a per-page summary index.
 * Here the index is the elementwise min and max of K over each page's valid
 * tokens: kmin, kmax [B][Hkv][ceil(capacity / page_size)][d_k], dtype of K
 * (min and max are exact).  first_page >= 0 rebuilds pages
 * [first_page, ceil(seq_len[b] / page_size)); first_page = -1 rebuilds only
 * the page holding slot seq_len[b] - 1 (the decode-step update).  Pages past
 * seq_len are not written. */
se_status se_page_meta_update(const se_cache* c, const void* k, void* kmin, void* kmax,
                              const int32_t* seq_len, int32_t page_size, int32_t first_page,
                              hipStream_t stream);

/* Append and summary-index update in one launch (the decode-step hook of a
 * Quest cache): writes k_new / v_new exactly as se_kv_append, then rebuilds
 * kmin / kmax of the page holding each written slot over the slots below the
 * new seq_len[b], then updates seq_len.  With slot == NULL this equals
 * se_kv_append followed by se_page_meta_update(first_page = -1).  Arguments
 * as for those two calls. */
se_status se_kv_append_meta(const se_cache* c, void* k, void* v, const void* k_new, const void* v_new,
                            const int32_t* slot, int32_t* seq_len, void* kmin, void* kmax, int32_t page_size,
                            hipStream_t stream);

/* Quest page selection.  tokendh.com explainer, section "历史太长,会撑爆什么"
 * (Quest picks pages dynamically from the query) and Netics blog
 * "SparseEngine 统一接入十五种稀疏注意力", section "SparseEngine 围绕 KV cache
 * 构建了什么" (page-selection methods choose KV pages per query).
 * Score of page p for query head h: sum_d max(q_hd * kmin_pd, q_hd * kmax_pd)
 * (an upper bound of q_h . k over the page), accumulated in fp32; the score of
 * a page for a KV head is the max over the heads of its group.  The view is
 * the top_pages best valid pages (ties to the lower page), ascending:
 *   view_idx int32 [B][Hkv][top_pages] (entries past view_len are -1),
 *   view_len int32 [B][Hkv] = min(top_pages, ceil(seq_len[b] / page_size)),
 *   page_score: NULL or float [B][Hkv][ceil(capacity / page_size)] (-inf for
 *   pages past seq_len).
 * ws: device workspace of se_workspace_bytes(SE_OP_QUEST, c, page_size, top_pages) bytes. */
se_status se_quest_select(const se_cache* c, const void* q, const void* kmin, const void* kmax,
                          const int32_t* seq_len, int32_t page_size, int32_t top_pages,
                          int32_t* view_idx, int32_t* view_len, float* page_score,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* One Quest decode step's cache update and page selection in one launch where
 * the shape allows (bf16, d_k 64 / 128 with G <= 16 or 32, latent 576 with
 * G <= 32, at most 8192 pages): the same results as
 *   se_kv_append_meta(c, k, v, k_new, v_new, NULL, seq_len, kmin, kmax, page_size)
 * followed by
 *   se_quest_select(c, q, kmin, kmax, seq_len, page_size, top_pages, view_idx,
 *                   view_len, page_score, ...)
 * (bit-identical K / V rows, metadata, seq_len, views and scores) as long as
 * kmin / kmax hold the min / max of each page's valid rows, as every call of
 * this library leaves them (the appended page's values are updated with the new
 * row rather than rebuilt from the cache); other shapes run those two calls'
 * kernels.  Arguments as for those calls.
 * ws: se_workspace_bytes(SE_OP_QUEST_APPEND, c, page_size, 0) bytes, 16-byte
 * aligned, zero-filled once before first use (se_workspace_init); the call
 * leaves its counters at zero. */
se_status se_quest_append_select(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                                 const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int32_t page_size,
                                 int32_t top_pages, int32_t* view_idx, int32_t* view_len, float* page_score,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* A whole Quest decode step (tokendh.com explainer, section "历史太长,会撑爆什么":
 * pages chosen per query from the summary index; section "把边界划在'生命周期'上":
 * attention over the chosen view): the same results, bit for bit, as
 *   se_quest_append_select(c, q, k, v, k_new, v_new, seq_len, kmin, kmax,
 *                          page_size, top_pages, view_idx, view_len, page_score, ...)
 * followed by
 *   se_sparse_decode_attn(c, q, k, v, seq_len, view_idx, view_len, top_pages,
 *                         page_size, scale, out, lse, NULL, 0, 0, ...)
 * (K / V rows, metadata, seq_len, out, lse, and the view and scores where
 * requested).  For bf16 GQA caches with d_k 64 / 128, G <= 16, a power-of-two
 * page size, at most 4096 pages and top_pages <= 2048 it runs in two launches:
 * the append and page scoring, then one launch in which every block selects its
 * unit's top pages from the scores and attends over its share of them (the view
 * never goes through memory); other shapes run the two calls' kernels.
 * view_idx int32 [B][Hkv][top_pages] / view_len int32 [B][Hkv]: NULL (both) or
 * the step's view; page_score: NULL or float [B][Hkv][ceil(capacity/page_size)].
 * Other arguments as for the two calls.
 * ws: se_workspace_bytes(SE_OP_QUEST_STEP, c, page_size, top_pages) bytes,
 * 16-byte aligned, zero-filled once before first use (se_workspace_init); the
 * call leaves its counters at zero. */
se_status se_quest_decode_step(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                               const void* v_new, int32_t* seq_len, void* kmin, void* kmax, int32_t page_size,
                               int32_t top_pages, float scale, float* out, float* lse, int32_t* view_idx,
                               int32_t* view_len, float* page_score, void* ws, size_t ws_bytes, hipStream_t stream);

/* FP8 KV rows (tokendh.com explainer, section "历史太长,会撑爆什么": KV
 * quantization keeps the history at lower precision with what is needed to
 * restore it).  Format: a stored row (one token of one KV head) is d_k OCP E4M3
 * codes (uint8 [B][Hkv][capacity][d_k]) and one scale byte s = e + 127 (E8M0,
 * uint8 [B][Hkv][capacity]); its values are code * 2^e, e being the smallest
 * exponent >= -126 with max |x| * 2^-e <= 448 over the row (0 for a zero row),
 * every code the nearest E4M3 value of x * 2^-e, ties to the even code.  Stored
 * values are exact in bf16: kmin / kmax (bf16) hold the min / max of the
 * stored K values and feed se_quest_select unchanged.  FP8 calls take a bf16
 * cache descriptor (q, metadata, source rows) without latent, d_k 64 or 128:
 * SE_ERR_DTYPE / SE_ERR_UNSUPPORTED otherwise.
 *
 * se_kv_quantize_fp8: rows [0, seq_len[b]) of bf16 K / V -> codes and scale
 * bytes; kmin / kmax (both NULL or both set) are rebuilt for every page below
 * seq_len from the stored values (page_size used only then). */
se_status se_kv_quantize_fp8(const se_cache* c, const void* k, const void* v, const int32_t* seq_len, void* k_q,
                             void* v_q, uint8_t* k_scale, uint8_t* v_scale, void* kmin, void* kmax, int32_t page_size,
                             hipStream_t stream);

/* Quantizes the new rows k_new / v_new (bf16 [B][Hkv][d_k]) into slot
 * seq_len[b] (nothing when seq_len[b] == capacity), updates kmin / kmax of the
 * page receiving it with the new stored K values (both NULL or both set; they
 * must hold that page's min / max, as every call here leaves them) and bumps
 * seq_len. */
se_status se_kv_append_fp8(const se_cache* c, void* k_q, void* v_q, uint8_t* k_scale, uint8_t* v_scale,
                           const void* k_new, const void* v_new, int32_t* seq_len, void* kmin, void* kmax,
                           int32_t page_size, hipStream_t stream);

/* se_sparse_decode_attn over FP8 rows: the same view, outputs, splits and
 * workspace (se_workspace_bytes(SE_OP_ATTN, ...)), attention over the stored
 * values; the operands are converted to bf16 in registers (exact) with the
 * row scale folded in.  G <= 16 (SE_ERR_UNSUPPORTED otherwise). */
se_status se_sparse_decode_attn_fp8(const se_cache* c, const void* q, const void* k_q, const void* v_q,
                                    const uint8_t* k_scale, const uint8_t* v_scale, const int32_t* seq_len,
                                    const int32_t* view_idx, const int32_t* view_len, int32_t view_cap,
                                    int32_t granularity, float scale, float* out, float* lse, float* logits,
                                    int32_t logit_cap, int32_t num_splits, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* The Quest decode step over FP8 rows: se_kv_append_fp8, se_quest_select (over
 * the stored values' page metadata) and se_sparse_decode_attn_fp8 in one call,
 * with bit-identical results (codes, scale bytes, kmin / kmax, seq_len, page
 * scores, views, out, lse).  Arguments as in those calls; view_idx / view_len
 * (both or neither) and page_score are optional outputs.  Workspace:
 * se_workspace_bytes(SE_OP_QUEST_STEP, c, page_size, top_pages), 16-byte aligned,
 * zero-filled once before first use; the call leaves its counters at zero.  GQA
 * with d_k 64 or 128, G <= 16 and a power-of-two page size, as the FP8 attention
 * (SE_ERR_UNSUPPORTED otherwise, before anything is written). */
se_status se_quest_decode_step_fp8(const se_cache* c, const void* q, void* k_q, void* v_q, uint8_t* k_scale,
                                   uint8_t* v_scale, const void* k_new, const void* v_new, int32_t* seq_len,
                                   void* kmin, void* kmax, int32_t page_size, int32_t top_pages, float scale,
                                   float* out, float* lse, int32_t* view_idx, int32_t* view_len, float* page_score,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* StreamingLLM view (Netics blog "SparseEngine 统一接入十五种稀疏注意力", section
 * "哪些情况下加速幅度会缩小": named there beside PyramidKV and SnapKV).  Unit
 * (b, h) attends over the first `sink` and the last `recent` positions below
 * the length L = min(seq_len[b] + pending, capacity): view_idx
 * [B][Hkv][view_cap] int32 gets those positions in ascending order (-1 after
 * them), view_len [B][Hkv] their count min(L, sink + recent).  pending = 0
 * gives the view of the cache as it is; pending = 1 the view it will have after
 * the next append, for se_kv_append_decode_attn.  Hand it to the attention with
 * granularity 1.  sink, recent >= 0, sink + recent >= 1 and
 * view_cap >= sink + recent, else SE_ERR_BUDGET; 0 <= pending <= capacity,
 * else SE_ERR_SHAPE. */
se_status se_streaming_view(const se_cache* c, const int32_t* seq_len, int32_t sink, int32_t recent,
                            int32_t* view_idx, int32_t* view_len, int32_t view_cap, int32_t pending,
                            hipStream_t stream);

/* PyramidKV layer budgets (same page and section; host computation, no GPU
 * work).  budgets: HOST int32 [n_layers]; layer l (0 = first) gets
 * min + (max - min) (n - 1 - l) / (n - 1) tokens with max = 2 avg - min, in
 * whole tokens summing to exactly n_layers * avg_budget: every layer takes the
 * floor, then the remaining tokens go one each to the layers with the largest
 * fractional parts (the lower layer first on ties).  Each layer then selects as
 * SnapKV does: se_snapkv_score_compact with its budget.  n_layers >= 1 (else
 * SE_ERR_SHAPE), 0 <= min_budget <= avg_budget (else SE_ERR_BUDGET). */
se_status se_pyramid_budgets(int32_t n_layers, int32_t avg_budget, int32_t min_budget, int32_t* budgets);

/* Chain Cache (tokendh.com explainer, section "聊天记录也能'续命':Chain Cache";
 * Netics blog, section "SparseEngine 围绕 KV cache 构建了什么": the
 * ChainCacheIndex ties a session to its retained per-layer KV, method metadata
 * and logical token prefix).  The logical prefix (tokens said) is kept apart
 * from the physical rows still stored; a new turn that continues a stored
 * prefix reuses that session's rows and only its new tokens are processed.
 *
 * se_chain_match (host computation, no GPU work): tokens / prefixes are HOST
 * int32 arrays; prefixes[s] (prefix_lens[s] tokens) is session s's logical
 * prefix.  *session = the session whose prefix `tokens` continues (the prefix
 * is a prefix of tokens), the longest one, the lower index on equal lengths;
 * -1 (and *matched_len 0) when none does. */
se_status se_chain_match(const int32_t* tokens, int32_t n_tokens, const int32_t* const* prefixes,
                         const int32_t* prefix_lens, int32_t n_prefixes, int32_t* session, int32_t* matched_len);

/* Position map after a compaction.  map_out int32 [B][Hkv][c_out->capacity]:
 * map_out[u][i] = map_in[u][kept[u][i]] for i < kept_len[b] (map_in NULL: the
 * identity, i.e. kept[u][i] itself), -1 for the remaining entries and for kept
 * entries outside [0, cap_in).  map_in int32 [B][Hkv][cap_in] or NULL; kept
 * int32 [B][Hkv][kept_stride] physical rows, ascending (e.g. SnapKV's kept
 * positions); kept_len int32 [B] (e.g. SnapKV's out_seq_len). */
se_status se_chain_remap(const se_cache* c_out, const int32_t* map_in, int32_t cap_in, const int32_t* kept,
                         int32_t kept_stride, const int32_t* kept_len, int32_t* map_out, hipStream_t stream);

/* Positions of n_new rows about to be appended after the seq_len[b] retained
 * rows: pos_map[u][seq_len[b] + j] = logical_len[b] + j (entries past the
 * capacity skipped).  Call before the rows are appended.  pos_map int32
 * [B][Hkv][capacity]; seq_len, logical_len int32 [B]. */
se_status se_chain_append_positions(const se_cache* c, int32_t* pos_map, const int32_t* seq_len,
                                    const int32_t* logical_len, int32_t n_new, hipStream_t stream);

/* Split-K flash decode over an AttentionView (tokendh.com explainer, section
 * "把边界划在'生命周期'上"; ai-feeds digest, section 方法 / 关键模块).
 *   view_idx: NULL = every slot below seq_len[b]; else int32 [B][Hkv][view_cap],
 *   entry e of unit u covering slots [view_idx*g, view_idx*g + g) with
 *   g = granularity (page size for page views, 1 for token views); only the
 *   first view_len[b][h] entries are read and slots >= seq_len[b] are skipped.
 *   out float [B][Hq][d_v] = softmax(scale * q . k) . v over the view (0 for an
 *   empty view); lse: NULL or float [B][Hq] natural-log sum of exp(scale q.k)
 *   (-inf for an empty view); logits: NULL or float [B][Hq][logit_cap], the
 *   scaled logit of view slot i (entry * g + offset) at index i, -inf where the
 *   slot holds no valid token (indices >= view_cap * g are not written);
 *   (n_q_heads / n_kv_heads) * logit_cap must not exceed 2^31 - 1 (SE_ERR_SHAPE).
 *   num_splits: 0 chooses the split-K factor; otherwise the number of chunks
 *   (1..256) each unit's view is cut into (results agree to rounding for any
 *   value).
 *   q, k, v and out must be 16-byte aligned (SE_ERR_ALIGN otherwise).
 *   ws: se_workspace_bytes(SE_OP_ATTN, c, view_cap * g, num_splits) bytes. */
se_status se_sparse_decode_attn(const se_cache* c, const void* q, const void* k, const void* v,
                                const int32_t* seq_len, const int32_t* view_idx,
                                const int32_t* view_len, int32_t view_cap, int32_t granularity,
                                float scale, float* out, float* lse, float* logits,
                                int32_t logit_cap, int32_t num_splits,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* se_sparse_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace, and the same results,
 * bit for bit.  Its split partials and ticket counters live in a static device
 * array of SE_NOALLOC_SCRATCH_BYTES bytes that each GPU the library runs on
 * holds until the process ends; the call allocates nothing.  Calls whose
 * workspace (se_workspace_bytes(SE_OP_ATTN, c, view_cap * granularity,
 * num_splits)) would exceed that size return SE_ERR_WORKSPACE and enqueue
 * nothing.  Every call on one GPU shares that GPU's array: calls that may run
 * concurrently on one GPU (different streams without ordering between them)
 * race and give undefined results.  Each call first clears the array's
 * counters with a fill kernel on `stream` (no memset node).  SE_ERR_HIP if the
 * array's device address cannot be obtained. */
#define SE_NOALLOC_SCRATCH_BYTES (32u << 20)
se_status se_sparse_decode_attn_noalloc(const se_cache* c, const void* q, const void* k, const void* v,
                                        const int32_t* seq_len, const int32_t* view_idx,
                                        const int32_t* view_len, int32_t view_cap, int32_t granularity,
                                        float scale, float* out, float* lse, float* logits,
                                        int32_t logit_cap, int32_t num_splits, hipStream_t stream);

/* A decode step's append and attention in one launch (the hooks' append-then-
 * attend, as for a SnapKV-compacted or H2O cache): the same results, bit for
 * bit, as
 *   se_kv_append(c, k, v, k_new, v_new, slot, seq_len)
 * followed by
 *   se_sparse_decode_attn(c, q, k, v, seq_len, view_idx, view_len, view_cap,
 *                         granularity, scale, out, lse, logits, logit_cap,
 *                         num_splits, ...).
 * The attention reads the new rows from k_new / v_new where the view meets the
 * slot they go to, one block per unit writes them into k / v, and seq_len is
 * updated once every block of its batch row has read the old value (bf16 GQA
 * caches the MFMA attention serves; other shapes run the two calls' kernels).
 * Arguments as for those calls; k_new / v_new must be 16-byte aligned.
 * ws: se_workspace_bytes(SE_OP_APPEND_ATTN, c, view_cap * granularity,
 * num_splits) bytes, zero-filled once before first use (se_workspace_init);
 * the call leaves its counters at zero. */
se_status se_kv_append_decode_attn(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                                   const void* v_new, const int32_t* slot, int32_t* seq_len,
                                   const int32_t* view_idx, const int32_t* view_len, int32_t view_cap,
                                   int32_t granularity, float scale, float* out, float* lse, float* logits,
                                   int32_t logit_cap, int32_t num_splits, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* SnapKV prefill-end eviction.  tokendh.com explainer, section
 * "把边界划在'生命周期'上": the method looks at how the last few prompt tokens
 * attend over the history, keeps the important part and physically deletes
 * the rest.  Every batch row has prompt_len valid slots.
 *   q_obs [B][Hq][window][d_k]: queries of prompt positions L - window + i.
 *   vote[j] (j < L - window) = sum over the group's heads and the window rows
 *   of the causal softmax weight the row gives key j (each row's softmax runs
 *   over keys 0 .. its own position); pooled = max-pool(vote, pool_kernel,
 *   stride 1, out-of-range ignored; pool_kernel odd, 1..129); kept = the
 *   budget - window best pooled
 *   positions (ties to the lower position) plus the window, ascending; with
 *   budget >= prompt_len every position is kept.
 *   kept_pos int32 [B][Hkv][budget] (-1 past min(budget, L)); k_out / v_out
 *   [B][Hkv][out->capacity][d] receive the kept rows in that order (bit copies);
 *   votes: NULL or float [B][Hkv][L - window]; out_seq_len: NULL or int32 [B]
 *   set to min(budget, L).  `out` describes k_out / v_out (same heads, widths,
 *   dtype; capacity >= min(budget, L)).
 *   ws: se_workspace_bytes(SE_OP_SNAPKV, c, prompt_len, window) bytes. */
se_status se_snapkv_score_compact(const se_cache* c, const void* q_obs, const void* k, const void* v,
                                  int32_t prompt_len, int32_t window, int32_t pool_kernel,
                                  int32_t budget, float scale, const se_cache* out, void* k_out,
                                  void* v_out, int32_t* kept_pos, float* votes,
                                  int32_t* out_seq_len, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* H2O accumulate-then-evict step.  tokendh.com explainer, sections
 * "历史太长,会撑爆什么" (a continuously accumulated score table plus physical
 * deletion) and "把边界划在'生命周期'上" (scores updated every decode step,
 * then the victim chosen).
 *   logits float [B][Hq][logit_cap], lse float [B][Hq]: from
 *   se_sparse_decode_attn over every slot below seq_len[b] (identity view).
 *   slot_pos int32 [B][Hkv][capacity] (token position held by a slot, -1 =
 *   free); acc float [B][Hkv][capacity] (accumulated score).
 *   evict_slot int32 [B][Hkv], in/out: on entry the slot that received the
 *   token at cur_pos (-1: it was appended at seq_len[b] - 1); on exit the
 *   evicted slot or -1.
 *   Per unit: the new slot gets position cur_pos and score 0; every occupied
 *   slot below seq_len[b] adds the sum over the group's heads of
 *   exp(logit - lse); if more than heavy + recent slots are occupied, the
 *   lowest-scoring slot with position <= cur_pos - recent (ties to the lower
 *   position) is freed (position -1, score 0). */
se_status se_h2o_accumulate_evict(const se_cache* c, const float* logits, const float* lse,
                                  int32_t logit_cap, const int32_t* seq_len, int32_t* slot_pos,
                                  float* acc, int32_t cur_pos, int32_t heavy_budget,
                                  int32_t recent_window, int32_t* evict_slot, hipStream_t stream);

/* A whole H2O decode step (tokendh.com explainer, section "把边界划在'生命周期'上":
 * the scores are updated at every decode step, then the victim is chosen): the
 * same results, bit for bit, as
 *   se_kv_append(c, k, v, k_new, v_new, slot_in, seq_len)
 *   se_sparse_decode_attn(c, q, k, v, seq_len, NULL, NULL, 0, 1, scale, out, lse,
 *                         logits, capacity, 1, ...)
 *   se_h2o_accumulate_evict(c, logits, lse, capacity, seq_len, slot_pos, acc,
 *                           cur_pos, heavy_budget, recent_window, evict)
 * where evict holds slot_in on entry (-1 everywhere when slot_in is NULL) and is
 * copied to evict_out on exit: slot_in int32 [B][Hkv] (or NULL) is the slot each
 * unit's new token goes to (the slot the previous step evicted), evict_out int32
 * [B][Hkv] receives the slot this step evicts (or -1).  slot_in and evict_out
 * must be different arrays (SE_ERR_SHAPE): every block of a batch row reads the
 * row's first slot_in entry.  Steps alternate the two arrays.  For bf16 GQA
 * caches with d_k 64 / 128, G <= 16, capacity <= 2048 and G * capacity <= 12288
 * it is one launch, in which the logits never leave the chip; other shapes run
 * the three calls' kernels.  lse: NULL or float [B][Hq].
 * ws: se_workspace_bytes(SE_OP_H2O_STEP, c, 0, 0) bytes, 16-byte aligned,
 * zero-filled once before first use (se_workspace_init); the call leaves its
 * counters at zero. */
se_status se_h2o_decode_step(const se_cache* c, const void* q, void* k, void* v, const void* k_new,
                             const void* v_new, const int32_t* slot_in, int32_t* seq_len, int32_t* slot_pos,
                             float* acc, int32_t cur_pos, int32_t heavy_budget, int32_t recent_window, float scale,
                             float* out, float* lse, int32_t* evict_out, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* H2O state at the end of a prefill (tokendh.com explainer, sections
 * "历史太长,会撑爆什么" and "把边界划在'生命周期'上": H2O's table accumulates the
 * attention every token receives).  scores[u][j] = sum over the group's heads
 * and the prompt queries i >= j of softmax_i(scale q_i . k)[j] (causal), from
 * q_prompt bf16 [B][Hq][prompt_len][d_k] and the prompt's rows k / v (cache c,
 * rows below prompt_len).  The kept slots are the heavy_budget best scores
 * below prompt_len - recent_window (ties to the lower position) and the recent
 * window, ascending (all positions when they fit): their rows are copied to
 * k_slots / v_slots (cache `slots`, capacity >= heavy + recent + 1), slot_pos
 * int32 [B][Hkv][slots.capacity] gets their positions (-1 after them) and acc
 * float [B][Hkv][slots.capacity] their scores (0 after them) — the state
 * se_h2o_accumulate_evict continues from.  scores: NULL or float
 * [B][Hkv][prompt_len].  bf16, d_k 64 / 128, G <= 16, prompt_len * G <= 2^30 and
 * B * Hkv * max(ceil(prompt_len * G / 1024), ceil(prompt_len / 512)) < 2^31 (SE_ERR_SHAPE
 * beyond, before any launch).
 * ws: se_workspace_bytes(SE_OP_H2O_PREFILL, c, prompt_len, recent_window) bytes,
 * zero-filled once before first use (its selection counters return to zero). */
se_status se_h2o_prefill_init(const se_cache* c, const void* q_prompt, const void* k, const void* v,
                              int32_t prompt_len, int32_t heavy_budget, int32_t recent_window, float scale,
                              const se_cache* slots, void* k_slots, void* v_slots, int32_t* slot_pos, float* acc,
                              float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* OmniKV filter-layer top-k.  tokendh.com explainer, section
 * "把边界划在'生命周期'上": some layers judge which history matters and later
 * layers reuse that judgement.
 *   score[j] = sum over the group's heads of exp(logit_hj - lse_h) for
 *   j < seq_len[b] (logits / lse from a full-view se_sparse_decode_attn);
 *   view_idx int32 [B][Hkv][top_k]: the top_k best slots (ties to the lower
 *   slot), ascending, -1 padded; view_len int32 [B][Hkv] = min(top_k, seq_len[b]);
 *   scores: NULL or float [B][Hkv][logit_cap] (entries past seq_len[b] not written).
 *   ws: se_workspace_bytes(SE_OP_OMNIKV, c, logit_cap, top_k) bytes (unused,
 *   may be NULL, when scores is given: the scores are staged there). */
se_status se_omnikv_topk(const se_cache* c, const float* logits, const float* lse, int32_t logit_cap,
                         const int32_t* seq_len, int32_t top_k, int32_t* view_idx,
                         int32_t* view_len, float* scores, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* Workspace bytes an operation needs for cache `c` (0 if none). */
size_t se_workspace_bytes(int32_t op, const se_cache* c, int32_t a0, int32_t a1);

/* Zero-fill `bytes` bytes of a workspace on `stream` with a fill kernel (no
 * memset node, so the call may be captured into a graph).  ws must be
 * 16-byte aligned unless bytes == 0. */
se_status se_workspace_init(void* ws, size_t bytes, hipStream_t stream);
const char* se_status_string(int32_t status);
int32_t se_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SE_H */
