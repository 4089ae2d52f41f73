/*
 * sparsekv.h -- C ABI of libsparsekv: single-token decode attention over a
 * paged bf16 KV cache that reads only a selected subset of it, for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources of the operations (web pages, cited by title and section):
 *  [ODA]  "On-Demand Attention: Language Models Know When to Recall"
 *         (arxiv-wiki summary). "Approach": local-first decoding with s = 4
 *         initial tokens and a recent window w = 2048, a recall head that
 *         scores the step from (h_{t-1}, E(x_t), h^L_t), a full recompute when
 *         q_t > theta, and commit of the selected pass's current-position KV
 *         into the preserved history. "Main results": the window includes the
 *         current token. "Developer perspective": a Local view and a paged
 *         full view of one preserved KV cache; the FP32 recall head and the
 *         conditional Full pass stay in one GPU execution flow.
 *  [DA]   "[Paper review] Language Models Can Control Their Own Attention"
 *         (blog review of Declarative Attention), section 3 "Method & Key
 *         Results": the mask is applied at KV-block granularity and the block
 *         table is rewritten so the attention kernel sees only kept blocks;
 *         section 1 "Key Terms": the global / focus / local modes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is DEVICE memory owned by the caller (for example
 *    torch tensors), unless a comment says otherwise. The library allocates
 *    nothing, copies nothing to the host and keeps no state between calls.
 *  - Every call is asynchronous on the caller's stream `stream` and never
 *    synchronizes with the host (the only exception is sk_workspace_error,
 *    which says so).
 *  - Return value: SK_OK (0) when the work was enqueued; a negative SK_E_*
 *    code when an argument is invalid (nothing is enqueued then); or
 *    -(1000 + hipError_t) when a kernel launch failed.
 *  - Errors that only the device can see (a block id outside the pool, a
 *    sequence length outside [1, max_blocks*16], an empty key set) set bits
 *    of the error word in the workspace header (SK_DEVERR_*). A request with
 *    an invalid length or an empty key set gets an all-zero output row; a
 *    request that hits an out-of-range block id has an unspecified output.
 *  - A workspace (see sk_workspace_bytes) must be cleared once with
 *    sk_workspace_init before first use; the kernels leave it ready for the
 *    next call. Calls that share one workspace must be ordered (for example
 *    issued on one stream); concurrent calls on one workspace race.
 *  - All entry points are reentrant and may be captured in a HIP graph: none
 *    of them records a memset or a host callback.
 *
 * Paged KV layout (sk_paged_kv)
 * -----------------------------
 *  The cache is a pool of physical blocks of 16 token positions. For every
 *  (physical block p, KV head g) there is one 4096-byte K tile and one
 *  4096-byte V tile, at byte offset (p * num_kv_heads + g) * 4096 of
 *  k_pool / v_pool. Inside a tile the 16 x 128 bf16 values are stored in the
 *  order the gfx950 matrix cores consume them:
 *    K tile: element (token t, dim d) at byte (d/8)*256 + t*16 + (d%8)*2
 *    V tile: element (token t, dim d) at byte (d/32)*1024 + (t/4)*256
 *            + (d%16)*16 + ((d%32)/16)*8 + (t%4)*2
 *  Callers do not need to know this order: sk_kv_write / sk_kv_read move
 *  tokens between row-major [count][num_kv_heads][128] bf16 arrays and the
 *  pool, and the decode calls commit the current token themselves.
 *  block_tables[b * max_blocks + i] is the physical block holding logical
 *  positions 16i .. 16i+15 of request b. seq_lens[b] = n, the number of
 *  visible positions INCLUDING the current token, which lives at position
 *  n-1 ([ODA] "Main results": the window counts the current token).
 */
#ifndef SPARSEKV_H
#define SPARSEKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define SK_OK 0
#define SK_E_NULL (-1)        /* a required pointer is NULL */
#define SK_E_SHAPE (-2)       /* unsupported shape: head_dim != 128, block_size != 16, Hq/Hkv > 16, ... */
#define SK_E_HEADS (-3)       /* num_q_heads is not a multiple of num_kv_heads */
#define SK_E_RANGE (-4)       /* a size or index argument is out of range */
#define SK_E_WORKSPACE (-5)   /* workspace too small for this call */
#define SK_E_LAUNCH_BASE (-1000) /* -(1000 + hipError_t): a launch failed */

/* ---- device error bits (workspace header word) ---- */
#define SK_DEVERR_BLOCK_ID 1  /* a block id outside [0, num_phys_blocks) */
#define SK_DEVERR_SEQ_LEN 2   /* seq_lens[b] outside [1, max_blocks*16] */
#define SK_DEVERR_EMPTY 4     /* a request's key set is empty */

/* ---- per-request view selectors (ragged batches) ---- */
#define SK_MODE_LOCAL 0
#define SK_MODE_FULL 1
#define SK_MODE_BLOCKS 2

/* ---- Declarative-Attention declared modes ([DA] section 1) ---- */
#define SK_DA_GLOBAL 0
#define SK_DA_FOCUS 1
#define SK_DA_LOCAL 2

typedef struct sk_paged_kv {
  void* k_pool;                 /* bf16 tiles, [num_phys_blocks][num_kv_heads][4096 B] */
  void* v_pool;                 /* bf16 tiles, same shape */
  const int32_t* block_tables;  /* [batch][max_blocks] logical block -> physical block */
  const int32_t* seq_lens;      /* [batch] visible positions n, current token included */
  int32_t batch;
  int32_t num_q_heads;          /* Hq; query head h reads KV head h / (Hq/Hkv) */
  int32_t num_kv_heads;         /* Hkv; Hq/Hkv must be in 1..16 */
  int32_t head_dim;             /* must be 128 */
  int32_t block_size;           /* must be 16 */
  int32_t max_blocks;           /* columns of block_tables */
  int64_t num_phys_blocks;      /* blocks in each pool */
} sk_paged_kv;

/* Bytes of workspace needed by every decode / recall call on up to `batch`
 * requests with up to `num_q_heads` query heads: a header (error word,
 * tickets) plus split partials. Depends only on its arguments. */
size_t sk_workspace_bytes(int32_t batch, int32_t num_q_heads);

/* Clears a workspace (error word, tickets) with a fill kernel on `stream`. */
int sk_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Reads the workspace error word: enqueues a copy on `stream`, WAITS for the
 * stream, and stores the SK_DEVERR_* bits in *err_out (host pointer).
 * This is the one call that synchronizes with the host. */
int sk_workspace_error(const void* ws, int32_t* err_out, hipStream_t stream);

/* Human-readable text of a status code (static storage, never NULL). */
const char* sk_status_str(int status);

/* Writes `count` tokens of request `request` at logical positions
 * pos0 .. pos0+count-1 into the pool. k, v: bf16 [count][num_kv_heads][128],
 * row-major. Used to fill a history (prefill) or to restore a cache.
 * Host-checked: 0 <= request < batch, 0 <= pos0, pos0 + count <= max_blocks*16;
 * count == 0 enqueues nothing (k and v may then be NULL).
 * Block ids outside the pool are skipped and reported in the error word of
 * `ws` when ws is not NULL. seq_lens is not read. */
int sk_kv_write(sk_paged_kv kv, int32_t request, int32_t pos0, int32_t count,
                const void* k, const void* v, void* ws, hipStream_t stream);

/* Inverse of sk_kv_write: copies positions pos0 .. pos0+count-1 of request
 * `request` out of the pool into row-major k_out, v_out
 * ([count][num_kv_heads][128] bf16). Positions in out-of-range blocks read
 * as zero and set the error bit when ws is not NULL. */
int sk_kv_read(sk_paged_kv kv, int32_t request, int32_t pos0, int32_t count,
               void* k_out, void* v_out, void* ws, hipStream_t stream);

/* Commit ([ODA] "Approach"): writes the current token of every request
 * (k_new, v_new: bf16 [batch][num_kv_heads][128]) into position
 * seq_lens[b]-1. When `sel` is not NULL, only requests with
 * sel[b] == sel_value are written. The decode calls below can do the same
 * commit themselves (their k_new / v_new arguments); this entry point is the
 * stand-alone form. */
int sk_kv_append(sk_paged_kv kv, const void* k_new, const void* v_new,
                 const int32_t* sel, int32_t sel_value, void* ws, hipStream_t stream);

/* Local-first view ([ODA] "Approach", "Main results"): for every request b
 * with n = seq_lens[b], attends the key positions
 *   [0, min(sinks, n))  union  [max(min(sinks, n), n - window), n)
 * with softmax scale `scale` (typically 1/sqrt(128)).
 *  q      : fp32 [batch][num_q_heads][128]
 *  out    : fp32 [batch][num_q_heads][128]; rows of requests that do not run
 *           are left untouched, so a later call may fill them
 *  k_new, v_new : NULL, or bf16 [batch][num_kv_heads][128] -- the current
 *           token's key/value, committed to position n-1 before it is
 *           attended (fused commit)
 *  sel    : NULL (every request runs) or int32 [batch]; request b runs iff
 *           sel[b] == sel_value
 *  ws     : workspace of at least sk_workspace_bytes(batch, num_q_heads)
 * Host-checked: sinks >= 0, window >= 1. */
int oda_decode_local(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                     int32_t sinks, int32_t window, float scale,
                     const int32_t* sel, int32_t sel_value,
                     float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* The Local view's tiles for one step ([ODA] "Approach": every layer of a step
 * attends the same sinks and window of its own cache, so the physical blocks of
 * that view are the same in every layer that shares the block tables and
 * lengths). oda_local_tiles writes, per request b, a row of
 * oda_local_tiles_bytes(...) / (4 * batch) int32 words: words 0-2 the length
 * seq_lens[b], the sinks and the window it was built for, word 3 + i the
 * physical block of tile i of request b's Local view (the sinks' blocks, then
 * the window's, in ascending order); words past the view's tiles are left as
 * they were. A request with an invalid length gets words 0-2 only.
 *  tab : int32 device memory of at least
 *        oda_local_tiles_bytes(batch, sinks, window, max_blocks) bytes
 *        (0 for an invalid argument)
 * oda_decode_local_tiles is oda_decode_local (same arguments, outputs, commits
 * and error bits, bit for bit) with such a table built on the same lengths
 * and block tables: a single-request launch requests its first tiles' blocks
 * from the table together with the length instead of after it. When words 0-2
 * differ from the request's current length and the call's sinks and window, or
 * the launch's split plan is not the one of the largest Local tile count, it
 * reads the block table as oda_decode_local does (a table from another step
 * gives the same results, only without the saving). Build the table again after
 * a block table changes.
 * Host-checked: tab non-NULL, sinks >= 0, window >= 1, tab_bytes large enough. */
size_t oda_local_tiles_bytes(int32_t batch, int32_t sinks, int32_t window, int32_t max_blocks);
int oda_local_tiles(sk_paged_kv kv, int32_t sinks, int32_t window, int32_t* tab, size_t tab_bytes,
                    hipStream_t stream);
int oda_decode_local_tiles(const float* q, sk_paged_kv kv, const int32_t* tab, size_t tab_bytes,
                           const void* k_new, const void* v_new, int32_t sinks, int32_t window,
                           float scale, const int32_t* sel, int32_t sel_value,
                           float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Full view ([ODA] "Approach": recompute the step over the whole preserved
 * history): attends positions [0, n). Arguments as oda_decode_local. For the
 * on-device gate, pass sel = the gate array written by oda_recall_score and
 * sel_value = 1: requests whose gate is 0 do no work, write nothing and
 * commit nothing, so a launch on a non-recall step costs only its dispatch.
 * Committing k_new here overwrites the Local pass's candidate at n-1, so the
 * slot ends up holding the selected pass's KV. */
int oda_decode_full(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                    float scale, const int32_t* sel, int32_t sel_value,
                    float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Local and Full views of one decoder layer straight from its raw q/k/v
 * projection ([ODA] "Approach": both passes run the layer's attention; the layer
 * is the Qwen3-family layer the pages name as backbone): the per-head finish that
 * sk_qkv_rope does in a launch of its own is applied while the decode kernel
 * stages its operands.
 *  qkv  : fp32 [batch][Hq + 2 Hkv][128], the projection W_qkv x per request
 *         (q heads, then k heads, then v heads), e.g. sk_gemv's output
 *  g_q, g_k : bf16 [128] RMSNorm gains of the q and k heads;  eps >= 0
 *  rope_base > 0 : each q and k head, RMS-normalised over its 128 values with
 *         its gains, is rotated at pos = n - 1 (rotate-half pairs (i, i + 64),
 *         angle pos * rope_base^(-i/64), computed and reduced in fp64)
 * The finished k and the raw v, rounded to bf16 (nearest even), are the current
 * token's candidate: committed to position n - 1 as k_new / v_new are. Other
 * arguments, the selector and errors as oda_decode_local / oda_decode_full. */
int oda_decode_local_qkv(const float* qkv, const uint16_t* g_q, const uint16_t* g_k, float eps,
                         float rope_base, sk_paged_kv kv, int32_t sinks, int32_t window, float scale,
                         const int32_t* sel, int32_t sel_value,
                         float* out, void* ws, size_t ws_bytes, hipStream_t stream);
int oda_decode_full_qkv(const float* qkv, const uint16_t* g_q, const uint16_t* g_k, float eps,
                        float rope_base, sk_paged_kv kv, float scale,
                        const int32_t* sel, int32_t sel_value,
                        float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Allocation-free form of oda_decode_full, for callers that cannot allocate or
 * pass a workspace (code under graph capture that may not call hipMalloc, tight
 * serving loops, harnesses that forbid allocation). Same computation, kernels and
 * results as oda_decode_full; the split tickets and partials live in a device array
 * inside the library (16 MiB per GPU, held until the process ends), so no `ws`.
 *  dev_err : NULL, or a caller-owned device int32 that receives the SK_DEVERR_*
 *            bits (OR-ed in; the caller clears it)
 * Limit: sk_workspace_bytes(batch, num_q_heads) <= 16 MiB (batch * num_q_heads up to
 * about 15700), else SK_E_WORKSPACE and nothing is enqueued. The first call on a GPU
 * looks up the array's address and enqueues its clearing on `stream`; it calls no
 * hipMalloc / hipFree. Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race; calls issued in order on
 * one stream do not. Other arguments and errors as oda_decode_full. */
int oda_decode_full_noalloc(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                            float scale, const int32_t* sel, int32_t sel_value,
                            float* out, int32_t* dev_err, hipStream_t stream);

/* Recall head and gate ([ODA] "Approach" and "Developer perspective"), FP32:
 *   a = W1 x_b + b1;  u = GELU(a) (exact erf form);  q_b = <w2, u> + b2;
 *   gate_b = (q_b > theta) ? 1 : 0          (strict comparison)
 *  x  : fp32 [batch][in_dim], the concatenation [h_{t-1}, E(x_t), h^L_t]
 *  W1 : fp32 [hidden][in_dim] row-major;  b1, w2 : fp32 [hidden];  b2 : fp32 [1]
 *  q_out : fp32 [batch];  gate_out : int32 [batch]
 * Host-checked: 1 <= batch <= 64, in_dim % 4 == 0, 1 <= in_dim <= 65536,
 * 1 <= hidden, ceil(hidden / 4) * batch <= 16384. The reduction order is fixed,
 * so results are deterministic. */
int oda_recall_score(const float* x, const float* W1, const float* b1, const float* w2,
                     const float* b2, int32_t batch, int32_t in_dim, int32_t hidden,
                     float theta, float* q_out, int32_t* gate_out,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Gate from given scores (no recall-head GEMV): for every request,
 *   out[b] = (scores[b] > theta) ? 1 : (fallback ? fallback[b] : 0).
 * With fallback = NULL this is the recall gate; with a per-request fallback
 * view (SK_MODE_LOCAL or SK_MODE_BLOCKS) it is the per-request view of a
 * ragged batch (SK_MODE_FULL == 1 when the score passes). */
int oda_gate_scores(const float* scores, int32_t batch, float theta,
                    const int32_t* fallback, int32_t* out, hipStream_t stream);

/* Declared mode -> logical keep mask ([DA] sections 1 and 3), one bit per
 * logical block (bit i of word i/32, little-endian), words per request =
 * (max_blocks + 31) / 32. decl: int32 [batch][4] =
 * {mode, focus_begin_block, focus_end_block, output_begin_block}.
 *  SK_DA_GLOBAL: every block holding a visible position (blocks < ceil(n/16));
 *  SK_DA_FOCUS : blocks in [focus_begin, focus_end) plus blocks >= output_begin,
 *                both cut at ceil(n/16);
 *  SK_DA_LOCAL : blocks overlapping the last `local_tokens` positions.
 * Bits of blocks >= ceil(n/16) are written as 0. */
int da_keep_mask(const int32_t* decl, sk_paged_kv kv, int32_t local_tokens,
                 uint32_t* keep_mask, hipStream_t stream);

/* Token ids of the mode tags ([DA] review page, section 1 "Key Terms"; chatpaper
 * abstract: the model writes <global>, <focus> and <local> into its chain of
 * thought, and a focus names one context segment, a "Magic Chunk"). Token
 * segment_base + k names segment k. The ids are the caller's tokenizer's. */
typedef struct sk_da_tags {
  int32_t global_tag;
  int32_t focus_tag;
  int32_t local_tag;
  int32_t segment_base;
} sk_da_tags;

/* Declaration parsing ([DA] section 3 and the chatpaper abstract: the engine
 * reads the declarations from the generated text like tool calls and derives
 * the attention mask). For every request b, this step's input token tokens[b]
 * advances a parser whose state persists in `state` (int32 [batch][4] =
 * {mode, focus_begin_block, focus_end_block, focus_pending}; initialise to
 * {SK_DA_GLOBAL, 0, 0, 0}):
 *   global_tag -> mode SK_DA_GLOBAL;   local_tag -> mode SK_DA_LOCAL
 *   (either clears a pending focus);   focus_tag -> focus pending (mode kept);
 *   any other token while a focus is pending clears it, and if it names
 *   segment k < num_segments the mode becomes SK_DA_FOCUS on that segment:
 *     [begin, end) = segments[b][k] (int32 [batch][num_segments][2], context
 *     positions) -> blocks [begin/16, ceil(end/16)), empty when end <= begin;
 *   any other token changes nothing.
 * The new mode applies to this very step (its input token is already parsed).
 * Then decl[b] = {mode, focus_begin_block, focus_end_block, output_begin[b]}
 * (the row da_keep_mask reads; output_begin: int32 [batch], the first logical
 * block of the model's own output) and keep_mask row b is written exactly as
 * da_keep_mask writes it; keep_mask may be NULL when only the declaration is
 * wanted (da_decode_declared reads it directly). One workgroup per request;
 * segments may be NULL when num_segments == 0. Host-checked: pointers,
 * num_segments >= 0, local_tokens >= 0, the paged-KV description. */
int da_declare(const int32_t* tokens, int32_t* state, const int32_t* segments,
               int32_t num_segments, const int32_t* output_begin, sk_da_tags tags,
               sk_paged_kv kv, int32_t local_tokens, int32_t* decl,
               uint32_t* keep_mask, hipStream_t stream);

/* ---- Dense layers of the weight-bearing decode step ----
 * A recall reruns the whole model for the current token ([ODA] "Approach": the
 * step is recomputed from the same prior state with Full attention), and the
 * recall head reads the final hidden state of the Local pass, so a decode step
 * carries the decoder's dense layers too. These entry points run one token
 * (batch 1) through a Qwen3-family decoder layer (the pages name the family but
 * give no layer structure; this is its published layer). Weights are bf16,
 * row-major [rows][cols]; activations fp32. Every call takes the decode calls'
 * selector: with sel != NULL and sel[0] != sel_value the launch does nothing
 * (the gated recall pass). Host-checked: pointers and sizes (SK_E_NULL,
 * SK_E_SHAPE, SK_E_RANGE); nothing is allocated. */

#define SK_PRO_NONE 0    /* x used as given, cols floats */
#define SK_PRO_RMSNORM 1 /* x <- x / sqrt(mean(x^2) + eps) * gamma, cols floats */
#define SK_EPI_STORE 0   /* y[r] = a_r (+ residual[r]) */
#define SK_EPI_SWIGLU 1  /* y[r] = SiLU(a_r) * a_{rows + r}: W holds 2*rows rows */

/* a_r = sum_c W[r][c] x'[c], x' from x by the prologue, fp32 accumulation in a
 * fixed order (deterministic); stored per the epilogue (SK_EPI_SWIGLU: gate rows
 * 0..rows-1 then up rows rows..2rows-1 of W, no residual). W: bf16 [rows or
 * 2*rows][cols]; gamma: bf16 [cols] (SK_PRO_RMSNORM only). cols % 512 == 0 with
 * cols / 512 in {1, 2, 3, 4, 6, 8, 12, 16}, 1 <= rows; y may be residual (in
 * place) but not x. */
int sk_gemv(const uint16_t* W, int32_t rows, int32_t cols, const float* x, int32_t prologue,
            const uint16_t* gamma, float eps, const float* residual, int32_t epilogue, float* y,
            const int32_t* sel, int32_t sel_value, hipStream_t stream);

/* Attention inputs of one token: x = h / sqrt(mean(h^2) + eps) * g_attn;
 * [q; k; v] = W_qkv x with W_qkv bf16 [(Hq + 2 Hkv) * 128][hidden] (written to
 * scratch, fp32 [(Hq + 2 Hkv) * 128], caller-owned); each q head and each k head
 * RMS-normalised over its 128 values with g_q / g_k (bf16 [128]); q and k rotated
 * by RoPE at pos = seq_lens[0] - 1 (rotate-half: pair (i, i + 64) turns by
 * pos * rope_base^(-i/64), angles and their sines in fp64). q_out: fp32
 * [Hq][128]; k_out, v_out: bf16 [Hkv][128], rounded to nearest even -- the
 * candidate the decode calls commit. Two launches. hidden % 512 == 0 with
 * hidden / 512 in {1, 2, 3, 4, 6, 8, 12, 16}, 1 <= Hkv, Hq % Hkv == 0. */
int sk_qkv_rope(const uint16_t* W_qkv, const float* h, const uint16_t* g_attn,
                const uint16_t* g_q, const uint16_t* g_k, int32_t hidden, int32_t q_heads,
                int32_t kv_heads, float eps, float rope_base, const int32_t* seq_lens,
                float* scratch, float* q_out, uint16_t* k_out, uint16_t* v_out,
                const int32_t* sel, int32_t sel_value, hipStream_t stream);

/* out = x / sqrt(mean(x^2) + eps) * gamma over dim values (gamma bf16 [dim]);
 * 1 <= dim <= 16384. */
int sk_rmsnorm(const float* x, const uint16_t* gamma, int32_t dim, float eps, float* out,
               const int32_t* sel, int32_t sel_value, hipStream_t stream);

/* out[i] = table[token[0]][i] widened to fp32 (table bf16 [vocab][hidden]), and
 * the same into out2 when out2 != NULL; a token outside [0, vocab) gives zeros. */
int sk_embed(const uint16_t* table, int32_t vocab, int32_t hidden, const int32_t* token,
             float* out, float* out2, const int32_t* sel, int32_t sel_value,
             hipStream_t stream);

/* out = (gate[0] == gate_value) ? a : b over dim floats (the step select). */
int sk_select(const int32_t* gate, int32_t gate_value, const float* a, const float* b,
              int32_t dim, float* out, hipStream_t stream);

/* Block-table rewrite plus attention over the kept blocks ([DA] section 3).
 * For every selected request b, the kept logical blocks (bits of keep_mask
 * row b below ceil(n/16)) are compacted in ascending logical order into
 *   gathered[b][i]     = block_tables[b][block_i]   (physical id)
 *   gathered_cnt[b][i] = min(16, n - 16*block_i)    (valid positions)
 *   num_kept[b]        = number of entries
 * (rows of [batch][max_blocks] int32), and the request attends exactly the
 * positions of those blocks. k_new / v_new, when given, are committed to
 * position n-1 in every case and attended when their block is kept.
 * Other arguments as oda_decode_local. */
int da_decode_blocks(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                     const uint32_t* keep_mask, int32_t* gathered, int32_t* gathered_cnt,
                     int32_t* num_kept, float scale, const int32_t* sel, int32_t sel_value,
                     float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* The two halves of da_decode_blocks, for callers that attend one rewritten
 * block table from several layers ([DA] section 3: the engine rewrites the
 * block table once per declaration; every attention layer of the step reads
 * the same kept blocks). da_gather writes gathered / gathered_cnt / num_kept
 * for every selected request exactly as da_decode_blocks does (one launch);
 * da_decode_gathered attends the given list (entries in ascending logical
 * order, as da_gather writes them) with the current token committed as in
 * da_decode_blocks (one launch). A physical id outside [0, num_phys_blocks)
 * sets SK_DEVERR_BLOCK_ID and attends nothing for that entry. */
int da_gather(sk_paged_kv kv, const uint32_t* keep_mask, int32_t* gathered,
              int32_t* gathered_cnt, int32_t* num_kept, const int32_t* sel, int32_t sel_value,
              void* ws, hipStream_t stream);
int da_decode_gathered(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                       const int32_t* gathered, const int32_t* gathered_cnt,
                       const int32_t* num_kept, float scale, const int32_t* sel,
                       int32_t sel_value, float* out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Per-request views of a batch in one launch ([ODA] "Approach": a step attends the
 * Full view when recalled, else its local-first view; [DA] section 3: a request may
 * instead attend the kept blocks of its rewritten block table). Request b attends
 *   view[b] == SK_MODE_FULL   : [0, n)                       (as oda_decode_full)
 *   view[b] == SK_MODE_LOCAL  : sinks + window               (as oda_decode_local)
 *   view[b] == SK_MODE_BLOCKS : its gathered list            (as da_decode_gathered)
 * and any other value runs nothing for b (out rows untouched, nothing committed).
 * k_new / v_new, when given, are committed to position n-1 of every running
 * request, as the single-view calls do. One launch instead of three: outputs
 * equal those of the three selector calls up to the order of the split merge
 * (the splits are planned over all running requests together).
 *  view     : int32 [batch], device memory (oda_gate_scores writes it)
 *  gathered, gathered_cnt, num_kept : da_gather's output for the SK_MODE_BLOCKS
 *             requests (read only for them)
 * Other arguments as oda_decode_local. Host-checked: view and the list arrays
 * non-NULL, sinks >= 0, window >= 1. */
int oda_decode_views(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                     int32_t sinks, int32_t window, float scale, const int32_t* view,
                     const int32_t* gathered, const int32_t* gathered_cnt,
                     const int32_t* num_kept, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Attention over the blocks a declared mode keeps ([DA] sections 1 and 3), with the
 * block-table rewrite done inside the decode kernel instead of through a keep mask and
 * a gathered list: decl and local_tokens as in da_keep_mask; the request attends exactly
 * the positions of the kept blocks, in ascending logical order, and commits k_new /
 * v_new (when given) as da_decode_blocks does. Outputs, commits and device error bits
 * are those of da_keep_mask followed by da_decode_blocks (the same tiles in the same
 * order, so bit for bit), in one launch and without the mask and list buffers. A mode
 * other than SK_DA_GLOBAL / SK_DA_FOCUS / SK_DA_LOCAL keeps nothing (SK_DEVERR_EMPTY,
 * zero row). NULL decl gives SK_E_NULL, local_tokens < 0 SK_E_RANGE; other arguments as
 * oda_decode_local. */
int da_decode_declared(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                       const int32_t* decl, int32_t local_tokens, float scale, const int32_t* sel,
                       int32_t sel_value, float* out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* ---- measurement helper (not part of the method) ---- */

/* Bandwidth reference for the decode rooflines: one launch of SK_STREAM_READ_GRID
 * workgroups (one per CU) reads `bytes` of device memory at `data` once, each
 * workgroup its own contiguous range (16-byte non-temporal loads, 1 KiB contiguous per
 * wave instruction, four loads per lane in flight), and writes one XOR checksum per
 * workgroup to sink[0 .. SK_STREAM_READ_GRID-1] (device uint32, caller-owned; the XOR
 * of all of them equals the XOR of all 32-bit words read). bytes must be a multiple of
 * 16 and data 16-byte aligned (SK_E_RANGE); NULL sink, or NULL data with bytes > 0,
 * gives SK_E_NULL. Asynchronous on `stream`. */
#define SK_STREAM_READ_GRID 256
int sk_stream_read(const void* data, uint64_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEKV_H */
