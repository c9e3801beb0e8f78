/*
 * tf.h - C ABI of a paged MLA latent KV cache with a DSA-style sparse indexer,
 * for one AMD Instinct MI355X (gfx950).
 *
 * The path, per layer and step:
 *   1. tf_latent_write      write each token's latent row (512 latent + 64 rope)
 *                           and its pooled index key into 512-row pages through a
 *                           per-stream page table;
 *   2. tf_indexer_logits    score query rows against the pooled keys (one per 4
 *                           tokens): l[t,j] = sum_h w[t,h] * ReLU(q[t,h] . k_j),
 *                           fp32, masked causally by the compressed length;
 *   3. tf_topk_blocks       select the top-k pooled blocks of each row
 *                           (tf_indexer_topk runs steps 2 and 3 one key block at
 *                           a time, without the whole logits buffer;
 *                           tf_indexer_topk_fused writes no logits at all;
 *                           tf_candidate_groups and tf_topk_in_candidates select
 *                           in two levels, candidate groups then keys);
 *   4. tf_sparse_mla_attn   absorbed-MLA softmax attention that gathers only the
 *                           selected latent rows from the pages (decode rows and
 *                           chunked-prefill rows alike);
 *   plus tf_latent_write_quantize (step 1 for fp8 pages, quantizing bf16 rows on
 *   the device), tf_dense_mla_attn (short contexts: attention over every visible
 *   token, with no indexer or top-k), tf_snapshot_copy (copy only the first `at` rows of a stream) and
 *   the host-side tf_kv_pool_plan / tf_prefill_chunk.
 *
 * Sources (web pages, by title and section):
 *   [#1142] "Proposal: GLM-5.3-Flash on CUDA takes its streams' KV pages from the
 *           core pool, and kept prompt states copy only their rows"
 *   [#1313] "GLM-5.3-Flash CUDA at TP=2: --parallel 8 at a 1M window is refused
 *           ... though KV pages would serve it"
 *   [#1732] "TF_GLM_KV_SHARE=n with TF_KV_PAGES=on keeps GLM's prompts as the
 *           pool's pages"
 *   [CPM]   "Running CHUNKED_PREFILL_SIZE above 1024 without the long-prompt
 *           memory problem"
 *
 * Conventions for every call:
 *   - Device pointers are caller-owned. The library never allocates, frees or
 *     synchronizes; it enqueues kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns.
 *   - Returns TF_OK or an error code. Arguments are validated on the host before
 *     any launch; on error nothing is enqueued and tf_last_error() (thread-local)
 *     names the argument and the fix. A launch failure reports TF_E_DEVICE.
 *   - Page ids and positions live in device memory, which the calls do not read
 *     on the host. A caller that holds a host copy of a table refuses a bad one
 *     before any launch with tf_check_page_table (TF_E_RANGE). On the device,
 *     kernels skip (writes) or produce NaN for (reads) any row whose page id
 *     falls outside [0, n_pages) or whose page index falls outside the table's
 *     stride, so a bad table never leads to an out-of-bounds access.
 *   - Every call is safe to capture in a HIP graph (no memset, no allocation).
 */
#ifndef TF_H_
#define TF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TF_OK = 0,
  TF_E_INVAL = 1,        /* an argument is malformed */
  TF_E_RANGE = 2,        /* a size or index is out of the supported range */
  TF_E_NOMEM = 3,        /* the plan's room cannot fund one window (refused at start) */
  TF_E_UNSUPPORTED = 4,  /* a shape the library has no kernel for */
  TF_E_DEVICE = 5        /* the HIP runtime reported an error */
} tf_status;

/* Latent row formats. FP8 rows are 512 OCP e4m3fn bytes and one fp32 scale; a
 * page keeps its rows' scales after its rows [#1313, "Proposal", step 1 item 3];
 * value = decode(byte) * scale. */
typedef enum { TF_LAT_BF16 = 0, TF_LAT_FP8E4M3_ROWSCALE = 1 } tf_lat_fmt;

/* Plan order [#1313]: ONE_WINDOW_FIRST funds one window, a page for each other
 * stream, then the prompt cache, then the rest as pages ("Why"); WINDOWS_FIRST
 * first sets aside n = min(lanes, 1 + (room - window) / (window + fixed))
 * windows ("Proposal", step 1 item 1). */
typedef enum { TF_PLAN_ONE_WINDOW_FIRST = 0, TF_PLAN_WINDOWS_FIRST = 1 } tf_plan_policy;

/* Geometry of one pool. One page id spans all n_caches caches (the 11 MLA layers
 * and the MTP layer in the pages) [#1142, "What happens now"]; pages hold 512 rows
 * [#1142, "GLM declares a kv_pool.Layout"]. */
typedef struct {
  int32_t n_caches;    /* >= 1 */
  int32_t page_rows;   /* must be 512 */
  int32_t latent_dim;  /* must be 512 */
  int32_t rope_dim;    /* 64 (0 allowed for byte accounting only) */
  int32_t pool_ratio;  /* tokens per pooled key: must be 4 */
  int32_t index_dim;   /* pooled key length in bf16: 64 or 128 */
  int32_t lat_fmt;     /* tf_lat_fmt */
} tf_geom;

/* Memory budget for the plan (all bytes per GPU). */
typedef struct {
  int64_t room_bytes;             /* what the pool, the fixed parts and the cache may use */
  int64_t window_tokens;          /* --context */
  int64_t lookahead_rows;         /* rows past the window a stream may write (1: MTP head) */
  int64_t fixed_bytes_per_stream; /* a stream's state outside the pages */
  int64_t cache_cap_bytes;        /* prompt cache cap */
  int32_t lanes;                  /* --parallel: streams */
  int32_t policy;                 /* tf_plan_policy */
} tf_budget;

/* Layout inside one page: for each cache c, the cache block at
 * c * cache_block_bytes holds, in order, the latent plane (page_rows rows of
 * lat_row_bytes), the fp32 scale plane (fp8 only: page_rows x 4 B), the rope
 * plane (page_rows x rope_row_bytes, bf16) and the pooled-key plane
 * (keys_per_page = page_rows / pool_ratio keys of pkey_row_bytes, bf16). */
typedef struct {
  tf_geom g;
  int64_t lat_row_bytes, rope_row_bytes, pkey_row_bytes, keys_per_page;
  int64_t off_latent, off_scale, off_rope, off_pkey;
  int64_t cache_block_bytes, page_bytes;
  int64_t bytes_per_token;        /* all planes, all caches */
  int64_t bytes_per_token_pages;  /* latent (+ scale) + pooled-key share, all caches: the
                                     pages' own count, 13,056 B for 12 bf16 caches [#1142] */
  /* budget results (all zero when no budget is given) */
  int64_t window_pages;           /* ceil((window + lookahead) / page_rows) */
  int64_t n_windows, stream_pages, total_pages, cache_bytes, fixed_bytes;
} tf_plan;

/* A view of one cache of a pool as seen by a set of streams.
 * Row t of stream b lives in page pt[b * pt_stride + t / 512] at slot t % 512;
 * pooled key j of stream b in page pt[b * pt_stride + j / 128] at slot j % 128.
 * A NULL pt keeps contiguous rows: stream b's page i is pool page
 * b * pt_stride + i, so a window is its pages in order and one address formula
 * serves both [#1142, "GLM declares a kv_pool.Layout"; #1313, "Proposal"]. */
typedef struct {
  void* pool;           /* device, n_pages * page_bytes bytes */
  const int32_t* pt;    /* device [streams][pt_stride] page ids, or NULL */
  int32_t pt_stride;    /* pages per stream in the table (the window for NULL) */
  int32_t n_streams;    /* streams (rows) of the table; stream ids outside [0, n_streams) read nothing */
  int32_t n_pages;      /* pages in the pool */
  int32_t cache;        /* which cache block of each page (0 <= cache < n_caches) */
} tf_kv_view;

/* Host only. Checks a page table before it is handed to the device [#1142, "GLM
 * declares a kv_pool.Layout": kernels take a page table; "Proposal": page ids come
 * from the host's plan]. pt_host is a host array [n_streams][pt_stride] of int32.
 * Every entry must be a pool page in [0, n_pages) or -1 (no page yet: reads of
 * such a row give NaN, writes to it are skipped). Returns TF_E_RANGE naming the
 * first stream, page index and id that break this, TF_E_INVAL for a NULL table
 * or non-positive sizes, TF_OK otherwise. Reads nothing but pt_host. */
tf_status tf_check_page_table(const int32_t* pt_host, int32_t n_streams, int32_t pt_stride, int32_t n_pages);

/* Host only. Fills `out` with the page layout of `g` and, when `budget` is not
 * NULL, the page budget in the pages' plan order [#1313, "Why" and "Proposal"].
 * Under WINDOWS_FIRST the streams hold max(n windows, one window + a page per
 * other stream). TF_E_NOMEM when the room cannot fund that; the message names
 * the room needed. */
tf_status tf_kv_pool_plan(const tf_geom* g, const tf_budget* budget, tf_plan* out);

/* Host only. Adaptive prefill chunk [CPM, 2.1]: with L = history_tokens,
 * chunk = clamp(round_down_to_256(2.0e8 / L), 256, 2048), 2048 at L = 0, and
 * never more than remaining_tokens. Returns 0 when remaining_tokens <= 0. */
int64_t tf_prefill_chunk(int64_t history_tokens, int64_t remaining_tokens);

/* Write rows and pooled keys into pages (a byte copy) [#1142, "GLM declares a
 * kv_pool.Layout": the writes take the page table].
 *   row i (i < n_rows) of stream row_stream[i] at position row_pos[i]:
 *     latent: bf16 [n_rows][512] or e4m3 bytes [n_rows][512] (fp8 format)
 *     row_scale: fp32 [n_rows] (fp8 only; else ignored, may be NULL)
 *     rope: bf16 [n_rows][rope_dim]
 *   pooled key i (i < n_pkeys) of stream pkey_stream[i] with index pkey_idx[i]:
 *     pkeys: bf16 [n_pkeys][index_dim]
 * All arrays are device memory. Rows whose page is out of range are skipped.
 * Writing a row that other streams share is the caller's contract to avoid. */
tf_status tf_latent_write(const tf_plan* p, tf_kv_view dst, int32_t n_rows,
                          const int32_t* row_stream, const int32_t* row_pos,
                          const void* latent, const float* row_scale, const void* rope,
                          int32_t n_pkeys, const int32_t* pkey_stream, const int32_t* pkey_idx,
                          const void* pkeys, void* stream);

/* The same write for fp8 pages, quantizing on the device [#1313, "Proposal",
 * step 1 item 3: fp8 rows on pages, each row's fp32 scale kept after the page's
 * rows, written through the table as the bf16 write is]. The pages fix no
 * quantization recipe; this one is per row:
 *   scale = amax / 448 (fp32 division; amax = max |x| over the row's 512 values),
 *   code_i = the e4m3fn value nearest to clamp(x_i / scale, -448, 448) (fp32
 *            division), ties to the even code, sign from the quotient (so a
 *            negative value that rounds to zero is coded -0),
 *   and an all-zero row gets scale 0 and +0 codes.
 * All arithmetic is IEEE fp32 (the divisions correctly rounded). The row's element
 * of largest magnitude is coded +-448 exactly whenever the scale is a normal fp32
 * number.
 *   latent: bf16 [n_rows][512], finite (non-finite values give unspecified codes)
 *   rope, pooled keys and every other argument as in tf_latent_write.
 * TF_E_INVAL unless the plan's format is TF_LAT_FP8E4M3_ROWSCALE. */
tf_status tf_latent_write_quantize(const tf_plan* p, tf_kv_view dst, int32_t n_rows,
                                   const int32_t* row_stream, const int32_t* row_pos,
                                   const void* latent, const void* rope,
                                   int32_t n_pkeys, const int32_t* pkey_stream, const int32_t* pkey_idx,
                                   const void* pkeys, void* stream);

/* Indexer logits [CPM, section 1]: for row r (stream row_stream[r], position
 * t = row_pos[r]) and pooled key j < n_c = min(t / 4 + 1, ld):
 *   logits[r * ld + j] = sum_h w[r * n_heads + h] * max(0, q[r][h] . key_j)
 * and -inf for n_c <= j < ld. q is bf16 [n_rows][n_heads][index_dim], w fp32
 * [n_rows][n_heads], logits fp32 [n_rows][ld]. Products are exact bf16 x bf16,
 * accumulated in fp32 (MFMA); the ReLU, weights and head sum in fp32.
 * n_valid (optional, device int32 [n_rows]) receives n_c.
 * Rows of streams whose tables name the same pages (a prefix held by reference,
 * [#1732] "What this changes") may be scored from one read of each shared page;
 * the results are the same bit for bit.
 * n_heads must be 4, 8 or 16; index_dim 64 or 128; ld >= 1. */
tf_status tf_indexer_logits(const tf_plan* p, tf_kv_view keys, int32_t n_rows,
                            const int32_t* row_stream, const int32_t* row_pos,
                            const void* q, const float* w, int32_t n_heads,
                            float* logits, int64_t ld, int32_t* n_valid, void* stream);

/* Top-k pooled blocks [CPM, sections 1 and 2.3]: for each row the k largest of
 * logits[r * ld + j], j < n_valid[r] (n_valid NULL: ld), ties to the lower index,
 * -0 equal to +0; written ascending to blocks [n_rows][k] and padded with -1
 * when fewer than k are visible. Long rows are split into key blocks whose
 * per-block top-k are merged (exact: topk(union) == topk(union of block top-k)).
 * ws: device workspace of at least tf_topk_workspace_bytes(n_rows, ld, k) bytes
 * (may be NULL when that is 0). 1 <= k <= 2048; NaN inputs are not supported. */
tf_status tf_topk_blocks(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid,
                         int32_t k, int32_t* blocks, void* ws, size_t ws_bytes, void* stream);
size_t tf_topk_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k);

/* Key-blocked indexer + top-k [CPM, section 2.3: score the rows against one key
 * block at a time, keep each block's top-k with its values, then take the top-k
 * of the candidates; exact, since topk(union) == topk(union of block top-k)]:
 * the blocks that tf_indexer_logits followed by tf_topk_blocks would select, bit
 * for bit, without the [n_rows][ld] logits buffer. Keys [0, ld) are scored in
 * key_block-key blocks (a multiple of 128 in 128..32768) into a workspace of
 * n_rows x key_block logits, whose per-block top-k candidates (order keys and
 * indices) wait in the workspace for the merge. Device memory is
 * tf_indexer_topk_workspace_bytes(n_rows, ld, k, key_block), flat in ld but
 * for the candidates (n_rows x blocks x k x 8 bytes). q, w, n_heads and the
 * masking are as for tf_indexer_logits; blocks, k and the tie rule as for
 * tf_topk_blocks. n_valid (optional, device int32 [n_rows]) receives n_c.
 * Limits: n_rows <= 65535, blocks x k <= 32,768 (TF_E_RANGE names the fix).
 * ws must be 16-byte aligned. The blocks run one after another on `stream`. */
tf_status tf_indexer_topk(const tf_plan* p, tf_kv_view keys, int32_t n_rows,
                          const int32_t* row_stream, const int32_t* row_pos, const void* q,
                          const float* w, int32_t n_heads, int64_t ld, int32_t k,
                          int32_t key_block, int32_t* blocks, int32_t* n_valid, void* ws,
                          size_t ws_bytes, void* stream);
size_t tf_indexer_topk_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k, int32_t key_block);

/* Fused indexer + top-k [CPM, section 2.3: only per-block top-k candidates leave the
 * scoring, and topk(union) == topk(union of block top-k) keeps the result exact;
 * section 1 on the [T, L] logits buffer this removes]: the blocks that
 * tf_indexer_logits followed by tf_topk_blocks would select, bit for bit, with no
 * logits written to memory. Each row's keys of every step-th page (about a sixteenth
 * of them, at least 2,048) are scored first, and a threshold is taken among those values
 * that about 2k of the row's keys should reach (at most the k-th largest of them). A
 * second scoring of every key, with the same arithmetic, keeps only the keys at or
 * above it (in key order, per key group of the launch). When at least k keys reach it,
 * the k-th largest logit does too, so the row's top k, ties with the k-th value
 * included, are candidates and their top k is the answer. A row with fewer than k
 * candidates or more than its slots hold (inputs far from an even spread: many equal
 * logits, large logits only in unsampled pages, rows much shorter than ld) is
 * re-scored and selected exactly inside the last kernel, more slowly. Rows of at most
 * max(4,096, 8k) keys, and calls of fewer than 64 rows of at most 262,144 keys (decode
 * batches: their logits are small, and the sample and threshold launches would cost
 * more than the buffer saves), are scored whole into the workspace and selected there,
 * by the kernels of the unfused pair. Arguments, masking, n_valid, the tie rule and -1
 * padding are those of tf_indexer_logits and tf_topk_blocks; NaN logits (missing pages)
 * order as there. ws: 256-byte aligned device workspace of at least
 * tf_indexer_topk_fused_workspace_bytes(n_rows, ld, k, n_heads) bytes, about
 * n_rows x (ld / 4 + 4 k x 8) for long rows: it grows with ld at a sixteenth of
 * the logits' rate (n_rows x ld x 4 and the top-k's own workspace when scored whole).
 * Limits: n_rows <= 65535, 1 <= k <= 2048, ld <= 2^24; four launches on `stream` (two
 * or three when scored whole). */
tf_status tf_indexer_topk_fused(const tf_plan* p, tf_kv_view keys, int32_t n_rows,
                                const int32_t* row_stream, const int32_t* row_pos, const void* q,
                                const float* w, int32_t n_heads, int64_t ld, int32_t k,
                                int32_t* blocks, int32_t* n_valid, void* ws, size_t ws_bytes,
                                void* stream);
size_t tf_indexer_topk_fused_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k, int32_t n_heads);

/* Two-level candidate selection [CPM, section 1: a layer publishes candidate
 * masks that the later low-ratio layers consume; section 2.3: its block pooling
 * over 8-key groups and top-2,048 groups, and the consumers' masking of
 * non-candidates before their own top-k]. The pages name the steps only; the
 * readings taken:
 *
 * tf_candidate_groups: each visible group of `group` consecutive keys (keys
 * j < n_valid[r]; the last group may be partial) scores the largest of its
 * logits, and cand [n_rows][n_cand] receives the top-n_cand groups of each row
 * as tf_topk_blocks selects (ties to the lower group, ascending, -1 padded).
 * logits are read only. 1 <= group <= 64, 1 <= n_cand <= 2048, n_rows <= 65535.
 * ws: 16-byte aligned device workspace of at least
 * tf_candidate_groups_workspace_bytes(n_rows, ld, group, n_cand) bytes.
 *
 * tf_topk_in_candidates: the consumer. blocks receives row r's top-k as
 * tf_topk_blocks selects it from the row with its visible keys outside its
 * candidate groups (cand [n_rows][n_cand], entries < 0 ignored) read as -inf,
 * the pages' masked_fill_ (fewer than k candidate keys: the lowest-index others
 * complete it). The masking happens as the keys are loaded: logits are read
 * only. ws: as for tf_topk_blocks (tf_topk_in_candidates_workspace_bytes). */
tf_status tf_candidate_groups(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid,
                              int32_t group, int32_t n_cand, int32_t* cand, void* ws, size_t ws_bytes,
                              void* stream);
size_t tf_candidate_groups_workspace_bytes(int32_t n_rows, int64_t ld, int32_t group, int32_t n_cand);
tf_status tf_topk_in_candidates(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid,
                                const int32_t* cand, int32_t n_cand, int32_t group, int32_t k,
                                int32_t* blocks, void* ws, size_t ws_bytes, void* stream);
size_t tf_topk_in_candidates_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k);

/* Sparse absorbed-MLA attention [#1313, "Step 2"; #1142, "What stays as it
 * is"]: for row r at position t, head h, with S = {s <= t : s / 4 in
 * blocks[r][*]} (entries < 0 ignored):
 *   z_s = softmax_scale * q[r][h] . [latent_s ; rope_s]   (576 values)
 *   out[r][h][:] = sum_s softmax(z)_s * latent_s           (fp32 [n_rows][n_heads][512])
 *   lse[r][h] = log sum_s exp(z_s)                          (optional fp32 [n_rows][n_heads])
 * An empty S gives out = 0 and lse = -inf. q is bf16 [n_rows][n_heads][576];
 * fp8 latent rows enter as decode(byte) * row scale. Products are exact and
 * accumulated in fp32; softmax weights keep 16 significant bits (a bf16
 * hi + lo pair) in the value product. n_heads <= 32; 1 <= k <= 2048.
 * ws: device workspace of at least tf_attn_workspace_bytes(n_rows, n_heads, k)
 * bytes for split partials (may be NULL when that is 0). */
tf_status tf_sparse_mla_attn(const tf_plan* p, tf_kv_view kv, int32_t n_rows,
                             const int32_t* row_stream, const int32_t* row_pos,
                             const void* q, int32_t n_heads, float softmax_scale,
                             const int32_t* blocks, int32_t k, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* The sparse pass for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and results as tf_sparse_mla_attn, bit for bit, with no workspace
 * argument. Its split partials live in a fixed scratch array inside the library
 * (tf_sparse_mla_attn_noalloc_max_bytes() bytes, 32 MiB, one copy per GPU, held
 * until the process ends); a call whose partials need more (see
 * tf_attn_workspace_bytes) is refused with TF_E_RANGE before any launch. The call
 * allocates nothing. Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (two streams, or two threads) race and must be serialized by
 * the caller. Nothing in the scratch needs clearing between calls; a call writes
 * every partial it reads. Other arguments and errors as for tf_sparse_mla_attn. */
tf_status tf_sparse_mla_attn_noalloc(const tf_plan* p, tf_kv_view kv, int32_t n_rows,
                                     const int32_t* row_stream, const int32_t* row_pos,
                                     const void* q, int32_t n_heads, float softmax_scale,
                                     const int32_t* blocks, int32_t k, float* out, float* lse,
                                     void* stream);
size_t tf_sparse_mla_attn_noalloc_max_bytes(void);

/* Dense absorbed-MLA attention [#1142, "What stays as it is", and the kernel
 * list of its proposal: the page-table kernels read the latent for dense
 * chunks as well as for the sparse gather]: the short-context pass that skips
 * the indexer and the top-k. Row r at position t = row_pos[r] attends every
 * token it sees within the first n_blocks pooled blocks:
 *   S = {s : s <= t and s < 4 * n_blocks}
 * and computes out and lse as tf_sparse_mla_attn does over that set (the pages
 * give no extent; with n_blocks >= t / 4 + 1 for every row it is plain causal
 * attention). It equals tf_sparse_mla_attn with blocks[r] = 0, 1, ..,
 * n_blocks - 1 for every row, bit for bit, and a stream's results do not
 * depend on which pages hold its rows. q, out, lse, the scale and the rows'
 * formats are as for tf_sparse_mla_attn; 1 <= n_blocks <= 2048 (8,192 tokens;
 * longer contexts take the sparse path, TF_E_RANGE otherwise). ws: device
 * workspace of at least tf_attn_workspace_bytes(n_rows, n_heads, n_blocks)
 * bytes (may be NULL when that is 0). */
tf_status tf_dense_mla_attn(const tf_plan* p, tf_kv_view kv, int32_t n_rows,
                            const int32_t* row_stream, const int32_t* row_pos,
                            const void* q, int32_t n_heads, float softmax_scale,
                            int32_t n_blocks, float* out, float* lse, void* ws,
                            size_t ws_bytes, void* stream);
size_t tf_attn_workspace_bytes(int32_t n_rows, int32_t n_heads, int32_t k);

/* Snapshot [#1142, "Proposal" piece 1]: for each i < n_streams, copy rows
 * [0, at) of every plane of every cache, and pooled keys [0, at / 4), from
 * stream src_stream[i] of `src` to stream dst_stream[i] of `dst` (two views of
 * the same geometry; their `cache` fields are ignored). Rows at or past `at`
 * are neither read nor written. `at` must be a multiple of 4 and fit both
 * tables' strides; the stream index arrays are device int32. A page the call both
 * reads and writes must sit at the same page index in both tables (a page the two
 * tables share copies onto itself); any other overlap of read and written pages
 * gives undefined bytes. The copy streams past the caches (non-temporal). */
tf_status tf_snapshot_copy(const tf_plan* p, tf_kv_view src, tf_kv_view dst, int32_t n_streams,
                           const int32_t* src_stream, const int32_t* dst_stream, int64_t at,
                           void* stream);

/* Thread-local message of the last error ("" after success). */
const char* tf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TF_H_ */
