// The extern "C" entry points: argument validation on the host, then one launcher
// per operation. Nothing here allocates, frees or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace tf {

static thread_local char g_err[512] = "";

tf_status set_error(tf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

tf_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(TF_E_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return TF_OK;
}

tf_status check_plan(const tf_plan* p) {
  if (!p) return set_error(TF_E_INVAL, "plan must not be NULL (fill it with tf_kv_pool_plan)");
  const tf_geom& g = p->g;
  if (g.page_rows != kPageRows || g.latent_dim != kLatent || g.pool_ratio != kPoolRatio ||
      (g.index_dim != 64 && g.index_dim != 128) || g.n_caches < 1 ||
      (g.lat_fmt != TF_LAT_BF16 && g.lat_fmt != TF_LAT_FP8E4M3_ROWSCALE))
    return set_error(TF_E_INVAL, "plan geometry is not one tf_kv_pool_plan produces");
  if (p->page_bytes != p->cache_block_bytes * g.n_caches || p->page_bytes <= 0)
    return set_error(TF_E_INVAL, "plan page_bytes is inconsistent: refill it with tf_kv_pool_plan");
  return TF_OK;
}

tf_status check_view(const tf_plan* p, const tf_kv_view& v, const char* name) {
  if (!v.pool) return set_error(TF_E_INVAL, "%s.pool must not be NULL", name);
  if (v.n_pages < 1) return set_error(TF_E_INVAL, "%s.n_pages=%d, need >= 1", name, v.n_pages);
  if (v.pt_stride < 1) return set_error(TF_E_INVAL, "%s.pt_stride=%d, need >= 1", name, v.pt_stride);
  if (v.n_streams < 1) return set_error(TF_E_INVAL, "%s.n_streams=%d, need >= 1", name, v.n_streams);
  if (v.cache < 0 || v.cache >= p->g.n_caches)
    return set_error(TF_E_RANGE, "%s.cache=%d outside [0, %d)", name, v.cache, p->g.n_caches);
  if (((uintptr_t)v.pool & 15) != 0) return set_error(TF_E_INVAL, "%s.pool must be 16-byte aligned", name);
  return TF_OK;
}

DevView make_view(const tf_plan* p, const tf_kv_view& v) {
  DevView d;
  d.pool = (char*)v.pool;
  d.pt = v.pt;
  d.pt_stride = v.pt_stride;
  d.n_streams = v.n_streams;
  d.n_pages = v.n_pages;
  d.page_bytes = p->page_bytes;
  d.cache_off = (int64_t)v.cache * p->cache_block_bytes;
  return d;
}

static bool aligned16(const void* x) { return ((uintptr_t)x & 15) == 0; }

}  // namespace tf

using namespace tf;

extern "C" const char* tf_last_error(void) { return g_err; }

extern "C" tf_status tf_check_page_table(const int32_t* pt_host, int32_t n_streams, int32_t pt_stride,
                                         int32_t n_pages) {
  clear_error();
  if (!pt_host) return set_error(TF_E_INVAL, "tf_check_page_table: pt_host must not be NULL");
  if (n_streams < 1 || pt_stride < 1 || n_pages < 1)
    return set_error(TF_E_INVAL, "tf_check_page_table: n_streams=%d, pt_stride=%d, n_pages=%d must be >= 1",
                     n_streams, pt_stride, n_pages);
  for (int64_t b = 0; b < n_streams; ++b)
    for (int64_t i = 0; i < pt_stride; ++i) {
      const int32_t p = pt_host[b * pt_stride + i];
      if (p < -1 || p >= n_pages)
        return set_error(TF_E_RANGE,
                         "tf_check_page_table: stream %lld page index %lld names page %d, outside the pool's "
                         "[0, %d) (use -1 for no page)",
                         (long long)b, (long long)i, p, n_pages);
    }
  return TF_OK;
}

extern "C" tf_status tf_latent_write(const tf_plan* p, tf_kv_view dst, int32_t n_rows,
                                     const int32_t* row_stream, const int32_t* row_pos,
                                     const void* latent, const float* row_scale, const void* rope,
                                     int32_t n_pkeys, const int32_t* pkey_stream,
                                     const int32_t* pkey_idx, const void* pkeys, void* stream) {
  clear_error();
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  if ((s = check_view(p, dst, "dst")) != TF_OK) return s;
  if (n_rows < 0 || n_pkeys < 0) return set_error(TF_E_INVAL, "tf_latent_write: negative counts");
  const bool fp8 = p->g.lat_fmt == TF_LAT_FP8E4M3_ROWSCALE;
  if (n_rows > 0) {
    if (!row_stream || !row_pos || !latent)
      return set_error(TF_E_INVAL, "tf_latent_write: row_stream, row_pos and latent are required");
    if (p->g.rope_dim > 0 && !rope) return set_error(TF_E_INVAL, "tf_latent_write: rope is required");
    if (fp8 && !row_scale) return set_error(TF_E_INVAL, "tf_latent_write: fp8 rows need row_scale");
    if (!aligned16(latent) || (rope && !aligned16(rope)))
      return set_error(TF_E_INVAL, "tf_latent_write: latent and rope must be 16-byte aligned");
  }
  if (n_pkeys > 0) {
    if (!pkey_stream || !pkey_idx || !pkeys)
      return set_error(TF_E_INVAL, "tf_latent_write: pkey_stream, pkey_idx and pkeys are required");
    if (!aligned16(pkeys)) return set_error(TF_E_INVAL, "tf_latent_write: pkeys must be 16-byte aligned");
  }
  if (n_rows == 0 && n_pkeys == 0) return TF_OK;
  return launch_latent_write(p, make_view(p, dst), n_rows, row_stream, row_pos, latent, row_scale, rope,
                             n_pkeys, pkey_stream, pkey_idx, pkeys, (hipStream_t)stream, false);
}

extern "C" tf_status tf_latent_write_quantize(const tf_plan* p, tf_kv_view dst, int32_t n_rows,
                                              const int32_t* row_stream, const int32_t* row_pos,
                                              const void* latent, const void* rope, int32_t n_pkeys,
                                              const int32_t* pkey_stream, const int32_t* pkey_idx,
                                              const void* pkeys, void* stream) {
  clear_error();
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  if (p->g.lat_fmt != TF_LAT_FP8E4M3_ROWSCALE)
    return set_error(TF_E_INVAL,
                     "tf_latent_write_quantize: the plan's rows are bf16; plan with lat_fmt "
                     "TF_LAT_FP8E4M3_ROWSCALE, or write bf16 rows with tf_latent_write");
  if ((s = check_view(p, dst, "dst")) != TF_OK) return s;
  if (n_rows < 0 || n_pkeys < 0) return set_error(TF_E_INVAL, "tf_latent_write_quantize: negative counts");
  if (n_rows > 0) {
    if (!row_stream || !row_pos || !latent)
      return set_error(TF_E_INVAL, "tf_latent_write_quantize: row_stream, row_pos and latent are required");
    if (p->g.rope_dim > 0 && !rope) return set_error(TF_E_INVAL, "tf_latent_write_quantize: rope is required");
    if (!aligned16(latent) || (rope && !aligned16(rope)))
      return set_error(TF_E_INVAL, "tf_latent_write_quantize: latent and rope must be 16-byte aligned");
  }
  if (n_pkeys > 0) {
    if (!pkey_stream || !pkey_idx || !pkeys)
      return set_error(TF_E_INVAL, "tf_latent_write_quantize: pkey_stream, pkey_idx and pkeys are required");
    if (!aligned16(pkeys)) return set_error(TF_E_INVAL, "tf_latent_write_quantize: pkeys must be 16-byte aligned");
  }
  if (n_rows == 0 && n_pkeys == 0) return TF_OK;
  return launch_latent_write(p, make_view(p, dst), n_rows, row_stream, row_pos, latent, nullptr, rope, n_pkeys,
                             pkey_stream, pkey_idx, pkeys, (hipStream_t)stream, true);
}

extern "C" tf_status tf_snapshot_copy(const tf_plan* p, tf_kv_view src, tf_kv_view dst,
                                      int32_t n_streams, const int32_t* src_stream,
                                      const int32_t* dst_stream, int64_t at, void* stream) {
  clear_error();
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  src.cache = 0;
  dst.cache = 0;
  if ((s = check_view(p, src, "src")) != TF_OK) return s;
  if ((s = check_view(p, dst, "dst")) != TF_OK) return s;
  if (n_streams < 0) return set_error(TF_E_INVAL, "tf_snapshot_copy: n_streams < 0");
  if (at < 0 || at % kPoolRatio != 0)
    return set_error(TF_E_INVAL, "tf_snapshot_copy: at=%lld must be a non-negative multiple of 4",
                     (long long)at);
  const int64_t pages = (at + kPageRows - 1) / kPageRows;
  if (pages > src.pt_stride || pages > dst.pt_stride)
    return set_error(TF_E_RANGE, "tf_snapshot_copy: at=%lld needs %lld pages, the tables hold %d and %d",
                     (long long)at, (long long)pages, src.pt_stride, dst.pt_stride);
  if (n_streams == 0 || at == 0) return TF_OK;
  if (!src_stream || !dst_stream)
    return set_error(TF_E_INVAL, "tf_snapshot_copy: src_stream and dst_stream are required");
  return launch_snapshot(p, src, dst, n_streams, src_stream, dst_stream, at, (hipStream_t)stream);
}

extern "C" tf_status tf_indexer_logits(const tf_plan* p, tf_kv_view keys, int32_t n_rows,
                                       const int32_t* row_stream, const int32_t* row_pos,
                                       const void* q, const float* w, int32_t n_heads, float* logits,
                                       int64_t ld, int32_t* n_valid, void* stream) {
  clear_error();
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  if ((s = check_view(p, keys, "keys")) != TF_OK) return s;
  if (n_rows < 0) return set_error(TF_E_INVAL, "tf_indexer_logits: n_rows < 0");
  if (ld < 1 || ld > (1LL << 30)) return set_error(TF_E_RANGE, "tf_indexer_logits: ld=%lld", (long long)ld);
  if (n_heads != 4 && n_heads != 8 && n_heads != 16)
    return set_error(TF_E_UNSUPPORTED, "tf_indexer_logits: n_heads=%d, built for 4, 8 or 16", n_heads);
  if (n_rows == 0) return TF_OK;
  if (!row_stream || !row_pos || !q || !w || !logits)
    return set_error(TF_E_INVAL, "tf_indexer_logits: row_stream, row_pos, q, w and logits are required");
  if (!aligned16(q)) return set_error(TF_E_INVAL, "tf_indexer_logits: q must be 16-byte aligned");
  return launch_indexer(p, make_view(p, keys), n_rows, row_stream, row_pos, q, w, n_heads, logits, ld,
                        n_valid, (hipStream_t)stream, 0, ld, ld, false);
}

extern "C" size_t tf_topk_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k) {
  if (n_rows <= 0 || ld <= 0 || k <= 0) return 0;
  return topk_ws_bytes(n_rows, ld, k);
}

extern "C" tf_status tf_topk_blocks(const float* logits, int64_t ld, int32_t n_rows,
                                    const int32_t* n_valid, int32_t k, int32_t* blocks, void* ws,
                                    size_t ws_bytes, void* stream) {
  clear_error();
  if (n_rows < 0) return set_error(TF_E_INVAL, "tf_topk_blocks: n_rows < 0");
  if (k < 1 || k > 2048) return set_error(TF_E_RANGE, "tf_topk_blocks: k=%d, need 1..2048", k);
  if (ld < 1 || ld > (1LL << 24)) return set_error(TF_E_RANGE, "tf_topk_blocks: ld=%lld", (long long)ld);
  if (n_rows == 0) return TF_OK;
  if (!logits || !blocks) return set_error(TF_E_INVAL, "tf_topk_blocks: logits and blocks are required");
  const size_t need = topk_ws_bytes(n_rows, ld, k);
  if (need == (size_t)-1)
    return set_error(TF_E_UNSUPPORTED, "tf_topk_blocks: ld=%lld with k=%d exceeds the blocked merge",
                     (long long)ld, k);
  if (need > 0 && (!ws || ws_bytes < need))
    return set_error(TF_E_INVAL, "tf_topk_blocks: workspace of %zu bytes needed, got %zu", need, ws_bytes);
  return launch_topk(logits, ld, n_rows, n_valid, k, blocks, ws, ws_bytes, (hipStream_t)stream);
}

// Key-blocked workspace: one block of logits, the blocks' candidates, then n_c.
static size_t idxtopk_ws(int32_t n_rows, int64_t ld, int32_t k, int32_t key_block, int64_t* nb_out) {
  const int64_t nb = (ld + key_block - 1) / key_block;
  if (nb_out) *nb_out = nb;
  return (size_t)n_rows * key_block * 4 + topk_cand_bytes(n_rows, (int32_t)nb, k) + ((size_t)n_rows * 4 + 15) / 16 * 16;
}

extern "C" size_t tf_indexer_topk_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k, int32_t key_block) {
  if (n_rows <= 0 || ld <= 0 || k <= 0 || key_block <= 0) return 0;
  return idxtopk_ws(n_rows, ld, k, key_block, nullptr);
}

extern "C" tf_status tf_indexer_topk(const tf_plan* p, tf_kv_view keys, int32_t n_rows,
                                     const int32_t* row_stream, const int32_t* row_pos, const void* q,
                                     const float* w, int32_t n_heads, int64_t ld, int32_t k,
                                     int32_t key_block, int32_t* blocks, int32_t* n_valid, void* ws,
                                     size_t ws_bytes, void* stream) {
  clear_error();
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  if ((s = check_view(p, keys, "keys")) != TF_OK) return s;
  if (n_rows < 0) return set_error(TF_E_INVAL, "tf_indexer_topk: n_rows < 0");
  if (n_rows > 65535) return set_error(TF_E_RANGE, "tf_indexer_topk: n_rows=%d, at most 65535 a call", n_rows);
  if (ld < 1 || ld > (1LL << 24)) return set_error(TF_E_RANGE, "tf_indexer_topk: ld=%lld", (long long)ld);
  if (k < 1 || k > 2048) return set_error(TF_E_RANGE, "tf_indexer_topk: k=%d, need 1..2048", k);
  if (key_block < kKeysPerPage || key_block > 32768 || key_block % kKeysPerPage != 0)
    return set_error(TF_E_INVAL, "tf_indexer_topk: key_block=%d, need a multiple of 128 in 128..32768", key_block);
  if (n_heads != 4 && n_heads != 8 && n_heads != 16)
    return set_error(TF_E_UNSUPPORTED, "tf_indexer_topk: n_heads=%d, built for 4, 8 or 16", n_heads);
  int64_t nb = 0;
  const size_t need = idxtopk_ws(n_rows, ld, k, key_block, &nb);
  if (nb * ((k + 3) / 4 * 4) > 32768)
    return set_error(TF_E_RANGE,
                     "tf_indexer_topk: %lld key blocks x %d candidates exceed the merge's 32,768; raise key_block",
                     (long long)nb, k);
  if (n_rows == 0) return TF_OK;
  if (!row_stream || !row_pos || !q || !w || !blocks)
    return set_error(TF_E_INVAL, "tf_indexer_topk: row_stream, row_pos, q, w and blocks are required");
  if (!aligned16(q)) return set_error(TF_E_INVAL, "tf_indexer_topk: q must be 16-byte aligned");
  if (!ws || ws_bytes < need || !aligned16(ws))
    return set_error(TF_E_INVAL, "tf_indexer_topk: a 16-byte aligned workspace of %zu bytes is needed, got %zu",
                     need, ws_bytes);
  const hipStream_t st = (hipStream_t)stream;
  const DevView v = make_view(p, keys);
  float* lbuf = (float*)ws;
  char* cand = (char*)ws + (size_t)n_rows * key_block * 4;
  int32_t* nv = n_valid ? n_valid : (int32_t*)(cand + topk_cand_bytes(n_rows, (int32_t)nb, k));
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t k0 = b * key_block, k1 = k0 + key_block < ld ? k0 + key_block : ld;
    if ((s = launch_indexer(p, v, n_rows, row_stream, row_pos, q, w, n_heads, lbuf, key_block, b == 0 ? nv : nullptr,
                            st, k0, k1, ld, true)) != TF_OK)
      return s;
    if ((s = launch_topk_block(lbuf, key_block, (int32_t)b, (int32_t)nb, ld, n_rows, nv, k, cand, st)) != TF_OK)
      return s;
  }
  return launch_topk_merge(key_block, (int32_t)nb, ld, n_rows, nv, k, blocks, cand, st);
}

extern "C" size_t tf_indexer_topk_fused_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k, int32_t n_heads) {
  if (n_rows <= 0 || ld <= 0 || k <= 0 || (n_heads != 4 && n_heads != 8 && n_heads != 16)) return 0;
  return indexer_topk_fused_ws_bytes(n_heads, n_rows, ld, k);
}

extern "C" tf_status tf_indexer_topk_fused(const tf_plan* p, tf_kv_view keys, int32_t n_rows,
                                           const int32_t* row_stream, const int32_t* row_pos, const void* q,
                                           const float* w, int32_t n_heads, int64_t ld, int32_t k, int32_t* blocks,
                                           int32_t* n_valid, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  if ((s = check_view(p, keys, "keys")) != TF_OK) return s;
  if (n_rows < 0) return set_error(TF_E_INVAL, "tf_indexer_topk_fused: n_rows < 0");
  if (n_rows > 65535) return set_error(TF_E_RANGE, "tf_indexer_topk_fused: n_rows=%d, at most 65535 a call", n_rows);
  if (ld < 1 || ld > (1LL << 24)) return set_error(TF_E_RANGE, "tf_indexer_topk_fused: ld=%lld", (long long)ld);
  if (k < 1 || k > 2048) return set_error(TF_E_RANGE, "tf_indexer_topk_fused: k=%d, need 1..2048", k);
  if (n_heads != 4 && n_heads != 8 && n_heads != 16)
    return set_error(TF_E_UNSUPPORTED, "tf_indexer_topk_fused: n_heads=%d, built for 4, 8 or 16", n_heads);
  if (n_rows == 0) return TF_OK;
  if (!row_stream || !row_pos || !q || !w || !blocks)
    return set_error(TF_E_INVAL, "tf_indexer_topk_fused: row_stream, row_pos, q, w and blocks are required");
  if (!aligned16(q)) return set_error(TF_E_INVAL, "tf_indexer_topk_fused: q must be 16-byte aligned");
  const size_t need = indexer_topk_fused_ws_bytes(n_heads, n_rows, ld, k);
  if (need == (size_t)-1)
    return set_error(TF_E_RANGE, "tf_indexer_topk_fused: no top-k block size fits %d rows of %lld keys, k=%d", n_rows,
                     (long long)ld, k);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255) != 0)
    return set_error(TF_E_INVAL,
                     "tf_indexer_topk_fused: a 256-byte aligned workspace of %zu bytes is needed, got %zu", need,
                     ws_bytes);
  return launch_indexer_topk_fused(p, make_view(p, keys), n_rows, row_stream, row_pos, q, w, n_heads, ld, k, blocks,
                                   n_valid, ws, (hipStream_t)stream);
}

// Candidate groups' workspace: the group scores (rows padded to whole quads), the
// rows' group counts, then the top-k's own.
static int64_t group_stride(int64_t ld, int32_t g) { return ((ld + g - 1) / g + 3) / 4 * 4; }

static size_t cand_ws(int32_t n_rows, int64_t ld, int32_t g, int32_t n_cand, size_t* topk_part) {
  const int64_t ldg = group_stride(ld, g);
  const size_t t = topk_ws_bytes(n_rows, ldg, n_cand);
  if (topk_part) *topk_part = t;
  if (t == (size_t)-1) return t;
  return (size_t)n_rows * ldg * 4 + ((size_t)n_rows * 4 + 15) / 16 * 16 + t;
}

extern "C" size_t tf_candidate_groups_workspace_bytes(int32_t n_rows, int64_t ld, int32_t group, int32_t n_cand) {
  if (n_rows <= 0 || ld <= 0 || group <= 0 || n_cand <= 0) return 0;
  return cand_ws(n_rows, ld, group, n_cand, nullptr);
}

extern "C" tf_status tf_candidate_groups(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid,
                                         int32_t group, int32_t n_cand, int32_t* cand, void* ws, size_t ws_bytes,
                                         void* stream) {
  clear_error();
  if (n_rows < 0) return set_error(TF_E_INVAL, "tf_candidate_groups: n_rows < 0");
  if (n_rows > 65535) return set_error(TF_E_RANGE, "tf_candidate_groups: n_rows=%d, at most 65535 a call", n_rows);
  if (ld < 1 || ld > (1LL << 24)) return set_error(TF_E_RANGE, "tf_candidate_groups: ld=%lld", (long long)ld);
  if (group < 1 || group > 64) return set_error(TF_E_RANGE, "tf_candidate_groups: group=%d, need 1..64", group);
  if (n_cand < 1 || n_cand > 2048)
    return set_error(TF_E_RANGE, "tf_candidate_groups: n_cand=%d, need 1..2048", n_cand);
  if (n_rows == 0) return TF_OK;
  if (!logits || !cand) return set_error(TF_E_INVAL, "tf_candidate_groups: logits and cand are required");
  size_t tpart = 0;
  const size_t need = cand_ws(n_rows, ld, group, n_cand, &tpart);
  if (need == (size_t)-1)
    return set_error(TF_E_UNSUPPORTED, "tf_candidate_groups: %lld groups with n_cand=%d exceed the blocked merge",
                     (long long)((ld + group - 1) / group), n_cand);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return set_error(TF_E_INVAL, "tf_candidate_groups: a 16-byte aligned workspace of %zu bytes is needed, got %zu",
                     need, ws_bytes);
  const hipStream_t st = (hipStream_t)stream;
  const int64_t ldg = group_stride(ld, group);
  float* scores = (float*)ws;
  int32_t* ngroups = (int32_t*)((char*)ws + (size_t)n_rows * ldg * 4);
  void* tws = tpart ? (char*)ngroups + ((size_t)n_rows * 4 + 15) / 16 * 16 : nullptr;
  tf_status s = launch_group_max(logits, ld, n_rows, n_valid, group, scores, ldg, ngroups, st);
  if (s != TF_OK) return s;
  return launch_topk(scores, ldg, n_rows, ngroups, n_cand, cand, tws, tpart, st);
}

extern "C" size_t tf_topk_in_candidates_workspace_bytes(int32_t n_rows, int64_t ld, int32_t k) {
  return tf_topk_workspace_bytes(n_rows, ld, k);
}

extern "C" tf_status tf_topk_in_candidates(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid,
                                           const int32_t* cand, int32_t n_cand, int32_t group, int32_t k,
                                           int32_t* blocks, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (n_rows < 0) return set_error(TF_E_INVAL, "tf_topk_in_candidates: n_rows < 0");
  if (k < 1 || k > 2048) return set_error(TF_E_RANGE, "tf_topk_in_candidates: k=%d, need 1..2048", k);
  if (ld < 1 || ld > (1LL << 24)) return set_error(TF_E_RANGE, "tf_topk_in_candidates: ld=%lld", (long long)ld);
  if (group < 1 || group > 64) return set_error(TF_E_RANGE, "tf_topk_in_candidates: group=%d, need 1..64", group);
  if (n_cand < 1) return set_error(TF_E_RANGE, "tf_topk_in_candidates: n_cand=%d, need >= 1", n_cand);
  if (n_rows == 0) return TF_OK;
  if (!logits || !cand || !blocks)
    return set_error(TF_E_INVAL, "tf_topk_in_candidates: logits, cand and blocks are required");
  const size_t need = topk_ws_bytes(n_rows, ld, k);
  if (need == (size_t)-1)
    return set_error(TF_E_UNSUPPORTED, "tf_topk_in_candidates: ld=%lld with k=%d exceeds the blocked merge",
                     (long long)ld, k);
  if (need > 0 && (!ws || ws_bytes < need))
    return set_error(TF_E_INVAL, "tf_topk_in_candidates: workspace of %zu bytes needed, got %zu", need, ws_bytes);
  return launch_topk(logits, ld, n_rows, n_valid, k, blocks, ws, ws_bytes, (hipStream_t)stream, cand, n_cand,
                     group);
}

extern "C" size_t tf_attn_workspace_bytes(int32_t n_rows, int32_t n_heads, int32_t k) {
  if (n_rows <= 0 || n_heads <= 0 || k <= 0) return 0;
  return attn_ws_bytes(n_rows, n_heads, k);
}

// Arguments of the sparse pass, checked before any launch (shared by its two entry points).
static tf_status check_sparse_attn(const char* fn, const tf_plan* p, const tf_kv_view& kv, int32_t n_rows,
                                   const int32_t* row_stream, const int32_t* row_pos, const void* q,
                                   int32_t n_heads, float softmax_scale, const int32_t* blocks, int32_t k,
                                   const float* out) {
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  if ((s = check_view(p, kv, "kv")) != TF_OK) return s;
  if (p->g.rope_dim != kRope) return set_error(TF_E_UNSUPPORTED, "%s: needs the 64-value rope plane", fn);
  if (n_rows < 0) return set_error(TF_E_INVAL, "%s: n_rows < 0", fn);
  if (n_heads < 1 || n_heads > 32) return set_error(TF_E_UNSUPPORTED, "%s: n_heads=%d, built for 1..32", fn, n_heads);
  if (k < 1 || k > 2048) return set_error(TF_E_RANGE, "%s: k=%d, need 1..2048", fn, k);
  if (!(softmax_scale == softmax_scale) || softmax_scale <= 0.f)
    return set_error(TF_E_INVAL, "%s: softmax_scale must be > 0", fn);
  if (n_rows == 0) return TF_OK;
  if (!row_stream || !row_pos || !q || !blocks || !out)
    return set_error(TF_E_INVAL, "%s: row_stream, row_pos, q, blocks and out are required", fn);
  if (!aligned16(q)) return set_error(TF_E_INVAL, "%s: q must be 16-byte aligned", fn);
  return TF_OK;
}

extern "C" tf_status tf_sparse_mla_attn(const tf_plan* p, tf_kv_view kv, int32_t n_rows,
                                        const int32_t* row_stream, const int32_t* row_pos,
                                        const void* q, int32_t n_heads, float softmax_scale,
                                        const int32_t* blocks, int32_t k, float* out, float* lse,
                                        void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  tf_status s = check_sparse_attn("tf_sparse_mla_attn", p, kv, n_rows, row_stream, row_pos, q, n_heads,
                                  softmax_scale, blocks, k, out);
  if (s != TF_OK || n_rows == 0) return s;
  const size_t need = attn_ws_bytes(n_rows, n_heads, k);
  if (need > 0 && (!ws || ws_bytes < need))
    return set_error(TF_E_INVAL, "tf_sparse_mla_attn: workspace of %zu bytes needed, got %zu", need, ws_bytes);
  return launch_attn(p, make_view(p, kv), n_rows, row_stream, row_pos, q, n_heads, softmax_scale, blocks,
                     k, out, lse, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" size_t tf_sparse_mla_attn_noalloc_max_bytes(void) { return attn_scratch_bytes(); }

extern "C" tf_status tf_sparse_mla_attn_noalloc(const tf_plan* p, tf_kv_view kv, int32_t n_rows,
                                                const int32_t* row_stream, const int32_t* row_pos,
                                                const void* q, int32_t n_heads, float softmax_scale,
                                                const int32_t* blocks, int32_t k, float* out, float* lse,
                                                void* stream) {
  clear_error();
  tf_status s = check_sparse_attn("tf_sparse_mla_attn_noalloc", p, kv, n_rows, row_stream, row_pos, q, n_heads,
                                  softmax_scale, blocks, k, out);
  if (s != TF_OK || n_rows == 0) return s;
  const size_t need = attn_ws_bytes(n_rows, n_heads, k);
  if (need > attn_scratch_bytes())
    return set_error(TF_E_RANGE,
                     "tf_sparse_mla_attn_noalloc: %d rows x %d heads x k=%d need %zu bytes of split partials, the "
                     "library's fixed scratch holds %zu; split the rows over calls or use tf_sparse_mla_attn",
                     n_rows, n_heads, k, need, attn_scratch_bytes());
  void* ws = nullptr;
  if (need > 0 && (s = attn_scratch(&ws)) != TF_OK) return s;
  return launch_attn(p, make_view(p, kv), n_rows, row_stream, row_pos, q, n_heads, softmax_scale, blocks,
                     k, out, lse, ws, need, (hipStream_t)stream);
}

extern "C" tf_status tf_dense_mla_attn(const tf_plan* p, tf_kv_view kv, int32_t n_rows,
                                       const int32_t* row_stream, const int32_t* row_pos,
                                       const void* q, int32_t n_heads, float softmax_scale,
                                       int32_t n_blocks, float* out, float* lse, void* ws,
                                       size_t ws_bytes, void* stream) {
  clear_error();
  tf_status s;
  if ((s = check_plan(p)) != TF_OK) return s;
  if ((s = check_view(p, kv, "kv")) != TF_OK) return s;
  if (p->g.rope_dim != kRope)
    return set_error(TF_E_UNSUPPORTED, "tf_dense_mla_attn: needs the 64-value rope plane");
  if (n_rows < 0) return set_error(TF_E_INVAL, "tf_dense_mla_attn: n_rows < 0");
  if (n_heads < 1 || n_heads > 32)
    return set_error(TF_E_UNSUPPORTED, "tf_dense_mla_attn: n_heads=%d, built for 1..32", n_heads);
  if (n_blocks < 1 || n_blocks > 2048)
    return set_error(TF_E_RANGE,
                     "tf_dense_mla_attn: n_blocks=%d, need 1..2048 (8,192 tokens); longer contexts go through "
                     "tf_indexer_logits, tf_topk_blocks and tf_sparse_mla_attn",
                     n_blocks);
  if (!(softmax_scale == softmax_scale) || softmax_scale <= 0.f)
    return set_error(TF_E_INVAL, "tf_dense_mla_attn: softmax_scale must be > 0");
  if (n_rows == 0) return TF_OK;
  if (!row_stream || !row_pos || !q || !out)
    return set_error(TF_E_INVAL, "tf_dense_mla_attn: row_stream, row_pos, q and out are required");
  if (!aligned16(q)) return set_error(TF_E_INVAL, "tf_dense_mla_attn: q must be 16-byte aligned");
  const size_t need = attn_ws_bytes(n_rows, n_heads, n_blocks);
  if (need > 0 && (!ws || ws_bytes < need))
    return set_error(TF_E_INVAL, "tf_dense_mla_attn: workspace of %zu bytes needed, got %zu", need, ws_bytes);
  return launch_attn(p, make_view(p, kv), n_rows, row_stream, row_pos, q, n_heads, softmax_scale, nullptr,
                     n_blocks, out, lse, ws, ws_bytes, (hipStream_t)stream);
}
