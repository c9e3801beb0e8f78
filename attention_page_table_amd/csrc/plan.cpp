// Host side: page layout, page budget and the adaptive prefill chunk.
//
// Layout of a page [#1142, "GLM declares a kv_pool.Layout"; #1313, "Proposal"
// step 1 item 3]: one page id spans every cache; inside a cache's block come the
// latent rows, the fp8 rows' fp32 scales after them, the rope rows, then the
// page's pooled keys (one per 4 rows).
// Budget [#1313, "Why" and "Proposal" step 1]: see tf_plan_policy in tf.h.
// Chunk [CPM, section 2.1]: clamp(round_down_to_256(2.0e8 / L), 256, 2048).
#include <limits.h>
#include <string.h>

#include "common.h"

namespace tf {
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace tf

using namespace tf;

extern "C" tf_status tf_kv_pool_plan(const tf_geom* g, const tf_budget* b, tf_plan* out) {
  clear_error();
  if (!g || !out) return set_error(TF_E_INVAL, "tf_kv_pool_plan: geom and out must not be NULL");
  if (g->n_caches < 1 || g->n_caches > 64)
    return set_error(TF_E_RANGE, "tf_kv_pool_plan: n_caches=%d, need 1..64", g->n_caches);
  if (g->page_rows != kPageRows)
    return set_error(TF_E_UNSUPPORTED, "tf_kv_pool_plan: page_rows=%d, only 512-row pages are built",
                     g->page_rows);
  if (g->latent_dim != kLatent)
    return set_error(TF_E_UNSUPPORTED, "tf_kv_pool_plan: latent_dim=%d, only 512 is built",
                     g->latent_dim);
  if (g->rope_dim != 0 && g->rope_dim != kRope)
    return set_error(TF_E_UNSUPPORTED, "tf_kv_pool_plan: rope_dim=%d, need 64 (or 0 for accounting)",
                     g->rope_dim);
  if (g->pool_ratio != kPoolRatio)
    return set_error(TF_E_UNSUPPORTED, "tf_kv_pool_plan: pool_ratio=%d, only 4 is built", g->pool_ratio);
  if (g->index_dim != 64 && g->index_dim != 128)
    return set_error(TF_E_UNSUPPORTED, "tf_kv_pool_plan: index_dim=%d, need 64 or 128", g->index_dim);
  if (g->lat_fmt != TF_LAT_BF16 && g->lat_fmt != TF_LAT_FP8E4M3_ROWSCALE)
    return set_error(TF_E_INVAL, "tf_kv_pool_plan: lat_fmt=%d is not a tf_lat_fmt", g->lat_fmt);

  tf_plan p;
  memset(&p, 0, sizeof(p));
  p.g = *g;
  const bool fp8 = g->lat_fmt == TF_LAT_FP8E4M3_ROWSCALE;
  p.lat_row_bytes = fp8 ? g->latent_dim : 2 * g->latent_dim;
  p.rope_row_bytes = 2 * g->rope_dim;
  p.pkey_row_bytes = 2 * g->index_dim;
  p.keys_per_page = g->page_rows / g->pool_ratio;
  p.off_latent = 0;
  p.off_scale = p.off_latent + (int64_t)g->page_rows * p.lat_row_bytes;
  p.off_rope = p.off_scale + (fp8 ? 4LL * g->page_rows : 0);
  p.off_pkey = p.off_rope + (int64_t)g->page_rows * p.rope_row_bytes;
  p.cache_block_bytes = p.off_pkey + p.keys_per_page * p.pkey_row_bytes;
  p.page_bytes = p.cache_block_bytes * g->n_caches;
  const int64_t scale_b = fp8 ? 4 : 0;
  p.bytes_per_token_pages =
      g->n_caches * (p.lat_row_bytes + scale_b + p.pkey_row_bytes / g->pool_ratio);
  p.bytes_per_token = p.bytes_per_token_pages + g->n_caches * p.rope_row_bytes;

  if (b) {
    if (b->lanes < 1) return set_error(TF_E_INVAL, "tf_kv_pool_plan: lanes=%d, need >= 1", b->lanes);
    if (b->room_bytes < 0 || b->window_tokens < 1 || b->lookahead_rows < 0 ||
        b->fixed_bytes_per_stream < 0 || b->cache_cap_bytes < 0)
      return set_error(TF_E_INVAL, "tf_kv_pool_plan: budget fields must be >= 0 (window >= 1)");
    if (b->policy != TF_PLAN_ONE_WINDOW_FIRST && b->policy != TF_PLAN_WINDOWS_FIRST)
      return set_error(TF_E_INVAL, "tf_kv_pool_plan: policy=%d is not a tf_plan_policy", b->policy);
    const int64_t P = p.page_bytes;
    const int64_t wp = cdiv(b->window_tokens + b->lookahead_rows, g->page_rows);
    const int64_t base_pages = wp + (b->lanes - 1);
    int64_t n = 1, stream_pages = base_pages;
    if (b->policy == TF_PLAN_WINDOWS_FIRST) {
      if (b->room_bytes >= wp * P) {
        const int64_t more = (b->room_bytes - wp * P) / (wp * P + b->fixed_bytes_per_stream);
        n = 1 + more < b->lanes ? 1 + more : b->lanes;
      }
      if (n < 1) n = 1;
      stream_pages = n * wp > base_pages ? n * wp : base_pages;
    }
    const int64_t fixed = (int64_t)b->lanes * b->fixed_bytes_per_stream;
    const int64_t need = stream_pages * P + fixed;
    if (b->room_bytes < need)
      return set_error(TF_E_NOMEM,
                       "tf_kv_pool_plan: %d streams at a %lld-token window need %lld bytes "
                       "(%lld pages + %lld fixed) and the room is %lld: lower the window or the lanes",
                       b->lanes, (long long)b->window_tokens, (long long)need,
                       (long long)stream_pages, (long long)fixed, (long long)b->room_bytes);
    const int64_t left = b->room_bytes - need;
    const int64_t cache = left < b->cache_cap_bytes ? left : b->cache_cap_bytes;
    p.window_pages = wp;
    p.n_windows = n;
    p.stream_pages = stream_pages;
    p.total_pages = stream_pages + (left - cache) / P;
    p.cache_bytes = cache;
    p.fixed_bytes = fixed;
  }
  *out = p;
  return TF_OK;
}

extern "C" int64_t tf_prefill_chunk(int64_t history, int64_t remaining) {
  const int64_t kMax = 2048, kMin = 256, kPage = 256;
  const double kBudget = 2.0e8;
  if (remaining <= 0) return 0;
  int64_t c = kMax;
  if (history > 0) {
    const int64_t raw = (int64_t)(kBudget / (double)history);  // floor for positive values
    c = (raw / kPage) * kPage;
    if (c < kMin) c = kMin;
    if (c > kMax) c = kMax;
  }
  return c < remaining ? c : remaining;
}
