// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tf.h"

namespace tf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPageRows = 512;
constexpr int kPoolRatio = 4;
constexpr int kKeysPerPage = kPageRows / kPoolRatio;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kRow = kLatent + kRope;

// A view of one cache of the pool, flattened for kernels.
struct DevView {
  char* pool;
  const int32_t* pt;
  int32_t pt_stride;
  int32_t n_streams;
  int32_t n_pages;
  int64_t page_bytes;
  int64_t cache_off;  // cache * cache_block_bytes
};

// Pool page of stream b's page index i, or -1 when the table cannot name one.
__device__ __forceinline__ int page_of(const DevView& v, int b, int i) {
  if (i < 0 || i >= v.pt_stride || b < 0 || b >= v.n_streams) return -1;
  int p = v.pt ? v.pt[(int64_t)b * v.pt_stride + i] : b * v.pt_stride + i;
  return (p >= 0 && p < v.n_pages) ? p : -1;
}

__device__ __forceinline__ char* cache_block(const DevView& v, int page) {
  return v.pool + (int64_t)page * v.page_bytes + v.cache_off;
}

// ---- host-side helpers (abi.cpp) -------------------------------------------------
tf_status set_error(tf_status s, const char* fmt, ...);
void clear_error();
DevView make_view(const tf_plan* p, const tf_kv_view& v);
tf_status check_plan(const tf_plan* p);
tf_status check_view(const tf_plan* p, const tf_kv_view& v, const char* name);
tf_status launch_status(const char* what);

// ---- launchers (one per translation unit) -----------------------------------------
tf_status launch_latent_write(const tf_plan* p, const DevView& v, int32_t n_rows,
                              const int32_t* row_stream, const int32_t* row_pos,
                              const void* latent, const float* row_scale, const void* rope,
                              int32_t n_pkeys, const int32_t* pkey_stream, const int32_t* pkey_idx,
                              const void* pkeys, hipStream_t st, bool quantize);
tf_status launch_snapshot(const tf_plan* p, const tf_kv_view& src, const tf_kv_view& dst,
                          int32_t n_streams, const int32_t* src_stream, const int32_t* dst_stream,
                          int64_t at, hipStream_t st);
// Scores keys [key0, kend) into logits[row * ld + (key - key0)]; n_c is clipped to
// ncap (the whole call: key0 = 0, kend = ncap = ld). `window`: one key block of a
// key-blocked call (its own kernel instance, same code).
tf_status launch_indexer(const tf_plan* p, const DevView& v, int32_t n_rows,
                         const int32_t* row_stream, const int32_t* row_pos, const void* q,
                         const float* w, int32_t n_heads, float* logits, int64_t ld,
                         int32_t* n_valid, hipStream_t st, int64_t key0, int64_t kend, int64_t ncap,
                         bool window);
// fused indexer + top-k (indexer.hip): sampled threshold, filtered scoring, selection
size_t indexer_topk_fused_ws_bytes(int32_t n_heads, int32_t n_rows, int64_t ld, int32_t k);
tf_status launch_indexer_topk_fused(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                                    const int32_t* row_pos, const void* q, const float* w, int32_t n_heads,
                                    int64_t ld, int32_t k, int32_t* blocks, int32_t* n_valid, void* ws,
                                    hipStream_t st);
size_t topk_ws_bytes(int32_t n_rows, int64_t ld, int32_t k);
// cand (nullable): keys outside the row's candidate groups of `group` keys read as -inf
tf_status launch_topk(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid,
                      int32_t k, int32_t* blocks, void* ws, size_t ws_bytes, hipStream_t st,
                      const int32_t* cand = nullptr, int32_t n_cand = 0, int32_t group = 1);
// key-blocked top-k: stage 1 of key block b (logits_blk is [n_rows][B]), then the merge
size_t topk_cand_bytes(int32_t n_rows, int32_t nb, int32_t k);
tf_status launch_topk_block(const float* logits_blk, int32_t B, int32_t b, int32_t nb, int64_t ncap,
                            int32_t n_rows, const int32_t* n_valid, int32_t k, void* cand, hipStream_t st);
tf_status launch_topk_merge(int32_t B, int32_t nb, int64_t ncap, int32_t n_rows, const int32_t* n_valid,
                            int32_t k, int32_t* blocks, void* cand, hipStream_t st);
// two-level candidate selection (candidates.hip)
tf_status launch_group_max(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid, int32_t g,
                           float* scores, int64_t ldg, int32_t* n_groups, hipStream_t st);
size_t attn_ws_bytes(int32_t n_rows, int32_t n_heads, int32_t k);
// the fixed device scratch of the allocation-free sparse pass (attention.hip): its size,
// and its address on the current device (looked up once per device)
size_t attn_scratch_bytes();
tf_status attn_scratch(void** ptr);
// blocks == nullptr runs the dense pass over the first k pooled blocks
tf_status launch_attn(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                      const int32_t* row_pos, const void* q, int32_t n_heads, float scale,
                      const int32_t* blocks, int32_t k, float* out, float* lse, void* ws,
                      size_t ws_bytes, hipStream_t st);

}  // namespace tf
