// Two-level candidate selection [CPM, section 1: one layer publishes candidate masks
// that the later low-ratio layers consume; section 2.3: its block pooling over 8-key
// groups and top-2,048 groups, and the consumers' masking of non-candidates before
// their top-k].
//
//   * group_max_kernel: each visible group of g consecutive keys scores the largest
//     of its visible logits (the last group may be partial); the top-n_cand groups
//     then come from the top-k kernels, ties to the lower group.
//   * mask_kernel: a consumer row's keys outside its candidate groups become -inf in
//     place (the pages' masked_fill_), before the top-k kernels take its top-k.
//
// Both stream a row once: group_max reads it (one group per thread, float4 loads when
// a group is whole quads) and writes a g-th of it; the mask writes only the
// non-candidate quads, testing a candidate bitmap built in LDS from the row's list.
#include "common.h"

namespace tf {

__global__ __launch_bounds__(256) void group_max_kernel(const float* logits, int64_t ld, int32_t n_rows,
                                                        const int32_t* n_valid, int32_t g, float* scores,
                                                        int64_t ldg, int32_t* n_groups, bool quads) {
  const int r = blockIdx.y;
  int64_t nv = n_valid ? n_valid[r] : ld;
  nv = nv < 0 ? 0 : (nv > ld ? ld : nv);
  const int64_t ng = (nv + g - 1) / g;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j == 0 && n_groups) n_groups[r] = (int32_t)ng;
  if (j >= ng) return;
  const float* row = logits + r * ld;
  const int64_t k0 = j * g;
  const int64_t k1 = k0 + g < nv ? k0 + g : nv;
  float m = -__builtin_inff();
  if (quads && k1 - k0 == g) {   // whole group of whole quads
    for (int64_t k = k0; k < k1; k += 4) {
      const float4 v = *(const float4*)(row + k);
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(v.x, v.y), __builtin_fmaxf(v.z, v.w)));
    }
  } else {
    for (int64_t k = k0; k < k1; ++k) m = __builtin_fmaxf(m, row[k]);
  }
  scores[r * ldg + j] = m;
}

constexpr int kMaskBitmapWords = 8192;   // candidate bitmap: up to 262,144 groups

__global__ __launch_bounds__(256) void mask_kernel(float* logits, int64_t ld, const int32_t* n_valid,
                                                   const int32_t* cand, int32_t n_cand, int32_t g, bool quads) {
  __shared__ uint32_t bits[kMaskBitmapWords];
  const int r = blockIdx.x;
  int64_t nv = n_valid ? n_valid[r] : ld;
  nv = nv < 0 ? 0 : (nv > ld ? ld : nv);
  const int64_t ng = (nv + g - 1) / g;
  const int words = (int)((ng + 31) / 32);
  for (int i = threadIdx.x; i < words; i += 256) bits[i] = 0u;
  __syncthreads();
  const int32_t* c = cand + (int64_t)r * n_cand;
  for (int i = threadIdx.x; i < n_cand; i += 256) {
    const int32_t x = c[i];
    if (x >= 0 && x < ng) atomicOr(&bits[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  float* row = logits + r * ld;
  const float ninf = -__builtin_inff();
  if (quads) {   // g a multiple of 4: a quad lies in one group
    const int64_t nq = nv / 4;
    for (int64_t q = threadIdx.x; q < nq; q += 256) {
      const int64_t grp = 4 * q / g;
      if (!((bits[grp >> 5] >> (grp & 31)) & 1u)) *(float4*)(row + 4 * q) = make_float4(ninf, ninf, ninf, ninf);
    }
    for (int64_t k = 4 * nq + threadIdx.x; k < nv; k += 256) {
      const int64_t grp = k / g;
      if (!((bits[grp >> 5] >> (grp & 31)) & 1u)) row[k] = ninf;
    }
  } else {
    for (int64_t k = threadIdx.x; k < nv; k += 256) {
      const int64_t grp = k / g;
      if (!((bits[grp >> 5] >> (grp & 31)) & 1u)) row[k] = ninf;
    }
  }
}

int64_t cand_max_groups() { return (int64_t)kMaskBitmapWords * 32; }

tf_status launch_group_max(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid, int32_t g,
                           float* scores, int64_t ldg, int32_t* n_groups, hipStream_t st) {
  const bool quads = g % 4 == 0 && ld % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  const unsigned gx = (unsigned)((ldg + 255) / 256);
  hipLaunchKernelGGL(group_max_kernel, dim3(gx, n_rows), dim3(256), 0, st, logits, ld, n_rows, n_valid, g, scores,
                     ldg, n_groups, quads);
  return launch_status("tf_candidate_groups");
}

tf_status launch_mask(float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid, const int32_t* cand,
                      int32_t n_cand, int32_t g, hipStream_t st) {
  const bool quads = g % 4 == 0 && ld % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  hipLaunchKernelGGL(mask_kernel, dim3(n_rows), dim3(256), 0, st, logits, ld, n_valid, cand, n_cand, g, quads);
  return launch_status("tf_topk_in_candidates");
}

}  // namespace tf
