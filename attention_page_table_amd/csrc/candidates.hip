// Two-level candidate selection [CPM, section 1: one layer publishes candidate masks
// that the later low-ratio layers consume; section 2.3: its block pooling over 8-key
// groups and top-2,048 groups, and the consumers' masking of non-candidates before
// their top-k].
//
//   * group_max_kernel: each visible group of g consecutive keys scores the largest
//     of its visible logits (the last group may be partial); the top-n_cand groups
//     then come from the top-k kernels, ties to the lower group. It streams a row
//     once (one group per thread, float4 loads when a group is whole quads) and
//     writes a g-th of it.
//   * The consumer's masking (the pages' masked_fill_ of non-candidates) is folded
//     into the top-k kernels' loads (their masked instances, topk.hip): a key
//     outside the row's candidate groups reads as -inf, and the logits are not
//     written.
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

tf_status launch_group_max(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid, int32_t g,
                           float* scores, int64_t ldg, int32_t* n_groups, hipStream_t st) {
  const bool quads = g % 4 == 0 && ld % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  const unsigned gx = (unsigned)((ldg + 255) / 256);
  hipLaunchKernelGGL(group_max_kernel, dim3(gx, n_rows), dim3(256), 0, st, logits, ld, n_rows, n_valid, g, scores,
                     ldg, n_groups, quads);
  return launch_status("tf_candidate_groups");
}

}  // namespace tf
