// Top-k pooled blocks per row: the k largest logits among a row's n_valid,
// ties to the lower index, -0 == +0, written ascending and padded with -1.
// [CPM, sections 1 and 2.3]: per-row (ragged) top-k; long rows are cut into key
// blocks whose top-k candidates are merged, which is exact:
// topk(union) == topk(union of per-block topk).
//
// Design: logits become order-preserving 32-bit keys in LDS; an MSB-first radix
// select (four 8-bit digit histograms with LDS atomics) finds the k-th largest
// key T and how many keys equal to T are taken; an ordered compaction (each
// thread owns a contiguous index range; two block scans) then writes the
// selected indices in ascending order, taking the keys equal to T lowest index
// first. No sort is needed because the output order is by index.
#include "common.h"

namespace tf {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the block; `total` receives the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t s = wsum[w];
    base += w < wid ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

struct SelShared {
  uint32_t hist[256];
  uint32_t wsum[16];
  uint32_t bin, rem;
};

// Finds T = the k-th largest of keys[0, n) (n > k >= 1) and rem = how many keys
// equal to T belong to the top k.
template <int NT>
__device__ void radix_select(const uint32_t* keys, int n, int k, SelShared& sh, uint32_t& T, uint32_t& rem) {
  uint32_t prefix = 0, mask = 0, r = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix sums over bins: thread t looks at bin 255 - t
    uint32_t c = 0;
    if (threadIdx.x < 256) c = sh.hist[255 - threadIdx.x];
    uint32_t tot;
    const uint32_t above = block_exclusive_scan<NT>(threadIdx.x < 256 ? c : 0u, sh.wsum, tot);
    if (threadIdx.x < 256 && above < r && r <= above + c) {
      sh.bin = 255 - threadIdx.x;
      sh.rem = r - above;
    }
    __syncthreads();
    prefix |= sh.bin << shift;
    mask |= 0xFFu << shift;
    r = sh.rem;
    __syncthreads();
  }
  T = prefix;
  rem = r;
}

// Ordered compaction: emit(pos, i) for every selected i in ascending order.
template <int NT, typename Emit>
__device__ void ordered_select(const uint32_t* keys, int n, uint32_t T, uint32_t rem, SelShared& sh, Emit emit) {
  const int per = (n + NT - 1) / NT;
  const int i0 = threadIdx.x * per;
  const int i1 = i0 + per < n ? i0 + per : n;
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan<NT>(eq, sh.wsum, tot);
  const uint32_t take_eq = eq_before >= rem ? 0u : (rem - eq_before < eq ? rem - eq_before : eq);
  const uint32_t pos0 = block_exclusive_scan<NT>(gt + take_eq, sh.wsum, tot);
  uint32_t pos = pos0, took = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    if (key > T || (key == T && took < take_eq)) {
      took += key == T;
      emit(pos++, i);
    }
  }
}

struct TopkArgs {
  const float* logits;
  int64_t ld;
  int32_t n_rows;
  const int32_t* n_valid;
  int32_t k;
  int32_t* blocks;
  int32_t blk;        // key block length (blocked mode)
  int32_t nblk;       // key blocks per row (blocked mode)
  uint32_t* ws_key;   // [n_rows][nblk][k]
  int32_t* ws_idx;    // [n_rows][nblk][k]
};

__device__ __forceinline__ int row_valid(const TopkArgs& a, int r) {
  int nv = a.n_valid ? a.n_valid[r] : (int)a.ld;
  if (nv < 0) nv = 0;
  if (nv > a.ld) nv = (int)a.ld;
  return nv;
}

// One workgroup per row; the row fits in LDS.
template <int NT>
__global__ __launch_bounds__(NT) void topk_single_kernel(TopkArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  const int n = row_valid(a, r);
  int32_t* out = a.blocks + (int64_t)r * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = a.logits + (int64_t)r * a.ld;
  for (int i = threadIdx.x; i < n; i += NT) smem[i] = order_key(row[i]);
  __syncthreads();
  uint32_t T, rem;
  radix_select<NT>(smem, n, a.k, sh, T, rem);
  ordered_select<NT>(smem, n, T, rem, sh, [&](uint32_t pos, int i) {
    if (pos < (uint32_t)a.k) out[pos] = i;
  });
}

// Blocked mode, stage 1: top-k candidates (key, index) of one key block of one row.
template <int NT>
__global__ __launch_bounds__(NT) void topk_stage1_kernel(TopkArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ SelShared sh;
  const int r = blockIdx.y;
  const int bb = blockIdx.x;
  const int nv = row_valid(a, r);
  const int i0 = bb * a.blk;
  int n = nv - i0;
  if (n > a.blk) n = a.blk;
  if (n < 0) n = 0;
  uint32_t* ck = a.ws_key + ((int64_t)r * a.nblk + bb) * a.k;
  int32_t* ci = a.ws_idx + ((int64_t)r * a.nblk + bb) * a.k;
  if (nv <= a.k) return;  // stage 2 writes the row directly
  const float* row = a.logits + (int64_t)r * a.ld + i0;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) {
      ck[i] = i < n ? order_key(row[i]) : 0u;
      ci[i] = i < n ? i0 + i : -1;
    }
    return;
  }
  for (int i = threadIdx.x; i < n; i += NT) smem[i] = order_key(row[i]);
  __syncthreads();
  uint32_t T, rem;
  radix_select<NT>(smem, n, a.k, sh, T, rem);
  ordered_select<NT>(smem, n, T, rem, sh, [&](uint32_t pos, int i) {
    if (pos < (uint32_t)a.k) {
      ck[pos] = smem[i];
      ci[pos] = i0 + i;
    }
  });
}

// Blocked mode, stage 2: merge the candidates of all key blocks of one row.
template <int NT>
__global__ __launch_bounds__(NT) void topk_stage2_kernel(TopkArgs a) {
  extern __shared__ uint32_t smem[];
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  const int nv = row_valid(a, r);
  int32_t* out = a.blocks + (int64_t)r * a.k;
  if (nv <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < nv ? i : -1;
    return;
  }
  const int nb_used = (nv + a.blk - 1) / a.blk;
  const int n = nb_used * a.k;
  uint32_t* keys = smem;
  int32_t* idx = (int32_t*)(smem + a.nblk * a.k);
  const uint32_t* ck = a.ws_key + (int64_t)r * a.nblk * a.k;
  const int32_t* ci = a.ws_idx + (int64_t)r * a.nblk * a.k;
  for (int i = threadIdx.x; i < n; i += NT) {
    keys[i] = ck[i];
    idx[i] = ci[i];
  }
  __syncthreads();
  uint32_t T, rem;
  radix_select<NT>(keys, n, a.k, sh, T, rem);
  ordered_select<NT>(keys, n, T, rem, sh, [&](uint32_t pos, int i) {
    if (pos < (uint32_t)a.k) out[pos] = idx[i];
  });
}

// Key-block length for the blocked mode, or 0 for one workgroup per row.
static int pick_block(int32_t n_rows, int64_t ld, int32_t k) {
  if (ld <= 4096 || (ld <= 32768 && n_rows >= 512)) return 0;
  int64_t B = 2048;
  while (B * B < ld * k && B < 32768) B *= 2;
  while (((ld + B - 1) / B) * k > 16384 && B < 32768) B *= 2;
  if (((ld + B - 1) / B) * k > 16384) return -1;
  return (int)B;
}

size_t topk_ws_bytes(int32_t n_rows, int64_t ld, int32_t k) {
  const int B = pick_block(n_rows, ld, k);
  if (B < 0) return (size_t)-1;
  if (B == 0) return 0;
  const int64_t nb = (ld + B - 1) / B;
  return (size_t)n_rows * nb * k * 8;
}

tf_status launch_topk(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid, int32_t k,
                      int32_t* blocks, void* ws, size_t ws_bytes, hipStream_t st) {
  TopkArgs a;
  a.logits = logits;
  a.ld = ld;
  a.n_rows = n_rows;
  a.n_valid = n_valid;
  a.k = k;
  a.blocks = blocks;
  const int B = pick_block(n_rows, ld, k);
  if (B == 0) {
    const size_t lds = (size_t)ld * 4;
    a.blk = (int)ld;
    a.nblk = 1;
    a.ws_key = nullptr;
    a.ws_idx = nullptr;
    hipFuncSetAttribute((const void*)topk_single_kernel<1024>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(topk_single_kernel<1024>, dim3(n_rows), dim3(1024), lds, st, a);
    return launch_status("tf_topk_blocks");
  }
  const int64_t nb = (ld + B - 1) / B;
  a.blk = B;
  a.nblk = (int32_t)nb;
  a.ws_key = (uint32_t*)ws;
  a.ws_idx = (int32_t*)((char*)ws + (size_t)n_rows * nb * k * 4);
  if (n_rows > 65535) return set_error(TF_E_RANGE, "tf_topk_blocks: at most 65535 rows in blocked mode");
  hipFuncSetAttribute((const void*)topk_stage1_kernel<256>, hipFuncAttributeMaxDynamicSharedMemorySize, B * 4);
  hipLaunchKernelGGL(topk_stage1_kernel<256>, dim3((unsigned)nb, n_rows), dim3(256), (size_t)B * 4, st, a);
  tf_status s = launch_status("tf_topk_blocks");
  if (s != TF_OK) return s;
  hipFuncSetAttribute((const void*)topk_stage2_kernel<1024>, hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)(nb * k * 8));
  hipLaunchKernelGGL(topk_stage2_kernel<1024>, dim3(n_rows), dim3(1024), (size_t)nb * k * 8, st, a);
  return launch_status("tf_topk_blocks");
}

}  // namespace tf
