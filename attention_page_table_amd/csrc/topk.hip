// Top-k pooled blocks per row: the k largest logits among a row's n_valid,
// ties to the lower index, -0 == +0, written ascending and padded with -1.
// [CPM, sections 1 and 2.3]: per-row (ragged) top-k; long rows are cut into key
// blocks whose top-k candidates are merged, which is exact:
// topk(union) == topk(union of per-block topk).
//
// Design: a workgroup of 1,024 threads owns a segment of up to 32,768 keys held in
// registers (each thread a contiguous run of E keys, loaded with 16-byte loads).
// Logits become order-preserving 32-bit keys. A most-significant-digit radix
// select in three passes (11 + 11 + 10 bits, 2,048-bin LDS histograms) finds the
// k-th largest key T and how many keys equal to T belong to the top k; an ordered
// compaction (two block scans over the threads' runs) then writes the selected
// indices ascending, taking keys equal to T lowest index first. No sort is needed
// because the output order is by index. Long rows: stage 1 selects per key block,
// stage 2 merges the blocks' candidates (kept in index order).
#include "common.h"

namespace tf {

constexpr int kNT = 1024;  // threads per workgroup
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelShared {
  uint32_t hist[kBins];
  uint32_t wsum[kNT / 64];
  uint32_t bin, rem;
};

// Exclusive scan over the workgroup; `total` receives the sum.
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
  for (int w = 0; w < kNT / 64; ++w) {
    const uint32_t s = wsum[w];
    base += w < wid ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// T = the k-th largest of the n > k valid keys (invalid slots hold 0, below every
// valid key), rem = how many keys equal to T belong to the top k.
template <int E>
__device__ void radix_select(const uint32_t (&key)[E], int k, SelShared& sh, uint32_t& T, uint32_t& rem) {
  uint32_t prefix = 0, mask = 0, r = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = threadIdx.x; i < kBins; i += kNT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0u && (key[e] & mask) == prefix) atomicAdd(&sh.hist[(key[e] >> shift) & dmask], 1u);
    __syncthreads();
    // suffix sums: thread t owns bins 2047 - 2t and 2046 - 2t (descending)
    const uint32_t c0 = sh.hist[kBins - 1 - 2 * threadIdx.x], c1 = sh.hist[kBins - 2 - 2 * threadIdx.x];
    uint32_t tot;
    const uint32_t above = block_exclusive_scan(c0 + c1, sh.wsum, tot);
    if (above < r && r <= above + c0) {
      sh.bin = kBins - 1 - 2 * threadIdx.x;
      sh.rem = r - above;
    } else if (above + c0 < r && r <= above + c0 + c1) {
      sh.bin = kBins - 2 - 2 * threadIdx.x;
      sh.rem = r - above - c0;
    }
    __syncthreads();
    prefix |= sh.bin << shift;
    mask |= dmask << shift;
    r = sh.rem;
    __syncthreads();
  }
  T = prefix;
  rem = r;
}

// Ordered compaction of a thread's contiguous run: emit(pos, e) for each selected key.
template <int E, typename Emit>
__device__ void ordered_select(const uint32_t (&key)[E], uint32_t T, uint32_t rem, SelShared& sh, Emit emit) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gt += key[e] > T;
    eq += key[e] == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(eq, sh.wsum, tot);
  const uint32_t take_eq = eq_before >= rem ? 0u : (rem - eq_before < eq ? rem - eq_before : eq);
  uint32_t pos = block_exclusive_scan(gt + take_eq, sh.wsum, tot);
  uint32_t took = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool eqT = key[e] == T;
    if (key[e] > T || (eqT && took < take_eq)) {
      took += eqT;
      emit(pos++, e);
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

// Keys of [0, n) of a float row, thread t taking the run [t*E, t*E + E).
template <int E>
__device__ __forceinline__ void load_keys(const float* row, int n, uint32_t (&key)[E]) {
  const int base = threadIdx.x * E;
  if ((E % 4) == 0 && ((uintptr_t)row & 15) == 0 && base + E <= n) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *(const float4*)(row + base + e);
      key[e] = order_key(v.x);
      key[e + 1] = order_key(v.y);
      key[e + 2] = order_key(v.z);
      key[e + 3] = order_key(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = base + e < n ? order_key(row[base + e]) : 0u;
  }
}

// One workgroup per row.
template <int E>
__global__ __launch_bounds__(kNT) void topk_row_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  const int n = row_valid(a, r);
  int32_t* out = a.blocks + (int64_t)r * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kNT) out[i] = i < n ? i : -1;
    return;
  }
  uint32_t key[E];
  load_keys<E>(a.logits + (int64_t)r * a.ld, n, key);
  uint32_t T, rem;
  radix_select<E>(key, a.k, sh, T, rem);
  const int base = threadIdx.x * E;
  ordered_select<E>(key, T, rem, sh, [&](uint32_t pos, int e) {
    if (pos < (uint32_t)a.k) out[pos] = base + e;
  });
}

// Blocked mode, stage 1: top-k candidates (key, index) of one key block of one row.
template <int E>
__global__ __launch_bounds__(kNT) void topk_stage1_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int r = blockIdx.y;
  const int bb = blockIdx.x;
  const int nv = row_valid(a, r);
  if (nv <= a.k) return;  // stage 2 writes the row directly
  const int i0 = bb * a.blk;
  int n = nv - i0;
  if (n > a.blk) n = a.blk;
  if (n < 0) n = 0;
  uint32_t* ck = a.ws_key + ((int64_t)r * a.nblk + bb) * a.k;
  int32_t* ci = a.ws_idx + ((int64_t)r * a.nblk + bb) * a.k;
  const float* row = a.logits + (int64_t)r * a.ld + i0;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kNT) {
      ck[i] = i < n ? order_key(row[i]) : 0u;
      ci[i] = i < n ? i0 + i : -1;
    }
    return;
  }
  uint32_t key[E];
  load_keys<E>(row, n, key);
  uint32_t T, rem;
  radix_select<E>(key, a.k, sh, T, rem);
  const int base = threadIdx.x * E;
  ordered_select<E>(key, T, rem, sh, [&](uint32_t pos, int e) {
    if (pos < (uint32_t)a.k) {
      ck[pos] = key[e];
      ci[pos] = i0 + base + e;
    }
  });
}

// Blocked mode, stage 2: merge the candidates of all key blocks of one row (they
// are in ascending index order, padding last in each block with key 0).
template <int E>
__global__ __launch_bounds__(kNT) void topk_stage2_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  const int nv = row_valid(a, r);
  int32_t* out = a.blocks + (int64_t)r * a.k;
  if (nv <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kNT) out[i] = i < nv ? i : -1;
    return;
  }
  const int nb_used = (nv + a.blk - 1) / a.blk;
  const int n = nb_used * a.k;
  const uint32_t* ck = a.ws_key + (int64_t)r * a.nblk * a.k;
  const int32_t* ci = a.ws_idx + (int64_t)r * a.nblk * a.k;
  uint32_t key[E];
  int32_t idx[E];
  const int base = threadIdx.x * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    key[e] = base + e < n ? ck[base + e] : 0u;
    idx[e] = base + e < n ? ci[base + e] : -1;
  }
  uint32_t T, rem;
  radix_select<E>(key, a.k, sh, T, rem);
  ordered_select<E>(key, T, rem, sh, [&](uint32_t pos, int e) {
    if (pos < (uint32_t)a.k) out[pos] = idx[e];
  });
}

// Key-block length for the blocked mode, or 0 for one workgroup per row.
static int pick_block(int32_t n_rows, int64_t ld, int32_t k) {
  if (ld <= 4096 || (ld <= 32768 && n_rows >= 128)) return 0;
  // few long rows: blocks of 2,048 .. 32,768 keys so that about 128 workgroups run,
  // with the merged candidates (blocks x k) at most 32,768
  int64_t B = 2048;
  while (B < 32768 && n_rows * ((ld + B - 1) / B) > 128) B *= 2;
  while (B < 32768 && ((ld + B - 1) / B) * k > 32768) B *= 2;
  if (((ld + B - 1) / B) * k > 32768) return -1;
  return (int)B;
}

size_t topk_ws_bytes(int32_t n_rows, int64_t ld, int32_t k) {
  const int B = pick_block(n_rows, ld, k);
  if (B < 0) return (size_t)-1;
  if (B == 0) return 0;
  const int64_t nb = (ld + B - 1) / B;
  return (size_t)n_rows * nb * k * 8;
}

template <int E>
static void launch_row(const TopkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(topk_row_kernel<E>, dim3(a.n_rows), dim3(kNT), 0, st, a);
}

template <int E>
static void launch_stage1(const TopkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(topk_stage1_kernel<E>, dim3(a.nblk, a.n_rows), dim3(kNT), 0, st, a);
}

template <int E>
static void launch_stage2(const TopkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(topk_stage2_kernel<E>, dim3(a.n_rows), dim3(kNT), 0, st, a);
}

// Smallest per-thread run E in {4, 8, 16, 32} that covers n keys.
static int run_for(int64_t n) { return n <= 4 * kNT ? 4 : (n <= 8 * kNT ? 8 : (n <= 16 * kNT ? 16 : 32)); }

tf_status launch_topk(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid, int32_t k,
                      int32_t* blocks, void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  TopkArgs a;
  a.logits = logits;
  a.ld = ld;
  a.n_rows = n_rows;
  a.n_valid = n_valid;
  a.k = k;
  a.blocks = blocks;
  const int B = pick_block(n_rows, ld, k);
  if (B == 0) {
    a.blk = (int)ld;
    a.nblk = 1;
    a.ws_key = nullptr;
    a.ws_idx = nullptr;
    switch (run_for(ld)) {
      case 4: launch_row<4>(a, st); break;
      case 8: launch_row<8>(a, st); break;
      case 16: launch_row<16>(a, st); break;
      default: launch_row<32>(a, st); break;
    }
    return launch_status("tf_topk_blocks");
  }
  const int64_t nb = (ld + B - 1) / B;
  a.blk = B;
  a.nblk = (int32_t)nb;
  a.ws_key = (uint32_t*)ws;
  a.ws_idx = (int32_t*)((char*)ws + (size_t)n_rows * nb * k * 4);
  if (n_rows > 65535) return set_error(TF_E_RANGE, "tf_topk_blocks: at most 65535 rows in blocked mode");
  switch (run_for(B)) {
    case 4: launch_stage1<4>(a, st); break;
    case 8: launch_stage1<8>(a, st); break;
    case 16: launch_stage1<16>(a, st); break;
    default: launch_stage1<32>(a, st); break;
  }
  tf_status s = launch_status("tf_topk_blocks");
  if (s != TF_OK) return s;
  switch (run_for(nb * k)) {
    case 4: launch_stage2<4>(a, st); break;
    case 8: launch_stage2<8>(a, st); break;
    case 16: launch_stage2<16>(a, st); break;
    default: launch_stage2<32>(a, st); break;
  }
  return launch_status("tf_topk_blocks");
}

}  // namespace tf
