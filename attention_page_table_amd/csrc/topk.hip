// Top-k pooled blocks per row: the k largest logits among a row's n_valid,
// ties to the lower index, -0 == +0, written ascending and padded with -1.
// [CPM, sections 1 and 2.3]: per-row (ragged) top-k; long rows are cut into key
// blocks whose top-k candidates are merged, which is exact:
// topk(union) == topk(union of per-block topk).
//
// Design: a workgroup of 1,024 threads owns a segment of up to 32,768 keys held in
// registers; wave w owns the contiguous index range [w*64E, (w+1)*64E) and its lane l
// holds indices w*64E + 64e + l (coalesced loads). Logits become order-preserving
// 32-bit keys. The bits above the highest bit in which the segment's keys differ
// (from OR/AND reductions) are common; a most-significant-digit radix select over
// the rest, in passes of at most 11 bits with 2,048-bin LDS histograms, finds the
// k-th largest key T and how many keys equal to T belong to the top k. An ordered
// compaction with wave ballots then writes the selected indices ascending, taking
// keys equal to T lowest index first. No sort is needed because the output order is
// by index. Long rows: stage 1 selects per key block, stage 2 merges the blocks'
// candidates (kept in index order).
#include "common.h"

namespace tf {

constexpr int kNT = 1024;  // threads per workgroup
constexpr int kWaves = kNT / 64;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int ctrl, int row_mask = 0xf>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, row_mask, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP: row shifts, then row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u<0x111>(x);        // row_shr:1
  x += dpp_u<0x112>(x);        // row_shr:2
  x += dpp_u<0x114>(x);        // row_shr:4
  x += dpp_u<0x118>(x);        // row_shr:8
  x += dpp_u<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_u<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// OR and AND of a value over the wave: within each row of 16 lanes by DPP, then the
// four rows through readlane (the results are wave-uniform).
__device__ __forceinline__ void wave_or_and(uint32_t& o, uint32_t& a) {
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0xB1, 0xf, 0xf, true);    // quad_perm [1,0,3,2]
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0xB1, 0xf, 0xf, true);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x4E, 0xf, 0xf, true);    // quad_perm [2,3,0,1]
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x4E, 0xf, 0xf, true);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x141, 0xf, 0xf, true);   // row_half_mirror
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x141, 0xf, 0xf, true);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x140, 0xf, 0xf, true);   // row_mirror
  a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x140, 0xf, 0xf, true);
  o = __builtin_amdgcn_readlane(o, 0) | __builtin_amdgcn_readlane(o, 16) | __builtin_amdgcn_readlane(o, 32) |
      __builtin_amdgcn_readlane(o, 48);
  a = __builtin_amdgcn_readlane(a, 0) & __builtin_amdgcn_readlane(a, 16) & __builtin_amdgcn_readlane(a, 32) &
      __builtin_amdgcn_readlane(a, 48);
}

struct SelShared {
  uint32_t hist[3][kBins];   // one histogram per radix pass, all cleared up front
  uint32_t wor[kWaves], wand[kWaves], wsum[kWaves], wgt[kWaves], weq[kWaves];
  uint32_t bin, rem;
};

// Exclusive prefix of the per-wave values v[0..kWaves) for this thread's wave, and
// their total, from one LDS read per lane and a wave prefix sum.
__device__ __forceinline__ uint32_t waves_before(const uint32_t* v, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t incl = wave_incl_scan(lane < kWaves ? v[lane] : 0u);
  total = __builtin_amdgcn_readlane(incl, kWaves - 1);
  return wid == 0 ? 0u : __builtin_amdgcn_readlane(incl, wid - 1);
}

// T = the k-th largest of the n > k valid keys (invalid slots hold 0, below every
// valid key), rem = how many keys equal to T belong to the top k. Three barriers per
// radix pass: after the histogram, after the wave totals, after the selected bin.
template <int E>
__device__ void radix_select(const uint32_t (&key)[E], int k, SelShared& sh, uint32_t& T, uint32_t& rem) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // common leading bits of the valid keys; clear the pass histograms
  {
    uint32_t o = 0u, an = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0u) {
        o |= key[e];
        an &= key[e];
      }
    wave_or_and(o, an);
    if (lane == 0) {
      sh.wor[wid] = o;
      sh.wand[wid] = an;
    }
    uint32_t* h = &sh.hist[0][0];
    for (int i = threadIdx.x * 4; i < 3 * kBins; i += kNT * 4) *(uint4*)&h[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  uint32_t orv = lane < kWaves ? sh.wor[lane] : 0u, andv = lane < kWaves ? sh.wand[lane] : 0xFFFFFFFFu;
  wave_or_and(orv, andv);
  const uint32_t diff = orv ^ andv;
  if (diff == 0u) {  // every valid key equal
    T = orv;
    rem = (uint32_t)k;
    return;
  }
  const int hb = 31 - __builtin_clz(diff);   // highest differing bit
  uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = andv & mask, r = (uint32_t)k;
  int top = hb + 1;   // bits [0, top) remain
  for (int p = 0; top > 0; ++p) {
    const int width = top > 11 ? 11 : top;
    const int shift = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = sh.hist[p];
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0u && (key[e] & mask) == prefix) atomicAdd(&h[(key[e] >> shift) & dmask], 1u);
    __syncthreads();
    // descending bins: thread t owns bins 2047 - 2t and 2046 - 2t
    const uint32_t c0 = h[kBins - 1 - 2 * threadIdx.x], c1 = h[kBins - 2 - 2 * threadIdx.x];
    const uint32_t incl = wave_incl_scan(c0 + c1);
    if (lane == 63) sh.wsum[wid] = incl;
    __syncthreads();
    uint32_t tot;
    const uint32_t above = waves_before(sh.wsum, tot) + incl - (c0 + c1);
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
    top = shift;
  }
  T = prefix;
  rem = r;
}

// Ordered compaction: emit(pos, e) for every selected key, in index order
// (wave-major, then e, then lane).
template <int E, typename Emit>
__device__ void ordered_select(const uint32_t (&key)[E], uint32_t T, uint32_t rem, SelShared& sh, Emit emit) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gt += __builtin_popcountll(__ballot(key[e] > T));
    eq += __builtin_popcountll(__ballot(key[e] == T));
  }
  if (lane == 0) {
    sh.wgt[wid] = gt;
    sh.weq[wid] = eq;
  }
  __syncthreads();
  // per wave (lane l < kWaves stands for wave l): keys equal to T before it, how many
  // of its own it takes, and the rank of its first selected key
  uint32_t eq_base, pos_base;
  {
    const uint32_t ge = lane < kWaves ? sh.wgt[lane] : 0u, we = lane < kWaves ? sh.weq[lane] : 0u;
    const uint32_t eq_incl = wave_incl_scan(we);
    const uint32_t eq_before = eq_incl - we;
    const uint32_t take = eq_before >= rem ? 0u : (rem - eq_before < we ? rem - eq_before : we);
    const uint32_t pos_incl = wave_incl_scan(ge + take);
    const int w0 = wid - 1;
    eq_base = wid == 0 ? 0u : __builtin_amdgcn_readlane(eq_incl, w0);
    pos_base = wid == 0 ? 0u : __builtin_amdgcn_readlane(pos_incl, w0);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool is_eq = key[e] == T;
    const uint64_t em = __ballot(is_eq);
    const bool take = key[e] > T || (is_eq && eq_base + lanes_below(em) < rem);
    const uint64_t tm = __ballot(take);
    if (take) emit(pos_base + lanes_below(tm), e);
    pos_base += __builtin_popcountll(tm);
    eq_base += __builtin_popcountll(em);
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

// index of this thread's e-th key within the segment
template <int E>
__device__ __forceinline__ int seg_index(int e) {
  return (threadIdx.x >> 6) * 64 * E + e * 64 + (threadIdx.x & 63);
}

template <int E>
__device__ __forceinline__ void load_keys(const float* row, int n, uint32_t (&key)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = seg_index<E>(e);
    key[e] = i < n ? order_key(row[i]) : 0u;
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
  ordered_select<E>(key, T, rem, sh, [&](uint32_t pos, int e) {
    if (pos < (uint32_t)a.k) out[pos] = seg_index<E>(e);
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
  ordered_select<E>(key, T, rem, sh, [&](uint32_t pos, int e) {
    if (pos < (uint32_t)a.k) {
      ck[pos] = key[e];
      ci[pos] = i0 + seg_index<E>(e);
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
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = seg_index<E>(e);
    key[e] = i < n ? ck[i] : 0u;
    idx[e] = i < n ? ci[i] : -1;
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
  // few long rows: blocks of 4,096 .. 32,768 keys so that about 64 workgroups run,
  // with the merged candidates (blocks x k) at most 32,768
  int64_t B = 4096;
  while (B < 32768 && n_rows * ((ld + B - 1) / B) > 64) B *= 2;
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
