// Top-k pooled blocks per row: the k largest logits among a row's n_valid,
// ties to the lower index, -0 == +0, written ascending and padded with -1.
// [CPM, sections 1 and 2.3]: per-row (ragged) top-k; long rows are cut into key
// blocks whose top-k candidates are merged, which is exact:
// topk(union) == topk(union of per-block topk).
//
// Design: a workgroup of 1,024 threads owns a segment of up to 32,768 keys held in
// registers; thread t holds the contiguous keys t*E .. t*E + E - 1 (16-byte loads).
// Logits become order-preserving 32-bit keys. The bits above the highest bit in which
// the segment's keys differ (from OR/AND reductions) are common; a most-significant-
// digit radix select over the rest, in passes of at most 11 bits with 2,048-bin LDS
// histograms, finds the k-th largest key T and how many keys equal to T belong to the
// top k. Every thread then counts its keys above T and equal to T; one block-wide
// prefix of the two counts gives each thread where its selected keys go and how many
// of its keys equal to T it takes, so the indices come out ascending, ties to the
// lower index, with no sort. Segments of 16 or 32 keys per thread first cut the keys
// down to a little more than k with a threshold taken from per-group maxima (each
// radix pass costs an LDS atomic per key and thread; at 8 keys per thread the cut
// measured slower than selecting on the whole segment). Long rows: stage 1 selects per
// key block, stage 2 merges the blocks' candidates (kept in index order).
#include "select.h"

namespace tf {

struct TopkArgs {
  const float* logits;
  int64_t ld;         // row stride of the logits
  int64_t ncap;       // n_valid is clipped here (the row's key count)
  int32_t n_rows;
  const int32_t* n_valid;
  int32_t k;
  int32_t* blocks;
  bool vec;           // 16-byte loads of logits rows
  int32_t blk;        // key block length (blocked mode)
  int32_t nblk;       // key blocks per row (blocked mode)
  int32_t kp;         // candidates per block in the workspace: k rounded up to a multiple of 4
  uint32_t* ws_key;   // [n_rows][nblk][kp]
  int32_t* ws_idx;    // [n_rows][nblk][kp]
  int32_t blk0;       // stage 1: key block of workgroup x = 0
  int64_t key0;       // stage 1: key at logits[r * ld + 0]
  const int32_t* cand;   // masked kernels: [n_rows][n_cand] candidate groups of `group` keys
  int32_t n_cand;
  int32_t group;
};

// Candidate bitmap of the masked kernels: the groups of one segment (at most 32,768 keys).
constexpr int kMaskWords = 32768 / 32 + 2;

// Masked kernels: the candidate groups among [g0, g0 + ng) as bits, from row r's list.
__device__ __forceinline__ void load_candidates(const TopkArgs& a, int r, int64_t g0, int ng, uint32_t* bits) {
  for (int i = threadIdx.x; i < (ng + 31) / 32; i += kNT) bits[i] = 0u;
  __syncthreads();
  const int32_t* c = a.cand + (int64_t)r * a.n_cand;
  for (int i = threadIdx.x; i < a.n_cand; i += kNT) {
    const int64_t x = (int64_t)c[i] - g0;
    if (c[i] >= 0 && x >= 0 && x < ng) atomicOr(&bits[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
}

// Masked kernels: load_keys with the thread's keys (segment positions base .. base +
// E - 1, keys key_base + position) outside the candidate groups read as -inf; bits
// start at group g0. With groups of whole quads (key_base and base are multiples of 4)
// one test covers a 16-byte load.
template <int E, bool VEC>
__device__ __forceinline__ void load_keys_masked(const float* seg, int n, const TopkArgs& a,
                                                 int64_t key_base, int64_t g0, const uint32_t* bits,
                                                 uint32_t (&key)[E]) {
  const int base = threadIdx.x * E;
  const int64_t k0 = key_base + base;
  int grp = (int)(k0 / a.group - g0);
  int rem = (int)(k0 % a.group);
  const uint32_t ninf = order_key(-__builtin_inff());
  if (VEC && a.group % 4 == 0) {
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
      const int i = base + 4 * j;
      const bool in = (bits[grp >> 5] >> (grp & 31)) & 1u;
      const float4 v = i < n ? *(const float4*)(seg + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      key[4 * j + 0] = i + 0 < n ? (in ? order_key(v.x) : ninf) : 0u;
      key[4 * j + 1] = i + 1 < n ? (in ? order_key(v.y) : ninf) : 0u;
      key[4 * j + 2] = i + 2 < n ? (in ? order_key(v.z) : ninf) : 0u;
      key[4 * j + 3] = i + 3 < n ? (in ? order_key(v.w) : ninf) : 0u;
      rem += 4;
      if (rem == a.group) {
        rem = 0;
        ++grp;
      }
    }
    return;
  }
  // every load issued before any is used (clamped indices), as in load_keys
  const int last = n > 0 ? n - 1 : 0;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = seg[base + e < n ? base + e : last];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = (bits[grp >> 5] >> (grp & 31)) & 1u;
    key[e] = base + e < n ? (in ? order_key(v[e]) : ninf) : 0u;
    if (++rem == a.group) {
      rem = 0;
      ++grp;
    }
  }
}

__device__ __forceinline__ int row_valid(const TopkArgs& a, int r) {
  int nv = a.n_valid ? a.n_valid[r] : (int)a.ld;
  if (nv < 0) nv = 0;
  if (nv > a.ncap) nv = (int)a.ncap;
  return nv;
}

// Waves per SIMD a kernel asks the compiler to leave room for: two workgroups of
// 1,024 threads per CU (8 waves per SIMD, at most 64 VGPRs) where the LDS allows it,
// so that one workgroup's loads overlap the other's selection.
template <int E>
constexpr int kWavesPerSimd = E >= 24 ? 8 : 4;

// One workgroup per row. MASK: keys outside the row's candidate groups read as -inf
// (a consumer's masking folded into the load; the logits are not written).
template <int E, bool MASK, bool VEC>
__device__ __forceinline__ void topk_row_body(const TopkArgs& a, SelShared& sh, CandShared& cs, uint32_t* bits) {
  const int r = blockIdx.x;
  const int n = row_valid(a, r);
  int32_t* out = a.blocks + (int64_t)r * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kNT) out[i] = i < n ? i : -1;
    return;
  }
  if constexpr (MASK) load_candidates(a, r, 0, (n + a.group - 1) / a.group, bits);
  uint32_t key[E];
  if constexpr (MASK) load_keys_masked<E, VEC>(a.logits + (int64_t)r * a.ld, n, a, 0, 0, bits, key);
  else load_keys<E, VEC>(a.logits + (int64_t)r * a.ld, n, key);
  const int base = threadIdx.x * E;
  select_topk<E>(key, a.k, sh, cs, [&](int e) { return base + e; },
                 [&](uint32_t pos, uint32_t, int32_t i) { out[pos] = i; });
}

template <int E, bool VEC>
__global__ __launch_bounds__(kNT, kWavesPerSimd<E>) void topk_row_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  __shared__ CandShared cs;
  topk_row_body<E, false, VEC>(a, sh, cs, nullptr);
}

template <int E, bool VEC>
__global__ __launch_bounds__(kNT, kWavesPerSimd<E>) void topk_row_masked_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  __shared__ CandShared cs;
  __shared__ uint32_t bits[kMaskWords];
  topk_row_body<E, true, VEC>(a, sh, cs, bits);
}

// Blocked mode, stage 1: top-k candidates (key, index) of one key block of one row, in
// index order, padded with key 0 to kp. MASK as for the row kernel.
template <int E, bool MASK, bool VEC>
__device__ __forceinline__ void topk_stage1_body(const TopkArgs& a, SelShared& sh, CandShared& cs, uint32_t* bits) {
  const int r = blockIdx.y;
  const int bb = blockIdx.x + a.blk0;
  const int nv = row_valid(a, r);
  if (nv <= a.k) return;  // stage 2 writes the row directly
  const int i0 = bb * a.blk;
  int n = nv - i0;
  if (n > a.blk) n = a.blk;
  if (n < 0) n = 0;
  uint32_t* ck = a.ws_key + ((int64_t)r * a.nblk + bb) * a.kp;
  int32_t* ci = a.ws_idx + ((int64_t)r * a.nblk + bb) * a.kp;
  const float* row = a.logits + (int64_t)r * a.ld + (i0 - a.key0);
  const int64_t g0 = MASK ? i0 / a.group : 0;
  if constexpr (MASK) load_candidates(a, r, g0, n > 0 ? (int)((i0 + n - 1) / a.group - g0 + 1) : 0, bits);
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.kp; i += kNT) {
      uint32_t kv = i < n ? order_key(row[i]) : 0u;
      if constexpr (MASK) {
        const int64_t gi = (int64_t)(i0 + i) / a.group - g0;
        if (i < n && !((bits[gi >> 5] >> (gi & 31)) & 1u)) kv = order_key(-__builtin_inff());
      }
      ck[i] = kv;
      ci[i] = i < n ? i0 + i : -1;
    }
    return;
  }
  uint32_t key[E];
  if constexpr (MASK) load_keys_masked<E, VEC>(row, n, a, i0, g0, bits, key);
  else load_keys<E, VEC>(row, n, key);
  const int base = i0 + threadIdx.x * E;
  for (int i = a.k + threadIdx.x; i < a.kp; i += kNT) {   // padding past k
    ck[i] = 0u;
    ci[i] = -1;
  }
  select_topk<E>(key, a.k, sh, cs, [&](int e) { return base + e; }, [&](uint32_t pos, uint32_t kv, int32_t i) {
    ck[pos] = kv;
    ci[pos] = i;
  });
}

template <int E, bool VEC>
__global__ __launch_bounds__(kNT, kWavesPerSimd<E>) void topk_stage1_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  __shared__ CandShared cs;
  topk_stage1_body<E, false, VEC>(a, sh, cs, nullptr);
}

template <int E, bool VEC>
__global__ __launch_bounds__(kNT, kWavesPerSimd<E>) void topk_stage1_masked_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  __shared__ CandShared cs;
  __shared__ uint32_t bits[kMaskWords];
  topk_stage1_body<E, true, VEC>(a, sh, cs, bits);
}

// Blocked mode, stage 2: merge the candidates of all key blocks of one row (they are in
// ascending index order, padding last in each block with key 0).
template <int E>
__global__ __launch_bounds__(kNT) void topk_stage2_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  __shared__ CandShared cs;
  const int r = blockIdx.x;
  const int nv = row_valid(a, r);
  int32_t* out = a.blocks + (int64_t)r * a.k;
  if (nv <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kNT) out[i] = i < nv ? i : -1;
    return;
  }
  const int nb_used = (nv + a.blk - 1) / a.blk;
  const int n = nb_used * a.kp;
  const uint32_t* ck = a.ws_key + (int64_t)r * a.nblk * a.kp;
  const int32_t* ci = a.ws_idx + (int64_t)r * a.nblk * a.kp;
  uint32_t key[E];
  int32_t idx[E];
  const int base = threadIdx.x * E;
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {   // kp is a multiple of 4: whole groups of four
    const int i = base + 4 * j;
    const uint4 kv = i < n ? *(const uint4*)(ck + i) : make_uint4(0u, 0u, 0u, 0u);
    const int4 iv = i < n ? *(const int4*)(ci + i) : make_int4(-1, -1, -1, -1);
    key[4 * j + 0] = kv.x;
    key[4 * j + 1] = kv.y;
    key[4 * j + 2] = kv.z;
    key[4 * j + 3] = kv.w;
    idx[4 * j + 0] = iv.x;
    idx[4 * j + 1] = iv.y;
    idx[4 * j + 2] = iv.z;
    idx[4 * j + 3] = iv.w;
  }
  select_topk<E>(key, a.k, sh, cs, [&](int e) { return idx[e]; },
                 [&](uint32_t pos, uint32_t, int32_t i) { out[pos] = i; });
}

// Key-block length for the blocked mode, or 0 for one workgroup per row. A few rows of
// up to 32,768 keys still take the blocked mode: one workgroup alone streams a long row
// from HBM and selects in it more slowly than many workgroups select in its blocks
// and a second launch merges their candidates.
static int pick_block(int32_t n_rows, int64_t ld, int32_t k) {
  if (ld <= 4096 || (ld <= 32768 && n_rows >= 128)) return 0;
  // few long rows: the shortest block of 4,096 .. 32,768 keys with at most 256 stage-1
  // workgroups (a decode batch of 8 rows x 32,768 keys: 64 blocks of 4,096; 8 rows x
  // 262,144: 136 of 16,384, which ran 29 against 41 us for 72 of 32,768), with the
  // merged candidates (blocks x kp) at most 32,768
  const int64_t kp = (k + 3) / 4 * 4;
  int64_t B = 4096;
  while (B < 32768 && n_rows * ((ld + B - 1) / B) > 256) B *= 2;
  while (B < 32768 && ((ld + B - 1) / B) * kp > 32768) B *= 2;
  if (((ld + B - 1) / B) * kp > 32768) return -1;
  return (int)B;
}

size_t topk_ws_bytes(int32_t n_rows, int64_t ld, int32_t k) {
  const int B = pick_block(n_rows, ld, k);
  if (B < 0) return (size_t)-1;
  if (B == 0) return 0;
  const int64_t nb = (ld + B - 1) / B;
  const int64_t kp = (k + 3) / 4 * 4;
  return (size_t)n_rows * nb * kp * 8;
}

template <int E>
static void launch_row(const TopkArgs& a, hipStream_t st) {
  if (a.cand && a.vec) hipLaunchKernelGGL((topk_row_masked_kernel<E, true>), dim3(a.n_rows), dim3(kNT), 0, st, a);
  else if (a.cand) hipLaunchKernelGGL((topk_row_masked_kernel<E, false>), dim3(a.n_rows), dim3(kNT), 0, st, a);
  else if (a.vec) hipLaunchKernelGGL((topk_row_kernel<E, true>), dim3(a.n_rows), dim3(kNT), 0, st, a);
  else hipLaunchKernelGGL((topk_row_kernel<E, false>), dim3(a.n_rows), dim3(kNT), 0, st, a);
}

template <int E>
static void launch_stage1(const TopkArgs& a, hipStream_t st, dim3 grid) {
  if (a.cand && a.vec) hipLaunchKernelGGL((topk_stage1_masked_kernel<E, true>), grid, dim3(kNT), 0, st, a);
  else if (a.cand) hipLaunchKernelGGL((topk_stage1_masked_kernel<E, false>), grid, dim3(kNT), 0, st, a);
  else if (a.vec) hipLaunchKernelGGL((topk_stage1_kernel<E, true>), grid, dim3(kNT), 0, st, a);
  else hipLaunchKernelGGL((topk_stage1_kernel<E, false>), grid, dim3(kNT), 0, st, a);
}

template <int E>
static void launch_stage2(const TopkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(topk_stage2_kernel<E>, dim3(a.n_rows), dim3(kNT), 0, st, a);
}

// Smallest per-thread run E in {4, 8, 16, 24, 28, 32} that covers n keys. 24 and 28
// keys a thread (rows of up to 28,672 keys) fit 64 VGPRs with no spill, where 32 spill
// 16 bytes a lane at the 64-VGPR bound of two workgroups per CU; only the row kernel
// takes 24 and 28 (the per-block kernels run 32).
static int run_for(int64_t n) {
  return n <= 4 * kNT ? 4
                      : (n <= 8 * kNT ? 8 : (n <= 16 * kNT ? 16 : (n <= 24 * kNT ? 24 : (n <= 28 * kNT ? 28 : 32))));
}

tf_status launch_topk(const float* logits, int64_t ld, int32_t n_rows, const int32_t* n_valid, int32_t k,
                      int32_t* blocks, void* ws, size_t ws_bytes, hipStream_t st, const int32_t* cand,
                      int32_t n_cand, int32_t group) {
  (void)ws_bytes;
  TopkArgs a;
  a.logits = logits;
  a.ld = ld;
  a.ncap = ld;
  a.blk0 = 0;
  a.key0 = 0;
  a.cand = cand;
  a.n_cand = n_cand;
  a.group = group;
  a.n_rows = n_rows;
  a.n_valid = n_valid;
  a.k = k;
  a.blocks = blocks;
  a.vec = ld % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  a.kp = (k + 3) / 4 * 4;
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
      case 24: launch_row<24>(a, st); break;
      case 28: launch_row<28>(a, st); break;
      default: launch_row<32>(a, st); break;
    }
    return launch_status("tf_topk_blocks");
  }
  const int64_t nb = (ld + B - 1) / B;
  a.blk = B;
  a.nblk = (int32_t)nb;
  a.ws_key = (uint32_t*)ws;
  a.ws_idx = (int32_t*)((char*)ws + (size_t)n_rows * nb * a.kp * 4);
  if (n_rows > 65535) return set_error(TF_E_RANGE, "tf_topk_blocks: at most 65535 rows in blocked mode");
  const dim3 g1((unsigned)a.nblk, (unsigned)n_rows);
  switch (run_for(B)) {
    case 4: launch_stage1<4>(a, st, g1); break;
    case 8: launch_stage1<8>(a, st, g1); break;
    case 16: launch_stage1<16>(a, st, g1); break;
    default: launch_stage1<32>(a, st, g1); break;
  }
  tf_status s = launch_status("tf_topk_blocks");
  if (s != TF_OK) return s;
  switch (run_for(nb * a.kp)) {
    case 4: launch_stage2<4>(a, st); break;
    case 8: launch_stage2<8>(a, st); break;
    case 16: launch_stage2<16>(a, st); break;
    default: launch_stage2<32>(a, st); break;
  }
  return launch_status("tf_topk_blocks");
}

// ---- key-blocked scoring [CPM, section 2.3]: stage 1 per key block, then the merge --------
// The caller scores one key block of B keys at a time into a [n_rows][B] buffer; each
// block's candidates go to its slot of the candidate workspace, and the merge runs once
// all blocks are in. n_valid holds the rows' full visible counts (clipped to ncap).

size_t topk_cand_bytes(int32_t n_rows, int32_t nb, int32_t k) {
  return (size_t)n_rows * nb * ((k + 3) / 4 * 4) * 8;
}

static TopkArgs block_args(const float* logits_blk, int32_t B, int32_t nb, int64_t ncap, int32_t n_rows,
                           const int32_t* n_valid, int32_t k, int32_t* blocks, void* cand) {
  TopkArgs a;
  a.logits = logits_blk;
  a.ld = B;
  a.ncap = ncap;
  a.n_rows = n_rows;
  a.n_valid = n_valid;
  a.k = k;
  a.blocks = blocks;
  a.vec = B % 4 == 0 && ((uintptr_t)logits_blk & 15) == 0;
  a.kp = (k + 3) / 4 * 4;
  a.blk = B;
  a.nblk = nb;
  a.ws_key = (uint32_t*)cand;
  a.ws_idx = (int32_t*)((char*)cand + (size_t)n_rows * nb * a.kp * 4);
  a.blk0 = 0;
  a.key0 = 0;
  a.cand = nullptr;
  a.n_cand = 0;
  a.group = 1;
  return a;
}

tf_status launch_topk_block(const float* logits_blk, int32_t B, int32_t b, int32_t nb, int64_t ncap,
                            int32_t n_rows, const int32_t* n_valid, int32_t k, void* cand, hipStream_t st) {
  TopkArgs a = block_args(logits_blk, B, nb, ncap, n_rows, n_valid, k, nullptr, cand);
  a.blk0 = b;
  a.key0 = (int64_t)b * B;
  const dim3 g1(1, (unsigned)n_rows);
  switch (run_for(B)) {
    case 4: launch_stage1<4>(a, st, g1); break;
    case 8: launch_stage1<8>(a, st, g1); break;
    case 16: launch_stage1<16>(a, st, g1); break;
    default: launch_stage1<32>(a, st, g1); break;
  }
  return launch_status("tf_indexer_topk");
}

tf_status launch_topk_merge(int32_t B, int32_t nb, int64_t ncap, int32_t n_rows, const int32_t* n_valid,
                            int32_t k, int32_t* blocks, void* cand, hipStream_t st) {
  TopkArgs a = block_args(nullptr, B, nb, ncap, n_rows, n_valid, k, blocks, cand);
  switch (run_for((int64_t)nb * a.kp)) {
    case 4: launch_stage2<4>(a, st); break;
    case 8: launch_stage2<8>(a, st); break;
    case 16: launch_stage2<16>(a, st); break;
    default: launch_stage2<32>(a, st); break;
  }
  return launch_status("tf_indexer_topk");
}

}  // namespace tf
