// Indexer logits on MFMA: l[t,j] = sum_h w[t,h] * ReLU(q[t,h] . k_j), fp32,
// masked to -inf for j >= n_c(t) = t/4 + 1.
// [CPM, section 1]: each chunk's query rows scored against the whole compressed
// prefix, output [T, max_seqlen_k] fp32, masked by the compressed lengths.
// [#1142, "GLM declares a kv_pool.Layout"]: the pooled keys are read through the
// page table.
//
// One v_mfma_f32_32x32x16_bf16 tile is 32 (row, head) pairs x 32 keys x 16 dims.
// Its 32 A-rows are arranged so that each lane's 16 accumulators are all the heads
// of the rows its half-wave holds, for one key: the ReLU, the weights and the head
// sum stay inside the lane (no shuffles) and each half-wave stores 32 consecutive
// keys of a row (128-byte stores).
//
// Two kernels:
//  * tile kernel (many rows of one stream, e.g. a prefill chunk; MFMA-bound): a
//    workgroup holds the queries of 4 x MT x (32/H) rows in registers and streams a
//    key range through LDS in 32-key subtiles (double-buffered global -> LDS loads,
//    16-byte chunks XOR-swizzled so the B-fragment reads are conflict-free); each
//    B fragment read from LDS feeds MT tiles. Workgroups whose rows are not all of
//    one stream take the per-row path.
//  * row kernel (few rows of distinct streams, e.g. a decode batch; HBM-bound): each
//    wave streams one row's keys straight into B fragments, one subtile ahead, with
//    the row's page ids preloaded across the lanes.
#include <type_traits>

#include "common.h"

namespace tf {

struct IdxArgs {
  DevView v;
  int64_t off_pkey;
  int32_t pkey_row_bytes;
  int32_t n_rows;
  const int32_t* row_stream;
  const int32_t* row_pos;
  const __bf16* q;
  const float* w;
  float* logits;   // logit of (row, key) at logits[row * ldo + key]: the caller's buffer
                   // shifted back by key0 elements (keys below key0 are never written)
  int64_t ldo;     // row stride of the logits
  int64_t key0;    // keys [key0, kend) are scored (key0 a multiple of 128)
  int64_t kend;
  int64_t ncap;    // n_c is clipped here (the full key count; n_valid receives it)
  int32_t* n_valid;
  int32_t keys_per_wg;   // multiple of 128
  int32_t n_kgroups;
};

typedef __attribute__((address_space(3))) void lds_void;

// max(x, 0) as one integer max on the bits: a float with the sign bit set (negative,
// -0) is a negative int32 and becomes +0; a non-negative float keeps its bits. A float
// max would first quiet signaling NaNs, one more instruction per value.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(__builtin_elementwise_max(__float_as_int(x), 0));
}

// sum_h w[h] * ReLU(acc[h]) over N values, in two independent chains so that
// consecutive FMAs do not wait on each other
template <int N, typename A>
__device__ __forceinline__ float weighted_relu_sum(const float* w, const A& acc, int off) {
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int h = 0; h < N; ++h) s[h & 1] = __builtin_fmaf(w[h], relu(acc[off + h]), s[h & 1]);
  return s[0] + s[1];
}

__device__ __forceinline__ int nc_of(const IdxArgs& a, int row) {
  const int pos = a.row_pos[row];
  if (pos < 0) return 0;
  const int64_t nc = (int64_t)pos / kPoolRatio + 1;
  return (int)(nc < a.ncap ? nc : a.ncap);
}

// ---- per-row path: one wave streams one row over keys [kb, ke) ---------------------------
// A-rows with bit 2 clear carry the row's heads (head 4 * (m / 8) + m % 4), the others are
// zero; lanes 0..31 then hold every head of key n = lane in accumulators 0..H-1.
template <int H, int D>
__device__ void index_one_row(const IdxArgs& a, int row, int64_t kb, int64_t ke, int lane, bool spec_page = false,
                              int spec_page_all = -1) {
  constexpr int KS = D / 16;
  const int g = lane >> 5, n = lane & 31;
  const int b = a.row_stream[row];
  const int nc = nc_of(a, row);
  const float ninf = -__builtin_inff();
  float* out = a.logits + (int64_t)row * a.ldo;
  bf16x8 aq[KS];
  {
    const int m = n;
    const int u = 4 * (m >> 3) + (m & 3);
    const bool live = ((m >> 2) & 1) == 0 && u < H;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      aq[ks] = live ? *(const bf16x8*)(a.q + ((int64_t)row * H + u) * D + ks * 16 + g * 8) : bf16x8{};
  }
  float wv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) wv[i] = i < H ? a.w[(int64_t)row * H + i] : 0.f;
  const int64_t kend = ke < nc ? ke : nc;   // keys that need scores
  // page ids of the range, one per lane (lane i: page index kb/128 + i)
  const int p0 = (int)(kb / kKeysPerPage);
  int my_page;
  if (spec_page) {
    // a one-page range of a table of at most 64 streams: lane s has already read
    // stream s's entry, so the page id does not wait for the row's stream id
    const int pb = b >= 0 && b < a.v.n_streams ? __builtin_amdgcn_readlane(spec_page_all, b) : -1;
    my_page = lane == 0 ? pb : -1;
  } else {
    my_page = page_of(a.v, b, p0 + lane);
  }
  auto page_at = [&](int64_t kt) { return __builtin_amdgcn_readlane(my_page, (int)(kt / kKeysPerPage) - p0); };
  auto load = [&](int64_t kt, bf16x8 (&bf)[KS]) {
    const int pg = page_at(kt);
    if (pg >= 0) {
      const char* kp = cache_block(a.v, pg) + a.off_pkey + (int64_t)((kt % kKeysPerPage) + n) * a.pkey_row_bytes + g * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[ks] = *(const bf16x8*)(kp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[ks] = bf16x8{};
    }
  };
  // three subtiles in flight: slot s holds subtile kb + 32 (3i + s)
  auto step = [&](int64_t kt, bf16x8 (&cur)[KS]) {
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[ks], cur[ks], acc, 0, 0, 0);
    const int pg = page_at(kt);
    if (kt + 96 < kend) load(kt + 96, cur);   // refill the slot three subtiles ahead
    const float s = weighted_relu_sum<H>(wv, acc, 0);
    const int64_t key = kt + n;
    if (g == 0 && key < ke) out[key] = key < nc ? (pg >= 0 ? s : __builtin_nanf("")) : ninf;
  };
  bf16x8 s0[KS], s1[KS], s2[KS];
  if (kb < kend) load(kb, s0);
  if (kb + 32 < kend) load(kb + 32, s1);
  if (kb + 64 < kend) load(kb + 64, s2);
  for (int64_t kt = kb; kt < kend; kt += 96) {
    step(kt, s0);
    if (kt + 32 < kend) step(kt + 32, s1);
    if (kt + 64 < kend) step(kt + 64, s2);
  }
  // keys past the compressed length
  for (int64_t key = (kend > kb ? kend : kb) + lane; key < ke; key += 64) out[key] = ninf;
}

// Per-row kernel: wave w of workgroup (key group kg, row group rg) takes row 4 rg + w.
// The row groups of one key group run on one XCD (workgroups 8 apart).
template <int H, int D>
__global__ __launch_bounds__(256) void indexer_rows_kernel(IdxArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n_rg = (a.n_rows + 3) / 4;
  const int id = blockIdx.x;
  const int rg = (id >> 3) % n_rg;
  const int kg = (id / (8 * n_rg)) * 8 + (id & 7);
  if (kg >= a.n_kgroups) return;
  const int row = rg * 4 + wave;
  if (row >= a.n_rows) return;
  const int64_t kb = a.key0 + (int64_t)kg * a.keys_per_wg;
  const int64_t ke = kb + a.keys_per_wg < a.kend ? kb + a.keys_per_wg : a.kend;
  // one-page ranges over a table of at most 64 streams: read every stream's entry for
  // the page now, beside the row's own stream id
  const bool spec = a.keys_per_wg == kKeysPerPage && a.v.n_streams <= 64;
  int spec_all = -1;
  if (spec) {
    const int pi = (int)(kb / kKeysPerPage);
    if (lane < a.v.n_streams && pi < a.v.pt_stride) {
      const int pg = a.v.pt ? a.v.pt[(int64_t)lane * a.v.pt_stride + pi] : lane * a.v.pt_stride + pi;
      spec_all = pg >= 0 && pg < a.v.n_pages ? pg : -1;
    }
  }
  if (kg == 0 && a.n_valid && lane == 0) a.n_valid[row] = nc_of(a, row);
  index_one_row<H, D>(a, row, kb, ke, lane, spec, spec_all);
}

// ---- tile path -----------------------------------------------------------------------------
constexpr int kChunk = 128;   // keys per LDS chunk: one page's pooled keys

template <int D>
struct KeyChunk {
  __bf16 k[kChunk * D];   // four 32-key subtiles; within each, 16-byte pieces swizzled by key
};

// Swizzled position of chunk c of key j in a subtile (chunks of 16 bytes, CH per key).
template <int CH>
__device__ __forceinline__ int swz(int j, int c) {
  return j * CH + (c ^ (j & (CH - 1)));
}

// WINDOW names the instance that scores one key block of a key-blocked call, so that
// profiles keep its launches apart from whole-range ones; the code is the same.
template <int H, int D, int MT, bool WINDOW>
__global__ __launch_bounds__(256, 2) void indexer_tile_kernel(IdxArgs a) {
  constexpr int RPT = 32 / H;   // query rows per MFMA tile
  constexpr int RH = 16 / H;    // rows per half-wave in the accumulators
  constexpr int KS = D / 16;    // MFMA k-steps
  constexpr int CH = D / 8;     // 16-byte chunks per key
  constexpr int ROWS = 4 * MT * RPT;
  constexpr int kMaxPages = 40;
  __shared__ KeyChunk<D> kc0, kc1;
  __shared__ int32_t pg_lds[kMaxPages];
  __shared__ int32_t uniform_flag;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int row_base = blockIdx.y * ROWS;
  const int64_t kb = a.key0 + (int64_t)blockIdx.x * a.keys_per_wg;
  const int64_t ke = kb + a.keys_per_wg < a.kend ? kb + a.keys_per_wg : a.kend;
  const int wave_row0 = row_base + wave * (MT * RPT);

  if (blockIdx.x == 0 && a.n_valid && tid < ROWS && row_base + tid < a.n_rows)
    a.n_valid[row_base + tid] = nc_of(a, row_base + tid);

  // all rows of the workgroup valid and of one stream?
  if (tid == 0) uniform_flag = 1;
  __syncthreads();
  const int b0 = a.row_stream[row_base < a.n_rows ? row_base : a.n_rows - 1];
  if (tid < ROWS && (row_base + tid >= a.n_rows || a.row_stream[row_base + tid] != b0)) uniform_flag = 0;
  __syncthreads();
  if (!uniform_flag) {
    // per-row path: each wave takes rows of the workgroup in turn
    for (int rr = wave; rr < ROWS; rr += 4) {
      const int row = row_base + rr;
      if (row < a.n_rows) {
        if (H == 16) index_one_row<16, D>(a, row, kb, ke, lane);
        else if (H == 8) index_one_row<8, D>(a, row, kb, ke, lane);
        else index_one_row<4, D>(a, row, kb, ke, lane);
      }
    }
    return;
  }

  // largest compressed length of the workgroup's rows: keys past it are -inf only
  int nc_max = 0, nc_min = 0x7fffffff;
  int rnc[MT][RH];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < RH; ++r) rnc[t][r] = nc_of(a, wave_row0 + t * RPT + g * RH + r);
  for (int rr = 0; rr < ROWS; ++rr) {
    const int c = nc_of(a, row_base + rr);
    nc_max = c > nc_max ? c : nc_max;
    nc_min = c < nc_min ? c : nc_min;
  }
  const int64_t kend = ke < nc_max ? ke : nc_max;

  // page ids of the key range
  const int p0 = (int)(kb / kKeysPerPage);
  if (tid < kMaxPages) pg_lds[tid] = page_of(a.v, b0, p0 + tid);

  // A fragments: lane supplies A-row m = n; m = 8a + 4b + c maps to tile row
  // b*RH + (4a+c)/H and head (4a+c)%H.
  bf16x8 afrag[MT][KS];
  {
    const int ma = n >> 3, mb = (n >> 2) & 1, mc = n & 3;
    const int u = 4 * ma + mc;
    const int trow = mb * RH + u / H;
    const int head = u % H;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int row = wave_row0 + t * RPT + trow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        afrag[t][ks] = *(const bf16x8*)(a.q + ((int64_t)row * H + head) * D + ks * 16 + g * 8);
    }
  }
  // weights of the (row, head) pairs of this lane's accumulators
  float wv[MT][16];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) wv[t][i] = a.w[(int64_t)(wave_row0 + t * RPT + g * RH + i / H) * H + (i % H)];
  // this lane's output rows, at key n
  float* optr[MT][RH];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < RH; ++r) optr[t][r] = a.logits + (int64_t)(wave_row0 + t * RPT + g * RH + r) * a.ldo + n;
  __syncthreads();

  // global -> LDS loads of one 128-key chunk (one page, since kb is a multiple of
  // 128): 32 * CH pieces of 16 bytes per subtile, 64 per wave-wide load; the lane that
  // fills swizzled position p loads the piece that belongs there. Keys past kend in
  // the chunk are read too (same page) and masked when scored.
  // The pieces a lane loads sit at the same offsets in every chunk: the lane's offsets
  // within a subtile are computed once (one or two of them), the subtile's start joins
  // the scalar base, and each load is a scalar base plus a vector offset.
  constexpr int kRowsPerSub = CH * 32 / 64;   // wave-wide loads per subtile
  constexpr int kPar = kRowsPerSub / 4;       // distinct in-subtile offsets per lane
  uint32_t dma_off[kPar];
#pragma unroll
  for (int pp = 0; pp < kPar; ++pp) {
    const int q = (wave + 4 * pp) * 64 + lane;
    const int j = q / CH, c = (q % CH) ^ (j & (CH - 1));
    dma_off[pp] = (uint32_t)(j * a.pkey_row_bytes + c * 16);
  }
  auto issue = [&](int64_t kt, __bf16* dst) __attribute__((always_inline)) {
    const int pg = __builtin_amdgcn_readfirstlane(pg_lds[(int)(kt / kKeysPerPage) - p0]);
    // a missing page reads any readable bytes: its keys' logits are written as NaN
    const char* base = pg >= 0 ? cache_block(a.v, pg) + a.off_pkey : a.v.pool;
#pragma unroll
    for (int u = 0; u < CH / 2; ++u) {
      const int i = wave + 4 * u;
      const char* bu = base + (int64_t)(u / kPar) * 32 * a.pkey_row_bytes;
      __builtin_amdgcn_global_load_lds((const void*)(bu + dma_off[u % kPar]), (lds_void*)&dst[i * 64 * 8], 16, 0,
                                       0);
    }
  };

  const float ninf = -__builtin_inff();
  const float qnan = __builtin_nanf("");
  // A chunk is four 32-key subtiles of MT tiles each. Tile (sub, t) accumulates into
  // acc[t]; its head sum and stores run while the next tile's MFMAs do (four VALU
  // instructions between consecutive MFMAs), so the two accumulators alternate and
  // the vector ALU works beside the matrix core (kPipe; with 128-dim keys and fewer
  // than 16 heads a lane holds several rows and the registers do not suffice, so
  // each tile's head sum follows its MFMAs there). The next subtile's B fragments are
  // read from LDS during the last tile's MFMAs, each right after its register is
  // consumed. Subtiles past kend are computed too (their keys are in the chunk's
  // page) and only keys < ke are stored. Modes: kOpen, every key of the chunk is
  // stored and visible to every row (no selects); kFull, every key is stored; kPart,
  // keys are tested against ke.
  constexpr int kOpen = 0, kFull = 1, kPart = 2;
  constexpr int kSubs = kChunk / 32;
  constexpr bool kPipe = H == 16 || D == 64;
  auto epilogue = [&](const f32x16& acc, int t, int64_t kt, bool pg_ok, auto mode) __attribute__((always_inline)) {
    constexpr int M = decltype(mode)::value;
    const int64_t key = kt + n;
#pragma unroll
    for (int r = 0; r < RH; ++r) {
      const float s = weighted_relu_sum<H>(&wv[t][r * H], acc, r * H);
      // non-temporal: the logits stream out past L2, which keeps the key chunks other
      // workgroups of the XCD read
      if (M == kOpen) {
        __builtin_nontemporal_store(s, &optr[t][r][kt]);
      } else {
        const float v = key < rnc[t][r] ? (pg_ok ? s : qnan) : ninf;
        if (M == kFull || key < ke) __builtin_nontemporal_store(v, &optr[t][r][kt]);
      }
    }
  };
  auto chunk_body = [&](int64_t kt0, const __bf16* src, bool pg_ok, auto mode) __attribute__((always_inline)) {
    f32x16 acc[MT];
    bf16x8 bfrag[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bfrag[ks] = *(const bf16x8*)&src[swz<CH>(n, 2 * ks + g) * 8];
#pragma unroll
    for (int sub = 0; sub < kSubs; ++sub) {
      const int64_t kt = kt0 + sub * 32;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        acc[t] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[t][ks], bfrag[ks], acc[t], 0, 0, 0);
          if (t == MT - 1 && sub + 1 < kSubs)
            bfrag[ks] = *(const bf16x8*)&src[(sub + 1) * 32 * D + swz<CH>(n, 2 * ks + g) * 8];
        }
        if constexpr (kPipe) {
          if (t > 0) epilogue(acc[t - 1], t - 1, kt, pg_ok, mode);
          else if (sub > 0) epilogue(acc[MT - 1], MT - 1, kt - 32, pg_ok, mode);
          // pin the interleave: per MFMA, the B read that refills its register (last
          // tile only) and four instructions of the previous tile's head sum
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (t == MT - 1 && sub + 1 < kSubs) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (t > 0 || sub > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
        } else {
          epilogue(acc[t], t, kt, pg_ok, mode);
        }
      }
    }
    if constexpr (kPipe) epilogue(acc[MT - 1], MT - 1, kt0 + (kSubs - 1) * 32, pg_ok, mode);
  };
  // which mode a chunk runs in, and the vector-memory operations it issues after the
  // next chunk's loads (its stores), so that the next barrier waits for the loads only
  auto chunk = [&](int64_t kt, const __bf16* src) __attribute__((always_inline)) -> bool {
    const bool pg_ok = pg_lds[(int)(kt / kKeysPerPage) - p0] >= 0;
    if (kt + kChunk <= ke && pg_ok && kt + kChunk <= nc_min) {
      chunk_body(kt, src, pg_ok, std::integral_constant<int, kOpen>{});
      return true;
    }
    if (kt + kChunk <= ke) {
      chunk_body(kt, src, pg_ok, std::integral_constant<int, kFull>{});
      return true;
    }
    chunk_body(kt, src, pg_ok, std::integral_constant<int, kPart>{});
    return false;
  };
  // Wait for this wave's loads of the chunk about to be published. After a chunk
  // that stored every key (a fixed number of stores, issued after the loads), the
  // stores may stay in flight: vector-memory operations complete in issue order.
  constexpr int kStores = (kChunk / 32) * MT * RH;
  static_assert(kStores < 64, "vmcnt holds at most 63");
  // s_waitcnt immediate for vmcnt(N) alone (expcnt and lgkmcnt at their maxima)
  constexpr int kWaitStores = (kStores & 15) | ((kStores >> 4) << 14) | 0x0F70;
  auto wait_loads = [&](bool stores_fixed) __attribute__((always_inline)) {
    if (stores_fixed) __builtin_amdgcn_s_waitcnt(kWaitStores);
    else __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  };
  // Two LDS chunks (distinct arrays, so the compiler sees that a chunk's reads and
  // the next chunk's loads touch different memory). Each wave waits for its own
  // loads of a chunk just before the barrier that publishes it, so the loads of the
  // next chunk overlap this one's MFMAs.
  if (kb < kend) issue(kb, kc0.k);
  bool fixed = false;   // nothing but the first chunk's loads in flight
  for (int64_t kt = kb; kt < kend; kt += 2 * kChunk) {
    wait_loads(fixed);
    __syncthreads();   // every wave's loads of chunk kt have landed; the other chunk is free
    if (kt + kChunk < kend) issue(kt + kChunk, kc1.k);
    fixed = chunk(kt, kc0.k) && kt + kChunk < kend;
    if (kt + kChunk >= kend) break;
    wait_loads(fixed);
    __syncthreads();
    if (kt + 2 * kChunk < kend) issue(kt + 2 * kChunk, kc0.k);
    fixed = chunk(kt + kChunk, kc1.k) && kt + 2 * kChunk < kend;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // keys past every row's compressed length
  const int64_t kf = kend > kb ? kend : kb;
  for (int rr = wave; rr < ROWS; rr += 4)
    for (int64_t key = kf + lane; key < ke; key += 64) a.logits[(int64_t)(row_base + rr) * a.ldo + key] = ninf;
}

template <int H, int D>
static tf_status launch_hd(IdxArgs a, int32_t n_rows, hipStream_t st, bool window) {
  constexpr int RPT = 32 / H;
  if (n_rows >= 64) {
    constexpr int MT = 2;
    constexpr int ROWS = 4 * MT * RPT;
    const int64_t rgroups = (n_rows + ROWS - 1) / ROWS;
    // about 1,024 workgroups (four per CU), each over a multiple of 128 keys (at most 4,096)
    const int64_t nk = a.kend - a.key0;
    int64_t kpw = (nk * rgroups + 1023) / 1024;
    kpw = (kpw + 127) / 128 * 128;
    if (kpw < 128) kpw = 128;
    if (kpw > 4096) kpw = 4096;
    a.keys_per_wg = (int32_t)kpw;
    const int64_t kgroups = (nk + kpw - 1) / kpw;
    a.n_kgroups = (int32_t)kgroups;
    if (rgroups > 65535) return set_error(TF_E_RANGE, "tf_indexer_logits: too many rows for one launch");
    if (window)
      hipLaunchKernelGGL((indexer_tile_kernel<H, D, MT, true>), dim3((unsigned)kgroups, (unsigned)rgroups),
                         dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((indexer_tile_kernel<H, D, MT, false>), dim3((unsigned)kgroups, (unsigned)rgroups),
                         dim3(256), 0, st, a);
  } else {
    // each wave one row; about 2,048 waves in all (eight per CU keep more key loads in
    // flight than four); a wave's range spans at most 64 pages
    const int n_rg = (n_rows + 3) / 4;
    const int64_t nk = a.kend - a.key0;
    int64_t kpw = (nk * n_rows + 2047) / 2048;
    kpw = (kpw + 127) / 128 * 128;
    if (kpw < 128) kpw = 128;
    if (kpw > 64 * 128) kpw = 64 * 128;
    a.keys_per_wg = (int32_t)kpw;
    const int64_t kgroups = (nk + kpw - 1) / kpw;
    a.n_kgroups = (int32_t)kgroups;
    const int64_t grid = ((kgroups + 7) / 8) * 8 * n_rg;
    if (grid > 0x7fffffffLL) return set_error(TF_E_RANGE, "tf_indexer_logits: too many keys for one launch");
    hipLaunchKernelGGL((indexer_rows_kernel<H, D>), dim3((unsigned)grid), dim3(256), 0, st, a);
  }
  return TF_OK;
}

tf_status launch_indexer(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                         const int32_t* row_pos, const void* q, const float* w, int32_t n_heads,
                         float* logits, int64_t ld, int32_t* n_valid, hipStream_t st, int64_t key0,
                         int64_t kend, int64_t ncap, bool window) {
  IdxArgs a;
  a.v = v;
  a.off_pkey = p->off_pkey;
  a.pkey_row_bytes = (int32_t)p->pkey_row_bytes;
  a.n_rows = n_rows;
  a.row_stream = row_stream;
  a.row_pos = row_pos;
  a.q = (const __bf16*)q;
  a.w = w;
  a.logits = (float*)((uintptr_t)logits - (uintptr_t)key0 * sizeof(float));   // never read below logits
  a.ldo = ld;
  a.key0 = key0;
  a.kend = kend;
  a.ncap = ncap;
  a.n_valid = n_valid;
  a.keys_per_wg = 128;
  a.n_kgroups = 1;
  const int D = p->g.index_dim;
  tf_status s;
  if (D == 128) {
    if (n_heads == 16) s = launch_hd<16, 128>(a, n_rows, st, window);
    else if (n_heads == 8) s = launch_hd<8, 128>(a, n_rows, st, window);
    else s = launch_hd<4, 128>(a, n_rows, st, window);
  } else {
    if (n_heads == 16) s = launch_hd<16, 64>(a, n_rows, st, window);
    else if (n_heads == 8) s = launch_hd<8, 64>(a, n_rows, st, window);
    else s = launch_hd<4, 64>(a, n_rows, st, window);
  }
  if (s != TF_OK) return s;
  return launch_status("tf_indexer_logits");
}

}  // namespace tf
