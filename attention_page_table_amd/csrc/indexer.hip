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
//    wave streams one row's keys straight into B fragments, three subtiles ahead, with
//    the row's page ids preloaded across the lanes. Its shared-page instance (ranges
//    of several pages, 16 heads) scores a row group of four streams that name the same
//    pages (a prefix held by reference) from one load of each page.
#include <type_traits>

#include "select.h"

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
  int32_t page_step;     // sampled scoring: logical page i is page i * page_step of the stream
  // filtered scoring: a key whose logit's order key is at least thr[row] goes to its
  // (row, key group) region of cap slots, in key order; cand_cnt counts them all
  const uint32_t* thr;
  uint32_t* cand_key;    // [n_rows][n_kgroups][cap] order keys
  int32_t* cand_idx;     // [n_rows][n_kgroups][cap] key indices
  int32_t* cand_cnt;     // [n_rows][n_kgroups]
  int32_t cap;
};

// What a tile-kernel instance computes (one instance each, so that profiles keep the
// launches apart): every key, one key block of a key-blocked call, a page sample, or
// the filtered candidates.
constexpr int kWhole = 0, kWindow = 1, kSample = 2, kFilter = 3;

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

// The row's visible keys: n_c = min(t / 4 + 1, ncap). Sampled scoring counts the
// logical keys of the sampled pages below n_c (a prefix of the logical keys, since
// page i of the sample is page i * page_step).
template <bool SAMPLED = false>
__device__ __forceinline__ int nc_of(const IdxArgs& a, int row) {
  const int pos = a.row_pos[row];
  if (pos < 0) return 0;
  int64_t nc = (int64_t)pos / kPoolRatio + 1;
  if (nc > a.ncap) nc = a.ncap;
  if (!SAMPLED) return (int)nc;
  const int64_t pl = (nc - 1) / kKeysPerPage;   // page of the last visible key
  const int64_t il = pl / a.page_step;           // last sampled page at or below it
  const int64_t c = il * kKeysPerPage + (il * a.page_step == pl ? nc - pl * kKeysPerPage : kKeysPerPage);
  return (int)(c < a.kend ? c : a.kend);
}

// Appends this lane's key to its row's region when `pass`, in lane order within each
// half-wave (half g holds the keys of one row): slot = count so far + passing lanes
// below it in the half. cnt is uniform over the half and grows by the half's passes.
__device__ __forceinline__ void append_candidate(const IdxArgs& a, bool pass, uint32_t u, int64_t key, int g,
                                                 int32_t off, int32_t& cnt) {
  const uint64_t m = __ballot(pass);
  const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
  const uint32_t below = g ? __builtin_amdgcn_mbcnt_hi(hi, 0u) : __builtin_amdgcn_mbcnt_lo(lo, 0u);
  const int32_t slot = cnt + (int32_t)below;
  if (pass && slot < a.cap) {
    a.cand_key[off + slot] = u;
    a.cand_idx[off + slot] = (int32_t)key;
  }
  cnt += (int32_t)__builtin_popcount(g ? hi : lo);
}

// ---- per-row path: one wave streams one row over keys [kb, ke) ---------------------------
// A-rows with bit 2 clear carry the row's heads (head 4 * (m / 8) + m % 4), the others are
// zero; lanes 0..31 then hold every head of key n = lane in accumulators 0..H-1.
template <int H, int D, int KIND>
__device__ void index_one_row(const IdxArgs& a, int row, int64_t kb, int64_t ke, int lane, int kg,
                              bool spec_page = false, int spec_page_all = -1) {
  constexpr bool FILTER = KIND == kFilter, SAMPLED = KIND == kSample;
  constexpr int KS = D / 16;
  const int g = lane >> 5, n = lane & 31;
  const int b = a.row_stream[row];
  const int nc = nc_of<SAMPLED>(a, row);
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
    my_page = page_of(a.v, b, SAMPLED ? (p0 + lane) * a.page_step : p0 + lane);
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
  // filtered: the row's threshold, region and count (lanes 0..31 hold the keys)
  const uint32_t thr = FILTER ? a.thr[row] : 0u;
  const int32_t off = FILTER ? (row * a.n_kgroups + kg) * a.cap : 0;
  int32_t cnt = 0;
  // three subtiles in flight: slot s holds subtile kb + 32 (3i + s)
  auto step = [&](int64_t kt, bf16x8 (&cur)[KS]) {
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[ks], cur[ks], acc, 0, 0, 0);
    const int pg = page_at(kt);
    if (kt + 96 < kend) load(kt + 96, cur);   // refill the slot three subtiles ahead
    const float s = weighted_relu_sum<H>(wv, acc, 0);
    const int64_t key = kt + n;
    if constexpr (FILTER) {
      const uint32_t u = order_key(pg >= 0 ? s : __builtin_nanf(""));
      append_candidate(a, g == 0 && key < ke && key < nc && u >= thr, u, key, g, off, cnt);
    } else {
      if (g == 0 && key < ke) out[key] = key < nc ? (pg >= 0 ? s : __builtin_nanf("")) : ninf;
    }
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
  if constexpr (FILTER) {
    if (lane == 0) a.cand_cnt[row * a.n_kgroups + kg] = cnt;
    return;
  }
  // keys past the compressed length
  for (int64_t key = (kend > kb ? kend : kb) + lane; key < ke; key += 64) out[key] = ninf;
}

// Four rows whose streams name the same pages over most of [kb, ke) (a prefix held by
// reference, [#1732] "What this changes"): each shared page is loaded once for all
// four rows. Wave w scores subtiles w, w + 4, w + 8, ... of the range (the w-th 32 keys
// of each page) for the four rows, as two MFMA tiles of two rows x 16 heads (lanes
// 0..31 hold the first row of a tile, lanes 32..63 the second; a lane holds one key and
// all 16 heads). A page the four do not share (bit i of shared clear for page
// kb / 128 + i; pgs[r][i] is row r's page id) is loaded and scored once per row. Each
// (row, key) is the same MFMA dot product, head sum and store as on the per-row path,
// so the logits are bit for bit the same.
template <int D>
__device__ void index_four_rows_shared(const IdxArgs& a, int row0, int64_t kb, int64_t ke, int wave, int lane,
                                       const int32_t (*pgs)[64], uint64_t shared) {
  constexpr int H = 16, KS = D / 16;
  const int g = lane >> 5, n = lane & 31;
  const float ninf = -__builtin_inff();
  const float qnan = __builtin_nanf("");
  int nc[2] = {0, 0}, ncmax = 0;   // nc[t]: this lane's row of tile t, row0 + 2 t + g
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = nc_of(a, row0 + r);
    ncmax = c > ncmax ? c : ncmax;
    if ((r & 1) == g) nc[r >> 1] = c;
  }
  const int64_t kend = ke < ncmax ? ke : ncmax;
  // A fragments as in the tile kernel: A-row m = 8a + 4b + c is head 4a + c of row b
  bf16x8 af[2][KS];
  {
    const int mb = (n >> 2) & 1, head = 4 * (n >> 3) + (n & 3);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        af[t][ks] = *(const bf16x8*)(a.q + ((int64_t)(row0 + 2 * t + mb) * H + head) * D + ks * 16 + g * 8);
  }
  float wv[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) wv[t][i] = a.w[(int64_t)(row0 + 2 * t + g) * H + i];
  float* out0 = a.logits + (int64_t)(row0 + g) * a.ldo;
  float* out1 = a.logits + (int64_t)(row0 + 2 + g) * a.ldo;
  const int p0 = (int)(kb / kKeysPerPage);
  // the page of subtile kt for row r (uniform: read from LDS)
  auto page_at = [&](int64_t kt, int r) { return pgs[r][(int)(kt / kKeysPerPage) - p0]; };
  auto load_pg = [&](int pg, int64_t kt, bf16x8 (&bf)[KS]) {
    if (pg >= 0) {
      const char* kp = cache_block(a.v, pg) + a.off_pkey + (int64_t)((kt % kKeysPerPage) + n) * a.pkey_row_bytes + g * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[ks] = *(const bf16x8*)(kp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[ks] = bf16x8{};
    }
  };
  auto load = [&](int64_t kt, bf16x8 (&bf)[KS]) { load_pg(page_at(kt, 0), kt, bf); };
  // two of the wave's subtiles in flight: slot s holds subtile kb + 32 wave + 128 (2 i + s)
  // (the row groups of a range request each page at about the same time, so the second
  // request of a page meets the first in L2)
  auto step = [&](int64_t kt, bf16x8 (&cur)[KS]) {
    const int64_t key = kt + n;
    if (!((shared >> ((int)(kt / kKeysPerPage) - p0)) & 1)) {
      // a page the rows do not share: each row's own page, scored by the tile that
      // holds the row; the row's half-wave stores
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pr = page_at(kt, r);
        load_pg(pr, kt, cur);
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[r >> 1][ks], cur[ks], acc, 0, 0, 0);
        const float s = weighted_relu_sum<H>(wv[r >> 1], acc, 0);
        if (g == (r & 1) && key < ke) {
          float* o = r >> 1 ? out1 : out0;
          o[key] = key < nc[r >> 1] ? (pr >= 0 ? s : qnan) : ninf;
        }
      }
      if (kt + 2 * kKeysPerPage < kend) load(kt + 2 * kKeysPerPage, cur);
      return;
    }
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][ks], cur[ks], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1][ks], cur[ks], acc1, 0, 0, 0);
    }
    const int pg = page_at(kt, 0);
    if (kt + 2 * kKeysPerPage < kend) load(kt + 2 * kKeysPerPage, cur);
    const float s0 = weighted_relu_sum<H>(wv[0], acc0, 0);
    const float s1 = weighted_relu_sum<H>(wv[1], acc1, 0);
    if (key < ke) {
      out0[key] = key < nc[0] ? (pg >= 0 ? s0 : qnan) : ninf;
      out1[key] = key < nc[1] ? (pg >= 0 ? s1 : qnan) : ninf;
    }
  };
  bf16x8 s0[KS], s1[KS];
  const int64_t k0 = kb + 32 * wave;
  if (k0 < kend) load(k0, s0);
  if (k0 + kKeysPerPage < kend) load(k0 + kKeysPerPage, s1);
  for (int64_t kt = k0; kt < kend; kt += 2 * kKeysPerPage) {
    step(kt, s0);
    if (kt + kKeysPerPage < kend) step(kt + kKeysPerPage, s1);
  }
  // keys past every row's compressed length: wave w fills row row0 + w
  float* o = a.logits + (int64_t)(row0 + wave) * a.ldo;
  for (int64_t key = (kend > kb ? kend : kb) + lane; key < ke; key += 64) o[key] = ninf;
}

// Per-row kernel: wave w of workgroup (key group kg, row group rg) takes row 4 rg + w.
// The row groups of one key group run on one XCD (workgroups 8 apart).
// SHARED (16 heads, whole calls, ranges of several pages, at least four rows): a row
// group whose streams name the same pages over at least half its range takes the
// shared-page path (indexer_shared_rows_kernel; the other calls run a kernel without it).
template <int H, int D, int KIND, bool SHARED>
__device__ __forceinline__ void rows_body(const IdxArgs& a) {
  constexpr bool SAMPLED = KIND == kSample;
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
    const int pi = (int)(kb / kKeysPerPage) * (SAMPLED ? a.page_step : 1);
    if (lane < a.v.n_streams && pi < a.v.pt_stride) {
      const int pg = a.v.pt ? a.v.pt[(int64_t)lane * a.v.pt_stride + pi] : lane * a.v.pt_stride + pi;
      spec_all = pg >= 0 && pg < a.v.n_pages ? pg : -1;
    }
  }
  if (kg == 0 && a.n_valid && lane == 0) a.n_valid[row] = nc_of<SAMPLED>(a, row);
  if constexpr (SHARED && H == 16 && KIND == kWhole) {
    // where the four streams of a row group name the same pages (a shared prefix) over
    // at least half the range, load those pages once for the four rows
    if (ke - kb > kKeysPerPage && (rg + 1) * 4 <= a.n_rows) {
      __shared__ int32_t pgs[4][64];
      const int p0 = (int)(kb / kKeysPerPage);
      const int np = (int)((ke - 1) / kKeysPerPage) - p0 + 1;
      pgs[wave][lane] = page_of(a.v, a.row_stream[row], p0 + lane);
      __syncthreads();
      const bool same =
          lane < np && pgs[0][lane] == pgs[1][lane] && pgs[0][lane] == pgs[2][lane] && pgs[0][lane] == pgs[3][lane];
      const uint64_t shared = __ballot(same);
      if (2 * __builtin_popcountll(shared) >= np) {
        index_four_rows_shared<D>(a, rg * 4, kb, ke, wave, lane, pgs, shared);
        return;
      }
    }
  }
  index_one_row<H, D, KIND>(a, row, kb, ke, lane, kg, spec, spec_all);
}

template <int H, int D, int KIND>
__global__ __launch_bounds__(256) void indexer_rows_kernel(IdxArgs a) {
  rows_body<H, D, KIND, false>(a);
}

template <int D>
__global__ __launch_bounds__(256) void indexer_shared_rows_kernel(IdxArgs a) {
  rows_body<16, D, kWhole, true>(a);
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

// KIND: kWhole, kWindow and kSample store logits (the same code; the sample's pages are
// strided through page_step); kFilter appends the keys at or above each row's threshold
// to the row's region for this workgroup's key group instead.
template <int H, int D, int MT, int KIND>
__global__ __launch_bounds__(256, 2) void indexer_tile_kernel(IdxArgs a) {
  constexpr bool FILTER = KIND == kFilter, SAMPLED = KIND == kSample;
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
    a.n_valid[row_base + tid] = nc_of<SAMPLED>(a, row_base + tid);

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
        if (H == 16) index_one_row<16, D, KIND>(a, row, kb, ke, lane, blockIdx.x);
        else if (H == 8) index_one_row<8, D, KIND>(a, row, kb, ke, lane, blockIdx.x);
        else index_one_row<4, D, KIND>(a, row, kb, ke, lane, blockIdx.x);
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
    for (int r = 0; r < RH; ++r) rnc[t][r] = nc_of<SAMPLED>(a, wave_row0 + t * RPT + g * RH + r);
  for (int rr = 0; rr < ROWS; ++rr) {
    const int c = nc_of<SAMPLED>(a, row_base + rr);
    nc_max = c > nc_max ? c : nc_max;
    nc_min = c < nc_min ? c : nc_min;
  }
  const int64_t kend = ke < nc_max ? ke : nc_max;

  // page ids of the key range
  const int p0 = (int)(kb / kKeysPerPage);
  if (tid < kMaxPages) pg_lds[tid] = page_of(a.v, b0, SAMPLED ? (p0 + tid) * a.page_step : p0 + tid);

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
  // filtered: each row's threshold, region offset and count so far
  uint32_t thr[MT][RH];
  int32_t coff[MT][RH], cnt[MT][RH];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < RH; ++r) {
      const int row = wave_row0 + t * RPT + g * RH + r;
      if constexpr (FILTER) {
        thr[t][r] = a.thr[row];
        coff[t][r] = (row * a.n_kgroups + (int)blockIdx.x) * a.cap;
        cnt[t][r] = 0;
      } else {
        optr[t][r] = a.logits + (int64_t)row * a.ldo + n;
      }
    }
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
  constexpr int kValu = FILTER ? 6 : 4;   // head-sum (and append) instructions per MFMA
  auto epilogue = [&](const f32x16& acc, int t, int64_t kt, bool pg_ok, auto mode) __attribute__((always_inline)) {
    constexpr int M = decltype(mode)::value;
    const int64_t key = kt + n;
#pragma unroll
    for (int r = 0; r < RH; ++r) {
      const float s = weighted_relu_sum<H>(&wv[t][r * H], acc, r * H);
      if constexpr (FILTER) {
        const bool in = M == kOpen || (key < rnc[t][r] && (M == kFull || key < ke));
        const uint32_t u = order_key(M == kOpen || pg_ok ? s : qnan);
        append_candidate(a, in && u >= thr[t][r], u, key, g, coff[t][r], cnt[t][r]);
        continue;
      }
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
          // tile only) and kValu instructions of the previous tile's head sum
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (t == MT - 1 && sub + 1 < kSubs) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (t > 0 || sub > 0) __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
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
    if constexpr (FILTER) {   // a data-dependent number of stores: the next wait takes them all
      if (kt + kChunk <= ke && pg_ok && kt + kChunk <= nc_min)
        chunk_body(kt, src, pg_ok, std::integral_constant<int, kOpen>{});
      else if (kt + kChunk <= ke)
        chunk_body(kt, src, pg_ok, std::integral_constant<int, kFull>{});
      else
        chunk_body(kt, src, pg_ok, std::integral_constant<int, kPart>{});
      return false;
    }
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
  if constexpr (FILTER) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < RH; ++r)
        if (n == 0) a.cand_cnt[(wave_row0 + t * RPT + g * RH + r) * a.n_kgroups + (int)blockIdx.x] = cnt[t][r];
    return;
  }
  // keys past every row's compressed length
  const int64_t kf = kend > kb ? kend : kb;
  for (int rr = wave; rr < ROWS; rr += 4)
    for (int64_t key = kf + lane; key < ke; key += 64) a.logits[(int64_t)(row_base + rr) * a.ldo + key] = ninf;
}

// Launch shape of a scoring call over nk keys: the tile kernel (n_rows >= 64) with
// about 1,024 workgroups (four per CU), each over a multiple of 128 keys (at most
// 4,096), or the row kernel with about 2,048 waves (eight per CU keep more key loads in
// flight than four), a wave's range spanning at most 64 pages.
struct IdxShape {
  bool tile;
  int64_t kpw, kgroups, grid_x, grid_y;
};

// wg_target: workgroups the tile kernel aims at; min_kpw: a floor on the keys per
// workgroup or wave (a multiple of 128).
static IdxShape idx_shape(int H, int32_t n_rows, int64_t nk, int64_t wg_target = 1024, int64_t min_kpw = 128) {
  IdxShape s;
  s.tile = n_rows >= 64;
  int64_t kpw;
  if (s.tile) {
    const int rows = 4 * 2 * (32 / H);   // 4 waves x MT = 2 tiles x 32 / H rows
    const int64_t rgroups = (n_rows + rows - 1) / rows;
    kpw = (nk * rgroups + wg_target - 1) / wg_target;
    kpw = (kpw + 127) / 128 * 128;
    kpw = kpw < min_kpw ? min_kpw : kpw;
    kpw = kpw < 128 ? 128 : (kpw > 4096 ? 4096 : kpw);
    s.kgroups = (nk + kpw - 1) / kpw;
    s.grid_x = s.kgroups;
    s.grid_y = rgroups;
  } else {
    kpw = (nk * n_rows + 2047) / 2048;
    kpw = (kpw + 127) / 128 * 128;
    kpw = kpw < min_kpw ? min_kpw : kpw;
    kpw = kpw < 128 ? 128 : (kpw > 64 * 128 ? 64 * 128 : kpw);
    s.kgroups = (nk + kpw - 1) / kpw;
    s.grid_x = ((s.kgroups + 7) / 8) * 8 * ((n_rows + 3) / 4);
    s.grid_y = 1;
  }
  s.kpw = kpw;
  return s;
}

template <int H, int D>
static tf_status launch_hd(IdxArgs a, int32_t n_rows, hipStream_t st, int kind, int64_t wg_target = 1024,
                           int64_t min_kpw = 128) {
  const IdxShape sh = idx_shape(H, n_rows, a.kend - a.key0, wg_target, min_kpw);
  a.keys_per_wg = (int32_t)sh.kpw;
  a.n_kgroups = (int32_t)sh.kgroups;
  if (sh.tile) {
    constexpr int MT = 2;
    if (sh.grid_y > 65535) return set_error(TF_E_RANGE, "tf_indexer_logits: too many rows for one launch");
    const dim3 grid((unsigned)sh.grid_x, (unsigned)sh.grid_y);
    switch (kind) {
      case kWhole: hipLaunchKernelGGL((indexer_tile_kernel<H, D, MT, kWhole>), grid, dim3(256), 0, st, a); break;
      case kWindow: hipLaunchKernelGGL((indexer_tile_kernel<H, D, MT, kWindow>), grid, dim3(256), 0, st, a); break;
      case kSample: hipLaunchKernelGGL((indexer_tile_kernel<H, D, MT, kSample>), grid, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((indexer_tile_kernel<H, D, MT, kFilter>), grid, dim3(256), 0, st, a); break;
    }
  } else {
    if (sh.grid_x > 0x7fffffffLL) return set_error(TF_E_RANGE, "tf_indexer_logits: too many keys for one launch");
    const dim3 grid((unsigned)sh.grid_x);
    switch (kind) {
      case kSample: hipLaunchKernelGGL((indexer_rows_kernel<H, D, kSample>), grid, dim3(256), 0, st, a); break;
      case kFilter: hipLaunchKernelGGL((indexer_rows_kernel<H, D, kFilter>), grid, dim3(256), 0, st, a); break;
      default:
        if (H == 16 && sh.kpw > kKeysPerPage && n_rows >= 4)
          hipLaunchKernelGGL((indexer_shared_rows_kernel<D>), grid, dim3(256), 0, st, a);
        else
          hipLaunchKernelGGL((indexer_rows_kernel<H, D, kWhole>), grid, dim3(256), 0, st, a);
        break;
    }
  }
  return TF_OK;
}

static IdxArgs base_args(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                         const int32_t* row_pos, const void* q, const float* w) {
  IdxArgs a;
  a.v = v;
  a.off_pkey = p->off_pkey;
  a.pkey_row_bytes = (int32_t)p->pkey_row_bytes;
  a.n_rows = n_rows;
  a.row_stream = row_stream;
  a.row_pos = row_pos;
  a.q = (const __bf16*)q;
  a.w = w;
  a.logits = nullptr;
  a.ldo = 0;
  a.key0 = 0;
  a.kend = 0;
  a.ncap = 0;
  a.n_valid = nullptr;
  a.keys_per_wg = 128;
  a.n_kgroups = 1;
  a.page_step = 1;
  a.thr = nullptr;
  a.cand_key = nullptr;
  a.cand_idx = nullptr;
  a.cand_cnt = nullptr;
  a.cap = 0;
  return a;
}

static tf_status launch_any(const tf_plan* p, IdxArgs a, int32_t n_heads, int32_t n_rows, hipStream_t st, int kind) {
  const int D = p->g.index_dim;
  if (D == 128) {
    if (n_heads == 16) return launch_hd<16, 128>(a, n_rows, st, kind);
    if (n_heads == 8) return launch_hd<8, 128>(a, n_rows, st, kind);
    return launch_hd<4, 128>(a, n_rows, st, kind);
  }
  if (n_heads == 16) return launch_hd<16, 64>(a, n_rows, st, kind);
  if (n_heads == 8) return launch_hd<8, 64>(a, n_rows, st, kind);
  return launch_hd<4, 64>(a, n_rows, st, kind);
}

tf_status launch_indexer(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                         const int32_t* row_pos, const void* q, const float* w, int32_t n_heads,
                         float* logits, int64_t ld, int32_t* n_valid, hipStream_t st, int64_t key0,
                         int64_t kend, int64_t ncap, bool window) {
  IdxArgs a = base_args(p, v, n_rows, row_stream, row_pos, q, w);
  a.logits = (float*)((uintptr_t)logits - (uintptr_t)key0 * sizeof(float));   // never read below logits
  a.ldo = ld;
  a.key0 = key0;
  a.kend = kend;
  a.ncap = ncap;
  a.n_valid = n_valid;
  const tf_status s = launch_any(p, a, n_heads, n_rows, st, window ? kWindow : kWhole);
  if (s != TF_OK) return s;
  return launch_status("tf_indexer_logits");
}

// ---- fused indexer + top-k [CPM, section 2.3: only per-block candidates leave the
// scoring; topk(union) == topk(union of per-block topk)] ---------------------------------
// Exactness needs only that at least k keys of a row reach its threshold: the k-th
// largest logit is then at or above it, so the row's top k, ties with the k-th value
// included, are all candidates, and their top k is the answer.
// 1. Page sample: the tile (or row) kernel scores every step-th page of each row into a
//    [n_rows][S] buffer (S about a sixteenth of the keys, at least 2,048), in a launch
//    of about 512 workgroups (one round on the chip).
// 2. Threshold: thr[r] = about the k'-th largest sampled order key (its top 16 bits),
//    k' = min(k, the sample's share of 2k), so that about 2k of the row's keys reach it
//    (0, which every key passes, when the sample holds at most k'). One wave a row.
// 3. Filtered scoring: every key again, with the same arithmetic, but a key leaves the
//    kernel only when its order key is >= thr[r], appended in key order to the region of
//    its (row, key group): no logits reach memory.
// 4. Selection: the top k of each row's candidates (the regions in key-group order are in
//    key order, so the tie rule holds), one wave a row for up to 2,048 candidates, the
//    whole workgroup for up to 32,768. A row with fewer than k candidates or an
//    overflowed region (more passes than slots) is re-scored inside the selection kernel
//    instead: three radix passes, a count and an emission, each scoring its keys anew.
// Rows of at most max(4,096, 8k) keys are scored whole into the workspace and selected
// there (the candidates would be a large share of the keys anyway), and so are calls of
// fewer than 64 rows of at most kFewRowsKeys keys: a decode batch's logits are small
// (8 rows x 32,768 keys: 1 MB), and its four dependent launches on few rows took 58 us
// against 33 us for the scoring and top-k kernels of the unfused pair.

constexpr int kMaxRegions = 512;   // key groups of the filtered pass
constexpr int64_t kFewRowsKeys = 1 << 18;   // longest rows a call of fewer than 64 scores whole
constexpr int kSelRows = 8;        // rows of a selection workgroup, one a wave
constexpr int kWaveCand = 24;      // candidates a lane holds in the one-wave selection

struct FusedPlan {
  bool direct;        // short rows: score whole rows into the sample buffer and select there
  int32_t step;       // sampled page stride
  int64_t S;          // sampled keys per row (a multiple of 128)
  IdxShape shape;     // the filtered pass's launch
  int64_t min_kpw;    // its floor on keys per workgroup (at most kMaxRegions key groups)
  int32_t cap;        // slots per (row, key group) region
  int32_t e_thr;      // lane values of the one-wave threshold (32, 64), or 0: the block one
  size_t off_smp, off_nvs, off_thr, off_nv, off_cnt, off_ck, off_ci, bytes;
  size_t off_tws, tws;   // direct: the top-k's own workspace (its blocked mode on few long rows)
};

static FusedPlan fused_plan(int H, int32_t n_rows, int64_t ld, int32_t k) {
  FusedPlan f = {};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const int64_t pages = (ld + kKeysPerPage - 1) / kKeysPerPage;
  if (ld <= 4096 || ld <= 8 * (int64_t)k || (n_rows < 64 && ld <= kFewRowsKeys)) {
    f.direct = true;
    f.step = 1;
    f.S = ld;
    f.off_smp = take((size_t)n_rows * ld * 4);
    f.off_nv = take((size_t)n_rows * 4);
    f.tws = topk_ws_bytes(n_rows, ld, k);
    if (f.tws == (size_t)-1) {
      f.bytes = (size_t)-1;
      return f;
    }
    f.off_tws = take(f.tws);
    f.bytes = at;
    return f;
  }
  int64_t sp = (pages + 15) / 16;
  if (sp < 16) sp = 16;
  f.step = (int32_t)((pages + sp - 1) / sp);
  sp = (pages + f.step - 1) / f.step;
  f.S = sp * kKeysPerPage;
  f.e_thr = f.S <= 2048 ? 32 : (f.S <= 4096 ? 64 : 0);
  int64_t mk = (ld + kMaxRegions - 1) / kMaxRegions;
  f.min_kpw = (mk + 127) / 128 * 128;
  f.shape = idx_shape(H, n_rows, ld, 1024, f.min_kpw);
  // slots: twice the passes expected of a row of ld keys (kpw * 2k / ld) plus 32, at
  // most kpw (the sample's threshold moves a row's candidates by up to about a half)
  int64_t cap = (int64_t)(2.0 * (double)f.shape.kpw * 2.0 * k / (double)ld) + 32;
  cap = (cap + 3) / 4 * 4;
  f.cap = (int32_t)(cap < f.shape.kpw ? cap : f.shape.kpw);
  const size_t regions = (size_t)n_rows * f.shape.kgroups;
  f.off_smp = take((size_t)n_rows * f.S * 4);
  f.off_nvs = take((size_t)n_rows * 4);
  f.off_thr = take((size_t)n_rows * 4);
  f.off_nv = take((size_t)n_rows * 4);
  f.off_cnt = take(regions * 4);
  f.off_ck = take(regions * f.cap * 4);
  f.off_ci = take(regions * f.cap * 4);
  f.bytes = at;
  return f;
}

size_t indexer_topk_fused_ws_bytes(int32_t n_heads, int32_t n_rows, int64_t ld, int32_t k) {
  return fused_plan(n_heads, n_rows, ld, k).bytes;
}

// k' = min(k, ceil(2k n / n_c)): the sample's share of 2k candidates (n sampled keys
// visible to a row of n_c keys)
__device__ __forceinline__ uint32_t sample_rank(int n, int pos, int64_t ncap, int32_t k) {
  const int64_t nc = pos < 0 ? 0 : ((int64_t)pos / kPoolRatio + 1 < ncap ? (int64_t)pos / kPoolRatio + 1 : ncap);
  int64_t kk = nc > 0 ? (2 * (int64_t)k * n + nc - 1) / nc : k;
  return (uint32_t)(kk < 1 ? 1 : (kk > k ? k : kk));
}

// One wave a row (four a workgroup); the sample (S <= 64 E) in registers.
template <int E>
__global__ __launch_bounds__(256) void fused_threshold_kernel(const float* smp, int32_t S, const int32_t* nv_s,
                                                             const int32_t* row_pos, int64_t ncap, int32_t k,
                                                             int32_t n_rows, uint32_t* thr) {
  __shared__ uint32_t hist[4][256];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.x * 4 + wid;
  if (r >= n_rows) return;
  int n = nv_s[r];
  n = n < 0 ? 0 : (n > S ? S : n);
  const uint32_t kk = sample_rank(n, row_pos[r], ncap, k);
  if ((uint32_t)n <= kk) {   // every visible key is a candidate
    if (lane == 0) thr[r] = 0u;
    return;
  }
  // every load issued before any is used: a load inside a branch on i < n would wait
  // for its own data before the next one starts
  uint32_t key[E];
  const float* row = smp + (int64_t)r * S;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = row[e * 64 + lane < n ? e * 64 + lane : n - 1];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = e * 64 + lane < n ? order_key(v[e]) : 0u;
  uint32_t T, rem;
  wave_select<E>(key, kk, 16, hist[wid], T, rem);
  if (lane == 0) thr[r] = T;
}

// Long samples: one workgroup a row, the exact k'-th largest.
template <int E>
__global__ __launch_bounds__(kNT) void fused_threshold_block_kernel(const float* smp, int32_t S,
                                                                   const int32_t* nv_s, const int32_t* row_pos,
                                                                   int64_t ncap, int32_t k, uint32_t* thr) {
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  int n = nv_s[r];
  n = n < 0 ? 0 : (n > S ? S : n);
  const uint32_t kk = sample_rank(n, row_pos[r], ncap, k);
  if ((uint32_t)n <= kk) {
    if (threadIdx.x == 0) thr[r] = 0u;
    return;
  }
  uint32_t key[E];
  load_keys<E, true>(smp + (int64_t)r * S, n, key);
  uint32_t T, rem;
  radix_select<E>(key, (int)kk, sh, T, rem);
  if (threadIdx.x == 0) thr[r] = T;
}

struct FusedSel {
  IdxArgs a;            // the filtered pass's arguments (regions; re-scoring)
  const int32_t* nv;    // n_c per row, from the filtered pass
  int32_t* n_valid;     // the caller's, optional
  int32_t k;
  int32_t* blocks;
};

// The top k of row `row` (n_c = nv > k) by re-scoring its keys, with the filtered
// pass's arithmetic (one row's heads on the A rows of the row kernel's layout; a
// product's value does not depend on where its operands sit in the tile): three
// most-significant-digit radix passes find the k-th largest order key T and how many
// keys equal to it are taken, then a pass counts each wave's keys above and equal to T
// and a last pass writes the selected indices, ascending. Wave w scores a contiguous
// run of 32-key subtiles, so the waves' runs are in key order.
template <int H, int D>
__device__ void rescore_select(const IdxArgs& a, int row, int nv, int k, int32_t* out, SelShared& sh) {
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = a.row_stream[row];
  bf16x8 aq[KS];
  {
    const int u = 4 * (n >> 3) + (n & 3);
    const bool live = ((n >> 2) & 1) == 0 && u < H;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      aq[ks] = live ? *(const bf16x8*)(a.q + ((int64_t)row * H + u) * D + ks * 16 + g * 8) : bf16x8{};
  }
  float wv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) wv[i] = i < H ? a.w[(int64_t)row * H + i] : 0.f;
  const int n_sub = (nv + 31) / 32;
  const int spw = (n_sub + kWaves - 1) / kWaves;
  const int s0 = wid * spw;
  const int s1 = s0 + spw < n_sub ? s0 + spw : n_sub;
  auto score = [&](int sub) -> uint32_t {
    const int64_t kt = (int64_t)sub * 32;
    const int pg = page_of(a.v, b, (int)(kt / kKeysPerPage));
    bf16x8 bf[KS];
    if (pg >= 0) {
      const char* kp = cache_block(a.v, pg) + a.off_pkey + (int64_t)((kt % kKeysPerPage) + n) * a.pkey_row_bytes + g * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[ks] = *(const bf16x8*)(kp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[ks] = bf16x8{};
    }
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[ks], bf[ks], acc, 0, 0, 0);
    const float s = weighted_relu_sum<H>(wv, acc, 0);
    return g == 0 && kt + n < nv ? order_key(pg >= 0 ? s : __builtin_nanf("")) : 0u;
  };
  uint32_t prefix = 0u, mask = 0u, rr = (uint32_t)k;
  uint32_t* h = sh.hist[0];
  for (int top = 32; top > 0;) {
    const int width = top > 11 ? 11 : top, shift = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = threadIdx.x; i < kBins; i += kNT) h[i] = 0u;
    __syncthreads();
    for (int sub = s0; sub < s1; ++sub) {
      const uint32_t u = score(sub);
      if (u != 0u && (u & mask) == prefix) atomicAdd(&h[(u >> shift) & dmask], 1u);
    }
    __syncthreads();
    // descending bins: thread t owns bins 2047 - 2t and 2046 - 2t
    const uint32_t c0 = h[kBins - 1 - 2 * threadIdx.x], c1 = h[kBins - 2 - 2 * threadIdx.x];
    const uint32_t incl = wave_incl_scan(c0 + c1);
    if (lane == 63) sh.wsum[wid] = incl;
    __syncthreads();
    uint32_t tot;
    const uint32_t above = waves_before(sh.wsum, tot) + incl - (c0 + c1);
    if (above < rr && rr <= above + c0) {
      sh.bin = kBins - 1 - 2 * threadIdx.x;
      sh.rem = rr - above;
    } else if (above + c0 < rr && rr <= above + c0 + c1) {
      sh.bin = kBins - 2 - 2 * threadIdx.x;
      sh.rem = rr - above - c0;
    }
    __syncthreads();
    prefix |= sh.bin << shift;
    mask |= dmask << shift;
    rr = sh.rem;
    top = shift;
    __syncthreads();
  }
  const uint32_t T = prefix, rem = rr;
  uint32_t gt = 0u, eq = 0u;
  for (int sub = s0; sub < s1; ++sub) {
    const uint32_t u = score(sub);
    gt += (uint32_t)__builtin_popcountll(__ballot(u > T));
    eq += (uint32_t)__builtin_popcountll(__ballot(u == T));
  }
  uint32_t gt_b, eq_b, gt_t, eq_t;
  block_scan2(lane == 0 ? gt : 0u, lane == 0 ? eq : 0u, sh.scan[0], gt_b, eq_b, gt_t, eq_t);
  uint32_t gtr = __builtin_amdgcn_readlane(gt_b, 0), eqr = __builtin_amdgcn_readlane(eq_b, 0);
  for (int sub = s0; sub < s1; ++sub) {
    const uint32_t u = score(sub);
    const bool is_gt = u > T, is_eq = u == T;
    const uint64_t mg = __ballot(is_gt), me = __ballot(is_eq);
    const uint32_t bg = gtr + __builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
    const uint32_t be = eqr + __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
    const uint32_t pos = bg + (be < rem ? be : rem);
    if ((is_gt || (is_eq && be < rem)) && pos < (uint32_t)k) out[pos] = sub * 32 + n;
    gtr += (uint32_t)__builtin_popcountll(mg);
    eqr += (uint32_t)__builtin_popcountll(me);
  }
  __syncthreads();   // the histogram and scan buffers are free for the next row
}

// Candidate p of a row (its regions' prefix counts in pre): region i with
// pre[i] <= p < pre[i + 1], found by walking on from i.
__device__ __forceinline__ int64_t cand_at(const IdxArgs& a, int row, const int32_t* pre, int p, int& i) {
  while (pre[i + 1] <= p) ++i;
  return (int64_t)(row * a.n_kgroups + i) * a.cap + (p - pre[i]);
}

// Selection, kSelRows rows a workgroup of 1,024 threads. Each of the first kSelRows
// waves reads its row's region counts (their prefix into LDS) and, when the row has at
// most 64 * kWaveCand candidates and no region overflowed, selects them alone
// (wave_select, then an emission in candidate order). Rows with more candidates take
// the whole workgroup (select_topk on up to 32,768), rows with too few or an overflow
// are re-scored (rescore_select), one row at a time.
template <int H, int D>
__global__ __launch_bounds__(kNT) void fused_select_kernel(FusedSel f) {
  constexpr int EB = 16;   // candidates a thread holds in the workgroup selection
  __shared__ SelShared sh;
  __shared__ CandShared cs;
  __shared__ int32_t pre[kSelRows][kMaxRegions + 1];
  __shared__ int32_t need[kSelRows], nvs[kSelRows];
  __shared__ uint32_t hist[kSelRows][256];
  const IdxArgs& a = f.a;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nk = a.n_kgroups;
  const uint32_t k = (uint32_t)f.k;
  if (wid < kSelRows) {
    const int row = blockIdx.x * kSelRows + wid;
    int nd = 0, nv = 0;
    uint32_t total = 0u;
    if (row < a.n_rows) {
      nv = f.nv[row];
      int32_t* out = f.blocks + (int64_t)row * f.k;
      if (f.n_valid && lane == 0) f.n_valid[row] = nv;
      if (nv <= f.k) {
        for (int i = lane; i < f.k; i += 64) out[i] = i < nv ? i : -1;
      } else {
        bool over = false;
        for (int i0 = 0; i0 < nk; i0 += 64) {
          const int i = i0 + lane;
          const int c = i < nk ? a.cand_cnt[row * nk + i] : 0;
          over |= c > a.cap;
          const uint32_t incl = wave_incl_scan((uint32_t)(c > a.cap ? a.cap : c));
          if (i < nk) pre[wid][i + 1] = (int32_t)(total + incl);
          total += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        }
        if (lane == 0) pre[wid][0] = 0;
        nd = (__ballot(over) != 0 || total < k) ? 2 : (total > 64u * kWaveCand ? 1 : 0);
      }
    }
    if (lane == 0) {
      need[wid] = row < a.n_rows && nv > f.k ? nd : -1;
      nvs[wid] = nv;
    }
    // the wave's lanes read what other lanes of it wrote to pre
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (row < a.n_rows && nv > f.k && nd == 0) {
      int32_t* out = f.blocks + (int64_t)row * f.k;
      uint32_t key[kWaveCand];
      int32_t idx[kWaveCand];
      // position e * 64 + lane, clamped to the last candidate (dropped below) so that
      // every load is issued before any is used; its region found by walking on from
      // the previous one when there are few regions, else by a search of its own (64
      // positions cross about 64 / (candidates per region) regions)
      const int32_t* pw = pre[wid];
      int i = 0;
#pragma unroll
      for (int e = 0; e < kWaveCand; ++e) {
        const int p = e * 64 + lane < (int)total ? e * 64 + lane : (int)total - 1;
        int64_t o;
        if (nk <= 16) {
          o = cand_at(a, row, pw, p, i);
        } else {
          int lo = 0, hi = nk;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pw[mid] <= p) lo = mid;
            else hi = mid;
          }
          o = (int64_t)(row * nk + lo) * a.cap + (p - pw[lo]);
        }
        key[e] = a.cand_key[o];
        idx[e] = a.cand_idx[o];
      }
#pragma unroll
      for (int e = 0; e < kWaveCand; ++e)
        if (e * 64 + lane >= (int)total) {
          key[e] = 0u;
          idx[e] = -1;
        }
      uint32_t T, rem;
      wave_select<kWaveCand>(key, k, 0, hist[wid], T, rem);
      uint32_t n_eq = 0u;
#pragma unroll
      for (int e = 0; e < kWaveCand; ++e) n_eq += (uint32_t)__builtin_popcountll(__ballot(key[e] == T));
      uint32_t base = 0u;
      if (n_eq == rem) {   // every key equal to T is taken: the keys >= T, in order
#pragma unroll
        for (int e = 0; e < kWaveCand; ++e) {
          const bool sel = key[e] >= T;
          const uint64_t m = __ballot(sel);
          const uint32_t pos =
              base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (sel && pos < k) out[pos] = idx[e];
          base += (uint32_t)__builtin_popcountll(m);
        }
      } else {
        uint32_t eqr = 0u;
#pragma unroll
        for (int e = 0; e < kWaveCand; ++e) {   // candidate order: position e * 64 + lane
          const bool is_gt = key[e] > T, is_eq = key[e] == T;
          const uint64_t mg = __ballot(is_gt), me = __ballot(is_eq);
          const uint32_t bg = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
          const uint32_t be = eqr + __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
          const uint32_t pos = bg + (be < rem ? be : rem);
          if ((is_gt || (is_eq && be < rem)) && pos < k) out[pos] = idx[e];
          base += (uint32_t)__builtin_popcountll(mg);
          eqr += (uint32_t)__builtin_popcountll(me);
        }
      }
    }
  }
  __syncthreads();
  for (int w = 0; w < kSelRows; ++w) {
    const int nd = need[w];
    if (nd <= 0) continue;
    const int row = blockIdx.x * kSelRows + w;
    const int nv = nvs[w];
    int32_t* out = f.blocks + (int64_t)row * f.k;
    const int32_t* pw = pre[w];
    const uint32_t total = (uint32_t)pw[nk];
    if (nd == 1 && total <= (uint32_t)(EB * kNT)) {
      uint32_t key[EB];
      int32_t idx[EB];
      const int p0 = (int)threadIdx.x * EB;
      int i = 0;
      if (p0 < (int)total) {   // the region holding position p0: pw[i] <= p0 < pw[i + 1]
        int hi = nk;
        while (hi - i > 1) {
          const int mid = (i + hi) >> 1;
          if (pw[mid] <= p0) i = mid;
          else hi = mid;
        }
      }
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        const int p = p0 + e;
        const int64_t o = cand_at(a, row, pw, p < (int)total ? p : (int)total - 1, i);
        key[e] = a.cand_key[o];
        idx[e] = a.cand_idx[o];
      }
#pragma unroll
      for (int e = 0; e < EB; ++e)
        if (p0 + e >= (int)total) {
          key[e] = 0u;
          idx[e] = -1;
        }
      select_topk<EB>(key, f.k, sh, cs, [&](int e) { return idx[e]; },
                      [&](uint32_t pos, uint32_t, int32_t ix) { out[pos] = ix; });
      __syncthreads();
    } else {
      rescore_select<H, D>(a, row, nv, f.k, out, sh);
    }
  }
}

template <int H, int D>
static tf_status fused_hd(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                          const int32_t* row_pos, const void* q, const float* w, int64_t ld, int32_t k,
                          int32_t* blocks, int32_t* n_valid, char* ws, hipStream_t st) {
  const FusedPlan f = fused_plan(H, n_rows, ld, k);
  if (f.bytes == (size_t)-1) return set_error(TF_E_RANGE, "tf_indexer_topk_fused: no top-k block size fits");
  IdxArgs a = base_args(p, v, n_rows, row_stream, row_pos, q, w);
  if (f.direct) {
    int32_t* nv = n_valid ? n_valid : (int32_t*)(ws + f.off_nv);
    a.logits = (float*)(ws + f.off_smp);
    a.ldo = ld;
    a.kend = ld;
    a.ncap = ld;
    a.n_valid = nv;
    tf_status s = launch_hd<H, D>(a, n_rows, st, kWhole);
    if (s == TF_OK) s = launch_status("tf_indexer_topk_fused");
    if (s != TF_OK) return s;
    return launch_topk((const float*)(ws + f.off_smp), ld, n_rows, nv, k, blocks, f.tws ? ws + f.off_tws : nullptr,
                       f.tws, st);
  }
  if ((int64_t)n_rows * f.shape.kgroups * f.cap >= 0x7fffffffLL || f.shape.kgroups > kMaxRegions)
    return set_error(TF_E_RANGE, "tf_indexer_topk_fused: %lld key groups of %d slots for %d rows exceed one launch",
                     (long long)f.shape.kgroups, f.cap, n_rows);
  float* smp = (float*)(ws + f.off_smp);
  int32_t* nvs = (int32_t*)(ws + f.off_nvs);
  uint32_t* thr = (uint32_t*)(ws + f.off_thr);
  int32_t* nv = (int32_t*)(ws + f.off_nv);
  // 1. page sample
  IdxArgs as = a;
  as.page_step = f.step;
  as.logits = smp;
  as.ldo = f.S;
  as.kend = f.S;
  as.ncap = ld;
  as.n_valid = nvs;
  tf_status s = launch_hd<H, D>(as, n_rows, st, kSample, 512);
  if (s == TF_OK) s = launch_status("tf_indexer_topk_fused");
  if (s != TF_OK) return s;
  // 2. thresholds
  const unsigned g4 = (unsigned)((n_rows + 3) / 4);
  if (f.e_thr == 32)
    hipLaunchKernelGGL(fused_threshold_kernel<32>, dim3(g4), dim3(256), 0, st, smp, (int32_t)f.S, nvs, row_pos, ld, k,
                       n_rows, thr);
  else if (f.e_thr == 64)
    hipLaunchKernelGGL(fused_threshold_kernel<64>, dim3(g4), dim3(256), 0, st, smp, (int32_t)f.S, nvs, row_pos, ld, k,
                       n_rows, thr);
  else if (f.S <= 8 * kNT)
    hipLaunchKernelGGL(fused_threshold_block_kernel<8>, dim3(n_rows), dim3(kNT), 0, st, smp, (int32_t)f.S, nvs, row_pos,
                       ld, k, thr);
  else if (f.S <= 16 * kNT)
    hipLaunchKernelGGL(fused_threshold_block_kernel<16>, dim3(n_rows), dim3(kNT), 0, st, smp, (int32_t)f.S, nvs,
                       row_pos, ld, k, thr);
  else if (f.S <= 32 * kNT)
    hipLaunchKernelGGL(fused_threshold_block_kernel<32>, dim3(n_rows), dim3(kNT), 0, st, smp, (int32_t)f.S, nvs,
                       row_pos, ld, k, thr);
  else
    return set_error(TF_E_RANGE, "tf_indexer_topk_fused: a sample of %lld keys exceeds 32,768", (long long)f.S);
  s = launch_status("tf_indexer_topk_fused");
  if (s != TF_OK) return s;
  // 3. filtered scoring
  IdxArgs af = a;
  af.kend = ld;
  af.ncap = ld;
  af.n_valid = nv;
  af.thr = thr;
  af.cand_cnt = (int32_t*)(ws + f.off_cnt);
  af.cand_key = (uint32_t*)(ws + f.off_ck);
  af.cand_idx = (int32_t*)(ws + f.off_ci);
  af.cap = f.cap;
  s = launch_hd<H, D>(af, n_rows, st, kFilter, 1024, f.min_kpw);
  if (s == TF_OK) s = launch_status("tf_indexer_topk_fused");
  if (s != TF_OK) return s;
  // 4. selection
  af.keys_per_wg = (int32_t)f.shape.kpw;
  af.n_kgroups = (int32_t)f.shape.kgroups;
  FusedSel fs;
  fs.a = af;
  fs.nv = nv;
  fs.n_valid = n_valid;
  fs.k = k;
  fs.blocks = blocks;
  hipLaunchKernelGGL((fused_select_kernel<H, D>), dim3((unsigned)((n_rows + kSelRows - 1) / kSelRows)), dim3(kNT), 0,
                     st, fs);
  return launch_status("tf_indexer_topk_fused");
}

tf_status launch_indexer_topk_fused(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                                    const int32_t* row_pos, const void* q, const float* w, int32_t n_heads,
                                    int64_t ld, int32_t k, int32_t* blocks, int32_t* n_valid, void* ws,
                                    hipStream_t st) {
  char* c = (char*)ws;
  if (p->g.index_dim == 128) {
    if (n_heads == 16) return fused_hd<16, 128>(p, v, n_rows, row_stream, row_pos, q, w, ld, k, blocks, n_valid, c, st);
    if (n_heads == 8) return fused_hd<8, 128>(p, v, n_rows, row_stream, row_pos, q, w, ld, k, blocks, n_valid, c, st);
    return fused_hd<4, 128>(p, v, n_rows, row_stream, row_pos, q, w, ld, k, blocks, n_valid, c, st);
  }
  if (n_heads == 16) return fused_hd<16, 64>(p, v, n_rows, row_stream, row_pos, q, w, ld, k, blocks, n_valid, c, st);
  if (n_heads == 8) return fused_hd<8, 64>(p, v, n_rows, row_stream, row_pos, q, w, ld, k, blocks, n_valid, c, st);
  return fused_hd<4, 64>(p, v, n_rows, row_stream, row_pos, q, w, ld, k, blocks, n_valid, c, st);
}

}  // namespace tf
