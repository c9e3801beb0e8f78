// Sparse absorbed-MLA attention over the selected latent rows, read through the
// page table. Decode rows and chunked-prefill rows run the same kernel.
// [#1313, "Step 2"]: a sparse row reads up to 2,048 latent rows of 1 KiB a layer
// (512 blocks x 4 tokens) and its 32 heads' absorbed queries are 32 KiB;
// [#1142, "What stays as it is"]: the sparse pass gathers the selected rows
// from the pages, and a stream's results do not depend on which pages hold it.
//
// Per row t and head h over S = {s <= t : s/4 selected}:
//   z_s = scale * q_h . [c_s ; r_s],  out_h = sum_s softmax(z)_s c_s,  lse_h.
//
// Design (gfx950). One workgroup of 4 waves takes (row, group of HG heads,
// split of the row's block list):
//   * the workgroup's token table (page and slot of every selected token) is
//     built once, in LDS;
//   * 32-token tiles (8 blocks; a block never straddles a 512-row page) are
//     gathered with 16-byte coalesced loads; the next tile's loads are issued
//     into registers before the current tile is computed; fp8 rows are widened
//     to bf16 exactly (the row scale is kept per token);
//   * S = Q K^T on MFMA with the heads as M (HG = 32: 32x32x16; HG = 16:
//     16x16x32), the 576-long contraction split over waves and summed through
//     LDS; the fp8 row scale multiplies the latent part of S;
//   * online softmax in fp32 (exp2 domain);
//   * O += P V on MFMA with P as a bf16 hi + lo pair (16 significant bits) and
//     V read from the LDS tile transposed; each wave owns 128 output columns;
//     the fp8 row scale is folded into P.
//   Decode rows (few rows, many CUs) split their block list and, with HG = 16,
//   their heads; the two head groups of one split sit on the same XCD (workgroup
//   i runs on XCD i mod 8) so the second gather hits L2. Partial (O, max, sum)
//   go to the workspace and a merge kernel combines them.
// The dense pass [#1142, "What stays as it is", and its proposal's kernel list: the
// page-table kernels read the latent for dense chunks as for the sparse gather]
// runs the same kernels with no block list: slot j is pooled block j, and a split
// stops at the row's last visible block. Its split ranges follow from the extent
// and the row count alone, so a stream's bits never depend on its pages.
// Three kernels: attn_kernel (the general one above), attn_kernel_w32 (bf16 rows,
// 32 heads: each wave gathers its own slice of the keys, below) and
// attn_decode_kernel (few rows: a row's 128 tokens in LDS at once, below). The
// 32-head one has a dense instance of its own, attn_dense_kernel_w32, that reads no
// block list; the others test for the list at run time.
#include <math.h>

#include <mutex>

#include "common.h"

namespace tf {

constexpr int kTileTok = 32;
constexpr int kRS = kRow + 8;       // LDS row stride in bf16 (1,168 bytes)
constexpr int kMaxWgTok = 4096;     // tokens one workgroup may own (k <= 1,024 blocks); its 16 KiB
                                    // token table still lets two workgroups share a CU (asserted below)
constexpr int kMasked = -1;         // token table: not attended
constexpr int kUnreadable = -2;     // token table: selected but the table names no page

struct AttnArgs {
  DevView v;
  int64_t off_scale, off_rope;
  int32_t lat_row_bytes;
  int32_t n_rows;
  const int32_t* row_stream;
  const int32_t* row_pos;
  const __bf16* q;
  int32_t n_heads;
  float scale_log2;  // softmax scale * log2(e)
  const int32_t* blocks;
  int32_t k;
  int32_t nsplit, slots_per_split, ngroups, n_units;
  float* out;
  float* lse;
  float* part_o;   // [n_rows][nsplit][32][512]
  float* part_ml;  // [n_rows][nsplit][32][2]  (max in log2 domain, sum)
};

// A row's block list, or none: the dense pass (blocks == nullptr) names slot j as
// pooled block j, so the row attends every token s <= t with s < 4 k.
__device__ __forceinline__ int block_at(const AttnArgs& a, int r, int slot) {
  return a.blocks ? a.blocks[(int64_t)r * a.k + slot] : slot;
}

// End of a split's slot range [j0, j1). In the dense pass the slots past the row's
// last visible block (t / 4) hold masked tokens only and are cut, keeping at least
// one slot so that the split still writes its (empty) partial for the merge.
__device__ __forceinline__ int dense_split_end(const AttnArgs& a, int j0, int t) {
  const int j1 = j0 + a.slots_per_split < a.k ? j0 + a.slots_per_split : a.k;
  const int jv = t >= 0 ? t / kPoolRatio + 1 : 0;
  const int lim = jv > j0 + 1 ? jv : j0 + 1;
  return j1 < lim ? j1 : lim;
}

__device__ __forceinline__ int split_end(const AttnArgs& a, int j0, int t) {
  return a.blocks ? (j0 + a.slots_per_split < a.k ? j0 + a.slots_per_split : a.k) : dense_split_end(a, j0, t);
}

// Row stride of the partial S tiles in floats, 16-byte aligned rows (vector reads in
// the softmax). 32x32 tiles: unpadded. Their 4-byte stores (one MFMA result: two rows
// of 32 tokens) measured free of bank conflicts at every stride tried, and the
// softmax's 16-byte reads (eight lanes a head, consecutive heads) are conflict-free
// only when a row is 128 bytes long: at 36 or 40 floats they cost 4 and 8 conflict
// cycles per read. 16x16 tiles: 36 (the four lane groups' rows 4 apart).
template <int HG>
constexpr int kSpartStride = HG == 32 ? kTileTok : kTileTok + 4;

template <int HG>
struct alignas(16) AttnShared {
  __bf16 kv[kTileTok][kRS];
  float spart[HG == 32 ? 4 : 2][HG][kSpartStride<HG>];
  __bf16 p_hi[HG][kTileTok + 8];
  __bf16 p_lo[HG][kTileTok + 8];
  float tsc[kTileTok];         // per-token value scale of the current tile (fp8)
  int32_t tt[kMaxWgTok];       // token table: page * 512 + slot, or kMasked / kUnreadable
  float m_run[HG], l_run[HG], alpha[HG];
  uint16_t lut[256];           // e4m3 -> bf16 bits
  int32_t bad;                 // a selected token the table could not name
};

__device__ __forceinline__ uint16_t e4m3_to_bf16_bits(uint32_t c) {
  const uint32_t sign = (c >> 7) << 15;
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 15u && m == 7u) return (uint16_t)(sign | 0x7FC0u);
  if (e == 0u) {
    if (m == 0u) return (uint16_t)sign;
    const uint32_t p = m >= 4u ? 2u : (m >= 2u ? 1u : 0u);   // value m * 2^-9 = 2^(p-9) * (m / 2^p)
    return (uint16_t)(sign | ((p - 9u + 127u) << 7) | ((m - (1u << p)) << (7u - p)));
  }
  return (uint16_t)(sign | ((e - 7u + 127u) << 7) | (m << 4));
}

// Nearest bf16, ties to even: the conversion instruction (v_cvt_pk_bf16_f32), where
// integer rounding took four instructions a value (the same bits for finite values, the
// only ones converted here: softmax weights and their residues).
__device__ __forceinline__ __bf16 bf16_rne(float x) { return (__bf16)x; }

// 2^x for a softmax weight (x <= 8): v_exp_f32 alone. exp2f adds a rescaling for
// x < -126 only, where the weight is below 2^-126 of the largest in its row and
// contributes nothing an fp32 sum keeps.
__device__ __forceinline__ float exp2_weight(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_to_f(__bf16 x) {
  return __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, x)) << 16);
}


typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// MFMA B fragment of 8 consecutive rows (K) of one column (N) from a row-major
// bf16 LDS tile, with two transpose reads (ds_read_b64_tr_b16). Within a 16-lane
// group, lane i receives, as element k, element i % 4 of the 8 bytes that lane
// 4k + i / 4 of the group addresses; so lane j of the group addresses row
// k0 + j / 4 (+ 4 for the second read), columns n0 + 4 (j % 4) .. + 3, and lane i
// ends up with rows k0 .. k0 + 7 of column n0 + i.
__device__ __forceinline__ bf16x8 bfrag_tr(const __bf16* tile, int stride, int k0, int n0, int j) {
  const __bf16* p = tile + (k0 + (j >> 2)) * stride + n0 + 4 * (j & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * stride));
  const short __attribute__((ext_vector_type(8))) v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Reductions over groups of 8 or 16 consecutive lanes with DPP (no LDS round trip).
template <int ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
template <int N>
__device__ __forceinline__ float group_max(float x) {
  x = __builtin_fmaxf(x, dpp<kQuadXor1>(x));
  x = __builtin_fmaxf(x, dpp<kQuadXor2>(x));
  x = __builtin_fmaxf(x, dpp<kHalfMirror>(x));
  if (N == 16) x = __builtin_fmaxf(x, dpp<kRowMirror>(x));
  return x;
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kHalfMirror>(x);
  if (N == 16) x += dpp<kRowMirror>(x);
  return x;
}

__device__ __forceinline__ int64_t row_base(const AttnArgs& a, int32_t tt) {
  return (int64_t)(tt >> 9) * a.v.page_bytes + a.v.cache_off;
}

// The token table of a workgroup's slots [j0, j1) (ntiles tiles of kTileTok tokens; slot
// j0 + q holds block q's four tokens): entry 4 q + c = page * 512 + slot of token
// 4 blk + c, or kMasked (no block, or past the row's position), or kUnreadable (the
// table names no page; `bad` is set). A thread takes blocks tid, tid + 256, ..: all
// their block ids are loaded at once (slots clamped into the list, the clamped ones
// dropped), then all their page ids (a block's four tokens share a page), so the table
// costs two dependent loads, not two per 256 tokens.
template <bool DENSE>
__device__ __forceinline__ void build_token_table(const AttnArgs& a, int r, int b, int t, int j0, int j1, int ntiles,
                                                  int32_t* tt, int32_t& bad, int tid) {
  constexpr int kBPT = kMaxWgTok / kPoolRatio / 256;   // blocks a thread takes at most
  const int nb = ntiles * kTileTok / kPoolRatio;
  int blk[kBPT];
#pragma unroll
  for (int u = 0; u < kBPT; ++u) {
    const int q = tid + 256 * u, slot = j0 + q;
    const int raw = DENSE ? slot : block_at(a, r, slot < j1 ? slot : (j1 > j0 ? j1 - 1 : 0));
    blk[u] = q < nb && slot < j1 ? raw : -1;
  }
  const bool b_ok = b >= 0 && b < a.v.n_streams;
  int page[kBPT];
#pragma unroll
  for (int u = 0; u < kBPT; ++u) {
    const int pi = blk[u] >= 0 ? blk[u] * kPoolRatio / kPageRows : 0;
    const bool in_tab = blk[u] >= 0 && b_ok && pi < a.v.pt_stride;
    const int64_t idx = in_tab ? (int64_t)b * a.v.pt_stride + pi : 0;
    const int p = a.v.pt ? a.v.pt[idx] : (int)idx;
    page[u] = in_tab && p >= 0 && p < a.v.n_pages ? p : -1;
  }
#pragma unroll
  for (int u = 0; u < kBPT; ++u) {
    const int q = tid + 256 * u;
    if (q >= nb) continue;
#pragma unroll
    for (int c = 0; c < kPoolRatio; ++c) {
      const int s = blk[u] * kPoolRatio + c;
      int32_t e = kMasked;
      if (blk[u] >= 0 && s <= t) {
        e = page[u] >= 0 ? page[u] * kPageRows + (s % kPageRows) : kUnreadable;
        if (page[u] < 0) bad = 1;
      }
      tt[kPoolRatio * q + c] = e;
    }
  }
}

// Pieces of one tile a thread loads: bf16 rows are 64 latent + 8 rope 16-byte
// pieces per token (9 per thread); fp8 rows 32 + 8 (5 per thread).
template <bool FP8>
struct Gather {
  static constexpr int kPieces = FP8 ? 40 : 72;
  static constexpr int kLatPieces = FP8 ? 32 : 64;
  static constexpr int kPerThread = kTileTok * kPieces / 256;
  uint4 v[kPerThread];
  float sc;  // this thread's token scale (threads < 32, fp8)

  __device__ __forceinline__ void issue(const AttnArgs& a, const int32_t* tt, int tok0, int tid) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int u = tid + i * 256;
      const int tok = u / kPieces, pc = u % kPieces;
      const int32_t e = tt[tok0 + tok];
      v[i] = make_uint4(0, 0, 0, 0);
      if (e >= 0) {
        const int64_t base = row_base(a, e);
        const int slot = e & 511;
        const char* src = pc < kLatPieces
                              ? a.v.pool + base + (int64_t)slot * a.lat_row_bytes + pc * 16
                              : a.v.pool + base + a.off_rope + (int64_t)slot * (kRope * 2) + (pc - kLatPieces) * 16;
        v[i] = *(const uint4*)src;
      }
    }
    if (FP8 && tid < kTileTok) {
      const int32_t e = tt[tok0 + tid];
      sc = 0.f;
      if (e >= 0) sc = *(const float*)(a.v.pool + row_base(a, e) + a.off_scale + 4LL * (e & 511));
    }
  }

  template <int HG>
  __device__ __forceinline__ void store(AttnShared<HG>& sh, const int32_t* tt, int tok0, int tid) const {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int u = tid + i * 256;
      const int tok = u / kPieces, pc = u % kPieces;
      if (!FP8) {
        *(uint4*)&sh.kv[tok][pc < 64 ? pc * 8 : kLatent + (pc - 64) * 8] = v[i];
      } else if (pc < 32) {
        const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t o8[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = w4[j];
          o8[2 * j] = (uint32_t)sh.lut[x & 255u] | ((uint32_t)sh.lut[(x >> 8) & 255u] << 16);
          o8[2 * j + 1] = (uint32_t)sh.lut[(x >> 16) & 255u] | ((uint32_t)sh.lut[x >> 24] << 16);
        }
        *(uint4*)&sh.kv[tok][pc * 16] = make_uint4(o8[0], o8[1], o8[2], o8[3]);
        *(uint4*)&sh.kv[tok][pc * 16 + 8] = make_uint4(o8[4], o8[5], o8[6], o8[7]);
      } else {
        *(uint4*)&sh.kv[tok][kLatent + (pc - 32) * 8] = v[i];
      }
    }
    if (tid < kTileTok) {
      const int32_t e = tt[tok0 + tid];
      sh.tsc[tid] = FP8 && e >= 0 ? sc : (e >= 0 ? 1.f : 0.f);
    }
  }
};

// MFMA fragment geometry. HG = 32: 32x32x16 (one wave covers 32 tokens, the 36
// k-steps split 9 per wave). HG = 16: 16x16x32 (a wave covers 16 tokens and half
// of the 18 k-steps).
template <int HG>
struct Frag;

template <>
struct Frag<32> {
  static constexpr int kParts = 4;  // partial S tiles summed in softmax
  typedef f32x16 acc_t;
  // k-steps of 16 dims; wave w takes latent steps 8w..8w+7 and rope step 32+w
  __device__ static int ks_dim(int wave, int i, int g) {
    const int ks = i < 8 ? wave * 8 + i : 32 + wave;
    return ks * 16 + g * 8;
  }
  static constexpr int kSteps = 9;
  __device__ static int tok_of_lane(int wave, int lane) { return lane & 31; }
  __device__ static int part_of(int wave) { return wave; }
  __device__ static acc_t mfma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr int kAccN = 16;
  __device__ static int row_of(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
  // A-operand lane geometry: head = lane % 32, k-slice half = lane / 32
  __device__ static int a_row(int lane) { return lane & 31; }
  __device__ static int a_half(int lane) { return lane >> 5; }
  static constexpr int kNT = 4;        // 32-column tiles per wave in P.V
  static constexpr int kNTW = 32;
  static constexpr int kPVsteps = 2;   // 16 tokens per k-step
  static constexpr int kPVk = 16;
};

template <>
struct Frag<16> {
  static constexpr int kParts = 2;
  typedef f32x4 acc_t;
  // k-steps of 32 dims; wave w: token half w%2, latent steps 8(w/2)..+7 and rope step 16 + w/2
  __device__ static int ks_dim(int wave, int i, int g) {
    const int ks = i < 8 ? (wave >> 1) * 8 + i : 16 + (wave >> 1);
    return ks * 32 + g * 8;
  }
  static constexpr int kSteps = 9;
  __device__ static int tok_of_lane(int wave, int lane) { return (wave & 1) * 16 + (lane & 15); }
  __device__ static int part_of(int wave) { return wave >> 1; }
  __device__ static acc_t mfma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr int kAccN = 4;
  __device__ static int row_of(int i, int lane) { return 4 * (lane >> 4) + i; }
  __device__ static int a_row(int lane) { return lane & 15; }
  __device__ static int a_half(int lane) { return lane >> 4; }
  static constexpr int kNT = 8;        // 16-column tiles per wave in P.V
  static constexpr int kNTW = 16;
  static constexpr int kPVsteps = 1;   // 32 tokens per k-step
  static constexpr int kPVk = 32;
};

// Online softmax of one 32-token tile for HG heads: 256 / HG threads per head, the
// partial S tiles summed, masked tokens at -inf; writes P (hi, lo) and the
// per-head rescale factor.
template <int HG, int NPARTS, bool FP8, typename SH>
__device__ __forceinline__ void softmax_tile(SH& sh, const int32_t* tt, const float* tsc, float scale_log2, int tid) {
  constexpr int TPH = 256 / HG, TPT = kTileTok / TPH;
  const int h = tid / TPH, p = tid % TPH;
  // this thread's TPT consecutive tokens: one vector read per partial tile and one
  // of the token table (the partials summed in the same order as one at a time)
  typedef float fv_t __attribute__((ext_vector_type(TPT)));
  typedef int32_t iv_t __attribute__((ext_vector_type(TPT)));
  typedef __bf16 bv_t __attribute__((ext_vector_type(TPT)));
  fv_t sv = *(const fv_t*)&sh.spart[0][h][p * TPT];
#pragma unroll
  for (int pp = 1; pp < NPARTS; ++pp) sv += *(const fv_t*)&sh.spart[pp][h][p * TPT];
  const iv_t tv = *(const iv_t*)&tt[p * TPT];
  float z[TPT];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int e = 0; e < TPT; ++e) {
    float v = sv[e] * scale_log2;
    if (tv[e] < 0) v = -__builtin_inff();   // not attended
    z[e] = v;
    tmax = __builtin_fmaxf(tmax, v);
  }
  tmax = group_max<TPH>(tmax);
  const float m_old = sh.m_run[h];
  const float m_new = __builtin_fmaxf(m_old, tmax);
  const float alpha = m_new == -__builtin_inff() ? 1.f : exp2f(m_old - m_new);
  float lsum = 0.f;
  bv_t phv, plv;
#pragma unroll
  for (int e = 0; e < TPT; ++e) {
    const int tok = p * TPT + e;
    const float pe = z[e] == -__builtin_inff() ? 0.f : exp2_weight(z[e] - m_new);
    lsum += pe;
    const float pv = FP8 ? pe * tsc[tok] : pe;
    const __bf16 hi = bf16_rne(pv);
    phv[e] = hi;
    plv[e] = bf16_rne(pv - bf16_to_f(hi));
  }
  *(bv_t*)&sh.p_hi[h][p * TPT] = phv;
  *(bv_t*)&sh.p_lo[h][p * TPT] = plv;
  lsum = group_sum<TPH>(lsum);
  __syncthreads();  // every thread of the head has read m_run
  if (p == 0) {
    sh.m_run[h] = m_new;
    sh.l_run[h] = sh.l_run[h] * alpha + lsum;
    sh.alpha[h] = alpha;
  }
}

// Final normalization (one split) or the split's partial (O, max, sum).
template <int HG, typename F, typename SH, int NT = F::kNT, int WCOLS = 128>
__device__ __forceinline__ void write_out(const AttnArgs& a, SH& sh, const typename F::acc_t* o, int r, int split,
                                          int h0, int wave, int lane, int tid) {
  const int col = F::a_row(lane);
  const bool bad = sh.bad != 0;   // a selected token the table could not name
  const float qnan = __builtin_nanf("");
  if (a.nsplit == 1) {
#pragma unroll
    for (int i = 0; i < F::kAccN; ++i) {
      const int m = F::row_of(i, lane);
      const int head = h0 + m;
      if (head >= a.n_heads) continue;
      const float l = sh.l_run[m];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* orow = a.out + ((int64_t)r * a.n_heads + head) * kLatent + wave * WCOLS + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) orow[nt * F::kNTW] = bad ? qnan : o[nt][i] * inv;
    }
    if (a.lse && tid < HG && h0 + tid < a.n_heads) {
      const float l = sh.l_run[tid];
      a.lse[(int64_t)r * a.n_heads + h0 + tid] =
          bad ? qnan : (l > 0.f ? (sh.m_run[tid] + log2f(l)) * 0.69314718055994531f : -__builtin_inff());
    }
  } else {
    float* po = a.part_o + ((int64_t)r * a.nsplit + split) * 32 * kLatent;
#pragma unroll
    for (int i = 0; i < F::kAccN; ++i) {
      const int m = F::row_of(i, lane);
      float* orow = po + (int64_t)(h0 + m) * kLatent + wave * WCOLS + col;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) orow[nt * F::kNTW] = o[nt][i];
    }
    if (tid < HG) {
      float* pm = a.part_ml + (((int64_t)r * a.nsplit + split) * 32 + h0 + tid) * 2;
      pm[0] = sh.m_run[tid];
      pm[1] = bad ? qnan : sh.l_run[tid];
    }
  }
}

template <int HG, bool FP8>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  typedef Frag<HG> F;
  __shared__ AttnShared<HG> sh;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  // ---- which (row, head group, split) ------------------------------------------
  int unit, hg;
  if (a.ngroups == 1) {
    unit = blockIdx.x;
    hg = 0;
  } else {  // the two head groups of a unit are 8 workgroups apart: same XCD
    unit = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    hg = (blockIdx.x >> 3) & 1;
  }
  if (unit >= a.n_units) return;
  const int r = unit % a.n_rows, split = unit / a.n_rows;
  const int h0 = hg * HG;
  const int b = a.row_stream[r];
  const int t = a.row_pos[r];
  const int j0 = split * a.slots_per_split;
  const int j1 = split_end(a, j0, t);
  const int ntok = (j1 > j0 ? j1 - j0 : 0) * kPoolRatio;
  const int ntiles = (ntok + kTileTok - 1) / kTileTok;

  if (FP8) sh.lut[tid] = e4m3_to_bf16_bits((uint32_t)tid);
  if (tid < HG) {
    sh.m_run[tid] = -__builtin_inff();
    sh.l_run[tid] = 0.f;
  }
  if (tid == 0) sh.bad = 0;
  __syncthreads();
  // ---- token table ----------------------------------------------------------------
  build_token_table<false>(a, r, b, t, j0, j1, ntiles, sh.tt, sh.bad, tid);
  // ---- query fragments --------------------------------------------------------------
  bf16x8 aq[F::kSteps];
  {
    const int head = h0 + F::a_row(lane);
    const __bf16* qr = a.q + ((int64_t)r * a.n_heads + head) * kRow;
#pragma unroll
    for (int i = 0; i < F::kSteps; ++i)
      aq[i] = head < a.n_heads ? *(const bf16x8*)(qr + F::ks_dim(wave, i, F::a_half(lane))) : bf16x8{};
  }
  typename F::acc_t o[F::kNT];
#pragma unroll
  for (int nt = 0; nt < F::kNT; ++nt) o[nt] = typename F::acc_t{};
  __syncthreads();

  Gather<FP8> gat;
  if (ntiles > 0) gat.issue(a, sh.tt, 0, tid);
  for (int it = 0; it < ntiles; ++it) {
    gat.store(sh, sh.tt, it * kTileTok, tid);
    if (it + 1 < ntiles) gat.issue(a, sh.tt, (it + 1) * kTileTok, tid);
    __syncthreads();
    // ---- S partials ---------------------------------------------------------------
    {
      typename F::acc_t accl{}, accr{};
      const int tok = F::tok_of_lane(wave, lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 bk = *(const bf16x8*)&sh.kv[tok][F::ks_dim(wave, i, F::a_half(lane))];
        accl = F::mfma(aq[i], bk, accl);
      }
      {
        const bf16x8 bk = *(const bf16x8*)&sh.kv[tok][F::ks_dim(wave, 8, F::a_half(lane))];
        accr = F::mfma(aq[8], bk, accr);
      }
      const float tsc = FP8 ? sh.tsc[tok] : 1.f;
#pragma unroll
      for (int i = 0; i < F::kAccN; ++i) sh.spart[F::part_of(wave)][F::row_of(i, lane)][tok] = accl[i] * tsc + accr[i];
    }
    __syncthreads();
    softmax_tile<HG, F::kParts, FP8>(sh, sh.tt + it * kTileTok, sh.tsc, a.scale_log2, tid);
    __syncthreads();
    // ---- O = alpha O + P V ------------------------------------------------------------
    {
      float al[F::kAccN];
#pragma unroll
      for (int i = 0; i < F::kAccN; ++i) al[i] = sh.alpha[F::row_of(i, lane)];
#pragma unroll
      for (int nt = 0; nt < F::kNT; ++nt)
#pragma unroll
        for (int i = 0; i < F::kAccN; ++i) o[nt][i] *= al[i];
      const int arow = F::a_row(lane), ahalf = F::a_half(lane);
      const int grp = lane >> 4, j = lane & 15;
#pragma unroll
      for (int ks = 0; ks < F::kPVsteps; ++ks) {
        const int tk = ks * F::kPVk + ahalf * 8;
        const bf16x8 ph = *(const bf16x8*)&sh.p_hi[arow][tk];
        const bf16x8 pl = *(const bf16x8*)&sh.p_lo[arow][tk];
#pragma unroll
        for (int nt = 0; nt < F::kNT; ++nt) {
          // this 16-lane group's 8 tokens and 16 columns of the B fragment
          const int k0 = ks * F::kPVk + (HG == 32 ? (grp >> 1) * 8 : grp * 8);
          const int n0 = wave * 128 + nt * F::kNTW + (HG == 32 ? (grp & 1) * 16 : 0);
          const bf16x8 vb = bfrag_tr(&sh.kv[0][0], kRS, k0, n0, j);
          o[nt] = F::mfma(ph, vb, o[nt]);
          o[nt] = F::mfma(pl, vb, o[nt]);
        }
      }
    }
    __syncthreads();
  }
  write_out<HG, F>(a, sh, o, r, split, h0, wave, lane, tid);
}

// ---- 32 heads, bf16 rows: each wave keeps its own slice of the keys ---------------------
// With 32 heads per workgroup, wave w's share of S is latent dims [128w, 128w+128) plus
// rope dims [16w, 16w+16), and its P.V columns are the same latent dims. So a wave
// gathers its slice of each 32-token tile straight into registers, already in the
// B-fragment order S wants, and runs its S partial from them; then it stores the
// slice's 128 latent columns in its own LDS region, for the transposed reads of P.V,
// and issues the next tile's gather into the same registers. No wave reads another's
// keys, so a tile needs two barriers (partial S -> softmax, softmax -> P.V) besides the
// one inside the softmax, and LDS carries each value twice instead of three times.
// LDS layouts of the sliced kernels, chosen by measured bank conflicts per instruction
// (no padded stride served both access forms of a tile):
// * a wave's V slice, 32 tokens x 128 columns: rows of 160 bf16 (the P.V transposed
//   reads, four rows x 64 bytes per half-wave, then land on disjoint banks), and the
//   16-byte piece c of row t stored at piece c ^ ((t >> 1) & 3), which spreads the
//   slice's 16-byte stores (consecutive tokens, one piece) over the banks. Unswizzled,
//   the stores cost 24 conflict cycles each at this stride; at 144 (stores 8, reads 2)
//   and 152 (0 and 2) no stride reached zero for both;
// * P (32 heads x 32 tokens): unpadded 64-byte rows, piece c of head h at
//   c ^ ((h >> 2) & 3): the softmax's 8-byte stores (four heads a half-wave) and P.V's
//   16-byte reads (16 heads, one piece) are both conflict-free, where 80-byte rows cost
//   the stores 4 cycles each.
constexpr int kVS = 160;
__device__ __forceinline__ int vslice_at(int t, int c) {   // bf16 offset of column c of token t
  return t * kVS + (((c >> 3) ^ ((t >> 1) & 3)) << 3) + (c & 7);
}
constexpr int kPS = kTileTok;
__device__ __forceinline__ int p_at(int h, int c) {        // bf16 offset of token c of head h
  return h * kPS + (((c >> 3) ^ ((h >> 2) & 3)) << 3) + (c & 7);
}
// bfrag_tr over the swizzled V slice: rows k0 + j / 4 and k0 + 4 + j / 4, columns
// n0 + 4 (j % 4) .. + 3 (n0 a multiple of 8: a lane's 8 bytes stay in one piece).
__device__ __forceinline__ bf16x8 bfrag_tr_vslice(const __bf16* tile, int k0, int n0, int j) {
  const int r = k0 + (j >> 2), c = n0 + 4 * (j & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + vslice_at(r, c)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + vslice_at(r + 4, c)));
  const short __attribute__((ext_vector_type(8))) v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

struct alignas(16) AttnSharedW {
  __bf16 vt[4][kTileTok * kVS];   // wave w: tokens x its 128 latent columns (vslice_at)
  float spart[4][32][kSpartStride<32>];
  __bf16 p_hi[32 * kPS];          // p_at
  __bf16 p_lo[32 * kPS];
  float tsc[kTileTok];
  int32_t tt[kMaxWgTok];
  float m_run[32], l_run[32], alpha[32];
  int32_t moved[2];   // by tile parity: some head's max moved in the tile (O needs a rescale)
  int32_t bad;
};

// Two workgroups of the 32-head kernels share a CU (__launch_bounds__(256, 2)), which
// LDS allows only while two copies of their shared state fit its 160 KiB; the token
// table (kMaxWgTok entries) is most of that state. Launch bounds do not count LDS, so
// a larger struct would silently halve the occupancy.
static_assert(2 * sizeof(AttnShared<32>) <= 160 * 1024, "two 32-head workgroups must fit one CU's LDS");
static_assert(2 * sizeof(AttnShared<16>) <= 160 * 1024, "two 16-head workgroups must fit one CU's LDS");
static_assert(2 * sizeof(AttnSharedW) <= 160 * 1024, "two sliced 32-head workgroups must fit one CU's LDS");

constexpr float kLazy = 8.f;

template <bool FP8>
__device__ __forceinline__ void softmax_tile_lazy(AttnSharedW& sh, const int32_t* tt, int it, float scale_log2,
                                                  int tid) {
  constexpr int TPH = 8, TPT = kTileTok / TPH;
  const int h = tid / TPH, p = tid % TPH;
  typedef float fv_t __attribute__((ext_vector_type(TPT)));
  typedef int32_t iv_t __attribute__((ext_vector_type(TPT)));
  typedef __bf16 bv_t __attribute__((ext_vector_type(TPT)));
  fv_t sv = *(const fv_t*)&sh.spart[0][h][p * TPT];
#pragma unroll
  for (int pp = 1; pp < 4; ++pp) sv += *(const fv_t*)&sh.spart[pp][h][p * TPT];
  const iv_t tv = *(const iv_t*)&tt[p * TPT];
  float z[TPT];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int e = 0; e < TPT; ++e) {
    float v = sv[e] * scale_log2;
    if (tv[e] < 0) v = -__builtin_inff();
    z[e] = v;
    tmax = __builtin_fmaxf(tmax, v);
  }
  tmax = group_max<TPH>(tmax);
  const float m_old = sh.m_run[h];
  const float m_new = (m_old == -__builtin_inff() || tmax > m_old + kLazy) ? tmax : m_old;
  const float alpha = m_new == m_old ? 1.f : (m_new == -__builtin_inff() ? 1.f : exp2f(m_old - m_new));
  float lsum = 0.f;
  bv_t phv, plv;
#pragma unroll
  for (int e = 0; e < TPT; ++e) {
    const float pe = z[e] == -__builtin_inff() ? 0.f : exp2_weight(z[e] - m_new);
    lsum += pe;
    const float pv = FP8 ? pe * sh.tsc[p * TPT + e] : pe;   // fp8 rows: the row scale joins P
    const __bf16 hi = bf16_rne(pv);
    phv[e] = hi;
    plv[e] = bf16_rne(pv - bf16_to_f(hi));
  }
  *(bv_t*)&sh.p_hi[p_at(h, p * TPT)] = phv;
  *(bv_t*)&sh.p_lo[p_at(h, p * TPT)] = plv;
  lsum = group_sum<TPH>(lsum);
  // the other parity's flag was last read in the previous tile's P.V (done: a barrier
  // since), and is next set in the next tile's softmax (a barrier after this one)
  if (tid == 0) sh.moved[(it + 1) & 1] = 0;
  __syncthreads();
  if (p == 0) {
    sh.m_run[h] = m_new;
    sh.l_run[h] = sh.l_run[h] * alpha + lsum;
    sh.alpha[h] = alpha;
    if (alpha != 1.f) sh.moved[it & 1] = 1;
  }
}

// FP8: rows of e4m3 codes and a row scale. A lane gathers its token's 64 codes at dims
// 128 w + 64 g .. + 63 (four 16-byte loads, where bf16 rows take eight) and widens them
// to bf16 exactly in registers (two codes per instruction); its k-steps take those dims
// in order (the queries are read to match), the row scale multiplies the latent part of
// S and joins P in the softmax.
template <bool DENSE, bool FP8>
__device__ __forceinline__ void attn_w32_body(const AttnArgs& a, AttnSharedW& sh) {
  typedef Frag<32> F;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  int unit, hg;
  if (a.ngroups == 1) {
    unit = blockIdx.x;
    hg = 0;
  } else {  // the two head groups of a unit are 8 workgroups apart: same XCD
    unit = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    hg = (blockIdx.x >> 3) & 1;
  }
  if (unit >= a.n_units) return;
  const int r = unit % a.n_rows, split = unit / a.n_rows;
  const int h0 = hg * 32;
  const int b = a.row_stream[r];
  const int t = a.row_pos[r];
  const int j0 = split * a.slots_per_split;
  const int j1 = DENSE ? dense_split_end(a, j0, t) : split_end(a, j0, t);
  const int ntok = (j1 > j0 ? j1 - j0 : 0) * kPoolRatio;
  const int ntiles = (ntok + kTileTok - 1) / kTileTok;

  if (tid < 32) {
    sh.m_run[tid] = -__builtin_inff();
    sh.l_run[tid] = 0.f;
    sh.tsc[tid] = 1.f;
  }
  if (tid == 0) {
    sh.bad = 0;
    sh.moved[0] = 0;
    sh.moved[1] = 0;
  }
  __syncthreads();
  // ---- token table ----------------------------------------------------------------
  build_token_table<DENSE>(a, r, b, t, j0, j1, ntiles, sh.tt, sh.bad, tid);
  // ---- query fragments (A: head = lane % 32, this wave's dims) ------------------------
  bf16x8 aq[F::kSteps];
  {
    const int head = h0 + F::a_row(lane);
    const __bf16* qr = a.q + ((int64_t)r * a.n_heads + head) * kRow;
#pragma unroll
    for (int i = 0; i < F::kSteps; ++i) {
      const int d = FP8 && i < 8 ? 128 * wave + 64 * F::a_half(lane) + 8 * i : F::ks_dim(wave, i, F::a_half(lane));
      aq[i] = head < a.n_heads ? *(const bf16x8*)(qr + d) : bf16x8{};
    }
  }
  F::acc_t o[F::kNT];
#pragma unroll
  for (int nt = 0; nt < F::kNT; ++nt) o[nt] = F::acc_t{};
  __syncthreads();

  // this lane's token of each tile and its 9 pieces of 8 dims: B[k][n] of S with
  // n = the token, k = the wave's dims (8 latent steps, then its rope step)
  const int tok = F::tok_of_lane(wave, lane), g = F::a_half(lane);
  bf16x8 kvr[F::kSteps];
  uint4 raw[4];   // fp8: the token's 64 codes of this lane's dims, widened when S needs them
  float sc = 0.f;  // fp8: the token's row scale
  // a token that is not attended (or whose page the table does not name) gets zeros:
  // its probability is 0, and 0 x V must not meet unwritten bytes
  auto gather = [&](int tile) __attribute__((always_inline)) {
    const int32_t e = sh.tt[tile * kTileTok + tok];
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) raw[j] = make_uint4(0, 0, 0, 0);
      kvr[8] = bf16x8{};
      sc = 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < F::kSteps; ++i) kvr[i] = bf16x8{};
    }
    if (e >= 0) {
      const int64_t base = row_base(a, e);
      const char* rowp = a.v.pool + base + (int64_t)(e & 511) * a.lat_row_bytes;
      const char* ropep = a.v.pool + base + a.off_rope + (int64_t)(e & 511) * (kRope * 2);
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) raw[j] = *(const uint4*)(rowp + wave * 128 + 64 * g + 16 * j);
        sc = *(const float*)(a.v.pool + base + a.off_scale + 4LL * (e & 511));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kvr[i] = *(const bf16x8*)(rowp + (wave * 128 + 16 * i + 8 * g) * 2);
      }
      kvr[8] = *(const bf16x8*)(ropep + (16 * wave + 8 * g) * 2);
    }
  };
  // fp8: codes 8i .. 8i + 7 of the lane's 64 as bf16 (exact: every e4m3 value is a bf16).
  // Each conversion turns the two codes of one half of a dword into one dword of two
  // bf16, the lower address in the lower half; the fragment is assembled from those
  // dwords as they are.
  auto widen = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w0 = (i & 1) ? raw[i >> 1].z : raw[i >> 1].x;
      const uint32_t w1 = (i & 1) ? raw[i >> 1].w : raw[i >> 1].y;
      u32x4 d;
      d[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false));
      d[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true));
      d[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false));
      d[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true));
      kvr[i] = __builtin_bit_cast(bf16x8, d);
    }
  };
  if (ntiles > 0) gather(0);
  __bf16* vt = &sh.vt[wave][0];
  for (int it = 0; it < ntiles; ++it) {
    // ---- S partial from the registers ------------------------------------------------
    if constexpr (FP8) widen();
    const float sc_tile = sc;
    F::acc_t accl{}, accr{};
#pragma unroll
    for (int i = 0; i < 8; ++i) accl = F::mfma(aq[i], kvr[i], accl);
    accr = F::mfma(aq[8], kvr[8], accr);
    // ---- the slice's latent columns to this wave's LDS region, then the next gather ----
#pragma unroll
    for (int i = 0; i < 8; ++i) *(bf16x8*)&vt[vslice_at(tok, FP8 ? 64 * g + 8 * i : 16 * i + 8 * g)] = kvr[i];
    if (it + 1 < ntiles) gather(it + 1);
#pragma unroll
    for (int i = 0; i < F::kAccN; ++i)
      sh.spart[wave][F::row_of(i, lane)][tok] = FP8 ? accl[i] * sc_tile + accr[i] : accl[i] + accr[i];
    if (FP8 && wave == 0 && lane < kTileTok) sh.tsc[tok] = sc_tile;   // the tile's row scales, for P
    __syncthreads();
    softmax_tile_lazy<FP8>(sh, sh.tt + it * kTileTok, it, a.scale_log2, tid);
    __syncthreads();
    {
      if (__builtin_amdgcn_readfirstlane(sh.moved[it & 1]) != 0) {   // some head's max moved
        float al[F::kAccN];
#pragma unroll
        for (int i = 0; i < F::kAccN; ++i) al[i] = sh.alpha[F::row_of(i, lane)];
#pragma unroll
        for (int nt = 0; nt < F::kNT; ++nt)
#pragma unroll
          for (int i = 0; i < F::kAccN; ++i) o[nt][i] *= al[i];
      }
      const int arow = F::a_row(lane), ahalf = F::a_half(lane);
      const int grp = lane >> 4, j = lane & 15;
#pragma unroll
      for (int ks = 0; ks < F::kPVsteps; ++ks) {
        const int tk = ks * F::kPVk + ahalf * 8;
        const bf16x8 ph = *(const bf16x8*)&sh.p_hi[p_at(arow, tk)];
        const bf16x8 pl = *(const bf16x8*)&sh.p_lo[p_at(arow, tk)];
#pragma unroll
        for (int nt = 0; nt < F::kNT; ++nt) {
          const int k0 = ks * F::kPVk + (grp >> 1) * 8;
          const int n0 = nt * F::kNTW + (grp & 1) * 16;
          const bf16x8 vb = bfrag_tr_vslice(vt, k0, n0, j);
          o[nt] = F::mfma(ph, vb, o[nt]);
          o[nt] = F::mfma(pl, vb, o[nt]);
        }
      }
    }
  }
  __syncthreads();
  write_out<32, F>(a, sh, o, r, split, h0, wave, lane, tid);
}

__global__ __launch_bounds__(256, 2) void attn_kernel_w32(AttnArgs a) {
  __shared__ AttnSharedW sh;
  attn_w32_body<false, false>(a, sh);
}

__global__ __launch_bounds__(256, 2) void attn_kernel_w32_fp8(AttnArgs a) {
  __shared__ AttnSharedW sh;
  attn_w32_body<false, true>(a, sh);
}

// The dense pass's instance: no block list to read (slot j is block j).
__global__ __launch_bounds__(256, 2) void attn_dense_kernel_w32(AttnArgs a) {
  __shared__ AttnSharedW sh;
  attn_w32_body<true, false>(a, sh);
}

__global__ __launch_bounds__(256, 2) void attn_dense_kernel_w32_fp8(AttnArgs a) {
  __shared__ AttnSharedW sh;
  attn_w32_body<true, true>(a, sh);
}

// ---- decode: every row of the workgroup in LDS at once ------------------------------------
// Few rows (decode): a workgroup of 8 waves owns 16 heads and at most 128 tokens of
// one row; wave w owns tokens 16w .. 16w + 15 from the page lookup to S:
//   * the loads that need nothing go out first: the wave's block ids and a third of
//     the queries (global -> LDS, so the workgroup reads its 18 KiB of queries once);
//     then the page ids; then every latent row of the wave goes global -> LDS
//     directly (one 1 KiB wave-wide load per token, no registers) and its rope rows
//     into registers, already in MFMA B-fragment order;
//   * S for the wave's 16 tokens on v_mfma_f32_16x16x32_bf16 (heads as M), kept in
//     registers; the per-head maxima and sums cross waves through LDS (two barriers);
//   * O = P V with K = 128: wave w owns columns 64w .. 64w + 63, P as a bf16 hi + lo
//     pair, V read transposed from the latent tile.
// bf16 rows only.
constexpr int kDecTok = 128;
constexpr int kDecWaves = 8;
constexpr int kDecRS = kLatent + 16;   // bf16 per LDS latent row (1,056 bytes: conflict-free transposes)
constexpr int kDecPS = kDecTok + 8;    // bf16 per P row
typedef __attribute__((address_space(3))) void lds_void;

struct alignas(16) DecShared {
  __bf16 lat[kDecTok][kDecRS];
  union {
    // queries, read by S only: k-step ks (32 dims) of head h, dims 8g .. 8g + 7 at
    // q[ks][g][h], so one A fragment is 1 KiB of consecutive bytes
    __bf16 q[18][4][16][8];
    struct {                     // then P as hi + lo
      __bf16 hi[16][kDecPS];
      __bf16 lo[16][kDecPS];
    } p;
  } qp;
  float wmax[kDecWaves][16], wsum[kDecWaves][16];
  float m_run[16], l_run[16];
  int32_t wbad[kDecWaves];       // a wave's selected token the table could not name
  int32_t bad;
};

__global__ __launch_bounds__(512, 1) void attn_decode_kernel(AttnArgs a) {
  typedef Frag<16> F;
  __shared__ DecShared sh;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  int unit, hg;
  if (a.ngroups == 1) {
    unit = blockIdx.x;
    hg = 0;
  } else {
    unit = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    hg = (blockIdx.x >> 3) & 1;
  }
  if (unit >= a.n_units) return;
  const int r = unit % a.n_rows, split = unit / a.n_rows;
  const int h0 = hg * 16;
  const int j0 = split * a.slots_per_split;

  // ---- loads with no dependence ------------------------------------------------------
  // Every address is made valid by clamping, so the loads carry no branches and stay
  // in flight together; what a clamped load returns is discarded by the selects below.
  // Lane i < 16 stands for token 16w + i (block slot j0 + 4w + i/4).
  const int b = a.row_stream[r];
  const int t = a.row_pos[r];
  const int j1 = split_end(a, j0, t);
  const int slot = j0 + 4 * wave + ((lane >> 2) & 3);
  const int blk_raw = block_at(a, r, slot < a.k ? slot : a.k - 1);
  {
    // query k-steps w, w + 8 and w + 16 (waves 2.. load k-step w again: same bytes)
    const int hq = h0 + (lane & 15) < a.n_heads ? h0 + (lane & 15) : a.n_heads - 1;   // heads past n_heads are never written
    const __bf16* qr = a.q + ((int64_t)r * a.n_heads + hq) * kRow + (lane >> 4) * 8;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int ks = u < 2 ? wave + 8 * u : (wave < 2 ? wave + 16 : wave);
      __builtin_amdgcn_global_load_lds((const void*)(qr + ks * 32), (lds_void*)&sh.qp.q[ks][0][0][0], 16, 0, 0);
    }
  }
  __asm__ volatile("" ::: "memory");
  const int blk = lane < 16 && slot < j1 ? blk_raw : -1;

  // ---- page of each token; byte offsets of its latent and rope rows -------------------
  const int s = blk * kPoolRatio + (lane & 3);
  const bool sel = blk >= 0 && s <= t;
  const int pi = s / kPageRows;
  const bool in_tab = sel && pi < a.v.pt_stride && b >= 0 && b < a.v.n_streams;
  const int64_t pidx = in_tab ? (int64_t)b * a.v.pt_stride + pi : 0;
  const int pg = a.v.pt ? a.v.pt[pidx] : (int)pidx;
  const int page = in_tab && pg >= 0 && pg < a.v.n_pages ? pg : -1;
  const bool valid = page >= 0;
  const int64_t base = valid ? (int64_t)page * a.v.page_bytes + a.v.cache_off : -1;
  const int64_t lat_off = valid ? base + (int64_t)(s % kPageRows) * a.lat_row_bytes : -1;
  const int64_t rope_off = valid ? base + a.off_rope + (int64_t)(s % kPageRows) * (kRope * 2) : 0;
  const uint64_t vmask = __ballot(valid);
  const bool wbad = __ballot(sel && !valid) != 0;
  if (lane == 0) sh.wbad[wave] = wbad;   // read after the barriers below

  // ---- every load of the wave at once ------------------------------------------------
  const int row0 = 16 * wave;
  const uint32_t lo_l = (uint32_t)lat_off, hi_l = (uint32_t)((uint64_t)lat_off >> 32);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = __builtin_amdgcn_readlane(lo_l, i), hi = __builtin_amdgcn_readlane(hi_l, i);
    const int64_t off = (int64_t)(((uint64_t)hi << 32) | lo);
    if (off >= 0)
      __builtin_amdgcn_global_load_lds((const void*)(a.v.pool + off + lane * 16), (lds_void*)&sh.lat[row0 + i][0],
                                       16, 0, 0);
  }
  // rope straight into the B fragments of the two rope k-steps: lane holds dims
  // 32 ks + 8 (lane / 16) .. + 7 of token lane % 16 (masked tokens read any readable
  // bytes: their scores never reach the softmax)
  bf16x8 br[2];
  {
    const uint32_t lo_r = (uint32_t)rope_off, hi_r = (uint32_t)((uint64_t)rope_off >> 32);
    const uint64_t ro = ((uint64_t)(uint32_t)__shfl((int)hi_r, lane & 15, 64) << 32) |
                        (uint32_t)__shfl((int)lo_r, lane & 15, 64);
    const char* rsrc = a.v.pool + ro + (lane >> 4) * 16;
    br[0] = *(const bf16x8*)rsrc;
    br[1] = *(const bf16x8*)(rsrc + 64);
  }
  // rows not attended are zero (P V multiplies them by 0)
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (!((vmask >> i) & 1)) *(uint4*)&sh.lat[row0 + i][lane * 8] = make_uint4(0, 0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's rows and query k-steps have landed
  __syncthreads();                      // every wave's query k-steps

  // ---- S for the wave's 16 tokens: lane holds heads 4(lane/16) .. + 3 of token lane % 16 ----
  float z[4];
  {
    f32x4 acc[2] = {};
    const int tok = row0 + (lane & 15);
    // every LDS read of S issued before the first MFMA, held there by a scheduling
    // barrier (left to itself the scheduler keeps two k-steps in flight, and the chain
    // waits on LDS latency at every step)
    bf16x8 aq[18], bk[16];
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      aq[ks] = *(const bf16x8*)&sh.qp.q[ks][lane >> 4][lane & 15][0];
      if (ks < 16) bk[ks] = *(const bf16x8*)&sh.lat[tok][ks * 32 + (lane >> 4) * 8];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks)
      acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ks], ks < 16 ? bk[ks] : br[ks - 16], acc[ks & 1], 0, 0, 0);
    const bool att = (vmask >> (lane & 15)) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = att ? (acc[0][i] + acc[1][i]) * a.scale_log2 : -__builtin_inff();
      const float m = group_max<16>(z[i]);
      if ((lane & 15) == 0) sh.wmax[wave][4 * (lane >> 4) + i] = m;
    }
  }
  __syncthreads();   // every wave's maxima; every wave is past its reads of the queries
  {
    // the waves' maxima of this lane's four heads: one 16-byte read per wave, all
    // issued before the first is used
    float4 wm[kDecWaves];
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) wm[w] = *(const float4*)&sh.wmax[w][4 * (lane >> 4)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * (lane >> 4) + i;
      float m = wm[0][i];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) m = __builtin_fmaxf(m, wm[w][i]);
      const float p = z[i] == -__builtin_inff() ? 0.f : exp2_weight(z[i] - m);
      const float ps = group_sum<16>(p);
      if ((lane & 15) == 0) sh.wsum[wave][h] = ps;
      if (wave == 0 && (lane & 15) == 0) sh.m_run[h] = m;
      const __bf16 hi = bf16_rne(p);
      sh.qp.p.hi[h][row0 + (lane & 15)] = hi;
      sh.qp.p.lo[h][row0 + (lane & 15)] = bf16_rne(p - bf16_to_f(hi));
    }
  }
  __syncthreads();
  if (tid < 16) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) l += sh.wsum[w][tid];
    sh.l_run[tid] = l;
  }
  if (tid == 16) {
    int32_t bad = 0;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) bad |= sh.wbad[w];
    sh.bad = bad;
  }
  // ---- O = P V: wave w owns columns 64w .. 64w + 63 (4 tiles of 16) ---------------------
  constexpr int kNTd = 4;
  // All four k-steps of 32 tokens run, whatever the split holds: a token it does not
  // attend has P = 0 and a zeroed row, so its products are exact zeros. Every LDS read
  // is issued before the first MFMA (held there by a scheduling barrier).
  constexpr int kKsd = kDecTok / 32;
  F::acc_t o[kNTd];
#pragma unroll
  for (int nt = 0; nt < kNTd; ++nt) o[nt] = F::acc_t{};
  {
    const int arow = lane & 15, grp = lane >> 4, j = lane & 15;
    bf16x8 ph[kKsd], pl[kKsd], vb[kKsd][kNTd];
#pragma unroll
    for (int ks = 0; ks < kKsd; ++ks) {
      ph[ks] = *(const bf16x8*)&sh.qp.p.hi[arow][ks * 32 + grp * 8];
      pl[ks] = *(const bf16x8*)&sh.qp.p.lo[arow][ks * 32 + grp * 8];
#pragma unroll
      for (int nt = 0; nt < kNTd; ++nt)
        vb[ks][nt] = bfrag_tr(&sh.lat[0][0], kDecRS, ks * 32 + grp * 8, wave * 64 + nt * 16, j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kKsd; ++ks) {
#pragma unroll
      for (int nt = 0; nt < kNTd; ++nt) o[nt] = F::mfma(ph[ks], vb[ks][nt], o[nt]);
#pragma unroll
      for (int nt = 0; nt < kNTd; ++nt) o[nt] = F::mfma(pl[ks], vb[ks][nt], o[nt]);
    }
  }
  __syncthreads();   // l_run, bad
  // ---- output: the wave's 16 x 64 block of O goes through LDS (the latent-tile columns
  // only this wave read in P V) so that each lane stores whole float4 runs of a row ----
  {
    float* ob = (float*)&sh.lat[0][wave * 64];   // 32 floats per latent-tile row
    constexpr int kOS = kDecRS / 2;
#pragma unroll
    for (int nt = 0; nt < kNTd; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = (4 * (lane >> 4) + i) * 64 + nt * 16 + (lane & 15);   // head * 64 + column
        ob[(f >> 5) * kOS + (f & 31)] = o[nt][i];
      }
    const bool bad = sh.bad != 0;
    const int c4 = 4 * (lane & 15);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int h = 4 * pp + (lane >> 4);
      const int f = h * 64 + c4;
      float4 v = *(const float4*)&ob[(f >> 5) * kOS + (f & 31)];
      if (a.nsplit == 1) {
        if (h0 + h < a.n_heads) {
          const float l = sh.l_run[h];
          const float inv = l > 0.f ? 1.f / l : 0.f;
          v = bad ? make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""))
                  : make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
          *(float4*)(a.out + ((int64_t)r * a.n_heads + h0 + h) * kLatent + wave * 64 + c4) = v;
        }
      } else {
        *(float4*)(a.part_o + (((int64_t)r * a.nsplit + split) * 32 + h0 + h) * kLatent + wave * 64 + c4) = v;
      }
    }
    if (wave == 0 && lane < 16) {
      const float l = sh.l_run[lane], m = sh.m_run[lane];
      if (a.nsplit == 1) {
        if (a.lse && h0 + lane < a.n_heads)
          a.lse[(int64_t)r * a.n_heads + h0 + lane] =
              bad ? __builtin_nanf("") : (l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -__builtin_inff());
      } else {
        float* pm = a.part_ml + (((int64_t)r * a.nsplit + split) * 32 + h0 + lane) * 2;
        pm[0] = m;
        pm[1] = bad ? __builtin_nanf("") : l;
      }
    }
  }
}

// Combine the splits of one (row, head): 128 threads, four columns each. The partial
// outputs of the first 16 splits are loaded before the split weights are known, so
// the two dependent rounds of loads overlap.
constexpr int kMergeBatch = 16;

__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a) {
  __shared__ float wgt[64];
  __shared__ float tot[2];
  // row r's merges run on the XCD that wrote its partials: workgroup h * n_rows + r (a
  // row's splits are n_rows workgroups apart, and workgroup i runs on XCD i mod 8)
  const int r = blockIdx.x % a.n_rows, h = blockIdx.x / a.n_rows;
  const int c4 = 4 * threadIdx.x;
  const float* po = a.part_o + ((int64_t)r * a.nsplit * 32 + h) * kLatent + c4;
  float4 v[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u)   // clamped split index: a split past nsplit gets weight 0
    v[u] = *(const float4*)(po + (int64_t)(u < a.nsplit ? u : a.nsplit - 1) * 32 * kLatent);
  const float* pml = a.part_ml + (int64_t)r * a.nsplit * 64;
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float2 ml = *(const float2*)&pml[((s < a.nsplit ? s : a.nsplit - 1) * 32 + h) * 2];
    const float m = s < a.nsplit ? ml.x : -__builtin_inff();
    const float l = s < a.nsplit ? ml.y : 0.f;
    bool nan = (m != m) || (l != l);
    float M = l > 0.f ? m : -__builtin_inff();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      M = __builtin_fmaxf(M, __shfl_xor(M, o, 64));
      nan |= __shfl_xor((int)nan, o, 64) != 0;
    }
    const float f = l > 0.f ? exp2f(m - M) : 0.f;
    float L = l * f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o, 64);
    wgt[s] = f;
    if (s == 0) {
      tot[0] = nan ? __builtin_nanf("") : L;
      tot[1] = M;
    }
  }
  __syncthreads();
  const float L = tot[0];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const float f = u < a.nsplit ? wgt[u] : 0.f;   // a split without an attended token has weight 0
    acc.x += f != 0.f ? v[u].x * f : 0.f;
    acc.y += f != 0.f ? v[u].y * f : 0.f;
    acc.z += f != 0.f ? v[u].z * f : 0.f;
    acc.w += f != 0.f ? v[u].w * f : 0.f;
  }
  // more splits (long block lists): the same, a batch of loads in flight at a time
  for (int s0 = kMergeBatch; s0 < a.nsplit; s0 += kMergeBatch) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      v[u] = *(const float4*)(po + (int64_t)(s0 + u < a.nsplit ? s0 + u : a.nsplit - 1) * 32 * kLatent);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float f = s0 + u < a.nsplit ? wgt[s0 + u] : 0.f;
      acc.x += f != 0.f ? v[u].x * f : 0.f;
      acc.y += f != 0.f ? v[u].y * f : 0.f;
      acc.z += f != 0.f ? v[u].z * f : 0.f;
      acc.w += f != 0.f ? v[u].w * f : 0.f;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *(float4*)(a.out + ((int64_t)r * a.n_heads + h) * kLatent + c4) =
      L != L ? make_float4(L, L, L, L) : make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse && threadIdx.x == 0)
    a.lse[(int64_t)r * a.n_heads + h] =
        L != L ? L : (L > 0.f ? (tot[1] + log2f(L)) * 0.69314718055994531f : -__builtin_inff());
}

struct SplitPlan {
  int nsplit, sps, ngroups, hg, n_units, grid;
  bool decode;  // all tiles in LDS at once (bf16, <= 128 tokens per workgroup)
};

// Few rows (decode): 16 heads and at most 128 tokens per workgroup, so a row is
// spread over many CUs. Many rows (prefill): all 32 heads and the whole block list
// (up to 4,096 tokens) per workgroup.
static SplitPlan pick_split(int32_t n_rows, int32_t n_heads, int32_t k, bool fp8) {
  SplitPlan p;
  const int tiles = (k + 7) / 8;
  p.hg = (n_heads <= 16 || n_rows < 128) ? 16 : 32;
  p.ngroups = (n_heads + p.hg - 1) / p.hg;
  p.decode = p.hg == 16 && !fp8 && n_rows < 128;
  int tiles_per;
  if (p.decode) {
    tiles_per = kDecTok / kTileTok;
  } else {
    int s = (256 + n_rows * p.ngroups - 1) / (n_rows * p.ngroups);
    if (s > tiles) s = tiles;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    tiles_per = (tiles + s - 1) / s;
    if (tiles_per * kTileTok > kMaxWgTok) tiles_per = kMaxWgTok / kTileTok;
  }
  if (tiles_per > tiles) tiles_per = tiles;
  p.sps = tiles_per * 8;
  p.nsplit = (k + p.sps - 1) / p.sps;
  p.n_units = n_rows * p.nsplit;
  p.grid = p.ngroups == 1 ? p.n_units : ((p.n_units + 7) / 8) * 16;
  return p;
}

// Split partials of the allocation-free entry point: a file-scope device array, one
// copy per GPU, held until the process ends. Host code never passes the array's name to
// a kernel (on the host it names a stand-in, not device memory): the device address is
// looked up once per device with hipGetSymbolAddress and kept.
constexpr size_t kScratchBytes = 32u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

size_t attn_scratch_bytes() { return kScratchBytes; }

tf_status attn_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(TF_E_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(TF_E_DEVICE, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(TF_E_DEVICE, "hipGetSymbolAddress of the attention scratch failed on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TF_OK;
}

size_t attn_ws_bytes(int32_t n_rows, int32_t n_heads, int32_t k) {
  // the larger of the two formats' needs (the format is not an argument here)
  SplitPlan p = pick_split(n_rows, n_heads, k, false);
  const SplitPlan q = pick_split(n_rows, n_heads, k, true);
  if (q.nsplit > p.nsplit) p = q;
  if (p.nsplit == 1) return 0;
  return (size_t)n_rows * p.nsplit * 32 * (kLatent + 2) * sizeof(float);
}

tf_status launch_attn(const tf_plan* pl, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                      const int32_t* row_pos, const void* q, int32_t n_heads, float scale,
                      const int32_t* blocks, int32_t k, float* out, float* lse, void* ws,
                      size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  AttnArgs a;
  a.v = v;
  a.off_scale = pl->off_scale;
  a.off_rope = pl->off_rope;
  a.lat_row_bytes = (int32_t)pl->lat_row_bytes;
  a.n_rows = n_rows;
  a.row_stream = row_stream;
  a.row_pos = row_pos;
  a.q = (const __bf16*)q;
  a.n_heads = n_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.blocks = blocks;
  a.k = k;
  const bool fp8 = pl->g.lat_fmt == TF_LAT_FP8E4M3_ROWSCALE;
  const SplitPlan p = pick_split(n_rows, n_heads, k, fp8);
  a.nsplit = p.nsplit;
  a.slots_per_split = p.sps;
  a.ngroups = p.ngroups;
  a.n_units = p.n_units;
  a.out = out;
  a.lse = lse;
  a.part_o = p.nsplit > 1 ? (float*)ws : nullptr;
  a.part_ml = p.nsplit > 1 ? a.part_o + (size_t)n_rows * p.nsplit * 32 * kLatent : nullptr;
  if (p.decode) {
    hipLaunchKernelGGL(attn_decode_kernel, dim3(p.grid), dim3(512), 0, st, a);
  } else if (p.hg == 16) {
    if (fp8) hipLaunchKernelGGL((attn_kernel<16, true>), dim3(p.grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<16, false>), dim3(p.grid), dim3(256), 0, st, a);
  } else {
    if (fp8 && blocks) hipLaunchKernelGGL(attn_kernel_w32_fp8, dim3(p.grid), dim3(256), 0, st, a);
    else if (fp8) hipLaunchKernelGGL(attn_dense_kernel_w32_fp8, dim3(p.grid), dim3(256), 0, st, a);
    else if (blocks) hipLaunchKernelGGL(attn_kernel_w32, dim3(p.grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(attn_dense_kernel_w32, dim3(p.grid), dim3(256), 0, st, a);
  }
  const char* name = blocks ? "tf_sparse_mla_attn" : "tf_dense_mla_attn";
  tf_status s = launch_status(name);
  if (s != TF_OK || p.nsplit == 1) return s;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(n_rows * n_heads), dim3(128), 0, st, a);
  return launch_status(name);
}

}  // namespace tf
