// Exact top-k selection on one workgroup of 1,024 threads, shared by the top-k kernels
// and the fused indexer selection: order-preserving keys, a most-significant-digit
// radix select with LDS histograms, and an emission of the selected keys in index
// order (ties to the lower index) from block-wide prefix counts.
#pragma once

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

// Sum and minimum of a value over the wave (wave-uniform results).
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)x, s, 64);
    x = x < y ? x : y;
  }
  return x;
}

// One wave's selection: T = the k-th largest of its n >= k valid keys (E a lane; invalid
// slots hold 0) and rem = how many keys equal to T belong to the top k. The bits above
// the highest one in which the keys differ are common; the rest are decided by a
// most-significant-digit radix select in digits of at most 8 bits, each digit from a
// 256-bin histogram of the keys matching the digits decided so far, in `hist` (256
// words of LDS that only this wave uses), down to lo_bit. With lo_bit > 0, T's bits
// below lo_bit are 0 and rem is not set: at least k keys are >= T.
template <int E>
__device__ void wave_select(const uint32_t (&key)[E], uint32_t k, int lo_bit, uint32_t* hist, uint32_t& T,
                            uint32_t& rem) {
  const int lane = threadIdx.x & 63;
  uint32_t o4[2] = {0u, 0u}, a4[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] != 0u) {
      o4[e & 1] |= key[e];
      a4[e & 1] &= key[e];
    }
  uint32_t o = o4[0] | o4[1], an = a4[0] & a4[1];
  wave_or_and(o, an);
  const uint32_t diff = o ^ an;
  if (diff == 0u) {   // every valid key equal
    T = o;
    rem = k;
    return;
  }
  const int hb = 31 - __builtin_clz(diff);
  uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = an & mask, r = k;
  for (int top = hb + 1; top > lo_bit;) {
    const int width = top - lo_bit < 8 ? top - lo_bit : 8;
    const int shift = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    *(uint4*)&hist[4 * lane] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0u && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> shift) & dmask], 1u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane l holds bins 255 - 4l .. 252 - 4l, so lanes in order walk the bins downwards
    const uint4 hv = *(const uint4*)&hist[4 * (63 - lane)];
    const uint32_t c = hv.x + hv.y + hv.z + hv.w;
    const uint32_t incl = wave_incl_scan(c);
    const uint64_t hit = __ballot(incl - c < r && r <= incl);
    const int hl = (int)__builtin_ctzll(hit);
    uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - c), hl);
    const uint32_t w3 = (uint32_t)__builtin_amdgcn_readlane((int)hv.w, hl);
    const uint32_t w2 = (uint32_t)__builtin_amdgcn_readlane((int)hv.z, hl);
    const uint32_t w1 = (uint32_t)__builtin_amdgcn_readlane((int)hv.y, hl);
    uint32_t bin = 4u * (63u - (uint32_t)hl) + 3u;
    if (above + w3 < r) {
      above += w3;
      --bin;
      if (above + w2 < r) {
        above += w2;
        --bin;
        if (above + w1 < r) {
          above += w1;
          --bin;
        }
      }
    }
    r -= above;
    prefix |= bin << shift;
    mask |= dmask << shift;
    top = shift;
  }
  T = prefix;
  rem = r;
}

struct alignas(16) SelShared {
  uint32_t hist[3][kBins];   // one histogram per radix pass, all cleared up front
  uint32_t wor[kWaves], wand[kWaves], wsum[kWaves];
  uint32_t scan[2][2][kWaves];   // two buffers of per-wave totals of two counts
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
// With first_pass_only, T is instead the lowest key of the first pass's bin that holds
// the k-th largest (at least k keys are >= T) and rem is not set.
template <int E>
__device__ void radix_select(const uint32_t (&key)[E], int k, SelShared& sh, uint32_t& T, uint32_t& rem,
                             bool first_pass_only = false) {
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
    if (first_pass_only) break;
  }
  T = prefix;
  rem = r;
}

// Exclusive block-wide prefix (in thread order) of two per-thread counts, and their
// totals. w is one of the two scan buffers; a caller alternates them, or leaves a
// barrier between two uses of one buffer.
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t (&w)[2][kWaves], uint32_t& a_before,
                                            uint32_t& b_before, uint32_t& a_tot, uint32_t& b_tot) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ai = wave_incl_scan(a), bi = wave_incl_scan(b);
  if (lane == 63) {
    w[0][wid] = ai;
    w[1][wid] = bi;
  }
  __syncthreads();
  const uint32_t aw = waves_before(w[0], a_tot), bw = waves_before(w[1], b_tot);
  a_before = aw + ai - a;
  b_before = bw + bi - b;
}

// emit(pos, e) for the keys above T and the first rem keys equal to T, pos ascending
// with the index (thread t holds the contiguous keys t*E + e).
template <int E, typename Emit>
__device__ __forceinline__ void ordered_emit(const uint32_t (&key)[E], uint32_t T, uint32_t rem,
                                             uint32_t (&w)[2][kWaves], Emit emit) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gt += key[e] > T ? 1u : 0u;
    eq += key[e] == T ? 1u : 0u;
  }
  uint32_t gt_b, eq_b, gt_t, eq_t;
  block_scan2(gt, eq, w, gt_b, eq_b, gt_t, eq_t);
  uint32_t pos = gt_b + (eq_b < rem ? eq_b : rem);
  uint32_t eq_i = eq_b;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool is_eq = key[e] == T;
    if (key[e] > T || (is_eq && eq_i < rem)) emit(pos++, e);
    eq_i += is_eq ? 1u : 0u;
  }
}

// Thread t's keys t*E .. t*E + E - 1 of a segment of n (invalid slots: 0). VEC: the
// segment is 16-byte aligned and every group of four that starts before n lies in the
// row, so groups load as one 16-byte access. (A compile-time choice: kernels are built
// once for each, so the 16-byte form's code does not carry the other.)
template <int E, bool VEC>
__device__ __forceinline__ void load_keys(const float* seg, int n, uint32_t (&key)[E]) {
  const int base = threadIdx.x * E;
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
      const int i = base + 4 * j;
      const float4 v = i < n ? *(const float4*)(seg + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      key[4 * j + 0] = i + 0 < n ? order_key(v.x) : 0u;
      key[4 * j + 1] = i + 1 < n ? order_key(v.y) : 0u;
      key[4 * j + 2] = i + 2 < n ? order_key(v.z) : 0u;
      key[4 * j + 3] = i + 3 < n ? order_key(v.w) : 0u;
    }
  } else {
    // every load issued before any is used (indices clamped into the segment): a load
    // under the test of its own index would wait for its data before the next starts
    const int last = n > 0 ? n - 1 : 0;
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = seg[base + e < n ? base + e : last];
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = base + e < n ? order_key(v[e]) : 0u;
  }
}

// ---- long segments: a sampled threshold first ---------------------------------------------
// Each thread splits its keys into S groups (S * 1,024 > k) and offers each group's
// maximum as a sample. One radix pass over the samples gives T0, the lowest key of the
// pass's bin that holds the k-th largest sample: at least k samples, which are distinct
// keys, are >= T0, so the top k lies among the keys >= T0 (ties with the k-th value
// included). Those candidates, usually a little over k, go in index order into LDS,
// where the exact selection runs on them, four per thread. With too few samples or too
// many candidates the caller selects on the whole segment instead.
constexpr int kCandCap = 4 * kNT;

struct alignas(16) CandShared {
  uint32_t key[kCandCap];
  int32_t idx[kCandCap];
};

// emit(pos, key, idx) for the k selected keys, pos ascending with the index; idx_of(e)
// names thread key e. False when the caller must select on the whole segment.
template <int E, int S, typename IdxOf, typename Emit>
__device__ bool select_sampled(const uint32_t (&key)[E], int k, SelShared& sh, CandShared& cs, IdxOf idx_of,
                               Emit emit) {
  static_assert(E % S == 0, "S groups of keys");
  constexpr int G = E / S;
  uint32_t smp[S];
  uint32_t nsmp = 0;
#pragma unroll
  for (int c = 0; c < S; ++c) {
    uint32_t m = 0u;
#pragma unroll
    for (int e = c * G; e < (c + 1) * G; ++e) m = key[e] > m ? key[e] : m;
    smp[c] = m;
    nsmp += m != 0u ? 1u : 0u;
  }
  uint32_t x0, x1, ns, x3;
  block_scan2(nsmp, 0u, sh.scan[0], x0, x1, ns, x3);
  if (ns <= (uint32_t)k) return false;
  uint32_t T0, unused;
  radix_select<S>(smp, k, sh, T0, unused, true);
  if (T0 == 0u) T0 = 1u;   // every valid key (invalid slots hold 0)
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) c += key[e] >= T0 ? 1u : 0u;
  uint32_t c_b, y1, C, y3;
  block_scan2(c, 0u, sh.scan[1], c_b, y1, C, y3);
  if (C > (uint32_t)kCandCap) return false;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] >= T0) {
      cs.key[c_b] = key[e];
      cs.idx[c_b] = idx_of(e);
      ++c_b;
    }
  __syncthreads();
  if (C == (uint32_t)k) {
    for (int i = threadIdx.x; i < k; i += kNT) emit((uint32_t)i, cs.key[i], cs.idx[i]);
    return true;
  }
  uint32_t ck[4];
  int32_t ci[4];
  {
    const uint4 kv = *(const uint4*)&cs.key[4 * threadIdx.x];
    const int4 iv = *(const int4*)&cs.idx[4 * threadIdx.x];
    const uint32_t kk[4] = {kv.x, kv.y, kv.z, kv.w};
    const int32_t ii[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = 4 * (int)threadIdx.x + e < (int)C;
      ck[e] = in ? kk[e] : 0u;
      ci[e] = in ? ii[e] : -1;
    }
  }
  uint32_t T, rem;
  radix_select<4>(ck, k, sh, T, rem);
  ordered_emit<4>(ck, T, rem, sh.scan[0], [&](uint32_t pos, int e) { emit(pos, ck[e], ci[e]); });
  return true;
}

// The k largest of a segment's keys (n_valid > k of them), in index order.
template <int E, typename IdxOf, typename Emit>
__device__ void select_topk(const uint32_t (&key)[E], int k, SelShared& sh, CandShared& cs, IdxOf idx_of,
                            Emit emit) {
  if constexpr (E >= 16) {
    bool done;
    if (k < kNT) done = select_sampled<E, 1>(key, k, sh, cs, idx_of, emit);
    else if (k < 2 * kNT) done = select_sampled<E, 2>(key, k, sh, cs, idx_of, emit);
    else done = select_sampled<E, 4>(key, k, sh, cs, idx_of, emit);
    if (done) return;
    __syncthreads();
  }
  uint32_t T, rem;
  radix_select<E>(key, k, sh, T, rem);
  ordered_emit<E>(key, T, rem, sh.scan[0], [&](uint32_t pos, int e) { emit(pos, key[e], idx_of(e)); });
}

}  // namespace tf
