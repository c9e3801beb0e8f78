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
// Design (gfx950, one workgroup of 4 waves per (row, split of its block list)):
//   * 32-token tiles (8 blocks; a block never straddles a 512-row page) are
//     gathered with 16-byte coalesced loads into an LDS tile [32][576] bf16;
//     fp8 rows are widened to bf16 exactly and their scales kept per token.
//   * S = Q K^T on v_mfma_f32_32x32x16_bf16 with the 32 heads as M; the 36
//     k-steps (32 latent + 4 rope) are split over the 4 waves and the partial
//     S tiles summed through LDS. The fp8 row scale multiplies the latent part.
//   * Online softmax in fp32 (exp2 domain).
//   * O += P V on MFMA with P as a bf16 hi + lo pair (16 significant bits) and
//     V read from the LDS tile transposed; each wave owns 128 of the 512 output
//     columns in 64 accumulator registers. The fp8 scale is folded into P.
//   * Rows with few tokens per CU (decode) split their block list; partial
//     (O, max, sum) go to the workspace and a small merge kernel combines them.
#include <math.h>

#include "common.h"

namespace tf {

constexpr int kTileTok = 32;
constexpr int kRS = kRow + 8;  // LDS row stride in bf16 (1,168 bytes)

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
  int32_t nsplit, slots_per_split;
  float* out;
  float* lse;
  float* part_o;   // [n_rows][nsplit][32][512]
  float* part_ml;  // [n_rows][nsplit][32][2]  (max in log2 domain, sum)
};

struct AttnShared {
  __bf16 kv[kTileTok][kRS];
  float spart[4][32][kTileTok + 1];
  __bf16 p_hi[32][kTileTok + 8];
  __bf16 p_lo[32][kTileTok + 8];
  float tsc[kTileTok];           // per-token value scale (1 for bf16 rows, 0 if masked)
  int64_t tlat[kTileTok];        // byte offset of the token's latent row in the pool, -1 masked
  int64_t trope[kTileTok];
  float m_run[32], l_run[32], alpha[32];
  uint16_t lut[256];             // e4m3 -> bf16 bits
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

__device__ __forceinline__ __bf16 bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return __builtin_bit_cast(__bf16, (uint16_t)u);
}

__device__ __forceinline__ float bf16_to_f(__bf16 x) {
  return __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, x)) << 16);
}

template <bool FP8>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int r = blockIdx.y, split = blockIdx.x;
  const int b = a.row_stream[r];
  const int t = a.row_pos[r];
  const int j0 = split * a.slots_per_split;
  const int j1 = j0 + a.slots_per_split < a.k ? j0 + a.slots_per_split : a.k;

  if (FP8) sh.lut[tid] = e4m3_to_bf16_bits((uint32_t)tid);
  if (tid < 32) {
    sh.m_run[tid] = -__builtin_inff();
    sh.l_run[tid] = 0.f;
  }

  // Query fragments of this wave's k-steps: latent steps 8w..8w+7, rope step 32+w.
  bf16x8 aq[9];
  {
    const __bf16* qr = a.q + ((int64_t)r * a.n_heads + n) * kRow + g * 8;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int ks = i < 8 ? wave * 8 + i : 32 + wave;
      aq[i] = n < a.n_heads ? *(const bf16x8*)(qr + ks * 16) : bf16x8{};
    }
  }
  f32x16 o[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) o[nt] = f32x16{};

  for (int j = j0; j < j1; j += 8) {
    // ---- token table of the tile ------------------------------------------------
    if (tid < kTileTok) {
      const int slot = j + tid / 4;
      const int blk = slot < j1 ? a.blocks[(int64_t)r * a.k + slot] : -1;
      const int s = blk * kPoolRatio + (tid & 3);
      int64_t lat = -1, rope = -1;
      float sc = 0.f;
      if (blk >= 0 && s <= t) {
        const int page = page_of(a.v, b, s / kPageRows);
        if (page >= 0) {
          const int64_t base = (int64_t)page * a.v.page_bytes + a.v.cache_off;
          const int slot_in = s % kPageRows;
          lat = base + (int64_t)slot_in * a.lat_row_bytes;
          rope = base + a.off_rope + (int64_t)slot_in * (kRope * 2);
          sc = FP8 ? *(const float*)(a.v.pool + base + a.off_scale + 4LL * slot_in) : 1.f;
        } else {
          sc = __builtin_nanf("");  // a selected token the table cannot name
        }
      }
      sh.tlat[tid] = lat;
      sh.trope[tid] = rope;
      sh.tsc[tid] = sc;
    }
    __syncthreads();
    // ---- gather: 16-byte pieces, consecutive threads along a row ------------------
    if (!FP8) {
      // 64 latent pieces + 8 rope pieces per token
      for (int u = tid; u < kTileTok * 72; u += 256) {
        const int tok = u / 72, pc = u % 72;
        const int64_t base = pc < 64 ? sh.tlat[tok] : sh.trope[tok];
        uint4 val = make_uint4(0, 0, 0, 0);
        if (base >= 0) val = *(const uint4*)(a.v.pool + base + (pc < 64 ? pc : pc - 64) * 16);
        *(uint4*)&sh.kv[tok][pc < 64 ? pc * 8 : kLatent + (pc - 64) * 8] = val;
      }
    } else {
      // 32 latent pieces of 16 e4m3 bytes + 8 rope pieces per token
      for (int u = tid; u < kTileTok * 40; u += 256) {
        const int tok = u / 40, pc = u % 40;
        if (pc < 32) {
          const int64_t base = sh.tlat[tok];
          uint4 val = make_uint4(0, 0, 0, 0);
          if (base >= 0) val = *(const uint4*)(a.v.pool + base + pc * 16);
          const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
          uint32_t outw[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t x = w4[i];
            outw[2 * i] = (uint32_t)sh.lut[x & 255u] | ((uint32_t)sh.lut[(x >> 8) & 255u] << 16);
            outw[2 * i + 1] = (uint32_t)sh.lut[(x >> 16) & 255u] | ((uint32_t)sh.lut[x >> 24] << 16);
          }
          *(uint4*)&sh.kv[tok][pc * 16] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
          *(uint4*)&sh.kv[tok][pc * 16 + 8] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
        } else {
          const int64_t base = sh.trope[tok];
          uint4 val = make_uint4(0, 0, 0, 0);
          if (base >= 0) val = *(const uint4*)(a.v.pool + base + (pc - 32) * 16);
          *(uint4*)&sh.kv[tok][kLatent + (pc - 32) * 8] = val;
        }
      }
    }
    __syncthreads();
    // ---- S partials: this wave's 9 k-steps --------------------------------------
    {
      f32x16 accl = {}, accr = {};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ks = wave * 8 + i;
        const bf16x8 bk = *(const bf16x8*)&sh.kv[n][ks * 16 + g * 8];
        accl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[i], bk, accl, 0, 0, 0);
      }
      {
        const bf16x8 bk = *(const bf16x8*)&sh.kv[n][(32 + wave) * 16 + g * 8];
        accr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[8], bk, accr, 0, 0, 0);
      }
      const float tsc = FP8 ? sh.tsc[n] : 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * g + (i & 3);
        sh.spart[wave][m][n] = accl[i] * tsc + accr[i];
      }
    }
    __syncthreads();
    // ---- online softmax: 8 threads per head, 4 tokens each ----------------------
    {
      const int h = tid >> 3, p = tid & 7;
      float z[4];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 4 * p + e;
        const float sc = sh.tsc[tok];
        float v = (sh.spart[0][h][tok] + sh.spart[1][h][tok] + sh.spart[2][h][tok] + sh.spart[3][h][tok]) *
                  a.scale_log2;
        if (sh.tlat[tok] < 0) v = sc != sc ? sc : -__builtin_inff();  // masked (NaN if unreadable)
        z[e] = v;
        tmax = __builtin_fmaxf(tmax, v);
        if (v != v) tmax = v;
      }
#pragma unroll
      for (int o2 = 1; o2 < 8; o2 <<= 1) {
        const float y = __shfl_xor(tmax, o2, 64);
        tmax = (y != y) ? y : __builtin_fmaxf(tmax, y);
      }
      const float m_old = sh.m_run[h];
      const float m_new = __builtin_fmaxf(m_old, tmax) + (tmax != tmax ? tmax : 0.f);
      const float alpha = m_new == -__builtin_inff() ? 1.f : exp2f(m_old - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 4 * p + e;
        const float pe = z[e] == -__builtin_inff() ? 0.f : exp2f(z[e] - m_new);
        lsum += pe;
        const float pv = FP8 ? pe * sh.tsc[tok] : pe;
        const __bf16 hi = bf16_rne(pv);
        sh.p_hi[h][tok] = hi;
        sh.p_lo[h][tok] = bf16_rne(pv - bf16_to_f(hi));
      }
#pragma unroll
      for (int o2 = 1; o2 < 8; o2 <<= 1) lsum += __shfl_xor(lsum, o2, 64);
      __syncthreads();  // every thread of the head has read m_run before it changes
      if (p == 0) {
        sh.m_run[h] = m_new;
        sh.l_run[h] = sh.l_run[h] * alpha + lsum;
        sh.alpha[h] = alpha;
      }
    }
    __syncthreads();
    // ---- O = alpha * O + P V: wave owns columns [128w, 128w + 128) ---------------
    {
      float al[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) al[i] = sh.alpha[8 * (i >> 2) + 4 * g + (i & 3)];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[nt][i] *= al[i];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 ph = *(const bf16x8*)&sh.p_hi[n][ks * 16 + g * 8];
        const bf16x8 pl = *(const bf16x8*)&sh.p_lo[n][ks * 16 + g * 8];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int d = wave * 128 + nt * 32 + n;
          bf16x8 vb;
#pragma unroll
          for (int e = 0; e < 8; ++e) vb[e] = sh.kv[ks * 16 + g * 8 + e][d];
          o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, vb, o[nt], 0, 0, 0);
          o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl, vb, o[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- write -----------------------------------------------------------------------
  if (a.nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 8 * (i >> 2) + 4 * g + (i & 3);
      if (m >= a.n_heads) continue;
      const float l = sh.l_run[m];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* orow = a.out + ((int64_t)r * a.n_heads + m) * kLatent + wave * 128 + n;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) orow[nt * 32] = o[nt][i] * inv;
    }
    if (a.lse && tid < a.n_heads) {
      const float l = sh.l_run[tid];
      a.lse[(int64_t)r * a.n_heads + tid] =
          l > 0.f ? (sh.m_run[tid] + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
    }
  } else {
    float* po = a.part_o + ((int64_t)r * a.nsplit + split) * 32 * kLatent;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 8 * (i >> 2) + 4 * g + (i & 3);
      float* orow = po + (int64_t)m * kLatent + wave * 128 + n;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) orow[nt * 32] = o[nt][i];
    }
    if (tid < 32) {
      float* pm = a.part_ml + (((int64_t)r * a.nsplit + split) * 32 + tid) * 2;
      pm[0] = sh.m_run[tid];
      pm[1] = sh.l_run[tid];
    }
  }
}

// Combine the splits of one (row, head): 128 threads x 4 columns.
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a) {
  const int r = blockIdx.x / a.n_heads, h = blockIdx.x % a.n_heads;
  const float* pml = a.part_ml + (int64_t)r * a.nsplit * 64;
  float M = -__builtin_inff();
  bool nan = false;
  for (int s = 0; s < a.nsplit; ++s) {
    const float m = pml[(s * 32 + h) * 2], l = pml[(s * 32 + h) * 2 + 1];
    if (m != m || l != l) nan = true;
    if (l > 0.f) M = __builtin_fmaxf(M, m);
  }
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int d = threadIdx.x * 4;
  for (int s = 0; s < a.nsplit; ++s) {
    const float m = pml[(s * 32 + h) * 2], l = pml[(s * 32 + h) * 2 + 1];
    if (!(l > 0.f)) continue;
    const float f = exp2f(m - M);
    L += l * f;
    const float4 v = *(const float4*)(a.part_o + (((int64_t)r * a.nsplit + s) * 32 + h) * kLatent + d);
    acc.x += v.x * f;
    acc.y += v.y * f;
    acc.z += v.z * f;
    acc.w += v.w * f;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float4 res = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (nan) res = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
  *(float4*)(a.out + ((int64_t)r * a.n_heads + h) * kLatent + d) = res;
  if (a.lse && threadIdx.x == 0)
    a.lse[(int64_t)r * a.n_heads + h] =
        nan ? __builtin_nanf("") : (L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -__builtin_inff());
}

static void pick_split(int32_t n_rows, int32_t k, int& nsplit, int& sps) {
  const int tiles = (k + 7) / 8;
  int s = (256 + n_rows - 1) / n_rows;
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  const int tiles_per = (tiles + s - 1) / s;
  sps = tiles_per * 8;
  nsplit = (k + sps - 1) / sps;
}

size_t attn_ws_bytes(int32_t n_rows, int32_t n_heads, int32_t k) {
  (void)n_heads;
  int ns, sps;
  pick_split(n_rows, k, ns, sps);
  if (ns == 1) return 0;
  return (size_t)n_rows * ns * 32 * (kLatent + 2) * sizeof(float);
}

tf_status launch_attn(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                      const int32_t* row_pos, const void* q, int32_t n_heads, float scale,
                      const int32_t* blocks, int32_t k, float* out, float* lse, void* ws,
                      size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  AttnArgs a;
  a.v = v;
  a.off_scale = p->off_scale;
  a.off_rope = p->off_rope;
  a.lat_row_bytes = (int32_t)p->lat_row_bytes;
  a.n_rows = n_rows;
  a.row_stream = row_stream;
  a.row_pos = row_pos;
  a.q = (const __bf16*)q;
  a.n_heads = n_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.blocks = blocks;
  a.k = k;
  int ns, sps;
  pick_split(n_rows, k, ns, sps);
  a.nsplit = ns;
  a.slots_per_split = sps;
  a.out = out;
  a.lse = lse;
  a.part_o = ns > 1 ? (float*)ws : nullptr;
  a.part_ml = ns > 1 ? (float*)ws + (size_t)n_rows * ns * 32 * kLatent : nullptr;
  if (n_rows > 65535) return set_error(TF_E_RANGE, "tf_sparse_mla_attn: at most 65535 rows per call");
  const bool fp8 = p->g.lat_fmt == TF_LAT_FP8E4M3_ROWSCALE;
  if (fp8) hipLaunchKernelGGL(attn_kernel<true>, dim3(ns, n_rows), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(attn_kernel<false>, dim3(ns, n_rows), dim3(256), 0, st, a);
  tf_status s = launch_status("tf_sparse_mla_attn");
  if (s != TF_OK || ns == 1) return s;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(n_rows * n_heads), dim3(128), 0, st, a);
  return launch_status("tf_sparse_mla_attn");
}

}  // namespace tf
