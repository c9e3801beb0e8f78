// Indexer logits on MFMA: l[t,j] = sum_h w[t,h] * ReLU(q[t,h] . k_j), fp32,
// masked to -inf for j >= n_c(t) = t/4 + 1.
// [CPM, section 1]: each chunk's query rows scored against the whole compressed
// prefix, output [T, max_seqlen_k] fp32, masked by the compressed lengths.
// [#1142, "GLM declares a kv_pool.Layout"]: the pooled keys are read through the
// page table.
//
// Design (gfx950): one v_mfma_f32_32x32x16_bf16 tile is 32 (row, head) pairs x
// 32 keys x 16 dims. The 32 A-rows are 32/H query rows of H heads each, arranged
// so that each lane's 16 accumulators are all H heads of 16/H rows for one key;
// the ReLU, the weights and the head sum then stay inside the lane (no shuffles),
// and each half-wave stores 32 consecutive keys of a row (128-byte stores).
// Queries stay in registers for the whole launch; keys stream through once per
// row tile, loaded straight from the page into MFMA B fragments. The rows of one
// tile share B only when their tables name the same page for the key tile (one
// stream, or shared prefix pages); otherwise each distinct page is a pass of its own.
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
  float* logits;
  int64_t ld;
  int32_t* n_valid;
  int32_t keys_per_wg;
};

template <int H, int D, int MT>
__global__ __launch_bounds__(256, 2) void indexer_kernel(IdxArgs a) {
  constexpr int RPT = 32 / H;   // query rows per MFMA tile
  constexpr int RH = 16 / H;    // rows per half-wave in the accumulators
  constexpr int KS = D / 16;    // MFMA k-steps
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;      // half-wave
  const int n = lane & 31;      // key column of this lane / A row of this lane
  const int wave_row0 = (blockIdx.y * 4 + wave) * (MT * RPT);

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
      for (int ks = 0; ks < KS; ++ks) {
        if (row < a.n_rows) {
          afrag[t][ks] = *(const bf16x8*)(a.q + ((int64_t)row * H + head) * D + ks * 16 + g * 8);
        } else {
          afrag[t][ks] = bf16x8{};
        }
      }
    }
  }
  // Weights of this lane's accumulators: value i is tile row g*RH + i/H, head i%H.
  float wv[MT][16];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = wave_row0 + t * RPT + g * RH + i / H;
      wv[t][i] = row < a.n_rows ? a.w[(int64_t)row * H + (i % H)] : 0.f;
    }
  }
  // Wave-uniform row facts.
  int rstream[MT][RPT], rnc[MT][RPT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int row = wave_row0 + t * RPT + j;
      int nc = -1, st = 0;
      if (row < a.n_rows) {
        const int pos = a.row_pos[row];
        st = a.row_stream[row];
        nc = pos >= 0 ? (int)((int64_t)pos / kPoolRatio + 1 < a.ld ? pos / kPoolRatio + 1 : a.ld) : 0;
      }
      rstream[t][j] = __builtin_amdgcn_readfirstlane(st);
      rnc[t][j] = __builtin_amdgcn_readfirstlane(nc);
    }
  }
  if (blockIdx.x == 0 && a.n_valid && lane < MT * RPT) {
    const int row = wave_row0 + lane;
    if (row < a.n_rows) {
      const int pos = a.row_pos[row];
      a.n_valid[row] = pos >= 0 ? (int)((int64_t)pos / kPoolRatio + 1 < a.ld ? pos / kPoolRatio + 1 : a.ld) : 0;
    }
  }

  const int64_t kb = (int64_t)blockIdx.x * a.keys_per_wg;
  const int64_t ke = kb + a.keys_per_wg < a.ld ? kb + a.keys_per_wg : a.ld;
  const float ninf = -__builtin_inff();
  const float qnan = __builtin_nanf("");

  for (int64_t kt = kb; kt < ke; kt += 32) {
    const int pidx = (int)(kt / kKeysPerPage);
    const int slot0 = (int)(kt % kKeysPerPage);
    const int64_t key = kt + n;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      int pg[RPT];
      bool need[RPT];
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        need[j] = rnc[t][j] > kt;
        pg[j] = need[j] ? page_of(a.v, rstream[t][j], pidx) : -2;
      }
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        // rows past their compressed length for the whole tile: -inf only
        const int row = wave_row0 + t * RPT + j;
        if (rnc[t][j] >= 0 && !need[j] && (j / RH) == g && key < a.ld)
          a.logits[(int64_t)row * a.ld + key] = ninf;
      }
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        if (!need[j]) continue;
        bool leader = true;
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
          if (need[jj] && pg[jj] == pg[j]) leader = false;
        if (!leader) continue;
        f32x16 acc = {};
        if (pg[j] >= 0) {
          const char* kp = cache_block(a.v, pg[j]) + a.off_pkey +
                           (int64_t)(slot0 + n) * a.pkey_row_bytes + g * 16;
          bf16x8 bfrag[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) bfrag[ks] = *(const bf16x8*)(kp + ks * 32);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[t][ks], bfrag[ks], acc, 0, 0, 0);
        }
        // epilogue: this lane holds rows g*RH + r (r < RH), all heads, key `key`
#pragma unroll
        for (int r = 0; r < RH; ++r) {
          const int tr = g * RH + r;
          // wave-uniform membership test per tile row, selected per half
          bool mine = false;
          int ncr = 0;
#pragma unroll
          for (int jj = 0; jj < RPT; ++jj) {
            if (jj == tr) {
              mine = need[jj] && pg[jj] == pg[j];
              ncr = rnc[t][jj];
            }
          }
          if (!mine || key >= a.ld) continue;
          float s = 0.f;
#pragma unroll
          for (int h = 0; h < H; ++h) s = __builtin_fmaf(wv[t][r * H + h], __builtin_fmaxf(acc[r * H + h], 0.f), s);
          const int row = wave_row0 + t * RPT + tr;
          a.logits[(int64_t)row * a.ld + key] = key < ncr ? (pg[j] >= 0 ? s : qnan) : ninf;
        }
      }
    }
  }
}

template <int H, int D, int MT>
static void launch_one(const IdxArgs& a, int rows_per_wg, hipStream_t st) {
  const int64_t kgroups = (a.ld + a.keys_per_wg - 1) / a.keys_per_wg;
  const int rgroups = (a.n_rows + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((indexer_kernel<H, D, MT>), dim3((unsigned)kgroups, (unsigned)rgroups), dim3(256), 0, st, a);
}

template <int H, int D>
static void launch_hd(const IdxArgs& a0, int32_t n_rows, hipStream_t st) {
  IdxArgs a = a0;
  constexpr int RPT = 32 / H;
  // Two tiles per wave when there are rows to fill them; one for small batches.
  const int mt = n_rows >= 8 * 4 * RPT ? 2 : 1;
  const int rows_per_wg = 4 * mt * RPT;
  const int64_t rgroups = (n_rows + rows_per_wg - 1) / rows_per_wg;
  // about 2048 workgroups in all, each over a multiple of 32 keys
  int64_t kpw = (a.ld * rgroups + 2047) / 2048;
  kpw = (kpw + 31) / 32 * 32;
  if (kpw < 32) kpw = 32;
  if (kpw > 4096) kpw = 4096;
  a.keys_per_wg = (int32_t)kpw;
  if (mt == 2) launch_one<H, D, 2>(a, rows_per_wg, st);
  else launch_one<H, D, 1>(a, rows_per_wg, st);
}

tf_status launch_indexer(const tf_plan* p, const DevView& v, int32_t n_rows, const int32_t* row_stream,
                         const int32_t* row_pos, const void* q, const float* w, int32_t n_heads,
                         float* logits, int64_t ld, int32_t* n_valid, hipStream_t st) {
  IdxArgs a;
  a.v = v;
  a.off_pkey = p->off_pkey;
  a.pkey_row_bytes = (int32_t)p->pkey_row_bytes;
  a.n_rows = n_rows;
  a.row_stream = row_stream;
  a.row_pos = row_pos;
  a.q = (const __bf16*)q;
  a.w = w;
  a.logits = logits;
  a.ld = ld;
  a.n_valid = n_valid;
  a.keys_per_wg = 32;
  const int D = p->g.index_dim;
  if ((ld + 2047) / 2048 * ((n_rows + 7) / 8) > 0x7fffffffLL)
    return set_error(TF_E_RANGE, "tf_indexer_logits: too many rows x keys for one launch");
  if (D == 128) {
    if (n_heads == 16) launch_hd<16, 128>(a, n_rows, st);
    else if (n_heads == 8) launch_hd<8, 128>(a, n_rows, st);
    else launch_hd<4, 128>(a, n_rows, st);
  } else {
    if (n_heads == 16) launch_hd<16, 64>(a, n_rows, st);
    else if (n_heads == 8) launch_hd<8, 64>(a, n_rows, st);
    else launch_hd<4, 64>(a, n_rows, st);
  }
  return launch_status("tf_indexer_logits");
}

}  // namespace tf
