// Latent / rope / pooled-key row writes through the page table, and the snapshot
// copy of a stream's first `at` rows. Both are byte copies, bound by HBM; the
// quantizing write turns bf16 latent rows into e4m3 codes and a row scale on the way.
//
// [#1142, "GLM declares a kv_pool.Layout"]: the writes take the page table; a
// null table keeps contiguous rows. [#1142, "Proposal" piece 1]: a kept state
// copies each cache's first at rows and the pooled keys up to at.
#include "common.h"

namespace tf {

struct WriteArgs {
  DevView v;
  int32_t n_rows, n_pkeys;
  const int32_t* row_stream;
  const int32_t* row_pos;
  const uint4* latent;   // n_rows * lat16 vectors
  const float* scale;    // fp8 only
  const uint4* rope;     // n_rows * rope16 vectors
  const int32_t* pkey_stream;
  const int32_t* pkey_idx;
  const uint4* pkeys;    // n_pkeys * key16 vectors
  int32_t lat16, rope16, key16;  // 16-byte vectors per latent row / rope row / key
  int64_t off_scale, off_rope, off_pkey;
  int32_t lat_row_bytes, rope_row_bytes, pkey_row_bytes;
  int32_t row_blocks;    // blocks that write rows; the rest write keys
  int32_t quantize;      // latent holds bf16 rows to code as e4m3 with a row scale
};

constexpr int kRowsPerBlock = 4;   // 64 threads per row
constexpr int kKeysPerBlock = 16;  // 16 threads per key

// e4m3fn code of q, |q| <= 448 (a finite value already clamped), rounding to nearest
// with ties to the even code. Below 2^-6 the codes step by 2^-9 (subnormals, and
// code 8 = 2^-6 continues them). Above, the fp32 mantissa is rounded to 3 bits
// (ties to even) and the exponent rebiased from 127 to 7; the clamp keeps the result
// at or below 0x7E (448), never the NaN code 0x7F. The sign comes from q's sign bit.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t bits = __float_as_uint(q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7FFFFFFFu;
  uint32_t code;
  if (mag < 0x3C800000u) {   // |q| < 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  } else {
    code = ((mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | code;
}

// One wave codes one 512-value row: lane l holds values 8l .. 8l+7 (16 bytes of
// bf16), the wave's max |x| gives scale = amax / 448, and the lane writes its 8
// codes as 8 contiguous bytes; lane 0 writes the scale.
__device__ __forceinline__ void quantize_row(const uint4 v, uint8_t* dst_codes, float* dst_scale, int lane) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, 64));
  const float scale = amax / 448.0f;
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = scale > 0.f ? x[i] / scale : 0.f;
    q = __builtin_fminf(__builtin_fmaxf(q, -448.0f), 448.0f);
    c[i >> 2] |= e4m3_code(q) << (8 * (i & 3));
  }
  *(uint2*)(dst_codes + 8 * lane) = make_uint2(c[0], c[1]);
  if (lane == 0) *dst_scale = scale;
}

// The source rows are read before the page lookup: they depend only on the row index,
// so the loads of the inputs and of the table overlap and each copy waits for one
// round trip instead of two. A row holds at most 64 16-byte vectors of latent and of
// rope (one a lane) and a key at most 16 (one a lane of its 16), which the launch checks.
__global__ __launch_bounds__(256) void latent_write_kernel(WriteArgs a) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < a.row_blocks) {
    const int r = blockIdx.x * kRowsPerBlock + tid / 64;
    const int lane = tid % 64;
    if (r >= a.n_rows) return;
    const int b = a.row_stream[r];
    const int t = a.row_pos[r];
    // unconditional loads (indices clamped into the row; a missing input reads the
    // latent row instead): no branch, so the table lookup below waits only for b and t
    const int nl = a.quantize ? kLatent * 2 / 16 : a.lat16;
    const uint4* src_l = a.latent + (int64_t)r * nl;
    const uint4 vl = src_l[lane < nl ? lane : nl - 1];
    const uint4 vr = a.rope16 > 0 ? a.rope[(int64_t)r * a.rope16 + (lane < a.rope16 ? lane : a.rope16 - 1)] : vl;
    const float vs = a.scale ? a.scale[r] : 0.f;
    if (t < 0) return;
    const int page = page_of(a.v, b, t / kPageRows);
    if (page < 0) return;
    char* blk = cache_block(a.v, page);
    const int slot = t % kPageRows;
    if (a.quantize) {
      quantize_row(vl, (uint8_t*)(blk + (int64_t)slot * a.lat_row_bytes), (float*)(blk + a.off_scale + 4LL * slot),
                   lane);
    } else if (lane < a.lat16) {
      ((uint4*)(blk + (int64_t)slot * a.lat_row_bytes))[lane] = vl;
    }
    if (lane < a.rope16) ((uint4*)(blk + a.off_rope + (int64_t)slot * a.rope_row_bytes))[lane] = vr;
    if (a.scale && lane == 0) *(float*)(blk + a.off_scale + 4LL * slot) = vs;
  } else {
    const int kk = (blockIdx.x - a.row_blocks) * kKeysPerBlock + tid / 16;
    const int lane = tid % 16;
    if (kk >= a.n_pkeys) return;
    const int b = a.pkey_stream[kk];
    const int j = a.pkey_idx[kk];
    const uint4 vk = a.pkeys[(int64_t)kk * a.key16 + (lane < a.key16 ? lane : a.key16 - 1)];
    // keep the key's load above the branch (left alone, the compiler sinks it past the
    // test of j, where it would wait for j first)
    __asm__ volatile("" ::"v"(vk.x), "v"(vk.y), "v"(vk.z), "v"(vk.w));
    if (j < 0) return;
    const int page = page_of(a.v, b, j / kKeysPerPage);
    if (page < 0 || lane >= a.key16) return;
    ((uint4*)(cache_block(a.v, page) + a.off_pkey + (int64_t)(j % kKeysPerPage) * a.pkey_row_bytes))[lane] = vk;
  }
}

tf_status launch_latent_write(const tf_plan* p, const DevView& v, int32_t n_rows,
                              const int32_t* row_stream, const int32_t* row_pos, const void* latent,
                              const float* row_scale, const void* rope, int32_t n_pkeys,
                              const int32_t* pkey_stream, const int32_t* pkey_idx, const void* pkeys,
                              hipStream_t st, bool quantize) {
  WriteArgs a;
  a.quantize = quantize ? 1 : 0;
  a.v = v;
  a.n_rows = n_rows;
  a.n_pkeys = n_pkeys;
  a.row_stream = row_stream;
  a.row_pos = row_pos;
  a.latent = (const uint4*)latent;
  a.scale = p->g.lat_fmt == TF_LAT_FP8E4M3_ROWSCALE && !quantize ? row_scale : nullptr;
  a.rope = (const uint4*)rope;
  a.pkey_stream = pkey_stream;
  a.pkey_idx = pkey_idx;
  a.pkeys = (const uint4*)pkeys;
  a.lat16 = (int32_t)(p->lat_row_bytes / 16);
  a.rope16 = (int32_t)(p->rope_row_bytes / 16);
  a.key16 = (int32_t)(p->pkey_row_bytes / 16);
  a.off_scale = p->off_scale;
  a.off_rope = p->off_rope;
  a.off_pkey = p->off_pkey;
  a.lat_row_bytes = (int32_t)p->lat_row_bytes;
  a.rope_row_bytes = (int32_t)p->rope_row_bytes;
  a.pkey_row_bytes = (int32_t)p->pkey_row_bytes;
  if (a.lat16 > 64 || a.rope16 > 64 || a.key16 > 16)
    return set_error(TF_E_UNSUPPORTED, "%s: rows wider than one vector a lane", quantize ? "tf_latent_write_quantize"
                                                                                         : "tf_latent_write");
  a.row_blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int key_blocks = (n_pkeys + kKeysPerBlock - 1) / kKeysPerBlock;
  hipLaunchKernelGGL(latent_write_kernel, dim3(a.row_blocks + key_blocks), dim3(256), 0, st, a);
  return launch_status(quantize ? "tf_latent_write_quantize" : "tf_latent_write");
}

// ---- snapshot -----------------------------------------------------------------------

struct SnapArgs {
  DevView src, dst;   // cache_off = 0: every cache of a page is copied
  const int32_t* src_stream;
  const int32_t* dst_stream;
  int64_t at;
  int32_t n_caches;
  int64_t cache_block_bytes;
  int64_t off_scale, off_rope, off_pkey;
  int32_t lat_row_bytes, rope_row_bytes, pkey_row_bytes;
  int32_t has_scale;
};

constexpr int kSnapUnitsPerBlock = 4096;  // 64 KiB of 16-byte units per block
constexpr int kSnapUnitsPerThread = kSnapUnitsPerBlock / 256;

// grid: x = chunk of a page's bytes, y = page index * n_caches + cache, z = stream pair.
// A thread copies units u0 + tid + 256 j, issuing all its loads before its first store
// (256 bytes in flight a thread instead of one load at a time). A unit past the chunk's
// range is taken as the chunk's first unit, whose bytes it copies again to the same
// place, so every load and store is unconditional. Loads and stores are non-temporal:
// a snapshot reads and writes each byte once, and streaming it past the caches leaves
// the Infinity Cache's other lines (and their write-backs) alone: with that cache full
// of dirty lines the copy ran 76 us against 104 us with cached accesses.
__global__ __launch_bounds__(256) void snapshot_kernel(SnapArgs a) {
  const int pidx = blockIdx.y / a.n_caches;
  const int c = blockIdx.y % a.n_caches;
  const int bs = a.src_stream[blockIdx.z];
  const int bd = a.dst_stream[blockIdx.z];
  const int ps = page_of(a.src, bs, pidx);
  const int pd = page_of(a.dst, bd, pidx);
  if (ps < 0 || pd < 0) return;
  const int64_t row0 = (int64_t)pidx * kPageRows;
  int64_t nr = a.at - row0;
  if (nr > kPageRows) nr = kPageRows;
  const int64_t nk = nr / kPoolRatio;
  // four contiguous ranges of the cache block, in 16-byte units
  const int64_t u_lat = nr * a.lat_row_bytes / 16;
  const int64_t u_sc = a.has_scale ? nr * 4 / 16 : 0;
  const int64_t u_rope = nr * a.rope_row_bytes / 16;
  const int64_t u_key = nk * a.pkey_row_bytes / 16;
  const int64_t total = u_lat + u_sc + u_rope + u_key;
  const int64_t u0 = (int64_t)blockIdx.x * kSnapUnitsPerBlock;
  if (u0 >= total) return;
  const char* s = cache_block(a.src, ps) + (int64_t)c * a.cache_block_bytes;
  char* d = cache_block(a.dst, pd) + (int64_t)c * a.cache_block_bytes;
  const int64_t u1 = u0 + kSnapUnitsPerBlock < total ? u0 + kSnapUnitsPerBlock : total;
  auto offset = [&](int j) {
    int64_t u = u0 + threadIdx.x + 256 * j;
    u = u < u1 ? u : u0;
    int64_t o = a.off_pkey + (u - u_lat - u_sc - u_rope) * 16;
    o = u < u_lat + u_sc + u_rope ? a.off_rope + (u - u_lat - u_sc) * 16 : o;
    o = u < u_lat + u_sc ? a.off_scale + (u - u_lat) * 16 : o;
    return u < u_lat ? u * 16 : o;
  };
  u32x4 v[kSnapUnitsPerThread];
#pragma unroll
  for (int j = 0; j < kSnapUnitsPerThread; ++j) v[j] = __builtin_nontemporal_load((const u32x4*)(s + offset(j)));
#pragma unroll
  for (int j = 0; j < kSnapUnitsPerThread; ++j) __builtin_nontemporal_store(v[j], (u32x4*)(d + offset(j)));
}

tf_status launch_snapshot(const tf_plan* p, const tf_kv_view& src, const tf_kv_view& dst,
                          int32_t n_streams, const int32_t* src_stream, const int32_t* dst_stream,
                          int64_t at, hipStream_t st) {
  SnapArgs a;
  a.src = make_view(p, src);
  a.dst = make_view(p, dst);
  a.src.cache_off = 0;
  a.dst.cache_off = 0;
  a.src_stream = src_stream;
  a.dst_stream = dst_stream;
  a.at = at;
  a.n_caches = p->g.n_caches;
  a.cache_block_bytes = p->cache_block_bytes;
  a.off_scale = p->off_scale;
  a.off_rope = p->off_rope;
  a.off_pkey = p->off_pkey;
  a.lat_row_bytes = (int32_t)p->lat_row_bytes;
  a.rope_row_bytes = (int32_t)p->rope_row_bytes;
  a.pkey_row_bytes = (int32_t)p->pkey_row_bytes;
  a.has_scale = p->g.lat_fmt == TF_LAT_FP8E4M3_ROWSCALE;
  const int64_t pages = (at + kPageRows - 1) / kPageRows;
  const int64_t max_units = p->cache_block_bytes / 16;
  const int64_t chunks = (max_units + kSnapUnitsPerBlock - 1) / kSnapUnitsPerBlock;
  if (pages * p->g.n_caches > 65535 || n_streams > 65535)
    return set_error(TF_E_RANGE, "tf_snapshot_copy: too many pages or streams for one launch");
  hipLaunchKernelGGL(snapshot_kernel, dim3((unsigned)chunks, (unsigned)(pages * p->g.n_caches), n_streams),
                     dim3(256), 0, st, a);
  return launch_status("tf_snapshot_copy");
}

}  // namespace tf
