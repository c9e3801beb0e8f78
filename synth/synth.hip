// Device twin of the seeded input generator in synth/__init__.py: the same
// SplitMix64 output function, the same Irwin-Hall(4) integer, the same single
// float32 multiply and round-to-nearest-even to bf16, the same integer e4m3
// encoding. No step of the attention method lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ int32_t normal_int(uint64_t key, uint64_t idx) {
  const uint64_t h = mix(key + (idx + 1) * kGamma);
  const uint32_t s = (uint32_t)(h & 0xFFFF) + (uint32_t)((h >> 16) & 0xFFFF) + (uint32_t)((h >> 32) & 0xFFFF) +
                     (uint32_t)(h >> 48);
  return (int32_t)s - 131070;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ int64_t rne_shift(int64_t a, int k) {
  if (k <= 0) return a;
  const int64_t q = a >> k, r = a - (q << k), half = 1LL << (k - 1);
  return q + ((r > half || (r == half && (q & 1))) ? 1 : 0);
}

__device__ __forceinline__ uint8_t e4m3_from_int(int32_t s) {
  const uint32_t sign = s < 0 ? 1u : 0u;
  int64_t a = s < 0 ? -(int64_t)s : s;
  if (a == 0) return (uint8_t)(sign << 7);
  int nb = 0;
  while (nb < 62 && (1LL << nb) <= a) ++nb;  // bit length
  int e = nb - 12;
  uint32_t code;
  if (e < -6) {
    code = (uint32_t)rne_shift(a, 2);
  } else {
    int64_t m4 = nb >= 4 ? rne_shift(a, nb - 4) : (a << (4 - nb));
    if (m4 >= 16) {
      e += 1;
      m4 = 8;
    }
    code = (uint32_t)(((e + 7) << 3) | (int)(m4 - 8));
  }
  return (uint8_t)((sign << 7) | code);
}

// element i of an [n_rows][cols] output takes generator index base + row * stride + col
__device__ __forceinline__ uint64_t gidx(uint64_t i, uint64_t cols, uint64_t base, uint64_t stride) {
  return base + (i / cols) * stride + (i % cols);
}

__global__ void fill_bf16(uint16_t* out, uint64_t n, uint64_t cols, uint64_t key, uint64_t base, uint64_t stride,
                          float c) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = bf16_bits((float)normal_int(key, gidx(i, cols, base, stride)) * c);
}

__global__ void fill_f32(float* out, uint64_t n, uint64_t cols, uint64_t key, uint64_t base, uint64_t stride,
                         float c) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = (float)normal_int(key, gidx(i, cols, base, stride)) * c;
}

__global__ void fill_e4m3(uint8_t* out, uint64_t n, uint64_t cols, uint64_t key, uint64_t base, uint64_t stride) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = e4m3_from_int(normal_int(key, gidx(i, cols, base, stride)));
}

__global__ void fill_scale8(float* out, uint64_t n, uint64_t key, uint64_t base, uint64_t stride, float c) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t h = mix(key + (base + i * stride + 1) * kGamma);
    const float u = (float)(uint32_t)(h >> 41) * 0x1p-23f;
    out[i] = (0.5f + u) * c;
  }
}

unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  return (unsigned)(g > 65536 ? 65536 : (g ? g : 1));
}

}  // namespace

extern "C" int tf_synth_bf16(void* out, uint64_t n_rows, uint64_t cols, uint64_t key, uint64_t base,
                             uint64_t stride, float c, void* stream) {
  const uint64_t n = n_rows * cols;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, (uint16_t*)out, n, cols, key,
                     base, stride, c);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int tf_synth_f32(void* out, uint64_t n_rows, uint64_t cols, uint64_t key, uint64_t base,
                            uint64_t stride, float c, void* stream) {
  const uint64_t n = n_rows * cols;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, (float*)out, n, cols, key,
                     base, stride, c);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int tf_synth_e4m3(void* out, uint64_t n_rows, uint64_t cols, uint64_t key, uint64_t base,
                             uint64_t stride, void* stream) {
  const uint64_t n = n_rows * cols;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_e4m3, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)out, n, cols, key,
                     base, stride);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int tf_synth_scale8(void* out, uint64_t n, uint64_t key, uint64_t base, uint64_t stride, float c,
                               void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_scale8, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, (float*)out, n, key, base,
                     stride, c);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
