// GPU twin of the seeded input generator in synth/__init__.py (same
// definition: SplitMix64 outputs, Box-Muller in fp64, one rounding from fp64
// to bfloat16).  Input generation only: none of the attention arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ inline uint16_t f64_to_bf16(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;
  u &= ~0x00001FFFFFFFFFFFull;
  const float f = (float)__longlong_as_double((long long)u);
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// out[r * ld + d] = bf16(std * N(0,1) drawn at index (base + r) * width + d)
__global__ void fill_normal(uint16_t* out, int64_t rows, int64_t width, int64_t ld, uint64_t key,
                            uint64_t base, double stdv) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * width) return;
  const int64_t r = idx / width, d = idx - r * width;
  const uint64_t n = (base + (uint64_t)r) * (uint64_t)width + (uint64_t)d;
  const uint64_t u = mix64(key + (n + 1) * kGamma);
  const double u1 = ((double)(u >> 32) + 0.5) * 2.3283064365386963e-10;   // 2^-32
  const double u2 = (double)(u & 0xFFFFFFFFull) * 2.3283064365386963e-10;
  const double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
  out[r * ld + d] = f64_to_bf16(z * stdv);
}

}  // namespace

extern "C" {

uint64_t synth_stream_key(uint64_t seed, uint64_t tensor, uint64_t layer) {
  const uint64_t k0 = mix64((seed + 1) * kGamma);
  const uint64_t k1 = mix64(k0 ^ ((tensor + 1) * kGamma));
  return mix64(k1 ^ ((layer + 1) * kGamma));
}

// Fills a rows x width block (row stride ld elements) of bf16 normals.
// Returns 0 on success, the hipError_t of the launch otherwise.
int synth_fill_normal_bf16(void* out, int64_t rows, int64_t width, int64_t ld, uint64_t seed,
                           uint64_t tensor, uint64_t layer, uint64_t base_row, double stdv,
                           void* stream) {
  if (rows <= 0 || width <= 0) return 0;
  const uint64_t key = synth_stream_key(seed, tensor, layer);
  const int64_t total = rows * width;
  hipLaunchKernelGGL(fill_normal, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, (uint16_t*)out, rows, width, ld, key, base_row, stdv);
  return (int)hipGetLastError();
}

}  // extern "C"
