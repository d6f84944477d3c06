// Streaming-read ceiling of the device, a measurement aid (mla_read_probe in
// include/mla.h): the HBM read rate that a plain streaming kernel reaches,
// against which the decode kernels' rates can be read.  Nothing on the
// decode or prefill path uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"   // include/mla.h (on the include path)

namespace {

constexpr int kGrid = 2048;   // workgroups of 256 threads, 4 waves each
constexpr int kDepth = 8;     // 1 KiB direct loads in flight per wave
static_assert(MLA_READ_PROBE_SINK_INTS == 4 * kGrid, "one sink int per wave");

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((address_space(3))) const i32x4 lds_i32x4_t;

// Workgroup x reads the 16-byte words [x n / G, (x + 1) n / G) of the buffer
// in 1 KiB pieces (64 words, one per lane); wave w takes pieces w, w + 4, ...
// with direct global->LDS loads (the way the decode kernels stream the cache),
// kDepth pieces in flight in its own LDS ring.  Once a piece has landed, each
// lane reads its own 16 bytes back and XORs them into a digest; each wave
// stores its digest to sink[4 x + w], so the XOR of all digests is the XOR
// of the buffer.
__global__ void __launch_bounds__(256) read_probe(const uint8_t* __restrict__ buf, size_t n16, int* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4][kDepth][1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t lo = n16 * blockIdx.x / kGrid, hi = n16 * (blockIdx.x + 1) / kGrid;
  const size_t pieces = (hi - lo + 63) / 64;
  const size_t mine = pieces > (size_t)wave ? (pieces - wave + 3) / 4 : 0;   // pieces w, w + 4, ... below `pieces`
  int acc = 0;
  auto word = [&](size_t k) { return lo + 64 * (wave + 4 * k) + lane; };
  auto digest = [&](size_t k) {
    if (word(k) < hi) {
      const i32x4 v = *(lds_i32x4_t*)((__attribute__((address_space(3))) uint8_t*)ring[wave][k % kDepth] + lane * 16);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  };
  for (size_t k = 0; k < mine; ++k) {
    if (word(k) < hi)
      __builtin_amdgcn_global_load_lds((const void*)(buf + 16 * word(k)),
                                       (__attribute__((address_space(3))) void*)ring[wave][k % kDepth], 16, 0, 0);
    if (k + 1 >= kDepth) {
      // piece k - kDepth + 1 has landed once at most kDepth - 1 loads are outstanding
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDepth - 1) : "memory");
      digest(k + 1 - kDepth);
      // its read is complete before the next load may overwrite the ring position
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (size_t k = mine > kDepth - 1 ? mine - (kDepth - 1) : 0; k < mine; ++k) digest(k);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) sink[blockIdx.x * 4 + wave] = acc;
}

}  // namespace

extern "C" mla_status mla_read_probe(const void* buf, size_t bytes, int32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return MLA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return MLA_ERR_RANGE;
  if (((uintptr_t)buf & 15u) != 0 || ((uintptr_t)sink & 3u) != 0) return MLA_ERR_ALIGN;
  hipLaunchKernelGGL(read_probe, dim3(kGrid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)buf, bytes / 16,
                     (int*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_DEVICE;
}
