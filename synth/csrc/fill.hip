// Device version of the seeded generator in synth/splitmix.py.
//
// Fills a bf16 buffer with table[u(start + i) >> 48], where u is the same
// counter-based SplitMix64 stream as the host versions, so the bits agree
// with numpy by construction.  Input generation only: nothing here belongs to
// the method under test, and the product library does not link it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t mix64_host(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// Each thread writes 8 consecutive values (one 16-byte store) per iteration.
__global__ void __launch_bounds__(256)
fill_normal_bf16(uint64_t s0, uint64_t start, int64_t count,
                 const uint16_t* __restrict__ table, uint16_t* __restrict__ out) {
  const int64_t n_vec = count / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n_vec; v += stride) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint64_t i0 = (uint64_t)(v * 8 + 2 * j);
      uint16_t a = table[mix64(s0 + (start + i0 + 1) * GOLDEN) >> 48];
      uint16_t b = table[mix64(s0 + (start + i0 + 2) * GOLDEN) >> 48];
      w[j] = (uint32_t)a | ((uint32_t)b << 16);
    }
    uint4 pk = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(out + v * 8) = pk;
  }
  // tail (count % 8 values), handled by the first threads of block 0
  const int64_t tail0 = n_vec * 8;
  if (blockIdx.x == 0 && (int64_t)threadIdx.x < count - tail0) {
    uint64_t i = (uint64_t)(tail0 + threadIdx.x);
    out[i] = table[mix64(s0 + (start + i + 1) * GOLDEN) >> 48];
  }
}

extern "C" int synth_fill_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t layer,
                                      uint64_t start, int64_t count,
                                      const uint16_t* table_dev, uint16_t* out_dev,
                                      hipStream_t stream) {
  if (count < 0 || table_dev == nullptr || (count > 0 && out_dev == nullptr)) return -1;
  if ((reinterpret_cast<uintptr_t>(out_dev) & 15) != 0) return -1;
  if (count == 0) return 0;
  const uint64_t s0 = mix64_host((seed << 32) ^ (tensor_id << 16) ^ layer);
  int64_t n_vec = count / 8;
  int64_t blocks = (n_vec + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_normal_bf16, dim3((unsigned)blocks), dim3(256), 0, stream,
                     s0, start, count, table_dev, out_dev);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
