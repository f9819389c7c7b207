/* Host (CPU) version of the seeded generator in synth/splitmix.py.
 *
 * Same counter-based SplitMix64 stream and the same N(0,1) bf16 table (passed
 * in by the caller), so every value is bit-identical to the numpy version; this
 * one only exists because it is ~50x faster on many cores.  Input generation
 * only: nothing here belongs to the method under test.
 */
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_start(uint64_t seed, uint64_t tensor_id, uint64_t layer) {
  return mix64((seed << 32) ^ (tensor_id << 16) ^ layer);
}

/* out[i] = table[u(start + i) >> 48] for i < count */
void synth_normal_bf16_host(uint64_t seed, uint64_t tensor_id, uint64_t layer,
                            uint64_t start, int64_t count,
                            const uint16_t* table, uint16_t* out) {
  const uint64_t s0 = synth_stream_start(seed, tensor_id, layer);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint64_t u = mix64(s0 + (start + (uint64_t)i + 1) * GOLDEN);
    out[i] = table[u >> 48];
  }
}
