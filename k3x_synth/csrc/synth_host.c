/* Host twin of the seeded expert-byte generator (see k3x_synth/__init__.py): the SplitMix64
 * output function of Steele, Lea and Flood (OOPSLA 2014), word i of the stream keyed by k
 * being fmix64(k + i * GAMMA).  Byte and scale extraction as in the Python and HIP versions.
 * Generator code only: no arithmetic of the routed-expert method. */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t fmix64(uint64_t z) {
  z += GAMMA;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t tensor_key(uint64_t seed, uint32_t layer, uint32_t expert, uint32_t tensor) {
  const uint64_t h = fmix64(seed);
  return fmix64(h ^ (((uint64_t)layer << 40) | ((uint64_t)expert << 8) | (uint64_t)tensor));
}

/* kind 0: n packed bytes starting at byte b0; kind 1: n scale bytes starting at scale b0. */
void k3x_synth_host_fill(uint8_t *dst, uint64_t b0, uint64_t n, uint64_t seed, uint32_t layer,
                         uint32_t expert, uint32_t tensor, int kind, uint32_t lo, uint32_t count) {
  const uint64_t key = tensor_key(seed, layer, expert, tensor);
  if (kind == 0) {
    uint64_t i = 0;
    while (i < n) {
      const uint64_t b = b0 + i;
      const uint64_t w = fmix64(key + (b >> 3) * GAMMA);
      for (uint64_t j = b & 7; j < 8 && i < n; ++j, ++i) dst[i] = (uint8_t)(w >> (8 * j));
    }
  } else {
    uint64_t i = 0;
    while (i < n) {
      const uint64_t s = b0 + i;
      const uint64_t w = fmix64(key + (s >> 1) * GAMMA);
      for (uint64_t j = s & 1; j < 2 && i < n; ++j, ++i) {
        const uint64_t h = j ? (w >> 32) : (w & 0xFFFFFFFFull);
        dst[i] = (uint8_t)(lo + ((h * count) >> 32));
      }
    }
  }
}
