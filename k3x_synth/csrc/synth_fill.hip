// Device-side twin of the seeded expert-byte generator in k3x_synth/__init__.py.
//
// Both sides implement, from its published definition, the SplitMix64 output function
// (Steele, Lea and Flood, OOPSLA 2014): word i of a stream keyed by k is
// fmix64(k + i * GAMMA), where fmix64 first adds GAMMA and then applies the two
// xor-shift-multiply rounds.  Packed-nibble tensors take byte b from byte (b % 8) of word
// b / 8 (little-endian); scale tensors take scale s from the 32-bit half (s % 2) of word
// s / 2 and map it to lo + floor(u32 * count / 2^32).
//
// This file holds no arithmetic of the routed-expert method: it only fills input buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kM1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kM2 = 0x94D049BB133111EBull;

__host__ __device__ inline uint64_t fmix64(uint64_t z) {
  z += kGamma;
  z = (z ^ (z >> 30)) * kM1;
  z = (z ^ (z >> 27)) * kM2;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t tensor_key(uint64_t seed, uint32_t layer, uint32_t expert,
                                               uint32_t tensor) {
  const uint64_t h = fmix64(seed);
  const uint64_t tag = ((uint64_t)layer << 40) | ((uint64_t)expert << 8) | (uint64_t)tensor;
  return fmix64(h ^ tag);
}

// One thread writes 16 bytes (two words) of packed nibbles.  per_expert is a multiple of 16.
__global__ void fill_packed(uint8_t* __restrict__ dst, uint64_t per_expert, uint32_t e0,
                            uint32_t n_experts, uint64_t seed, uint32_t layer, uint32_t tensor) {
  const uint64_t chunks_per_expert = per_expert / 16;
  const uint64_t total = chunks_per_expert * n_experts;
  for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t e = c / chunks_per_expert;
    const uint64_t w = 2 * (c - e * chunks_per_expert);  // first word index within the expert
    const uint64_t key = tensor_key(seed, layer, e0 + (uint32_t)e, tensor);
    uint4 v;
    const uint64_t a = fmix64(key + w * kGamma);
    const uint64_t b = fmix64(key + (w + 1) * kGamma);
    v.x = (uint32_t)a;
    v.y = (uint32_t)(a >> 32);
    v.z = (uint32_t)b;
    v.w = (uint32_t)(b >> 32);
    reinterpret_cast<uint4*>(dst)[c] = v;
  }
}

// One thread writes 4 scale bytes (two words).  per_expert is a multiple of 4.
__global__ void fill_scale(uint8_t* __restrict__ dst, uint64_t per_expert, uint32_t e0,
                           uint32_t n_experts, uint64_t seed, uint32_t layer, uint32_t tensor,
                           uint32_t lo, uint32_t count) {
  const uint64_t chunks_per_expert = per_expert / 4;
  const uint64_t total = chunks_per_expert * n_experts;
  for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t e = c / chunks_per_expert;
    const uint64_t w = 2 * (c - e * chunks_per_expert);
    const uint64_t key = tensor_key(seed, layer, e0 + (uint32_t)e, tensor);
    const uint64_t a = fmix64(key + w * kGamma);
    const uint64_t b = fmix64(key + (w + 1) * kGamma);
    const uint32_t h[4] = {(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
    uint32_t out = 0;
    for (int i = 0; i < 4; ++i) {
      const uint32_t s = lo + (uint32_t)(((uint64_t)h[i] * count) >> 32);
      out |= (s & 0xFFu) << (8 * i);
    }
    reinterpret_cast<uint32_t*>(dst)[c] = out;
  }
}

}  // namespace

extern "C" {

// Fills dst = [n_experts][per_expert bytes] with the stream bytes of experts e0..e0+n-1.
// kind 0: packed nibbles (per_expert % 16 == 0); kind 1: scale bytes in lo..lo+count-1
// (per_expert % 4 == 0).  Returns 0 on success, -1 on bad arguments, -4 on a HIP error.
int k3x_synth_fill(void* dst, uint64_t per_expert, uint32_t e0, uint32_t n_experts,
                   uint64_t seed, uint32_t layer, uint32_t tensor, int kind, uint32_t lo,
                   uint32_t count, void* stream) {
  if (!dst || n_experts == 0 || per_expert == 0) return -1;
  if (((uintptr_t)dst & 15) != 0) return -1;
  const hipStream_t s = (hipStream_t)stream;
  const int block = 256;
  if (kind == 0) {
    if (per_expert % 16) return -1;
    const uint64_t total = per_expert / 16 * n_experts;
    uint64_t grid = (total + block - 1) / block;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(fill_packed, dim3((unsigned)grid), dim3(block), 0, s, (uint8_t*)dst,
                       per_expert, e0, n_experts, seed, layer, tensor);
  } else if (kind == 1) {
    if (per_expert % 4 || count == 0 || lo + count > 256) return -1;
    const uint64_t total = per_expert / 4 * n_experts;
    uint64_t grid = (total + block - 1) / block;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(fill_scale, dim3((unsigned)grid), dim3(block), 0, s, (uint8_t*)dst,
                       per_expert, e0, n_experts, seed, layer, tensor, lo, count);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
