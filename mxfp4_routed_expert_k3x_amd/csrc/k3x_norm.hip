// Hidden-state helpers for chaining MoE layers (kimi-k3-in-c README, Part II section 5
// "Kernels with a floating point contract"): RMSNorm with the sum of squares in double, eps
// inside the square root, unit weight; and the bf16 residual update.
//
// rmsnorm: one wave per token.  Lane L owns the 8-element chunks whose index is L mod 64 and
// sums their squares (exact in double) in ascending order; partials fold p[L] += p[L + s]
// for s = 32 .. 1, so the sum is reproducible bit for bit.
#include "k3x_internal.h"

namespace k3x {
namespace {

// x and out may be the same buffer: each lane rewrites only chunks it has finished reading.
__global__ __launch_bounds__(256) void rmsnorm_bf16(const uint16_t* x, int32_t T, int32_t H,
                                                    float eps, uint16_t* out) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  const int chunks = H / 8;
  double ss = 0.0;
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = (double)bf16_bits_to_f32(w[j] & 0xFFFFu);
      const double hi = (double)bf16_bits_to_f32(w[j] >> 16);
      ss = ss + lo * lo;
      ss = ss + hi * hi;
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) ss = ss + __shfl_down(ss, s, kWave);
  ss = __shfl(ss, 0, kWave);
  const float inv = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
  uint4* orow = reinterpret_cast<uint4*>(out + (size_t)t * H);
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_bits_to_f32(w[j] & 0xFFFFu) * inv;
      const float hi = bf16_bits_to_f32(w[j] >> 16) * inv;
      o[j] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    }
    orow[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void residual_add_bf16(uint16_t* __restrict__ x,
                                                         const float* __restrict__ y,
                                                         int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  uint4 v = reinterpret_cast<uint4*>(x)[i];
  const float4 y0 = reinterpret_cast<const float4*>(y)[2 * i];
  const float4 y1 = reinterpret_cast<const float4*>(y)[2 * i + 1];
  const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = bf16_bits_to_f32(w[j] & 0xFFFFu) + ys[2 * j];
    const float hi = bf16_bits_to_f32(w[j] >> 16) + ys[2 * j + 1];
    w[j] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
  }
  reinterpret_cast<uint4*>(x)[i] = make_uint4(w[0], w[1], w[2], w[3]);
}

// Residual update of one layer fused with the RMSNorm that starts the next: x_out[t] <-
// bf16(x[t] + y[t]) and out[t] <- rmsnorm(x_out[t]), one wave per token.  The updated chunks
// stay in registers (NC per lane) for the norm; the squares are summed in the same order as
// rmsnorm_bf16, so both outputs equal those of the two separate launches bit for bit.  x_out
// may be x (each lane rewrites only the chunks it has read).
template <int NC>
__global__ __launch_bounds__(256) void residual_rmsnorm_bf16(const uint16_t* x,
                                                             const float* __restrict__ y,
                                                             int32_t T, int32_t H, float eps,
                                                             uint16_t* x_out,
                                                             uint16_t* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  uint4* xw = reinterpret_cast<uint4*>(x_out + (size_t)t * H);
  const float4* yr = reinterpret_cast<const float4*>(y + (size_t)t * H);
  const int chunks = H / 8;
  uint4 nv[NC];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    if (c < chunks) {
      const uint4 v = xr[c];
      const float4 y0 = yr[2 * c], y1 = yr[2 * c + 1];
      const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = f32_to_bf16_bits(bf16_bits_to_f32(w[j] & 0xFFFFu) + ys[2 * j]);
        const uint32_t hi = f32_to_bf16_bits(bf16_bits_to_f32(w[j] >> 16) + ys[2 * j + 1]);
        o[j] = lo | (hi << 16);
        const double dl = (double)bf16_bits_to_f32(lo);
        const double dh = (double)bf16_bits_to_f32(hi);
        ss = ss + dl * dl;
        ss = ss + dh * dh;
      }
      nv[i] = make_uint4(o[0], o[1], o[2], o[3]);
      xw[c] = nv[i];
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) ss = ss + __shfl_down(ss, s, kWave);
  ss = __shfl(ss, 0, kWave);
  const float inv = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
  uint4* orow = reinterpret_cast<uint4*>(out + (size_t)t * H);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    if (c < chunks) {
      const uint32_t w[4] = {nv[i].x, nv[i].y, nv[i].z, nv[i].w};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = bf16_bits_to_f32(w[j] & 0xFFFFu) * inv;
        const float hi = bf16_bits_to_f32(w[j] >> 16) * inv;
        o[j] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
      }
      orow[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

}  // namespace

hipError_t launch_residual_rmsnorm(const uint16_t* x, const float* y, int32_t T, int32_t H,
                                   float eps, uint16_t* x_out, uint16_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (H <= 64 * 8 * 8)
    return launch("residual_rmsnorm_bf16", residual_rmsnorm_bf16<8>, dim3((T + 3) / 4),
                  dim3(256), 0, s, x, y, T, H, eps, x_out, out);
  return launch("residual_rmsnorm_bf16", residual_rmsnorm_bf16<32>, dim3((T + 3) / 4), dim3(256),
                0, s, x, y, T, H, eps, x_out, out);
}

hipError_t launch_rmsnorm(const uint16_t* x, int32_t T, int32_t H, float eps, uint16_t* out,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  return launch("rmsnorm_bf16", rmsnorm_bf16, dim3((T + 3) / 4), dim3(256), 0, s, x, T, H, eps,
                out);
}

hipError_t launch_residual(uint16_t* x, const float* y, int32_t T, int32_t H, hipStream_t s) {
  const int64_t n8 = (int64_t)T * H / 8;
  if (n8 == 0) return hipSuccess;
  return launch("residual_add_bf16", residual_add_bf16, dim3((unsigned)((n8 + 255) / 256)),
                dim3(256), 0, s, x, y, n8);
}

}  // namespace k3x
