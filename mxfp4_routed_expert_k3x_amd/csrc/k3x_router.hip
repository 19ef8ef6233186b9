// Sigmoid + correction-bias top-k router (kimi-k3-in-c README, Part II section 9 "Picking 16
// experts of 896"): logits as double dot products, the unbiased sigmoid score, the bias added
// for selection only, repeated argmax with ties to the lower expert, gates from the unbiased
// scores renormalised by their float sum and scaled by routed_scale.
//
// Kernel 1 (route_scores): one wave per (expert, token block).  The expert's weight row
// stays in registers while the wave walks its tokens.  Lane L owns the 8-element chunks
// whose index is L mod 64 and sums their exact bf16*bf16 products in double, in ascending
// order; the 64 lane partials are then folded p[L] += p[L + s] for s = 32 .. 1 with
// down-shuffles.  The float logit goes through a double sigmoid rounded once to float.
// This fixes the summation order completely, so the scores are reproducible bit for bit.
//
// Kernel 2 (route_select): one wave per token.  The selection scores c = s + bias live in
// LDS; each of the topk rounds takes every lane's best untaken expert and reduces them with
// a butterfly under the total order (larger c first, then lower index), so ties go to the
// lower expert and -0 equals +0 as in an IEEE compare.
#include "k3x_internal.h"

namespace k3x {
namespace {

constexpr int kRouteTokBlock = 32;  // tokens per wave in route_scores

// NC = 8-element chunks each lane keeps in registers: hidden <= 64 * 8 * NC
template <int NC>
__global__ __launch_bounds__(256) void route_scores(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ W, int32_t T,
                                                    int32_t H, int32_t E,
                                                    float* __restrict__ scores) {
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (e >= E) return;
  const int chunks = H / 8;
  const int t0 = blockIdx.y * kRouteTokBlock;
  const int t1 = min(T, t0 + kRouteTokBlock);

  // this lane's chunks of the weight row, widened to double once
  uint4 wv[NC];
  int nmine = 0;
  const uint4* wrow = reinterpret_cast<const uint4*>(W + (size_t)e * H);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    if (c < chunks) {
      wv[i] = wrow[c];
      nmine = i + 1;
    }
  }

  for (int t = t0; t < t1; ++t) {
    const uint4* xrow = reinterpret_cast<const uint4*>(x + (size_t)t * H);
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (i < nmine) {
        const uint4 xv = xrow[lane + kWave * i];
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
        const uint32_t ws[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double xl = (double)bf16_bits_to_f32(xs[j] & 0xFFFFu);
          const double wl = (double)bf16_bits_to_f32(ws[j] & 0xFFFFu);
          acc = acc + xl * wl;  // the product is exact in double
          const double xh = (double)bf16_bits_to_f32(xs[j] >> 16);
          const double wh = (double)bf16_bits_to_f32(ws[j] >> 16);
          acc = acc + xh * wh;
        }
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) acc = acc + __shfl_down(acc, s, kWave);
    if (lane == 0) {
      const float l = (float)acc;
      scores[(size_t)t * E + e] = (float)(1.0 / (1.0 + exp(-(double)l)));
    }
  }
}

// (c, index) total order: true when candidate b beats a.  Index -1 means "no candidate".
__device__ __forceinline__ bool beats(float cb, int ib, float ca, int ia) {
  if (ib < 0) return false;
  if (ia < 0) return true;
  return cb > ca || (cb == ca && ib < ia);
}

__global__ __launch_bounds__(64) void route_select(const float* __restrict__ scores,
                                                   const float* __restrict__ bias, int32_t E,
                                                   int32_t topk, int32_t renorm, float rscale,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ gates_out) {
  extern __shared__ float lds[];
  float* c = lds;       // [E] selection scores
  float* sel = lds + E; // [topk] chosen unbiased scores, selection order
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* s_t = scores + (size_t)t * E;
  for (int e = lane; e < E; e += kWave) c[e] = s_t[e] + (bias ? bias[e] : 0.0f);
  __syncthreads();

  uint64_t taken = 0;  // bit m: expert lane + 64 m already chosen
  const int per_lane = (E + kWave - 1) / kWave;
  for (int j = 0; j < topk; ++j) {
    float bc = 0.0f;
    int bi = -1;
    for (int m = 0; m < per_lane; ++m) {
      const int e = lane + kWave * m;
      if (e < E && !((taken >> m) & 1ull)) {
        const float v = c[e];
        if (beats(v, e, bc, bi)) {
          bc = v;
          bi = e;
        }
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float oc = __shfl_xor(bc, s, kWave);
      const int oi = __shfl_xor(bi, s, kWave);
      if (beats(oc, oi, bc, bi)) {
        bc = oc;
        bi = oi;
      }
    }
    // every lane now holds the same winner
    if ((bi % kWave) == lane) taken |= 1ull << (bi / kWave);
    if (lane == 0) {
      idx_out[(size_t)t * topk + j] = bi;
      sel[j] = s_t[bi];
    }
  }
  __syncthreads();
  if (lane == 0) {
    float sum = 0.0f;
    if (renorm)
      for (int j = 0; j < topk; ++j) sum = sum + sel[j];
    sel[topk] = sum;  // slot reserved past the chosen scores
  }
  __syncthreads();
  const float sum = sel[topk];
  for (int j = lane; j < topk; j += kWave) {
    float w = sel[j];
    if (renorm && sum > 0.0f) w = w / sum;
    gates_out[(size_t)t * topk + j] = w * rscale;
  }
}

}  // namespace

hipError_t launch_route(const k3x_router_desc& r, const uint16_t* x, int32_t T, int32_t* idx,
                        float* gates, float* scores, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int E = r.n_experts, H = r.hidden;
  dim3 g1((E + 3) / 4, (T + kRouteTokBlock - 1) / kRouteTokBlock);
  const uint16_t* W = static_cast<const uint16_t*>(r.weight);
  {
    LaunchTimer lt("route_scores", s);
    if (H <= 64 * 8 * 8)
      hipLaunchKernelGGL(route_scores<8>, g1, dim3(256), 0, s, x, W, T, H, E, scores);
    else
      hipLaunchKernelGGL(route_scores<32>, g1, dim3(256), 0, s, x, W, T, H, E, scores);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = sizeof(float) * ((size_t)E + (size_t)r.topk + 1);
  {
    LaunchTimer lt("route_select", s);
    hipLaunchKernelGGL(route_select, dim3(T), dim3(64), lds, s, scores, r.bias, E, r.topk,
                       r.renorm, r.routed_scale, idx, gates);
  }
  return hipGetLastError();
}

}  // namespace k3x
