// Sigmoid + correction-bias top-k router (kimi-k3-in-c README, Part II section 9 "Picking 16
// experts of 896"): logits as double dot products, the unbiased sigmoid score, the bias added
// for selection only, repeated argmax with ties to the lower expert, gates from the unbiased
// scores renormalised by their float sum and scaled by routed_scale.
//
// Kernel 1 (route_scores): one wave per (expert, block of 4 tokens); for hidden sizes that are
// multiples of 512 a block of 4 tokens takes two experts per wave and a single token one.  The
// weight rows stay in registers while the wave sums the block's tokens side by side, each
// staged chunk widened once for both experts.  Lane L owns the
// 8-element chunks whose index is L mod 64 and sums their exact bf16*bf16 products in double,
// in ascending order; the 64 lane partials are then folded p[L] += p[L + s] for s = 32 .. 1
// with down-shuffles.  The float logit goes through a double sigmoid rounded once to float
// (for a block of tokens lane k then takes token k's, so the block's sigmoids run side by side).
// This fixes the summation order completely, so the scores are reproducible bit for bit.
// For widths that are multiples of 512 (up to 8192) the row is loaded whole and at once (a
// fixed number of 16-byte chunks per lane) and the block's tokens are staged in LDS while the
// row is in flight; other widths take a guarded loop that reads the tokens from memory.
// A single-token variant (route_scores_residual) first forms the token itself: the previous
// layer's residual update and this layer's RMSNorm, in the order of the standalone kernels.
//
// Kernel 2 (route_select): one workgroup per token.  Up to 1024 experts and 16 picks the
// experts are ranked by sorting networks over (selection key, index) words
// (select_topk_bitonic, which the fused single-token decode also runs); beyond that a radix
// select (select_topk) finds the selection score of the topk-th expert under the total order
// (larger c first, then lower index) on order-preserving integer keys, so ties go to the lower
// expert and -0 equals +0 as in an IEEE compare, and puts the chosen experts in selection
// order by their rank.
#include "k3x_internal.h"
#include "k3x_select.h"

namespace k3x {
namespace {

constexpr int kRouteTokBlock = 4;  // tokens per wave in route_scores, summed side by side

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

  // the block's tokens are summed side by side (independent chains, each in the fixed order)
  double acc[kRouteTokBlock];
#pragma unroll
  for (int k = 0; k < kRouteTokBlock; ++k) acc[k] = 0.0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (i < nmine) {
      const uint32_t ws[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
      for (int k = 0; k < kRouteTokBlock; ++k) {
        if (t0 + k < t1) {
          const uint4 xv = reinterpret_cast<const uint4*>(x + (size_t)(t0 + k) * H)[lane + kWave * i];
          const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const double xl = (double)bf16_bits_to_f32(xs[j] & 0xFFFFu);
            const double wl = (double)bf16_bits_to_f32(ws[j] & 0xFFFFu);
            acc[k] = acc[k] + xl * wl;  // the product is exact in double
            const double xh = (double)bf16_bits_to_f32(xs[j] >> 16);
            const double wh = (double)bf16_bits_to_f32(ws[j] >> 16);
            acc[k] = acc[k] + xh * wh;
          }
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kRouteTokBlock; ++k) {
    if (t0 + k < t1) {
      double a = acc[k];
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) a = a + __shfl_down(a, s, kWave);
      if (lane == 0) {
        const float l = (float)a;
        scores[(size_t)(t0 + k) * E + e] = (float)(1.0 / (1.0 + exp(-(double)l)));
      }
    }
  }
}

// The same scores for H = 512 * NCH: the wave's weight rows (EPW experts) are requested first
// (NCH chunks per lane and row, no guards), the NT-token block is staged in LDS meanwhile, then
// summed in the order above; each staged chunk of a token is widened once and used for every
// one of the wave's experts.  Slots of tokens past T are zero-filled and their sums dropped.
template <int NCH, int NT, int EPW>
__global__ __launch_bounds__(256) void route_scores_staged(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ W,
                                                           int32_t T, int32_t H, int32_t E,
                                                           float* __restrict__ scores) {
  extern __shared__ uint4 xs[];  // [NT][H / 8]
  const int lane = threadIdx.x % kWave;
  const int e0 = (blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * EPW;
  const int t0 = blockIdx.y * NT;
  const int nt = min(NT, T - t0);
  const int cpr = NCH * kWave;
  uint4 wv[EPW][NCH];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < EPW; ++u) {
    const int e = e0 + u < E ? e0 + u : E - 1;
    const uint4* wrow = reinterpret_cast<const uint4*>(W + (size_t)e * H);
#pragma unroll
    for (int i = 0; i < NCH; ++i) wv[u][i] = wrow[lane + kWave * i];
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int i = threadIdx.x; i < NT * cpr; i += blockDim.x)
    xs[i] = i < nt * cpr ? reinterpret_cast<const uint4*>(x + (size_t)(t0 + i / cpr) * H)[i % cpr]
                         : make_uint4(0, 0, 0, 0);
  __syncthreads();
  if (e0 >= E) return;
  double acc[EPW][NT];
#pragma unroll
  for (int u = 0; u < EPW; ++u)
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[u][k] = 0.0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const uint4 xv = xs[k * cpr + lane + kWave * i];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      double xd[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xd[2 * j] = (double)bf16_bits_to_f32(xw[j] & 0xFFFFu);
        xd[2 * j + 1] = (double)bf16_bits_to_f32(xw[j] >> 16);
      }
#pragma unroll
      for (int u = 0; u < EPW; ++u) {
        const uint32_t ws[4] = {wv[u][i].x, wv[u][i].y, wv[u][i].z, wv[u][i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[u][k] = acc[u][k] + xd[2 * j] * (double)bf16_bits_to_f32(ws[j] & 0xFFFFu);
          acc[u][k] = acc[u][k] + xd[2 * j + 1] * (double)bf16_bits_to_f32(ws[j] >> 16);
        }
      }
    }
    if (NT > 1) {  // one chunk's tokens live at a time
#pragma unroll
      for (int u = 0; u < EPW; ++u)
#pragma unroll
        for (int k = 0; k < NT; ++k) asm volatile("" : "+v"(acc[u][k]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // each token's sum ends in lane 0; lane k then takes token k's, so the block's sigmoids run
  // side by side instead of one after another in lane 0
#pragma unroll
  for (int u = 0; u < EPW; ++u) {
    double mine = 0.0;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      double a = acc[u][k];
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) a = a + __shfl_down(a, s, kWave);
      const uint64_t bits = __builtin_bit_cast(uint64_t, a);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, 0);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), 0);
      if (lane == k) mine = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    }
    if (lane < nt && e0 + u < E) {
      const float l = (float)mine;
      scores[(size_t)(t0 + lane) * E + e0 + u] = (float)(1.0 / (1.0 + exp(-(double)l)));
    }
  }
}

// Single-token scores with the hidden-state update and the RMSNorm that precede the router
// folded in (README Part II section 5): xr = bf16(x + y_prev) (x itself when y_prev is NULL),
// xn = bf16(xr * inv), inv = (float)(1 / sqrt(sum of squares / H + eps)) with the squares of
// xr summed in double in the order of the standalone RMSNorm (lane L's chunks L + 64 i
// ascending, the low then the high half of each pair, then the fold s = 32 .. 1), and the
// scores of xn in route_scores_staged's order.  The workgroup builds xr in LDS once; each wave
// then sums the squares itself, so no second barrier is needed, and scores its expert.
// Workgroup 0 stores xr (when x_next is given) and xn.  H = 512 * NCH.
template <int NCH>
__global__ __launch_bounds__(256) void route_scores_residual(
    const uint16_t* __restrict__ x, const float* __restrict__ y_prev, float eps,
    const uint16_t* __restrict__ W, int32_t H, int32_t E, float* __restrict__ scores,
    uint16_t* __restrict__ x_next, uint16_t* __restrict__ xn) {
  constexpr int cpr = NCH * kWave;
  __shared__ uint4 xs[cpr];
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  uint4 wv[NCH];
  const uint4* wrow = reinterpret_cast<const uint4*>(W + (size_t)(e < E ? e : E - 1) * H);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NCH; ++i) wv[i] = wrow[lane + kWave * i];
  __builtin_amdgcn_sched_barrier(0);
  for (int c = threadIdx.x; c < cpr; c += blockDim.x) {
    uint4 v = reinterpret_cast<const uint4*>(x)[c];
    if (y_prev) {
      const float4 y0 = reinterpret_cast<const float4*>(y_prev)[2 * c];
      const float4 y1 = reinterpret_cast<const float4*>(y_prev)[2 * c + 1];
      const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = f32_to_bf16_bits(bf16_bits_to_f32(w[j] & 0xFFFFu) + ys[2 * j]) |
               (f32_to_bf16_bits(bf16_bits_to_f32(w[j] >> 16) + ys[2 * j + 1]) << 16);
      v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    xs[c] = v;
  }
  __syncthreads();
  if (e >= E) return;
  uint4 xv[NCH];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    xv[i] = xs[lane + kWave * i];
    const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
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
  const bool store = blockIdx.x == 0 && threadIdx.x < kWave;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
    const uint32_t ws[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = f32_to_bf16_bits(bf16_bits_to_f32(xw[j] & 0xFFFFu) * inv);
      const uint32_t hi = f32_to_bf16_bits(bf16_bits_to_f32(xw[j] >> 16) * inv);
      o[j] = lo | (hi << 16);
      acc = acc + (double)bf16_bits_to_f32(lo) * (double)bf16_bits_to_f32(ws[j] & 0xFFFFu);
      acc = acc + (double)bf16_bits_to_f32(hi) * (double)bf16_bits_to_f32(ws[j] >> 16);
    }
    if (store) {
      const int c = lane + kWave * i;
      reinterpret_cast<uint4*>(xn)[c] = make_uint4(o[0], o[1], o[2], o[3]);
      if (x_next) reinterpret_cast<uint4*>(x_next)[c] = xv[i];
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc = acc + __shfl_down(acc, s, kWave);
  if (lane == 0) {
    const float l = (float)acc;
    scores[e] = (float)(1.0 / (1.0 + exp(-(double)l)));
  }
}

typedef void (*ResidualScoresKernel)(const uint16_t*, const float*, float, const uint16_t*,
                                     int32_t, int32_t, float*, uint16_t*, uint16_t*);

template <int... N>
ResidualScoresKernel residual_kernel(int nch) {
  constexpr ResidualScoresKernel k[] = {route_scores_residual<N>...};
  return k[nch - 1];
}

typedef void (*ScoresKernel)(const uint16_t*, const uint16_t*, int32_t, int32_t, int32_t, float*);

template <int... N>
ScoresKernel staged_kernel(int nch, int nt) {
  constexpr ScoresKernel k1[] = {route_scores_staged<N, 1, 1>...};
  constexpr ScoresKernel k4[] = {route_scores_staged<N, kRouteTokBlock, 2>...};
  return (nt == 1 ? k1 : k4)[nch - 1];
}

// Kernel 2: one workgroup of kSelThreads per token (select_topk, k3x_select.h).
template <int M>
__global__ __launch_bounds__(kSelThreads) void route_select(const float* __restrict__ scores,
                                                            const float* __restrict__ bias,
                                                            int32_t E, int32_t topk,
                                                            int32_t renorm, float rscale,
                                                            int32_t* __restrict__ idx_out,
                                                            float* __restrict__ gates_out) {
  extern __shared__ float dyn[];  // [4][topk]
  const size_t t = blockIdx.x;
  select_topk<M>(scores + t * E, bias, E, topk, renorm, rscale, dyn, idx_out + t * topk,
                 gates_out + t * topk);
}

// The same for up to 1024 experts and 16 picks (select_topk_bitonic, k3x_select.h).
__global__ __launch_bounds__(kSelThreads) void route_select_bitonic(const float* __restrict__ scores,
                                                                    const float* __restrict__ bias,
                                                                    int32_t E, int32_t topk,
                                                                    int32_t renorm, float rscale,
                                                                    int32_t* __restrict__ idx_out,
                                                                    float* __restrict__ gates_out) {
  const size_t t = blockIdx.x;
  select_topk_bitonic(scores + t * E, bias, E, topk, renorm, rscale, idx_out + t * topk,
                      gates_out + t * topk);
}

}  // namespace

hipError_t launch_route_select(const k3x_router_desc& r, int32_t T, const float* scores,
                               int32_t* idx, float* gates, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int E = r.n_experts;
  if (select_bitonic_supported(E, r.topk))
    return launch("route_select", route_select_bitonic, dim3(T), dim3(kSelThreads), 0, s,
                  scores, r.bias, E, r.topk, r.renorm, r.routed_scale, idx, gates);
  const uint32_t lds = (uint32_t)(sizeof(float) * 4 * (size_t)r.topk);
  if (E <= kSelThreads * 4)
    return launch("route_select", route_select<4>, dim3(T), dim3(kSelThreads), lds, s, scores,
                  r.bias, E, r.topk, r.renorm, r.routed_scale, idx, gates);
  return launch("route_select", route_select<16>, dim3(T), dim3(kSelThreads), lds, s, scores,
                r.bias, E, r.topk, r.renorm, r.routed_scale, idx, gates);
}

hipError_t launch_route(const k3x_router_desc& r, const uint16_t* x, int32_t T, int32_t* idx,
                        float* gates, float* scores, hipStream_t s) {
  hipError_t err = launch_route_scores(r, x, T, scores, s);
  if (err != hipSuccess) return err;
  return launch_route_select(r, T, scores, idx, gates, s);
}

hipError_t launch_route_scores(const k3x_router_desc& r, const uint16_t* x, int32_t T,
                               float* scores, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int E = r.n_experts, H = r.hidden;
  const uint16_t* W = static_cast<const uint16_t*>(r.weight);
  hipError_t err;
  if (H % 512 == 0 && H <= 8192) {
    const int nt = T == 1 ? 1 : kRouteTokBlock;
    const int epw = nt == 1 ? 1 : 2;  // experts per wave (route_scores_staged's EPW)
    dim3 g((E + 4 * epw - 1) / (4 * epw), (T + nt - 1) / nt);
    err = launch("route_scores",
                 staged_kernel<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(H / 512, nt),
                 g, dim3(256), (uint32_t)(sizeof(uint16_t) * (size_t)nt * H), s, x, W, T, H, E,
                 scores);
  } else {
    dim3 g1((E + 3) / 4, (T + kRouteTokBlock - 1) / kRouteTokBlock);
    if (H <= 64 * 8 * 8)
      err = launch("route_scores", route_scores<8>, g1, dim3(256), 0, s, x, W, T, H, E, scores);
    else
      err = launch("route_scores", route_scores<32>, g1, dim3(256), 0, s, x, W, T, H, E, scores);
  }
  return err;
}

bool route_scores_residual_supported(const k3x_router_desc& r, int32_t T) {
  return T == 1 && r.hidden % 512 == 0 && r.hidden <= 8192;
}

hipError_t launch_route_scores_residual(const k3x_router_desc& r, const uint16_t* x,
                                        const float* y_prev, float eps, uint16_t* x_next,
                                        uint16_t* xn, float* scores, hipStream_t s) {
  const int E = r.n_experts, H = r.hidden;
  return launch("route_scores",
                residual_kernel<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(H / 512),
                dim3((E + 3) / 4), dim3(256), 0, s, x, y_prev, eps,
                static_cast<const uint16_t*>(r.weight), H, E, scores, x_next, xn);
}

}  // namespace k3x
