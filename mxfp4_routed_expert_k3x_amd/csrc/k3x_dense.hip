// The dense parts of the latent MoE block around the routed experts (kimi-k3-in-c README,
// Part II section 9, the k3_moe listing): the down-projection of the full-width input into the
// expert latent, the up-projection back, the two shared experts that run on the original
// input and are added unweighted, and the RMSNorm of the aggregate of the routed experts
// (README Part II section 5, the RMSNorm of the floating point contract, with its weight).
//
// Two row-streaming kernels over bf16 weights, for decode-sized batches (up to 8 tokens a
// launch; larger batches run in passes, each reading the weights again):
//   latent_in:  the rows of the router Wr [E][D], down [L][D], sh1 [S][D] and sh3 [S][D] all
//               read x, so one launch streams all E + L + 2 S of them: the router's scores
//               (the logit rounded to float, then a double sigmoid rounded once, as the
//               router's own kernel), z = bf16(down . x), and for each shared row j the rows
//               sh1[j] and sh3[j] back to back in one wave, g and u parked per lane and
//               s[j] = bf16(act(g, u)) evaluated 64 at a time.
//   latent_out: output row n is the fp32 sum of up[n] . a and sh2[n] . s, streamed as one row
//               of L + S columns against [a | s]; the launch stages a = bf16(RMSNorm_w(acc))
//               (the aggregate of the routed experts) and s in LDS itself.
// Every dot product is the contract's bf16 matmul (README Part II section 5): exact products,
// summed in double, rounded once to float; the double sum runs in a fixed 64-way order (lane
// L sums, in ascending order, the 8-element chunks whose index is L mod 64; the partials fold
// p[L] += p[L + s] for s = 32 .. 1), so every result is reproducible bit for bit.  The
// activations sit in LDS once per launch; each wave streams whole weight rows (lane L reads
// the 16-byte chunks L, L + 64, ...: one load instruction covers 1 KB of a row), one row ahead
// of the arithmetic.
#include <type_traits>

#include "k3x_internal.h"

namespace k3x {
namespace {

constexpr int kTok = 8;  // tokens per launch at most (staged: 8 * 2 * 9728 B <= 160 KB)
constexpr int kDenseWaves = 8;
constexpr int kDenseThreads = kDenseWaves * kWave;

struct DenseArgs {
  int32_t t0, nt;          // tokens [t0, t0 + nt) of this launch
  int32_t rows;            // rows streamed by the launch
  // latent_in
  const uint16_t* x;       // [T][D]
  const uint16_t* wr;      // router [E][D]
  float* scores;           // fp32 [T][E]
  int32_t E;
  const uint16_t* down;    // [L][D]
  const uint16_t* sh1;     // [S][D]
  const uint16_t* sh3;     // [S][D]
  uint16_t* z;             // bf16 [T][L]
  uint16_t* s;             // bf16 [T][S] shared experts' activation
  int32_t L, S, D;
  int32_t act;             // shared experts' activation (k3x_activation) and caps
  float b1, b2;
  // latent_out
  const uint16_t* up;      // [D][L]
  const uint16_t* sh2;     // [D][S]
  const float* acc;        // fp32 [T][L]
  const float* norm_w;     // fp32 [L] or null
  float eps;
  int32_t norm;            // 0: a = bf16(acc)
  float* out;              // fp32 [T][D]
};

// A double from lane + n of the same row of 16 lanes (DPP row_shl:n; 0 past the row).
template <int N>
__device__ __forceinline__ double row_shl(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, 0x100 + N, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), 0x100 + N, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The fixed 64-way fold of the lane partials, p[L] += p[L + s] for s = 32 .. 1, exact for
// lane 0 (the steps inside a row of 16 lanes read their partner with DPP); the sum is read
// from lane 0 (uniform).
__device__ __forceinline__ double fold64_d(double p) {
  p = p + __shfl_down(p, 32, kWave);
  p = p + __shfl_down(p, 16, kWave);
  p = p + row_shl<8>(p);
  p = p + row_shl<4>(p);
  p = p + row_shl<2>(p);
  p = p + row_shl<1>(p);
  return p;
}

__device__ __forceinline__ float fold64(double p) {
  const float f = (float)fold64_d(p);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), 0));
}

// This wave's rows [r0, r1) of `rows`, split evenly over every wave of the grid; a boundary
// that falls inside the pair region [pair0, rows) at an odd offset moves up by one, so the two
// rows of a pair stay in one wave.
__device__ __forceinline__ void wave_range(int rows, int pair0, int& r0, int& r1) {
  const int nw = gridDim.x * kDenseWaves;
  const int w = blockIdx.x * kDenseWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  auto bound = [&](int v) {
    int b = (int)((int64_t)rows * v / nw);
    if (b > pair0 && ((b - pair0) & 1)) ++b;
    return b < rows ? b : rows;
  };
  r0 = bound(w);
  r1 = bound(w + 1);
}

// Streams rows [r0, r1) against the staged activations xs[NT][NCH * 64]: base(r, pa, pb)
// gives the first 16-byte chunk of row r in its two parts (lane L reads chunks L, L + 64, ...
// of pa for i < na, then L, L + 64, ... of pb).  Each part is summed on its own (kSplit; else
// na == NCH) and emit(r, t, A, B) receives the two sums of token t, the same on every lane.
// stage() (run by every thread of the block, with its barriers) fills xs; the wave's first
// row is requested before it, so the row's latency overlaps the staging.  The last row is
// summed by a second copy of the loop body that requests nothing after it (a wave has only a
// few rows, and a re-read of its last row would often miss the cache).
// 16 bytes of a weight row, loaded non-temporal: each row is read once per launch, in whole
// cache lines per load instruction, so its lines may leave the caches first (the block's
// activations and the next launch's data stay).
__device__ __forceinline__ uint4 stream_load16(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int NCH, int NT, bool kSplit, class Base, class Stage, class Emit>
__device__ __forceinline__ void stream_dense(int r0, int r1, int na, const uint4* xs, int lane,
                                             Base base, Stage stage, Emit emit) {
  uint4 cur[NCH], nxt[NCH];  // the next row is loaded while this one is summed
  auto load = [&](uint4 (&b)[NCH], int r) {
    const uint4 *pa, *pb;  // uniform row bases; the lane's chunks are added at the load
    base(r, pa, pb);
    pb = pb - kWave * na;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NCH; ++i) b[i] = stream_load16((i < na ? pa : pb) + lane + kWave * i);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (r0 < r1) load(cur, r0);
  stage();
  // row r; kNext: the next row is requested first and becomes the current one after
  auto row = [&](int r, auto next) {
    constexpr bool kNext = decltype(next)::value;
    if constexpr (kNext) load(nxt, r + 1);
    // the activations are read again for every row (kept out of registers)
    int xo = lane;
    asm volatile("" : "+v"(xo));
    double acc[NT], accA[kSplit ? NT : 1];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t] = 0.0;
      if (kSplit) accA[t] = 0.0;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (kSplit && i == na) {  // chunk na starts the second part: park the first (uniform)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          accA[t] = acc[t];
          acc[t] = 0.0;
        }
      }
      const uint32_t wv[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
      double wd[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wd[2 * q] = (double)bf16_bits_to_f32(wv[q] & 0xFFFFu);
        wd[2 * q + 1] = (double)bf16_bits_to_f32(wv[q] >> 16);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint4 xv = xs[(t * NCH + i) * kWave + xo];
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[t] = __builtin_fma(wd[2 * q], (double)bf16_bits_to_f32(xw[q] & 0xFFFFu), acc[t]);
          acc[t] = __builtin_fma(wd[2 * q + 1], (double)bf16_bits_to_f32(xw[q] >> 16), acc[t]);
        }
      }
      if (NT > 1) {  // one chunk's activations live at a time
#pragma unroll
        for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(acc[t]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float B = fold64(acc[t]);
      const float A = kSplit ? fold64(accA[t]) : B;
      emit(r, t, A, B);
    }
    if constexpr (kNext) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) cur[i] = nxt[i];
    }
  };
#pragma unroll 1
  for (int r = r0; r < r1 - 1; ++r) row(r, std::true_type{});
  if (r0 < r1) row(r1 - 1, std::false_type{});
}

// Zero-fills the staged slots of tokens nt .. NT - 1 (their sums are computed and dropped).
template <int NT>
__device__ __forceinline__ void zero_tail(uint4* xs, int nt, int cpr) {
  for (int i = nt * cpr + threadIdx.x; i < NT * cpr; i += kDenseThreads) xs[i] = make_uint4(0, 0, 0, 0);
}

// The gated activation of one shared-expert pair, each exp and tanh the float nearest its
// double value, products and quotients in fp32 left to right.
__device__ __forceinline__ float glu_exact(float g, float u, int act, float b1, float b2) {
  const float ex = (float)exp(-(double)g);
  if (act == K3X_ACT_SITU) {
    const float tg = (float)tanh((double)(g / b1));
    const float sg = 1.0f / (1.0f + ex);
    const float av = b1 * tg * sg;
    const float tu = (float)tanh((double)(u / b2));
    return av * (b2 * tu);
  }
  return (g / (1.0f + ex)) * u;
}

template <int NCH, int NT>
__global__ __launch_bounds__(kDenseThreads) void latent_in(DenseArgs a) {
  extern __shared__ uint4 xs[];  // [NT][D / 8]
  const int lane = threadIdx.x % kWave;
  const int cpr = NCH * kWave;
  auto stage = [&]() {
    for (int i = threadIdx.x; i < a.nt * cpr; i += kDenseThreads)
      xs[i] = reinterpret_cast<const uint4*>(a.x + (size_t)(a.t0 + i / cpr) * a.D)[i % cpr];
    zero_tail<NT>(xs, a.nt, cpr);
    __syncthreads();
  };
  const int E = a.E, L = a.L, S = a.S, P = E + L;  // P: first row of the shared pairs
  int r0, r1;
  wave_range(a.rows, P, r0, r1);
  // rows [0, E): router; [E, P): down; P + 2 j and P + 2 j + 1: sh1[j] and sh3[j]
  auto base = [&](int r, const uint4*& pa, const uint4*& pb) {
    const int j = (r - P) >> 1;
    const uint16_t* w = r < E   ? a.wr + (size_t)r * a.D
                        : r < P ? a.down + (size_t)(r - E) * a.D
                        : ((r - P) & 1) ? a.sh3 + (size_t)j * a.D
                                        : a.sh1 + (size_t)j * a.D;
    pa = pb = reinterpret_cast<const uint4*>(w);
  };
  float gst[NT];                // g of the current pair, per token
  float pg = 0.0f, pu = 0.0f;   // parked pairs: lane k holds the k-th
  int po = 0, np = 0;           // its output index; number parked (uniform)
  auto flush = [&]() {
    if (lane < np) a.s[po] = (uint16_t)f32_to_bf16_bits(glu_exact(pg, pu, a.act, a.b1, a.b2));
    np = 0;
  };
  stream_dense<NCH, NT, false>(r0, r1, NCH, xs, lane, base, stage, [&](int r, int t, float, float v) {
    const int tt = a.t0 + t;
    if (r < E) {
      if (lane == 0 && t < a.nt)
        a.scores[(size_t)tt * E + r] = (float)(1.0 / (1.0 + exp(-(double)v)));
    } else if (r < P) {
      if (lane == 0 && t < a.nt) a.z[(size_t)tt * L + (r - E)] = (uint16_t)f32_to_bf16_bits(v);
    } else if (((r - P) & 1) == 0) {
      gst[t] = v;
    } else if (t < a.nt) {
      if (np == kWave) flush();
      if (lane == np) {
        pg = gst[t];
        pu = v;
        po = tt * S + ((r - P) >> 1);
      }
      ++np;
    }
  });
  flush();
}

// Staging of latent_out: xs[t] = [bf16(RMSNorm_w(acc[t])) | s[t]].  The sum of squares of
// acc[t] is taken by wave t in double in the fixed 64-way order; inv = (float)(1 / sqrt(ss / L
// + eps)); a = bf16((acc * inv) * w).
__device__ void stage_out(const DenseArgs& a, uint4* xs, int cpr) {
  __shared__ float s_inv[kTok];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int L = a.L, S = a.S, lc = L / 8, sc = S / 8;
  if (a.norm && wave < a.nt) {
    const float4* xr = reinterpret_cast<const float4*>(a.acc + (size_t)(a.t0 + wave) * L);
    double ss = 0.0;
    for (int c = lane; c < lc; c += kWave) {
      const float4 v0 = xr[2 * c], v1 = xr[2 * c + 1];
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = ss + (double)v[j] * (double)v[j];
    }
    ss = fold64_d(ss);
    if (lane == 0) s_inv[wave] = (float)(1.0 / sqrt(ss / (double)L + (double)a.eps));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.nt * lc; i += kDenseThreads) {
    const int t = i / lc, c = i % lc;
    const float4* xr = reinterpret_cast<const float4*>(a.acc + (size_t)(a.t0 + t) * L);
    const float4 v0 = xr[2 * c], v1 = xr[2 * c + 1];
    float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    if (a.norm) {
      const float inv = s_inv[t];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * inv * (a.norm_w ? a.norm_w[8 * c + j] : 1.0f);
    }
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = f32_to_bf16_bits(v[2 * j]) | (f32_to_bf16_bits(v[2 * j + 1]) << 16);
    xs[t * cpr + c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  for (int i = threadIdx.x; i < a.nt * sc; i += kDenseThreads) {
    const int t = i / sc, c = i % sc;
    xs[t * cpr + lc + c] = reinterpret_cast<const uint4*>(a.s + (size_t)(a.t0 + t) * S)[c];
  }
  __syncthreads();
}

template <int NCH, int NT>
__global__ __launch_bounds__(kDenseThreads) void latent_out(DenseArgs a) {
  extern __shared__ uint4 xs[];  // [NT][(L + S) / 8]
  const int lane = threadIdx.x % kWave;
  const int cpr = NCH * kWave;
  auto stage = [&]() {
    zero_tail<NT>(xs, a.nt, cpr);
    stage_out(a, xs, cpr);
  };
  int r0, r1;
  wave_range(a.rows, a.rows, r0, r1);
  const int na = a.L / (8 * kWave);  // chunks per lane taken from up
  auto base = [&](int r, const uint4*& pa, const uint4*& pb) {
    pa = reinterpret_cast<const uint4*>(a.up + (size_t)r * a.L);
    pb = reinterpret_cast<const uint4*>(a.sh2 + (size_t)r * a.S);
  };
  stream_dense<NCH, NT, true>(r0, r1, na, xs, lane, base, stage, [&](int r, int t, float o, float f) {
    if (lane == 0 && t < a.nt) a.out[(size_t)(a.t0 + t) * a.D + r] = o + f;
  });
}

typedef void (*DenseKernel)(DenseArgs);

// Instantiations by chunks per lane: latent_in for D = 512 .. 8192, latent_out for
// L + S = 1024 .. 9728 (the most whose 8 staged tokens fit in LDS).
template <int... N>
DenseKernel in_kernel(int n, int nt) {
  constexpr DenseKernel k1[] = {latent_in<N, 1>...}, k8[] = {latent_in<N, kTok>...};
  return (nt == 1 ? k1 : k8)[n - 1];
}
template <int... N>
DenseKernel out_kernel(int n, int nt) {
  constexpr DenseKernel k1[] = {latent_out<N, 1>...}, k8[] = {latent_out<N, kTok>...};
  return (nt == 1 ? k1 : k8)[n - 2];
}

}  // namespace

LatentLayout latent_layout(const k3x_latent_desc& d, const k3x_pool& p, int32_t E, int32_t T,
                           int32_t topk) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  LatentLayout L{};
  size_t off = 0;
  L.scores = off;
  off = up(off + sizeof(float) * (size_t)T * E + 16);
  L.idx = off;
  off = up(off + sizeof(int32_t) * (size_t)T * topk + 16);
  L.gates = off;
  off = up(off + sizeof(float) * (size_t)T * topk + 16);
  L.z = off;
  off = up(off + sizeof(uint16_t) * (size_t)T * p.H + 16);
  L.acc = off;
  off = up(off + sizeof(float) * (size_t)T * p.H + 16);
  L.s = off;
  off = up(off + sizeof(uint16_t) * (size_t)T * d.shared_inter + 16);
  L.moe = off;
  return L;
}

hipError_t launch_latent(const k3x_latent_desc& d, const k3x_pool& p, const k3x_router_desc& r,
                         const uint16_t* x, int32_t T, float* out, uint8_t* ws,
                         const LatentLayout& L, const MoeLayout& ML, hipStream_t s) {
  DenseArgs a{};
  a.L = p.H;
  a.S = d.shared_inter;
  a.D = d.hidden;
  a.x = x;
  a.wr = static_cast<const uint16_t*>(r.weight);
  a.E = r.n_experts;
  a.scores = reinterpret_cast<float*>(ws + L.scores);
  a.down = static_cast<const uint16_t*>(d.down);
  a.sh1 = static_cast<const uint16_t*>(d.sh1);
  a.sh3 = static_cast<const uint16_t*>(d.sh3);
  a.up = static_cast<const uint16_t*>(d.up);
  a.sh2 = static_cast<const uint16_t*>(d.sh2);
  a.z = reinterpret_cast<uint16_t*>(ws + L.z);
  a.s = reinterpret_cast<uint16_t*>(ws + L.s);
  a.acc = reinterpret_cast<const float*>(ws + L.acc);
  a.norm_w = d.norm_weight;
  a.eps = d.eps;
  a.norm = d.latent_norm ? 1 : 0;
  a.act = d.shared_activation;
  a.b1 = d.situ_b1;
  a.b2 = d.situ_b2;
  a.out = out;
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
  float* gates = reinterpret_cast<float*>(ws + L.gates);
  const int ncu = device_cu_count();

  // the router's scores on the full width, z = bf16(down . x), s = bf16(act(sh1 . x, sh3 . x))
  hipError_t e = hipSuccess;
  const int kin = a.D / (8 * kWave), tin = kTok;
  a.rows = a.E + a.L + 2 * a.S;
  for (int t0 = 0; e == hipSuccess && t0 < T; t0 += tin) {
    a.t0 = t0;
    a.nt = std::min(tin, T - t0);
    const int blocks = std::max(1, std::min(ncu, (a.rows + kDenseWaves - 1) / kDenseWaves));
    e = launch("latent_in", in_kernel<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(kin, a.nt), dim3(blocks), dim3(kDenseThreads),
               (uint32_t)(sizeof(uint16_t) * (size_t)(a.nt == 1 ? 1 : kTok) * a.D), s, a);
  }
  // the top-k selection, then the routed experts on the latent
  if (e == hipSuccess) e = launch_route_select(r, T, a.scores, idx, gates, s);
  if (e == hipSuccess)
    e = launch_moe(p, a.z, T, idx, gates, r.topk, const_cast<float*>(a.acc), ws + L.moe, ML, s);
  // out = up . a + sh2 . s, a = bf16(RMSNorm_w(acc))
  const int kout = (a.L + a.S) / (8 * kWave), tout = kTok;
  a.rows = a.D;
  for (int t0 = 0; e == hipSuccess && t0 < T; t0 += tout) {
    a.t0 = t0;
    a.nt = std::min(tout, T - t0);
    const int blocks = std::max(1, std::min(ncu, (a.rows + kDenseWaves - 1) / kDenseWaves));
    e = launch("latent_out", out_kernel<2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18,
                                      19>(kout, a.nt), dim3(blocks), dim3(kDenseThreads),
               (uint32_t)(sizeof(uint16_t) * (size_t)(a.nt == 1 ? 1 : kTok) * (a.L + a.S)), s,
               a);
  }
  return e;
}

}  // namespace k3x
