// The expert forward of one token in the pages' floating point contract (kimi-k3-in-c README,
// Part II section 4, the MXFP4 matmul; section 5, "double, always"): every matvec sums, per
// row, its groups in sequence in double -- each group the sequential double sum of its exact
// products, times its scale, a NaN scale byte (255) skipping the group -- and rounds the row
// once to float; h = act(g, u) stays in fp32; the slots are combined in fp32 in slot order.
//
// contract_rows streams rows three ahead of the arithmetic (as the decode kernels do): lane L
// turns its groups L and 64 + L into terms, which are parked in LDS for a batch of 16 rows;
// then one lane per row adds the row's terms in group order.  The W1/W3 rows alternate, so a
// row's g and u end up in neighbouring lanes, which evaluate h with the exact activation (each
// exponential and tanh the float nearest its double value).  contract_combine adds the slots.
// A skipped group adds +0.0, which leaves the accumulator unchanged: it starts at +0.0 and a
// sum of these terms is never -0.0.
#include "k3x_internal.h"

namespace k3x {
namespace {

constexpr int kCThreads = 256;
constexpr int kCWaves = kCThreads / kWave;
constexpr int kCBatch = 16;          // rows whose terms are parked before their chains run
constexpr int kCMaxGroups = 128;     // K <= 4096
constexpr int kCStride = kCMaxGroups + 1;

struct ContractArgs {
  const uint8_t* wa;  // W1 (w13) or W2 packed, expert 0
  const uint8_t* sa;
  const uint8_t* wb;  // W3 (w13)
  const uint8_t* sb;
  int64_t st_wa, st_sa, st_wb, st_sb;
  int32_t K;          // H for w13, I for w2
  int32_t rows;       // I for w13, H for w2
  const uint16_t* x;  // w13: bf16 [K]
  const float* h;     // w2: fp32 [topk][K]
  const int32_t* idx; // [topk]
  int32_t topk, E;
  uint8_t* ws;        // w13 writes the drop count at offset 0
  float* out;         // w13: h fp32 [topk][I]; w2: d fp32 [topk][H]
  int32_t act;
  float b1, b2;
};

__device__ __forceinline__ bool expert_ok(int e, int E) { return e >= 0 && e < E; }

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

typedef float cf32x2 __attribute__((ext_vector_type(2)));

// part += x[2B] * w[2B], then x[2B + 1] * w[2B + 1], for byte B of one dword of nibbles.
template <int B>
__device__ __forceinline__ double byte_terms(uint32_t dw, const float* x, double part) {
  const cf32x2 w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw, 1.0f, B);
  part = __builtin_fma((double)x[2 * B], (double)w[0], part);
  return __builtin_fma((double)x[2 * B + 1], (double)w[1], part);
}

// The term of one group: the sequential double sum of its 32 products (exact in double), in
// element order, times its scale (+0.0 for a NaN scale byte).  x: the group's 32 inputs.
__device__ __forceinline__ double group_term(const uint4& q, uint32_t s, const float (&x)[32]) {
  const uint32_t dw[4] = {q.x, q.y, q.z, q.w};
  double part = 0.0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    part = byte_terms<0>(dw[d], x + 8 * d, part);
    part = byte_terms<1>(dw[d], x + 8 * d, part);
    part = byte_terms<2>(dw[d], x + 8 * d, part);
    part = byte_terms<3>(dw[d], x + 8 * d, part);
  }
  return s == 255u ? 0.0 : part * (double)e8m0_to_f32(s);
}

// fp32 inputs of this lane's groups L (x0) and 64 + L (x1); zero past the last group.
__device__ __forceinline__ void load_inputs_bf16(const uint16_t* row, int lane, int ng,
                                                 float (&x0)[32], float (&x1)[32]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = lane + 64 * h;
    float* dst = h ? x1 : x0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = g < ng ? *reinterpret_cast<const uint4*>(row + 32 * g + 8 * c) : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[8 * c + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
        dst[8 * c + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      }
    }
  }
}
__device__ __forceinline__ void load_inputs_f32(const float* row, int lane, int ng,
                                                float (&x0)[32], float (&x1)[32]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = lane + 64 * h;
    float* dst = h ? x1 : x0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 v = g < ng ? reinterpret_cast<const float4*>(row + 32 * g)[c] : make_float4(0, 0, 0, 0);
      dst[4 * c] = v.x;
      dst[4 * c + 1] = v.y;
      dst[4 * c + 2] = v.z;
      dst[4 * c + 3] = v.w;
    }
  }
}

struct CRow {
  uint4 q0, q1;
  uint32_t s0, s1;
};

// Items: W13 -- item 2 p and 2 p + 1 are the W1 and W3 rows r of slot j (p = j I + r);
// W2 -- item p is the W2 row r of slot j (p = j H + r).
template <bool kW13>
__global__ __launch_bounds__(kCThreads) void contract_rows(ContractArgs a) {
  __shared__ double terms[kCWaves][kCBatch][kCStride];
  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int ng = a.K / kGroup;
  const int my_idx = lane < a.topk ? a.idx[lane] : -1;
  if (kW13 && blockIdx.x == 0 && threadIdx.x < kWave) {
    const unsigned long long bad = __ballot(lane < a.topk && !expert_ok(my_idx, a.E));
    if (lane == 0) *reinterpret_cast<int64_t*>(a.ws) = __popcll(bad);
  }
  const int per_item = kW13 ? 2 : 1;
  const int total = a.topk * a.rows * per_item;
  const int nw = gridDim.x * kCWaves;
  const int w = blockIdx.x * kCWaves + wv;
  int i0 = (int)((int64_t)total * w / nw), i1 = (int)((int64_t)total * (w + 1) / nw);
  if (kW13) {  // whole (W1, W3) pairs per wave
    i0 &= ~1;
    i1 = w + 1 == nw ? total : (i1 & ~1);
  }
  const uint32_t wrow = (uint32_t)a.K / 2, srow = (uint32_t)ng;
  const uint32_t oa = lane < ng ? 16u * lane : 0u, ob = lane + 64 < ng ? 16u * (lane + 64) : 0u;
  const uint32_t sa = lane < ng ? (uint32_t)lane : 0u, sb = lane + 64 < ng ? (uint32_t)lane + 64u : 0u;

  float x0[32], x1[32];
  int xslot = -1;
  if (kW13) load_inputs_bf16(a.x, lane, ng, x0, x1);

  auto item_ptrs = [&](int it, const uint8_t*& wp, const uint8_t*& sp, int& slot, int& r) {
    const int p = kW13 ? it >> 1 : it;
    slot = p / a.rows;
    r = p - slot * a.rows;
    int e = __builtin_amdgcn_readlane(my_idx, slot);
    if (!expert_ok(e, a.E)) e = 0;  // a dropped slot reads expert 0 and is never used
    const bool b = kW13 && (it & 1);
    wp = (b ? a.wb : a.wa) + (size_t)e * (b ? a.st_wb : a.st_wa) + (size_t)r * wrow;
    sp = (b ? a.sb : a.sa) + (size_t)e * (b ? a.st_sb : a.st_sa) + (size_t)r * srow;
  };
  CRow ring[4];
  auto load = [&](int i, int it) {
    const int ii = it < i1 ? it : i1 - 1;
    const uint8_t *wp, *sp;
    int slot, r;
    item_ptrs(ii, wp, sp, slot, r);
    __builtin_amdgcn_sched_barrier(0);
    ring[i].q0 = *reinterpret_cast<const uint4*>(wp + oa);
    ring[i].q1 = *reinterpret_cast<const uint4*>(wp + ob);
    ring[i].s0 = sp[sa];
    ring[i].s1 = sp[sb];
    __builtin_amdgcn_sched_barrier(0);
  };
  if (i0 >= i1) return;
  load(0, i0);
  load(1, i0 + 1);
  load(2, i0 + 2);
  int q = 0, bstart = i0;
  // one lane per parked row: its terms in group order, one rounding to float
  auto chains = [&](int n) {
    __builtin_amdgcn_wave_barrier();
    float v = 0.0f;
    if (lane < n) {
      double acc = 0.0;
      for (int g = 0; g < ng; ++g) acc = acc + terms[wv][lane][g];
      v = (float)acc;
    }
    if (kW13) {
      const float u = __shfl_xor(v, 1, kWave);
      const int p = (bstart + lane) >> 1;
      const int slot = p / a.rows, r = p - slot * a.rows;
      const int e = __shfl(my_idx, slot < a.topk ? slot : 0, kWave);  // every lane takes part
      if (lane < n && (lane & 1) == 0 && expert_ok(e, a.E))
        a.out[(size_t)slot * a.rows + r] = glu_exact(v, u, a.act, a.b1, a.b2);
    } else if (lane < n) {
      const int p = bstart + lane;
      const int slot = p / a.rows, r = p - slot * a.rows;
      a.out[(size_t)slot * a.rows + r] = v;
    }
    __builtin_amdgcn_wave_barrier();
  };
#pragma unroll 1
  for (int it = i0; it < i1; it += 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cur = it + k;
      load((k + 3) % 4, cur + 3);
      if (cur < i1) {
        if (!kW13) {  // W2: the slot's h, when the slot changes
          const int slot = cur / a.rows;
          if (slot != xslot) {
            load_inputs_f32(a.h + (size_t)slot * a.K, lane, ng, x0, x1);
            xslot = slot;
          }
        }
        const CRow& rb = ring[k];
        if (lane < ng) terms[wv][q][lane] = group_term(rb.q0, rb.s0, x0);
        if (lane + 64 < ng) terms[wv][q][lane + 64] = group_term(rb.q1, rb.s1, x1);
        if (++q == kCBatch) {
          chains(q);
          q = 0;
          bstart = cur + 1;
        }
      }
    }
  }
  if (q > 0) chains(q);
}

// y[r] = sum over valid slots j, in slot order, of gates[j] * d[j][r]; each product and each
// sum rounded to fp32.
__global__ __launch_bounds__(256) void contract_combine(const float* __restrict__ d,
                                                        const float* __restrict__ gates,
                                                        const int32_t* __restrict__ idx,
                                                        int32_t topk, int32_t E, int32_t H,
                                                        float* __restrict__ y) {
#pragma clang fp contract(off)  // the product and the sum are rounded separately
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= H) return;
  float acc = 0.0f;
  for (int j = 0; j < topk; ++j) {
    if (!expert_ok(idx[j], E)) continue;
    acc = acc + gates[j] * d[(size_t)j * H + r];
  }
  y[r] = acc;
}

}  // namespace

bool contract_supported(const k3x_pool& p, int32_t T, int32_t topk) {
  return T == 1 && topk <= 64 && p.H / kGroup <= kCMaxGroups && p.I / kGroup <= kCMaxGroups;
}

size_t contract_ws(const k3x_pool& p, int32_t topk, size_t* off_h, size_t* off_d) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = up(16);
  *off_h = off;
  off = up(off + sizeof(float) * (size_t)topk * p.I);
  *off_d = off;
  off = up(off + sizeof(float) * (size_t)topk * p.H);
  return off;
}

hipError_t launch_contract(const k3x_pool& p, const uint16_t* x, const int32_t* idx,
                           const float* gates, int32_t topk, float* y, uint8_t* ws,
                           hipStream_t s) {
  size_t off_h, off_d;
  contract_ws(p, topk, &off_h, &off_d);
  const int ncu = device_cu_count();
  ContractArgs a{};
  a.wa = p.base[0];
  a.sa = p.base[1];
  a.wb = p.base[2];
  a.sb = p.base[3];
  a.st_wa = p.stride[0];
  a.st_sa = p.stride[1];
  a.st_wb = p.stride[2];
  a.st_sb = p.stride[3];
  a.K = p.H;
  a.rows = p.I;
  a.x = x;
  a.idx = idx;
  a.topk = topk;
  a.E = p.E;
  a.ws = ws;
  a.out = reinterpret_cast<float*>(ws + off_h);
  a.act = p.act;
  a.b1 = p.b1;
  a.b2 = p.b2;
  hipError_t e = launch("w13_contract", contract_rows<true>, dim3(2 * ncu), dim3(kCThreads), 0, s, a);
  if (e != hipSuccess) return e;
  ContractArgs b = a;
  b.wa = p.base[4];
  b.sa = p.base[5];
  b.wb = nullptr;
  b.sb = nullptr;
  b.st_wa = p.stride[4];
  b.st_sa = p.stride[5];
  b.K = p.I;
  b.rows = p.H;
  b.x = nullptr;
  b.h = reinterpret_cast<const float*>(ws + off_h);
  b.out = reinterpret_cast<float*>(ws + off_d);
  e = launch("w2_contract", contract_rows<false>, dim3(2 * ncu), dim3(kCThreads), 0, s, b);
  if (e != hipSuccess) return e;
  return launch("combine_contract", contract_combine, dim3((p.H + 255) / 256), dim3(256), 0, s,
                reinterpret_cast<const float*>(ws + off_d), gates, idx, topk, p.E, p.H, y);
}

}  // namespace k3x
