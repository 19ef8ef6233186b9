// Single-token decode of the routed experts in the reference arithmetic order.
//
// Source: kimi-k3-in-c README, Part II section 4 "Reduction one: the experts already ship at
// half a byte" (y = W.x taken straight from the nibbles, one power-of-two scale per group
// of 32, scale byte 255 zeroes its group) and section 9 "Picking 16 experts of 896" (the
// routed-expert loop and the slot-order weighted combine).  The activation is SwiGLU with h
// rounded to bf16 before W2.
//
// Every dot product is formed in one fixed order:
//   - a group of 32 is summed sequentially in fp32, element by element (the products of a
//     bf16 activation and an E2M1 value are exact, so a fused multiply-add gives the same
//     bits as a multiply followed by an add);
//   - the group sum is multiplied by its exact power-of-two scale;
//   - the group sums are added by a pairwise tree over groups in index order, zero-padded to
//     a power of two: lane L holds groups 2L and 2L+1 and adds them; lanes then combine with
//     partners at distance 1, 2, 4, 8, 16, 32, so each addition joins two adjacent subtrees
//     (IEEE addition is commutative, so which lane holds which operand does not matter).
// The exponential inside silu is the float nearest to exp(-g) (evaluated in double), and the
// combine multiplies and adds with separate roundings.  With these rules the result is a
// function of the inputs alone, independent of the launch shape.
//
// Decode is bound by HBM: each lane streams 32 contiguous bytes (two whole MX groups) of a
// weight row per load pair, so a wave reads whole rows with fully coalesced 16-byte loads;
// dequantization is in registers (gfx950 FP4 -> f32 conversion, two weights per
// instruction) and nothing dequantized is ever written.  Sixteen rows of one slot form a work
// item; loads run three rows ahead of the arithmetic, and lane r keeps row r's sum.
#include "k3x_internal.h"

// Products and sums below are rounded one at a time unless written as an explicit fma.
#pragma clang fp contract(off)

namespace k3x {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 16;  // rows per work item

struct DecodeArgs {
  const uint8_t* wa;  // W1 (w13) or W2 (w2) packed, expert 0
  const uint8_t* sa;
  const uint8_t* wb;  // W3 (w13), unused for w2
  const uint8_t* sb;
  int64_t st_wa, st_sa, st_wb, st_sb;
  int32_t K;          // reduction length: H for w13, I for w2
  int32_t rows;       // rows per expert: I for w13, H for w2
  const uint16_t* act;  // w13: x [1][H]; w2: h [topk][I]
  const int32_t* idx;   // [topk]
  int32_t topk, E;
  uint8_t* ws;          // w13 writes the drop count at offset 0
  void* out;            // w13: h bf16 [topk][I]; w2: d fp32 [topk][H]
};

__device__ __forceinline__ bool expert_ok(int e, int E) { return e >= 0 && e < E; }

// E2M1 values (unscaled) of the two nibbles of byte B of a dword: element 2B (low nibble)
// and element 2B + 1 (high nibble).
template <int B>
__device__ __forceinline__ f32x2 e2m1_pair(uint32_t dw) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw, 1.0f, B);
}

// p <- p + x[k] * w[k] for the 8 elements of one dword, in element order.
__device__ __forceinline__ float dot8(uint32_t dw, const float* x, float p) {
  const f32x2 w0 = e2m1_pair<0>(dw), w1 = e2m1_pair<1>(dw);
  const f32x2 w2 = e2m1_pair<2>(dw), w3 = e2m1_pair<3>(dw);
  p = __builtin_fmaf(x[0], w0[0], p);
  p = __builtin_fmaf(x[1], w0[1], p);
  p = __builtin_fmaf(x[2], w1[0], p);
  p = __builtin_fmaf(x[3], w1[1], p);
  p = __builtin_fmaf(x[4], w2[0], p);
  p = __builtin_fmaf(x[5], w2[1], p);
  p = __builtin_fmaf(x[6], w3[0], p);
  p = __builtin_fmaf(x[7], w3[1], p);
  return p;
}

// Sequential fp32 sum of one group: sum_c x[c] * E2M1[nibble c], c = 0..31 in order.
__device__ __forceinline__ float group_sum(const uint4& q, const float (&x)[32]) {
  float p = 0.0f;
  p = dot8(q.x, x + 0, p);
  p = dot8(q.y, x + 8, p);
  p = dot8(q.z, x + 16, p);
  p = dot8(q.w, x + 24, p);
  return p;
}

// bf16 activations of two groups (64 elements at e0) -> floats.
__device__ __forceinline__ void load_act(const uint16_t* __restrict__ row, int e0, bool ok,
                                         float (&x0)[32], float (&x1)[32]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 v = ok ? *reinterpret_cast<const uint4*>(row + e0 + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float* dst = c < 4 ? x0 : x1;
    const int o = (c % 4) * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[o + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      dst[o + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
  }
}

// One row of one matrix for this lane: its two groups and their scale bytes.
struct RowBits {
  uint4 q0, q1;
  uint32_t sc;  // two scale bytes (groups 2L, 2L+1) in the low 16 bits
};

__device__ __forceinline__ RowBits load_row(const uint8_t* wrow, const uint8_t* srow, int lane,
                                            bool ok) {
  RowBits r;
  if (ok) {
    const uint4* p = reinterpret_cast<const uint4*>(wrow + 32 * lane);
    r.q0 = p[0];
    r.q1 = p[1];
    r.sc = *reinterpret_cast<const uint16_t*>(srow + 2 * lane);
  } else {
    r.q0 = r.q1 = make_uint4(0, 0, 0, 0);
    r.sc = 0;
  }
  return r;
}

// Leaf of the tree for this lane: (group 2L sum * scale) + (group 2L+1 sum * scale).
__device__ __forceinline__ float row_leaf(const RowBits& r, const float (&x0)[32],
                                          const float (&x1)[32]) {
  const float p0 = group_sum(r.q0, x0) * e8m0_to_f32(r.sc & 0xFFu);
  const float p1 = group_sum(r.q1, x1) * e8m0_to_f32((r.sc >> 8) & 0xFFu);
  return p0 + p1;
}

// Sum of one row's lane leaves in tree order: partners at distance 1, 2, ..., 32.  Every
// lane ends with the same total.
__device__ __forceinline__ float tree_sum(float v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v = v + __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ void keep_row(int lane, int r, float gv, float uv, float& g, float& u) {
  if (lane == r) {
    g = gv;
    u = uv;
  }
}

// Work items of one wave: the die's contiguous share of the items, cut into contiguous runs
// per wave, so a wave keeps its slot (and its activation registers) for long stretches.
__device__ __forceinline__ void wave_items(int items, int& i0, int& i1) {
  int die, rank, per_die;
  xcd_rank(die, rank, per_die);
  const int wave = threadIdx.x / kWave;
  const int waves_per_die = per_die * (blockDim.x / kWave);
  const int wave_rank = rank * (blockDim.x / kWave) + wave;
  const int chunk = (items + kNumXcd - 1) / kNumXcd;
  const int lo = die * chunk;
  const int hi = min(items, lo + chunk);
  const int n = max(0, hi - lo);
  const int per = (n + waves_per_die - 1) / waves_per_die;
  i0 = min(hi, lo + wave_rank * per);
  i1 = min(hi, i0 + per);
}

// g = W1 x and u = W3 x for 16 rows of one slot, then h = bf16(silu(g) * u).
__global__ __launch_bounds__(256) void w13_decode_exact(DecodeArgs a) {
  const int lane = threadIdx.x % kWave;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int bad = 0;
    for (int j = 0; j < a.topk; ++j) bad += expert_ok(a.idx[j], a.E) ? 0 : 1;
    *reinterpret_cast<int64_t*>(a.ws) = bad;
  }
  const int ngroups = a.K / kGroup;
  const bool lane_ok = 2 * lane < ngroups;
  float x0[32], x1[32];
  load_act(a.act, 64 * lane, lane_ok, x0, x1);

  const int per_slot = a.rows / kRows;
  int i0, i1;
  wave_items(a.topk * per_slot, i0, i1);
  const size_t wrow = (size_t)a.K / 2, srow = (size_t)ngroups;
  for (int it = i0; it < i1; ++it) {
    const int slot = it / per_slot;
    const int r0 = (it % per_slot) * kRows;
    const int e = a.idx[slot];
    if (!expert_ok(e, a.E)) continue;
    const uint8_t* w1 = a.wa + (size_t)e * a.st_wa + (size_t)r0 * wrow;
    const uint8_t* s1 = a.sa + (size_t)e * a.st_sa + (size_t)r0 * srow;
    const uint8_t* w3 = a.wb + (size_t)e * a.st_wb + (size_t)r0 * wrow;
    const uint8_t* s3 = a.sb + (size_t)e * a.st_sb + (size_t)r0 * srow;

    // rows r0..r0+15, loads issued three rows ahead; lane r keeps row r's sums
    float g = 0.0f, u = 0.0f;
    RowBits a0, a1, a2, a3, c0, c1, c2, c3;
    a0 = load_row(w1, s1, lane, lane_ok);
    c0 = load_row(w3, s3, lane, lane_ok);
    a1 = load_row(w1 + wrow, s1 + srow, lane, lane_ok);
    c1 = load_row(w3 + wrow, s3 + srow, lane, lane_ok);
    a2 = load_row(w1 + 2 * wrow, s1 + 2 * srow, lane, lane_ok);
    c2 = load_row(w3 + 2 * wrow, s3 + 2 * srow, lane, lane_ok);
#pragma unroll 1
    for (int r = 0; r < kRows; r += 4) {
      a3 = load_row(w1 + (r + 3) * wrow, s1 + (r + 3) * srow, lane, lane_ok);
      c3 = load_row(w3 + (r + 3) * wrow, s3 + (r + 3) * srow, lane, lane_ok);
      keep_row(lane, r, tree_sum(row_leaf(a0, x0, x1)), tree_sum(row_leaf(c0, x0, x1)), g, u);
      if (r + 4 < kRows) {
        a0 = load_row(w1 + (r + 4) * wrow, s1 + (r + 4) * srow, lane, lane_ok);
        c0 = load_row(w3 + (r + 4) * wrow, s3 + (r + 4) * srow, lane, lane_ok);
      }
      keep_row(lane, r + 1, tree_sum(row_leaf(a1, x0, x1)), tree_sum(row_leaf(c1, x0, x1)), g, u);
      if (r + 5 < kRows) {
        a1 = load_row(w1 + (r + 5) * wrow, s1 + (r + 5) * srow, lane, lane_ok);
        c1 = load_row(w3 + (r + 5) * wrow, s3 + (r + 5) * srow, lane, lane_ok);
      }
      keep_row(lane, r + 2, tree_sum(row_leaf(a2, x0, x1)), tree_sum(row_leaf(c2, x0, x1)), g, u);
      if (r + 6 < kRows) {
        a2 = load_row(w1 + (r + 6) * wrow, s1 + (r + 6) * srow, lane, lane_ok);
        c2 = load_row(w3 + (r + 6) * wrow, s3 + (r + 6) * srow, lane, lane_ok);
      }
      keep_row(lane, r + 3, tree_sum(row_leaf(a3, x0, x1)), tree_sum(row_leaf(c3, x0, x1)), g, u);
    }
    if (lane < kRows) {
      const float ex = (float)exp(-(double)g);
      const float hv = (g / (1.0f + ex)) * u;
      uint16_t* h = static_cast<uint16_t*>(a.out);
      h[(size_t)slot * a.rows + r0 + lane] = (uint16_t)f32_to_bf16_bits(hv);
    }
  }
}

// d = W2 h for 16 rows of one slot.
__global__ __launch_bounds__(256) void w2_decode_exact(DecodeArgs a) {
  const int lane = threadIdx.x % kWave;
  const int ngroups = a.K / kGroup;
  const bool lane_ok = 2 * lane < ngroups;
  const int per_slot = a.rows / kRows;
  int i0, i1;
  wave_items(a.topk * per_slot, i0, i1);
  const size_t wrow = (size_t)a.K / 2, srow = (size_t)ngroups;
  float x0[32], x1[32];
  int have = -1;
  for (int it = i0; it < i1; ++it) {
    const int slot = it / per_slot;
    const int r0 = (it % per_slot) * kRows;
    const int e = a.idx[slot];
    if (!expert_ok(e, a.E)) continue;
    if (slot != have) {
      load_act(a.act + (size_t)slot * a.K, 64 * lane, lane_ok, x0, x1);
      have = slot;
    }
    const uint8_t* w2 = a.wa + (size_t)e * a.st_wa + (size_t)r0 * wrow;
    const uint8_t* s2 = a.sa + (size_t)e * a.st_sa + (size_t)r0 * srow;
    float dsum = 0.0f, dummy = 0.0f;
    RowBits b0, b1, b2, b3;
    b0 = load_row(w2, s2, lane, lane_ok);
    b1 = load_row(w2 + wrow, s2 + srow, lane, lane_ok);
    b2 = load_row(w2 + 2 * wrow, s2 + 2 * srow, lane, lane_ok);
#pragma unroll 1
    for (int r = 0; r < kRows; r += 4) {
      b3 = load_row(w2 + (r + 3) * wrow, s2 + (r + 3) * srow, lane, lane_ok);
      keep_row(lane, r, tree_sum(row_leaf(b0, x0, x1)), 0.0f, dsum, dummy);
      if (r + 4 < kRows) b0 = load_row(w2 + (r + 4) * wrow, s2 + (r + 4) * srow, lane, lane_ok);
      keep_row(lane, r + 1, tree_sum(row_leaf(b1, x0, x1)), 0.0f, dsum, dummy);
      if (r + 5 < kRows) b1 = load_row(w2 + (r + 5) * wrow, s2 + (r + 5) * srow, lane, lane_ok);
      keep_row(lane, r + 2, tree_sum(row_leaf(b2, x0, x1)), 0.0f, dsum, dummy);
      if (r + 6 < kRows) b2 = load_row(w2 + (r + 6) * wrow, s2 + (r + 6) * srow, lane, lane_ok);
      keep_row(lane, r + 3, tree_sum(row_leaf(b3, x0, x1)), 0.0f, dsum, dummy);
    }
    if (lane < kRows) static_cast<float*>(a.out)[(size_t)slot * a.rows + r0 + lane] = dsum;
  }
}

// y[r] = sum_j gates[j] * d[j][r] over valid slots in slot order, each product and each sum
// rounded separately.  One thread per row.
__global__ __launch_bounds__(256) void combine_exact(const float* __restrict__ d,
                                                     const int32_t* __restrict__ idx,
                                                     const float* __restrict__ gates,
                                                     int32_t topk, int32_t H, int32_t E,
                                                     float* __restrict__ y) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= H) return;
  float dv[64];
#pragma unroll
  for (int j = 0; j < 64; ++j)
    if (j < topk) dv[j] = expert_ok(idx[j], E) ? d[(size_t)j * H + r] : 0.0f;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 64; ++j)
    if (j < topk && expert_ok(idx[j], E)) acc = acc + gates[j] * dv[j];
  y[r] = acc;
}

int decode_grid(const void* fn) {
  static int cached[2] = {0, 0};
  const int which = fn == reinterpret_cast<const void*>(&w13_decode_exact) ? 0 : 1;
  if (!cached[which]) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu < 1)
      per_cu = 2;
    cached[which] = per_cu;
  }
  return device_cu_count() * cached[which];
}

}  // namespace

bool decode_exact_supported(const k3x_pool& p, int32_t T, int32_t topk) {
  return T == 1 && topk <= 64 && p.H / kGroup <= 128 && p.I / kGroup <= 128 &&
         p.H % kRows == 0 && p.I % kRows == 0;
}

size_t decode_exact_ws(const k3x_pool& p, int32_t topk, size_t* off_h, size_t* off_d) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = up(16);
  *off_h = off;
  off = up(off + sizeof(uint16_t) * (size_t)topk * p.I);
  *off_d = off;
  off = up(off + sizeof(float) * (size_t)topk * p.H);
  return off;
}

hipError_t launch_decode_exact(const k3x_pool& p, const uint16_t* x, const int32_t* idx,
                               const float* gates, int32_t topk, float* y, uint8_t* ws,
                               hipStream_t s) {
  size_t off_h, off_d;
  decode_exact_ws(p, topk, &off_h, &off_d);
  DecodeArgs a{};
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
  a.act = x;
  a.idx = idx;
  a.topk = topk;
  a.E = p.E;
  a.ws = ws;
  a.out = ws + off_h;
  {
    LaunchTimer lt("w13_decode", s);
    hipLaunchKernelGGL(w13_decode_exact,
                       dim3(decode_grid(reinterpret_cast<const void*>(&w13_decode_exact))),
                       dim3(256), 0, s, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  DecodeArgs b = a;
  b.wa = p.base[4];
  b.sa = p.base[5];
  b.wb = nullptr;
  b.sb = nullptr;
  b.st_wa = p.stride[4];
  b.st_sa = p.stride[5];
  b.K = p.I;
  b.rows = p.H;
  b.act = reinterpret_cast<const uint16_t*>(ws + off_h);
  b.out = ws + off_d;
  {
    LaunchTimer lt("w2_decode", s);
    hipLaunchKernelGGL(w2_decode_exact,
                       dim3(decode_grid(reinterpret_cast<const void*>(&w2_decode_exact))),
                       dim3(256), 0, s, b);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    LaunchTimer lt("moe_combine", s);
    hipLaunchKernelGGL(combine_exact, dim3((p.H + 255) / 256), dim3(256), 0, s,
                       reinterpret_cast<const float*>(ws + off_d), idx, gates, topk, p.H, p.E, y);
  }
  return hipGetLastError();
}

}  // namespace k3x
