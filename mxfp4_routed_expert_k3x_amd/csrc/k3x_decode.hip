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
//     128 leaves (a zero leaf leaves every sum unchanged, so this is the tree over the groups
//     padded to any power of two): lane L holds groups L and 64 + L; each half of the tree is
//     formed by lanes combining with partners at distance 1, 2, 4, 8, 16, 32, so each
//     addition joins two adjacent subtrees, and the root adds the two halves (IEEE addition
//     is commutative, so which lane holds which operand does not matter).
// The exponential inside silu is the float nearest to exp(-g) (evaluated in double), and the
// combine multiplies and adds with separate roundings.  With these rules the result is a
// function of the inputs alone, independent of the launch shape.
//
// Decode is bound by HBM: lane L reads group L of a weight row, then group 64 + L, so each
// load instruction of a wave covers up to 1 KB of the row contiguously (whole cache lines);
// loads go through buffer descriptors whose range is the row, so lanes past its last group
// issue no request.  Dequantization is in registers (gfx950 FP4 -> f32 conversion, two
// weights per instruction) and nothing dequantized is ever written.  Two launches: W1/W3
// (each wave streams a contiguous run of rows over all slots and writes h; called from the
// router path it first selects the experts itself), then W2 with the weighted combine in its
// epilogue (each workgroup owns a block of output rows of every slot, so the slot-order sum
// happens in LDS and the per-slot W2 outputs never reach memory; rows of 65..96 groups share
// the load of their second halves two rows at a time, and a wave's two slots run as one
// pipeline across the change of slot).  Loads run two rows ahead of the
// arithmetic (three or more measured slower: the launch streams best with few requests in
// flight per CU).
#include <atomic>

#include "k3x_internal.h"
#include "k3x_select.h"

// Products and sums below are rounded one at a time unless written as an explicit fma.
#pragma clang fp contract(off)

namespace k3x {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

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
  int32_t gact;         // k3x_activation of the W1/W3 epilogue
  float b1, b2;         // SiTU-GLU caps
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

// The bf16 activations of this lane's groups L and 64 + L, as loaded: raw[4 h + c] holds
// elements 8c .. 8c + 7 of group L + 64 h.  Lanes past the last group read the last group
// (act_to_f32 zeroes them), so the loads are unconditional and can be issued early, their
// conversion waiting until the first weight rows are in flight.
__device__ __forceinline__ void load_act_raw(const uint16_t* __restrict__ row, int lane,
                                             int ngroups, uint4 (&raw)[8]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = min(lane + 64 * h, ngroups - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[4 * h + c] = *reinterpret_cast<const uint4*>(row + 32 * g + 8 * c);
  }
}

// raw -> floats of groups L (x0) and 64 + L (x1); zero past the last group.  The raw words
// pass through an empty asm, so the conversion stays where it is called (after the first
// weight rows are requested) instead of being hoisted next to the loads.
__device__ __forceinline__ void act_to_f32(const uint4 (&raw)[8], int lane, int ngroups,
                                           float (&x0)[32], float (&x1)[32]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool ok = lane + 64 * h < ngroups;
    float* dst = h ? x1 : x0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = raw[4 * h + c];
      asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[8 * c + 2 * j] = ok ? bf16_bits_to_f32(w[j] & 0xFFFFu) : 0.0f;
        dst[8 * c + 2 * j + 1] = ok ? bf16_bits_to_f32(w[j] >> 16) : 0.0f;
      }
    }
  }
}

// One row of one matrix for this lane: groups L and 64 + L and their scale bytes.
struct RowBits {
  uint4 q0, q1;
  uint32_t s0, s1;
};

// The two leaves of this lane: group L sum * scale (half A) and group 64 + L sum * scale
// (half B).
__device__ __forceinline__ void row_leaves(const RowBits& r, const float (&x0)[32],
                                           const float (&x1)[32], float& la, float& lb) {
  la = group_sum(r.q0, x0) * e8m0_to_f32(r.s0);
  lb = group_sum(r.q1, x1) * e8m0_to_f32(r.s1);
}

// Rows of one wave.  The rows of all slots form one sequence g = slot * rows + r; each die
// takes a contiguous, balanced share of it, and each wave of the die a contiguous, balanced
// run of that share, so every wave streams nearly the same number of rows and the expert
// (and, for W2, the slot's activations) changes at most a few times along a run.
template <int kThreads>
__device__ __forceinline__ void wave_rows(int total, int& g0, int& g1) {
  int die, rank, per_die;
  xcd_rank(die, rank, per_die);
  constexpr int wpb = kThreads / kWave;
  const int W = per_die * wpb;
  const int w = rank * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lo = (int)((int64_t)total * die / kNumXcd);
  const int hi = (int)((int64_t)total * (die + 1) / kNumXcd);
  const int n = hi - lo;
  g0 = lo + (int)((int64_t)n * w / W);
  g1 = lo + (int)((int64_t)n * (w + 1) / W);
}

// Loads row r of one matrix of expert e through buffer descriptors whose range is the row
// (the row's bytes, the row's scale bytes): wave-uniform row addresses plus per-lane offsets.
// Lanes past the last group get an offset beyond the range, so the buffer unit returns zeros
// for them without a memory request; their activations are zero as well, so their leaves are
// zero.  The load is unconditional (callers clamp r to a real row), so the loop body has no
// branches and loads stay in flight across rows.
struct LaneOffsets {
  uint32_t wa, wb, sa, sb;  // weight bytes and scale bytes of groups L and 64 + L
};

// Cache policy of the weight and scale loads: non-temporal.  A token reads each expert row
// once, its weight bytes in whole cache lines per load instruction, so the stream's lines may
// leave the caches first.  (The prefill's weight loads must not use it: each of them takes half
// of every line it touches, and the other half is read one K block later.)
constexpr int kStreamLoad = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ void load_row(RowBits& b, const uint8_t* wexp, const uint8_t* sexp,
                                         int r, uint32_t wrow, uint32_t srow,
                                         const LaneOffsets& o) {
  const __amdgpu_buffer_rsrc_t rw = row_rsrc(wexp + (size_t)r * wrow, wrow);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(sexp + (size_t)r * srow, srow);
  const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rw, o.wa, 0, kStreamLoad);
  const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rw, o.wb, 0, kStreamLoad);
  b.q0 = make_uint4(v0[0], v0[1], v0[2], v0[3]);
  b.q1 = make_uint4(v1[0], v1[1], v1[2], v1[3]);
  b.s0 = __builtin_amdgcn_raw_buffer_load_b8(rs, o.sa, 0, kStreamLoad);
  b.s1 = __builtin_amdgcn_raw_buffer_load_b8(rs, o.sb, 0, kStreamLoad);
}

// Reduce-scatter of eight leaves per vector (rows 0..3 of half A, then rows 0..3 of half B)
// across the wave, in tree order: distances 1, 2, 4 halve the set (lane L keeps entry
// L & 7), distances 8 .. 32 finish each half's tree, and a last exchange at distance 4 adds
// the two halves of a row.  On return v[m][0] of lane L is the full sum of row (L & 3).
template <int NV>
__device__ __forceinline__ void reduce8(float (&v)[NV][8], int lane) {
  const bool b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1;
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    float a[4], c[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // entries 2j, 2j+1 -> entry 2j + b0
      const float k = b0 ? v[m][2 * j + 1] : v[m][2 * j];
      const float s = b0 ? v[m][2 * j] : v[m][2 * j + 1];
      a[j] = k + __shfl_xor(s, 1, kWave);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // -> entry 4j + 2 b1 + b0
      const float k = b1 ? a[2 * j + 1] : a[2 * j];
      const float s = b1 ? a[2 * j] : a[2 * j + 1];
      c[j] = k + __shfl_xor(s, 2, kWave);
    }
    const float k = b2 ? c[1] : c[0], s = b2 ? c[0] : c[1];
    float t = k + __shfl_xor(s, 4, kWave);  // entry L & 7
#pragma unroll
    for (int d = 8; d < kWave; d <<= 1) t = t + __shfl_xor(t, d, kWave);
    v[m][0] = t + __shfl_xor(t, 4, kWave);  // half A + half B of row L & 3
  }
}

// Per-lane load offsets of a row of K/32 groups (lanes past the last group get an offset
// outside the row's descriptor range).
__device__ __forceinline__ LaneOffsets lane_offsets(int lane, int ngroups) {
  constexpr uint32_t kOutside = 0x40000000u;
  LaneOffsets lo;
  lo.wa = lane < ngroups ? 16u * lane : kOutside;
  lo.wb = lane + 64 < ngroups ? 16u * (lane + 64) : kOutside;
  lo.sa = lane < ngroups ? (uint32_t)lane : kOutside;
  lo.sb = lane + 64 < ngroups ? (uint32_t)lane + 64u : kOutside;
  return lo;
}

// Streams rows r0 .. rlast of one expert (one matrix, or W1 and W3 side by side when kW13)
// against the activations x0/x1: rows are loaded two ahead of the arithmetic and finished
// four at a time.  prep() runs once the first two rows are requested (it fills x0/x1 from
// activations already in flight).  After each group of four rows r .. r + 3 every lane calls
// emit(r + lane, sum_a, sum_b, valid, n): lanes 0..3 with valid set hold the full dot
// products of row r + lane (sum_b only when kW13), and n (the same on every lane) is the
// number of valid rows in the group.
template <bool kW13, typename Prep, typename Emit>
__device__ __forceinline__ void stream_rows(const uint8_t* wa, const uint8_t* sa,
                                            const uint8_t* wb, const uint8_t* sb, int r0,
                                            int rlast, uint32_t wrow, uint32_t srow,
                                            const LaneOffsets& lo, const float (&x0)[32],
                                            const float (&x1)[32], int lane, Prep prep,
                                            Emit emit) {
  RowBits A[4] = {}, C[4] = {};
  // row r into buffer i (rows past the segment re-read rlast); the scheduling barriers keep
  // the loads where they stand, two rows ahead of the arithmetic
  auto load = [&](int i, int r) {
    const int rr = r <= rlast ? r : rlast;
    __builtin_amdgcn_sched_barrier(0);
    load_row(A[i], wa, sa, rr, wrow, srow, lo);
    if (kW13) load_row(C[i], wb, sb, rr, wrow, srow, lo);
    __builtin_amdgcn_sched_barrier(0);
  };
  load(0, r0);
  load(1, r0 + 1);
  prep();
#pragma unroll 1
  for (int r = r0; r <= rlast; r += 4) {
    float v[kW13 ? 2 : 1][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load((i + 2) % 4, r + i + 2);
      row_leaves(A[i], x0, x1, v[0][i], v[0][4 + i]);
      if (kW13) row_leaves(C[i], x0, x1, v[kW13 ? 1 : 0][i], v[kW13 ? 1 : 0][4 + i]);
    }
    reduce8(v, lane);
    emit(r + lane, v[0][0], v[kW13 ? 1 : 0][0], lane < 4 && r + lane <= rlast,
         min(4, rlast - r + 1));
  }
}

// Rows of 64 < G <= 96 groups (W2 at I = 3072): the second half of a row (groups 64 .. G - 1)
// has at most 32 groups, so two rows share one load there: lanes 0..31 take groups 64 + L of
// the even row, lanes 32..63 groups 64 + (L - 32) of the odd row, and every lane's arithmetic
// is used.  The sums keep the same tree: each row's second half is the subtree of groups
// 64..95 (lanes of one half-wave, distances 1..16) joined to the zero subtree of groups
// 96..127 by an explicit + 0, and the root adds the two halves.
struct PairLanes {
  uint32_t wa, wb, sa, sb;  // group L of a row; group 64 + (L & 31) of the even / odd row
};

__device__ __forceinline__ PairLanes pair_lanes(int lane, int ngroups, uint32_t wrow,
                                                uint32_t srow) {
  constexpr uint32_t kOutside = 0x40000000u;
  const int g = 64 + (lane & 31);
  const bool odd = lane >= 32;
  PairLanes o;
  o.wa = 16u * lane;
  o.sa = (uint32_t)lane;
  o.wb = g < ngroups ? (odd ? wrow : 0u) + 16u * g : kOutside;
  o.sb = g < ngroups ? (odd ? srow : 0u) + (uint32_t)g : kOutside;
  return o;
}

struct PairBits {
  uint4 a0, a1, b;        // first halves of the even and odd rows, shared second half
  uint32_t s0, s1, sb;
};

// Rows r and r + 1 (r + 1 past rlast: the odd row is absent, its loads return zeros).
__device__ __forceinline__ void load_pair(PairBits& p, const uint8_t* wexp, const uint8_t* sexp,
                                          int r, int rlast, uint32_t wrow, uint32_t srow,
                                          const PairLanes& o) {
  const int r1 = r + 1 <= rlast ? r + 1 : r;
  const uint32_t nrows = r1 > r ? 2u : 1u;
  const __amdgpu_buffer_rsrc_t w0 = row_rsrc(wexp + (size_t)r * wrow, wrow);
  const __amdgpu_buffer_rsrc_t w1 = row_rsrc(wexp + (size_t)r1 * wrow, wrow);
  const __amdgpu_buffer_rsrc_t wb = row_rsrc(wexp + (size_t)r * wrow, nrows * wrow);
  const __amdgpu_buffer_rsrc_t s0 = row_rsrc(sexp + (size_t)r * srow, srow);
  const __amdgpu_buffer_rsrc_t s1 = row_rsrc(sexp + (size_t)r1 * srow, srow);
  const __amdgpu_buffer_rsrc_t sb = row_rsrc(sexp + (size_t)r * srow, nrows * srow);
  const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(w0, o.wa, 0, kStreamLoad);
  const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(w1, o.wa, 0, kStreamLoad);
  const auto vb = __builtin_amdgcn_raw_buffer_load_b128(wb, o.wb, 0, kStreamLoad);
  p.a0 = make_uint4(v0[0], v0[1], v0[2], v0[3]);
  p.a1 = make_uint4(v1[0], v1[1], v1[2], v1[3]);
  p.b = make_uint4(vb[0], vb[1], vb[2], vb[3]);
  p.s0 = __builtin_amdgcn_raw_buffer_load_b8(s0, o.sa, 0, kStreamLoad);
  p.s1 = __builtin_amdgcn_raw_buffer_load_b8(s1, o.sa, 0, kStreamLoad);
  p.sb = __builtin_amdgcn_raw_buffer_load_b8(sb, o.sb, 0, kStreamLoad);
}

// Activations of the paired layout: x0 = group L, x1 = group 64 + (L & 31) (zero past G).
__device__ __forceinline__ void load_act_raw_pair(const uint16_t* __restrict__ row, int lane,
                                                  int ngroups, uint4 (&raw)[8]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = min(h ? 64 + (lane & 31) : lane, ngroups - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[4 * h + c] = *reinterpret_cast<const uint4*>(row + 32 * g + 8 * c);
  }
}

__device__ __forceinline__ void act_to_f32_pair(const uint4 (&raw)[8], int lane, int ngroups,
                                                float (&x0)[32], float (&x1)[32]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool ok = (h ? 64 + (lane & 31) : lane) < ngroups;
    float* dst = h ? x1 : x0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = raw[4 * h + c];
      asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[8 * c + 2 * j] = ok ? bf16_bits_to_f32(w[j] & 0xFFFFu) : 0.0f;
        dst[8 * c + 2 * j + 1] = ok ? bf16_bits_to_f32(w[j] >> 16) : 0.0f;
      }
    }
  }
}

// Four rows from two pairs: A[r] = first-half leaves of row r, B[0] = second halves of rows 0
// (lanes 0..31) and 1 (lanes 32..63), B[1] the same for rows 2 and 3.  Returns, in lane L < 4,
// the full sum of row L.
__device__ __forceinline__ float reduce_pairs(const float (&A)[4], const float (&B)[2], int lane) {
  const bool b0 = lane & 1, b1 = (lane >> 1) & 1;
  float a[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // rows 2j, 2j + 1 -> row 2j + b0
    const float k = b0 ? A[2 * j + 1] : A[2 * j];
    const float s = b0 ? A[2 * j] : A[2 * j + 1];
    a[j] = k + __shfl_xor(s, 1, kWave);
  }
  float t;
  {
    const float k = b1 ? a[1] : a[0], s = b1 ? a[0] : a[1];
    t = k + __shfl_xor(s, 2, kWave);  // row L & 3
  }
#pragma unroll
  for (int d = 4; d < kWave; d <<= 1) t = t + __shfl_xor(t, d, kWave);  // first half, row L & 3
  float u;
  {
    const float k = b0 ? B[1] : B[0], s = b0 ? B[0] : B[1];
    u = k + __shfl_xor(s, 1, kWave);
  }
#pragma unroll
  for (int d = 2; d < 32; d <<= 1) u = u + __shfl_xor(u, d, kWave);  // groups 64..95
  u = u + 0.0f;  // joined to the zero subtree of groups 96..127
  // second half of row r sits in lane (r >> 1) + 32 (r & 1)
  const int r = lane & 3;
  const float ub = __shfl(u, (r >> 1) + 32 * (r & 1), kWave);
  return t + ub;
}

// The three leaves of one pair (first halves of the even and odd rows, the shared second half).
__device__ __forceinline__ void pair_leaves(const PairBits& p, const float (&x0)[32],
                                            const float (&x1)[32], float& a0, float& a1,
                                            float& b) {
  a0 = group_sum(p.a0, x0) * e8m0_to_f32(p.s0);
  a1 = group_sum(p.a1, x0) * e8m0_to_f32(p.s1);
  b = group_sum(p.b, x1) * e8m0_to_f32(p.sb);
}

// Rows r0 .. rlast of W2 for one or two slots in the paired layout, as one stream: the pairs
// of the first slot, then those of the second (s1 < 0: none), one pair loaded ahead of the
// arithmetic also across the change of slot, so the loads never drain in between (a wave
// whose two slots ran as separate streams waited a full memory latency at the change).  Both
// slots' activations are requested up front; the second's are widened when its first pair
// comes up.  Rows are finished four at a time (two pairs); with an odd number of pairs per
// slot one group of four holds the last pair of the first slot and the first of the second.
// Every lane calls emit(s, r, sum, valid) after each group: lane L < 4 with valid set holds
// the full sum of row r of slot s.
template <typename Emit>
__device__ __forceinline__ void stream_pairs2(const DecodeArgs& a, int s0, int e0, int s1,
                                              int e1, int r0, int rlast, uint32_t wrow,
                                              uint32_t srow, const PairLanes& po, int lane,
                                              int ngroups, Emit emit) {
  const int np = (rlast - r0 + 2) / 2;  // pairs per slot
  const bool two = s1 >= 0;
  const int Q = two ? 2 * np : np;
  const int sl1 = two ? s1 : s0, ex1 = two ? e1 : e0;
  const uint8_t* w0 = a.wa + (size_t)e0 * a.st_wa;
  const uint8_t* c0 = a.sa + (size_t)e0 * a.st_sa;
  const uint8_t* w1 = a.wa + (size_t)ex1 * a.st_wa;
  const uint8_t* c1 = a.sa + (size_t)ex1 * a.st_sa;
  uint4 ra[8], rb[8];
  load_act_raw_pair(a.act + (size_t)s0 * a.K, lane, ngroups, ra);
  load_act_raw_pair(a.act + (size_t)sl1 * a.K, lane, ngroups, rb);
  PairBits P[2] = {};
  // pair q of the stream into buffer i (pairs past the end re-read the last one)
  auto load = [&](int i, int q) {
    const int qq = q < Q ? q : Q - 1;
    const bool second = qq >= np;
    const int r = r0 + 2 * (second ? qq - np : qq);
    __builtin_amdgcn_sched_barrier(0);
    load_pair(P[i], second ? w1 : w0, second ? c1 : c0, r, rlast, wrow, srow, po);
    __builtin_amdgcn_sched_barrier(0);
  };
  // pairs q (against xa) and q + 1 (against xb), then their rows
  auto quad = [&](int q, const float (&xa0)[32], const float (&xa1)[32], const float (&xb0)[32],
                  const float (&xb1)[32]) __attribute__((always_inline)) {
    float A[4], B[2];
    load(1, q + 1);
    pair_leaves(P[0], xa0, xa1, A[0], A[1], B[0]);
    load(0, q + 2);
    pair_leaves(P[1], xb0, xb1, A[2], A[3], B[1]);
    const float v = reduce_pairs(A, B, lane);
    // lane L < 4: row L & 1 of pair q + (L >> 1)
    const int qq = q + ((lane >> 1) & 1);
    const bool second = qq >= np;
    const int r = r0 + 2 * (second ? qq - np : qq) + (lane & 1);
    emit(second ? sl1 : s0, r, v, lane < 4 && qq < Q && r <= rlast);
  };
  load(0, 0);
  float x0[32], x1[32];
  act_to_f32_pair(ra, lane, ngroups, x0, x1);
  const bool odd = np & 1;
  int q = 0;
#pragma unroll 1
  for (; q < np - 1; q += 2) quad(q, x0, x1, x0, x1);  // groups within the first slot
  if (!two) {
    if (odd) quad(q, x0, x1, x0, x1);  // the last pair alone
    return;
  }
  float y0[32], y1[32];
  act_to_f32_pair(rb, lane, ngroups, y0, y1);
  if (odd) {  // the group that holds both slots
    quad(q, x0, x1, y0, y1);
    q += 2;
  }
#pragma unroll 1
  for (; q < Q; q += 2) quad(q, y0, y1, y0, y1);
}

// g = W1 x, u = W3 x, h = bf16(silu(g) * u) (or of SiTU-GLU, with each tanh the float nearest
// to its double value, products and quotients in fp32 left to right) for every (slot, row)
// of this wave's run.  A run is cut at slot boundaries into segments of one expert; a dropped
// slot's segment is skipped.  The finished (g, u) pairs are parked in the wave's LDS slice
// and their activations evaluated up to 64 at a time, one per lane, so the double-precision
// exponentials and tanh do not hold up the row loop.  Workgroup 0 also writes the number of
// dropped slots.
constexpr int kW13Threads = 256;
// Dynamic LDS the launch reserves (and the kernel leaves unused) so that one 4-wave workgroup
// runs per CU: with one wave per SIMD the launch streams its rows faster than with two (fewer
// concurrent streams; the bytes in flight still suffice), and much faster than with half a
// wave per SIMD.
constexpr uint32_t kW13LdsLimiter = 96 * 1024;

// With kSel the launch also picks the token's experts: every workgroup runs the router's
// selection (select_topk_bitonic) on the scores of route_scores while its activations load, and
// workgroup 0 writes the picks and gates for the W2 launch and the caller.
struct SelArgs {
  const float* scores;  // [E] sigmoid scores of the token
  const float* bias;    // [E] correction bias or NULL
  int32_t E, renorm;
  float rscale;
  int32_t* idx_out;     // [topk]
  float* gates_out;     // [topk]
};

template <bool kSel>
__global__ __launch_bounds__(kW13Threads) void decode_w13(DecodeArgs a, SelArgs sel) {
  const int lane = threadIdx.x % kWave;
  const int ngroups = a.K / kGroup;
  uint4 xr[8];
  load_act_raw(a.act, lane, ngroups, xr);
  int my_idx;
  if constexpr (kSel) {
    __shared__ int32_t s_idx[kWave];
    __shared__ float s_gate[kWave];
    select_topk_bitonic(sel.scores, sel.bias, sel.E, a.topk, sel.renorm, sel.rscale, s_idx,
                        s_gate);
    __syncthreads();
    my_idx = lane < a.topk ? s_idx[lane] : -1;
    if (blockIdx.x == 0 && threadIdx.x < a.topk) {
      sel.idx_out[threadIdx.x] = s_idx[threadIdx.x];
      sel.gates_out[threadIdx.x] = s_gate[threadIdx.x];
    }
  } else {
    my_idx = lane < a.topk ? a.idx[lane] : -1;
  }
  if (blockIdx.x == 0 && threadIdx.x < kWave) {
    const unsigned long long bad = __ballot(lane < a.topk && !expert_ok(my_idx, a.E));
    if (lane == 0) *reinterpret_cast<int64_t*>(a.ws) = __popcll(bad);
  }
  const uint32_t wrow = (uint32_t)a.K / 2, srow = (uint32_t)ngroups;
  const LaneOffsets lo = lane_offsets(lane, ngroups);
  int g0, g1;
  wave_rows<kW13Threads>(a.topk * a.rows, g0, g1);

  float x0[32], x1[32];

  __shared__ float s_g[4][kWave], s_u[4][kWave];
  __shared__ int32_t s_o[4][kWave];
  const int wv = threadIdx.x / kWave;
  uint16_t* hout = static_cast<uint16_t*>(a.out);
  int nbuf = 0;  // parked rows of this wave (the same on every lane)
  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();
    if (lane < nbuf) {
      const float gv = s_g[wv][lane], uv = s_u[wv][lane];
      const float ex = (float)exp(-(double)gv);
      float hv;
      if (a.gact == K3X_ACT_SITU) {
        const float tg = (float)tanh((double)(gv / a.b1));
        const float sg = 1.0f / (1.0f + ex);
        const float av = a.b1 * tg * sg;
        const float tu = (float)tanh((double)(uv / a.b2));
        hv = av * (a.b2 * tu);
      } else {
        hv = (gv / (1.0f + ex)) * uv;
      }
      hout[s_o[wv][lane]] = (uint16_t)f32_to_bf16_bits(hv);
    }
    __builtin_amdgcn_wave_barrier();
    nbuf = 0;
  };

  for (int gs = g0; gs < g1;) {
    const int slot = gs / a.rows;
    const int r0 = gs - slot * a.rows;
    const int n = min(g1 - gs, a.rows - r0);  // rows of this segment
    const int e = __builtin_amdgcn_readlane(my_idx, slot);
    gs += n;
    if (!expert_ok(e, a.E)) continue;
    const int obase = slot * a.rows;
    stream_rows<true>(a.wa + (size_t)e * a.st_wa, a.sa + (size_t)e * a.st_sa,
                      a.wb + (size_t)e * a.st_wb, a.sb + (size_t)e * a.st_sb, r0, r0 + n - 1,
                      wrow, srow, lo, x0, x1, lane,
                      [&]() { act_to_f32(xr, lane, ngroups, x0, x1); },
                      [&](int r, float gv, float uv, bool valid, int nv) {
                        if (valid) {
                          s_g[wv][nbuf + lane] = gv;
                          s_u[wv][nbuf + lane] = uv;
                          s_o[wv][nbuf + lane] = obase + r;
                        }
                        nbuf += nv;
                        if (nbuf > kWave - 4) flush();
                      });
  }
  flush();
}

// y = sum_j gates[j] * (W2_j h_j) over valid slots in slot order, with the combine in the
// epilogue: workgroup b owns output rows [b R, b R + R) of every slot, so it holds all the
// terms of its rows.  Wave w streams the block's rows of slots w, w + 8, ... (one expert
// each, against that slot's h) and parks d[slot][row] in LDS; after a barrier one thread per
// row adds the slots in order, each product and each sum rounded separately.  d never
// reaches memory.
constexpr int kW2Waves = 8;

__global__ __launch_bounds__(kW2Waves * kWave) void decode_w2_combine(DecodeArgs a,
                                                                      const float* __restrict__ gates,
                                                                      float* __restrict__ y,
                                                                      int32_t R) {
  extern __shared__ float dsh[];  // [topk][R]
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int my_idx = lane < a.topk ? a.idx[lane] : -1;
  const float my_gate = lane < a.topk ? gates[lane] : 0.0f;
  const int rb0 = blockIdx.x * R;
  const int rlast = rb0 + min(R, a.rows - rb0) - 1;
  const int nr = rlast - rb0 + 1;
  const int ngroups = a.K / kGroup;
  const uint32_t wrow = (uint32_t)a.K / 2, srow = (uint32_t)ngroups;
  const LaneOffsets lo = lane_offsets(lane, ngroups);
  const bool paired = ngroups > kWave && ngroups <= kWave + 32;
  const PairLanes po = pair_lanes(lane, ngroups, wrow, srow);

  if (paired) {
    // the wave's valid slots two at a time, each two as one stream
    auto park = [&](int slot, int r, float dv, bool valid) {
      if (valid) dsh[slot * R + r - rb0] = dv;
    };
    int pend = -1, pend_e = -1;
    for (int slot = wave; slot < a.topk; slot += kW2Waves) {
      const int e = __builtin_amdgcn_readlane(my_idx, slot);
      if (!expert_ok(e, a.E)) continue;
      if (pend < 0) {
        pend = slot;
        pend_e = e;
        continue;
      }
      stream_pairs2(a, pend, pend_e, slot, e, rb0, rlast, wrow, srow, po, lane, ngroups, park);
      pend = -1;
    }
    if (pend >= 0)
      stream_pairs2(a, pend, pend_e, -1, -1, rb0, rlast, wrow, srow, po, lane, ngroups, park);
  } else {
    float x0[32], x1[32];
    for (int slot = wave; slot < a.topk; slot += kW2Waves) {
      const int e = __builtin_amdgcn_readlane(my_idx, slot);
      if (!expert_ok(e, a.E)) continue;
      uint4 hr[8];
      float* d = dsh + slot * R - rb0;
      load_act_raw(a.act + (size_t)slot * a.K, lane, ngroups, hr);
      stream_rows<false>(a.wa + (size_t)e * a.st_wa, a.sa + (size_t)e * a.st_sa, nullptr,
                         nullptr, rb0, rlast, wrow, srow, lo, x0, x1, lane,
                         [&]() { act_to_f32(hr, lane, ngroups, x0, x1); },
                         [&](int r, float dv, float, bool valid, int) {
                           if (valid) d[r] = dv;
                         });
    }
  }
  __syncthreads();
  if (threadIdx.x < nr) {
    float acc = 0.0f;
    for (int j = 0; j < a.topk; ++j) {
      const int e = __builtin_amdgcn_readlane(my_idx, j);
      const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_gate), j));
      if (expert_ok(e, a.E)) acc = acc + g * dsh[j * R + threadIdx.x];
    }
    y[rb0 + threadIdx.x] = acc;
  }
}

// Workgroups per CU is a property of the kernel and the architecture, so one cached value
// serves every device; concurrent first calls store the same value.
int decode_w13_grid() {
  static std::atomic<int> per_cu{0};
  int n = per_cu.load(std::memory_order_relaxed);
  if (!n) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_w13<true>, kW13Threads, kW13LdsLimiter) !=
            hipSuccess ||
        n < 1)
      n = 1;
    per_cu.store(n, std::memory_order_relaxed);
  }
  return device_cu_count() * n;
}

}  // namespace

bool decode_exact_supported(const k3x_pool& p, int32_t T, int32_t topk) {
  return T == 1 && topk <= 64 && p.H / kGroup <= 128 && p.I / kGroup <= 128;
}

size_t decode_exact_ws(const k3x_pool& p, int32_t topk, size_t* off_h) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = up(16);
  *off_h = off;
  off = up(off + sizeof(uint16_t) * (size_t)topk * p.I);
  return off;
}

namespace {

// The two launches of the single-token decode; sel.scores set means the W1/W3 launch also
// selects the experts (a.idx then names where the picks go).
hipError_t launch_decode(const k3x_pool& p, const uint16_t* x, const int32_t* idx,
                         const float* gates, int32_t topk, float* y, uint8_t* ws,
                         const SelArgs& sel, hipStream_t s) {
  size_t off_h;
  decode_exact_ws(p, topk, &off_h);
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
  a.gact = p.act;
  a.b1 = p.b1;
  a.b2 = p.b2;
  hipError_t err = sel.scores ? launch("w13_decode", decode_w13<true>, dim3(decode_w13_grid()),
                                       dim3(kW13Threads), kW13LdsLimiter, s, a, sel)
                              : launch("w13_decode", decode_w13<false>, dim3(decode_w13_grid()),
                                       dim3(kW13Threads), kW13LdsLimiter, s, a, sel);
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
  b.out = nullptr;
  // one workgroup per compute unit, each owning a block of R output rows
  const int ncu = device_cu_count();
  const int R = std::min((p.H + ncu - 1) / ncu, kW2Waves * kWave);  // one thread per row
  const int nblk = (p.H + R - 1) / R;
  return launch("w2_combine_decode", decode_w2_combine, dim3(nblk), dim3(kW2Waves * kWave),
                (uint32_t)(sizeof(float) * topk * R), s, b, gates, y, R);
}

}  // namespace

hipError_t launch_decode_exact(const k3x_pool& p, const uint16_t* x, const int32_t* idx,
                               const float* gates, int32_t topk, float* y, uint8_t* ws,
                               hipStream_t s) {
  return launch_decode(p, x, idx, gates, topk, y, ws, SelArgs{}, s);
}

bool decode_routed_supported(const k3x_router_desc& r, const k3x_pool& p, int32_t T) {
  return decode_exact_supported(p, T, r.topk) && select_bitonic_supported(r.n_experts, r.topk);
}

hipError_t launch_decode_routed(const k3x_router_desc& r, const k3x_pool& p, const uint16_t* x,
                                float* scores, int32_t* idx, float* gates, float* y, uint8_t* ws,
                                hipStream_t s) {
  hipError_t err = launch_route_scores(r, x, 1, scores, s);
  if (err != hipSuccess) return err;
  const SelArgs sel{scores, r.bias, r.n_experts, r.renorm, r.routed_scale, idx, gates};
  return launch_decode(p, x, idx, gates, r.topk, y, ws, sel, s);
}

bool decode_routed_residual_supported(const k3x_router_desc& r, const k3x_pool& p, int32_t T) {
  return decode_routed_supported(r, p, T) && route_scores_residual_supported(r, T);
}

hipError_t launch_decode_routed_residual(const k3x_router_desc& r, const k3x_pool& p,
                                         const uint16_t* x, const float* y_prev, float eps,
                                         uint16_t* x_next, uint16_t* xn, float* scores,
                                         int32_t* idx, float* gates, float* y, uint8_t* ws,
                                         hipStream_t s) {
  hipError_t err = launch_route_scores_residual(r, x, y_prev, eps, x_next, xn, scores, s);
  if (err != hipSuccess) return err;
  const SelArgs sel{scores, r.bias, r.n_experts, r.renorm, r.routed_scale, idx, gates};
  return launch_decode(p, xn, idx, gates, r.topk, y, ws, sel, s);
}

}  // namespace k3x
