// Top-k selection of the sigmoid + correction-bias router (kimi-k3-in-c README, Part II
// section 9 "Picking 16 experts of 896") as a device function of one 256-thread workgroup,
// run once per token by the router's selection kernel.
#pragma once

#include "k3x_internal.h"

namespace k3x {

// (c, index) total order: true when candidate b beats a.  Index -1 means "no candidate".
__device__ __forceinline__ bool beats(float cb, int ib, float ca, int ia) {
  if (ib < 0) return false;
  if (ia < 0) return true;
  return cb > ca || (cb == ca && ib < ia);
}

// Order-preserving 32-bit key of a selection score: a larger float gives a larger key, and
// -0 is first made +0 so that the two compare equal, as in an IEEE compare.
__device__ __forceinline__ uint32_t score_key(float c) {
  const uint32_t b = c == 0.0f ? 0u : __float_as_uint(c);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
// Thread t clears histogram bin t (one thread per 8-bit digit value), so the workgroup has
// exactly as many threads as bins.
static_assert(kSelThreads == 256, "one thread per histogram bin");

// Wave-wide scans with DPP row shifts inside each row of 16 lanes and lane reads across
// rows (no LDS round trips).
// DPP controls: row_shr:n = 0x110 + n, row_ror:n = 0x120 + n.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {  // 0 where the row has no source
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Inclusive prefix sum over the lanes of the wave, in lane order.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v, int lane) {
  v += dpp0<0x111>(v);
  v += dpp0<0x112>(v);
  v += dpp0<0x114>(v);
  v += dpp0<0x118>(v);
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

// AND and OR over the wave, the same on every lane.
__device__ __forceinline__ void wave_and_or(uint32_t& a, uint32_t& o) {
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x128, 0xF, 0xF, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x128, 0xF, 0xF, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x124, 0xF, 0xF, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x124, 0xF, 0xF, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x122, 0xF, 0xF, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x122, 0xF, 0xF, false);
  a &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x121, 0xF, 0xF, false);
  o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x121, 0xF, 0xF, false);
  const uint32_t a_all = (uint32_t)__builtin_amdgcn_readlane((int)a, 0) &
                         (uint32_t)__builtin_amdgcn_readlane((int)a, 16) &
                         (uint32_t)__builtin_amdgcn_readlane((int)a, 32) &
                         (uint32_t)__builtin_amdgcn_readlane((int)a, 48);
  const uint32_t o_all = (uint32_t)__builtin_amdgcn_readlane((int)o, 0) |
                         (uint32_t)__builtin_amdgcn_readlane((int)o, 16) |
                         (uint32_t)__builtin_amdgcn_readlane((int)o, 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)o, 48);
  a = a_all;
  o = o_all;
}

// Thread tid's experts e = tid + 256 m (m < M): the unbiased score sc, the selection score
// c = sc + bias (zero past E) and whether e < E.  Every load is issued before any is used
// (indices past E read expert E - 1), so the workgroup waits for memory once.
template <int M>
__device__ __forceinline__ void load_scores(const float* __restrict__ s_t,
                                            const float* __restrict__ bias, int32_t E,
                                            float (&sc)[M], float (&c)[M], bool (&ok)[M]) {
  const int tid = threadIdx.x;
  float sv[M], bv[M];
#pragma unroll
  for (int m = 0; m < M; ++m) sv[m] = s_t[min(tid + kSelThreads * m, E - 1)];
#pragma unroll
  for (int m = 0; m < M; ++m) bv[m] = bias ? bias[min(tid + kSelThreads * m, E - 1)] : 0.0f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    ok[m] = tid + kSelThreads * m < E;
    sc[m] = ok[m] ? sv[m] : 0.0f;
    c[m] = ok[m] ? sc[m] + bv[m] : 0.0f;
  }
}

// One workgroup of 256 threads per token; thread i owns experts i + 256 m (m < M).
//  1. The key of the topk-th largest selection score is found by a radix select over 8-bit
//     digits, each pass building a 256-bin LDS histogram of the keys that match the digits
//     fixed so far and walking it from the top.  The leading digits every key shares (scores
//     of one binade share their top byte) are taken as they are, without a pass; the
//     histograms alternate between two buffers, so a pass needs two barriers.
//  2. The chosen set is every expert whose key is larger, plus, among the experts whose key
//     equals it, the ones of lowest index until topk are taken -- exactly the experts the
//     repeated argmax (larger score first, lower index on ties) would pick.  Each wave's
//     ballots give every key its place among the larger ones, or its index rank among the
//     equal ones, so the chosen experts are packed without atomics.
//  3. Each chosen expert's slot is its rank in that total order; the gates are the unbiased
//     scores in slot order, renormalised by their float sum (added in slot order).
template <int M>
__device__ __forceinline__ void select_topk(const float* __restrict__ s_t,
                                            const float* __restrict__ bias, int32_t E,
                                            int32_t topk, int32_t renorm, float rscale,
                                            float* dyn, int32_t* idx_out, float* gates_out) {
  // dyn: LDS [topk] c, [topk] s, [topk] e (as int), [topk] ranked s
  float* sel_c = dyn;
  float* sel_s = dyn + topk;
  int* sel_e = reinterpret_cast<int*>(dyn + 2 * topk);
  float* ranked = dyn + 3 * topk;
  __shared__ uint32_t hist[2][256];
  __shared__ uint32_t s_and[kSelWaves], s_or[kSelWaves];
  __shared__ uint32_t s_prefix, s_rem;
  __shared__ uint32_t s_cnt[2][M * kSelWaves];  // larger / equal keys per (m, wave), then
                                                // their exclusive prefix sums
  __shared__ uint32_t s_ngt;
  __shared__ float s_sum;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;

  float sc[M], c[M];
  uint32_t key[M];
  bool ok[M];
  load_scores<M>(s_t, bias, E, sc, c, ok);
#pragma unroll
  for (int m = 0; m < M; ++m) key[m] = score_key(c[m]);

  // bits every key shares: their AND equals their OR there
  uint32_t kand = ~0u, kor = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (tid + kSelThreads * m < E) {
      kand &= key[m];
      kor |= key[m];
    }
  wave_and_or(kand, kor);
  if (lane == 0) {
    s_and[wv] = kand;
    s_or[wv] = kor;
  }
  hist[0][tid] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    kand &= s_and[w];
    kor |= s_or[w];
  }
  const uint32_t diff = kand ^ kor;
  // the first digit that differs (none: every key equal, no pass)
  const int top = diff ? (31 - __clz(diff)) / 8 * 8 : -8;
  uint32_t mask = top >= 24 ? 0u : ~0u << (top + 8);
  uint32_t prefix = kand & mask, rem = (uint32_t)topk;
  int buf = 0;
  for (int shift = top; shift >= 0; shift -= 8, buf ^= 1) {
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (tid + kSelThreads * m < E && (key[m] & mask) == prefix)
        atomicAdd(&hist[buf][(key[m] >> shift) & 255u], 1u);
    __syncthreads();
    hist[buf ^ 1][tid] = 0;  // the next pass's buffer, last read before the barrier above
    if (tid < kWave) {
      // lane l sums bins 255-4l .. 252-4l (descending); an inclusive scan over lanes gives
      // the number of keys in all bins from 255 down to the lane's lowest bin
      uint32_t hb[4], local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = hist[buf][255 - 4 * tid - i];
        local += hb[i];
      }
      const uint32_t incl = wave_incl_sum(local, tid);
      const uint32_t excl = incl - local;
      if (excl < rem && rem <= incl) {  // exactly one lane
        uint32_t above = excl;
        int bin = 255 - 4 * tid - 3;
        uint32_t left = rem - above;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (above < rem && rem <= above + hb[i]) {
            bin = 255 - 4 * tid - i;
            left = rem - above;
            break;
          }
          above += hb[i];
        }
        s_prefix = prefix | ((uint32_t)bin << shift);
        s_rem = left;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    rem = s_rem;
    mask |= 255u << shift;
  }

  // prefix is now the key of the topk-th expert; rem of the experts with that key are
  // taken, those of lowest index.  Per (m, wave): how many keys are larger, how many equal.
  const uint64_t below_me = (1ull << lane) - 1ull;
  uint64_t bgt[M], beq[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool ok = tid + kSelThreads * m < E;
    bgt[m] = __ballot(ok && key[m] > prefix);
    beq[m] = __ballot(ok && key[m] == prefix);
  }
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      s_cnt[0][m * kSelWaves + wv] = (uint32_t)__popcll(bgt[m]);
      s_cnt[1][m * kSelWaves + wv] = (uint32_t)__popcll(beq[m]);
    }
  }
  __syncthreads();
  if (tid < kWave) {  // exclusive prefix sums in index order (m, then wave)
    static_assert(M * kSelWaves <= kWave, "one lane per (m, wave)");
    const bool in = tid < M * kSelWaves;
    const uint32_t g0 = in ? s_cnt[0][tid] : 0u, q0 = in ? s_cnt[1][tid] : 0u;
    const uint32_t g = wave_incl_sum(g0, tid), q = wave_incl_sum(q0, tid);
    if (in) {
      s_cnt[0][tid] = g - g0;
      s_cnt[1][tid] = q - q0;
    }
    if (tid == kWave - 1) s_ngt = g;  // every larger key
  }
  __syncthreads();
  const uint32_t ngt = s_ngt;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    int pos = -1;
    if ((bgt[m] >> lane) & 1ull)
      pos = (int)(s_cnt[0][m * kSelWaves + wv] + (uint32_t)__popcll(bgt[m] & below_me));
    if ((beq[m] >> lane) & 1ull) {
      const uint32_t eb = s_cnt[1][m * kSelWaves + wv] + (uint32_t)__popcll(beq[m] & below_me);
      if (eb < rem) pos = (int)(ngt + eb);
    }
    if (pos >= 0) {
      sel_c[pos] = c[m];
      sel_s[pos] = sc[m];
      sel_e[pos] = tid + kSelThreads * m;
    }
  }
  __syncthreads();
  if (topk <= kWave) {
    // one wave, one pick per lane: ranks and the slot-order sum read the other picks with
    // lane reads instead of a loop over LDS
    if (tid < kWave) {
      const bool mine = tid < topk;
      const float ci = mine ? sel_c[tid] : 0.0f;
      const int ei = mine ? sel_e[tid] : -1;
      const float si = mine ? sel_s[tid] : 0.0f;
      int r = 0;
      for (int j = 0; j < topk; ++j) {
        const float cj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ci), j));
        const int ej = __builtin_amdgcn_readlane(ei, j);
        r += beats(cj, ej, ci, ei) ? 1 : 0;
      }
      if (mine) {
        idx_out[r] = ei;
        ranked[r] = si;
      }
      __builtin_amdgcn_wave_barrier();
      const float rs = mine ? ranked[tid] : 0.0f;
      float sum = 0.0f;
      if (renorm)
        for (int j = 0; j < topk; ++j)
          sum = sum + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), j));
      if (mine) {
        float w = rs;
        if (renorm && sum > 0.0f) w = w / sum;
        gates_out[tid] = w * rscale;
      }
    }
    return;
  }
  // slot of each chosen expert = its rank under (larger c, then lower index)
  for (int i = tid; i < topk; i += kSelThreads) {
    const float ci = sel_c[i];
    const int ei = sel_e[i];
    int r = 0;
    for (int j = 0; j < topk; ++j) r += beats(sel_c[j], sel_e[j], ci, ei) ? 1 : 0;
    idx_out[r] = ei;
    ranked[r] = sel_s[i];
  }
  __syncthreads();
  if (tid == 0) {
    float sum = 0.0f;
    if (renorm)
      for (int j = 0; j < topk; ++j) sum = sum + ranked[j];
    s_sum = sum;
  }
  __syncthreads();
  const float sum = s_sum;
  for (int j = tid; j < topk; j += kSelThreads) {
    float w = ranked[j];
    if (renorm && sum > 0.0f) w = w / sum;
    gates_out[j] = w * rscale;
  }
}

// ---------------------------------------------------------------------------------------
// The same selection for topk <= 16 and E <= 1024 as sorting networks over registers, with
// no histogram, atomic or scalar round trip on the way.  Each expert is one 64-bit word:
// its selection key above, the complement of its index below (0 when absent), so the words
// order exactly as the picks do (larger selection score first, lower index on ties).
//  1. Thread tid holds experts tid + 256 m (m < 4); every four lanes (a quad) hold 16 words
//     and sort them with a bitonic network (element r + 4 (lane & 3) is register r of that
//     lane; partners one or two elements away sit in the same lane, four or eight away in
//     the neighbouring lanes of the quad).  Quads sort in alternating directions.
//  2. Two sorted lists of 16 in opposite directions give the 16 largest of their union as
//     the element-wise larger of the two (a bitonic sequence), sorted by a clean-up network.
//     Four such rounds, the partner quad 1, 2, 4, 8 quads away and each round's result in the
//     direction its next partner needs, leave the wave's 16 largest in every quad.
//  3. Wave 0 merges the four waves' lists the same way (every other list read reversed); its
//     first topk elements are the picks in slot order.  The gates follow from the unbiased
//     scores as above.
// Steps 1-3 are the fallback.  First the workgroup narrows the field: the 16th largest of the
// 64 quad maxima is a lower bound of the 16th largest word (16 quads hold a word at least that
// large), so every pick is among the words at or above it — about 18 of 896 router scores.
// If at most 64 words qualify, wave 0 sorts just those (one word per lane, a bitonic network
// over the lanes of half the wave when at most 32 do); otherwise the networks above run.
// ---------------------------------------------------------------------------------------
namespace bitonic {

__device__ __forceinline__ uint64_t join(uint32_t lo, uint32_t hi) {
  return ((uint64_t)hi << 32) | lo;
}

// Word of lane ^ X by DPP: X < 4 within the quad (quad_perm), X = 4 or 8 within the row of 16.
template <int X>
__device__ __forceinline__ uint32_t dpp_xor32(uint32_t v) {
  if constexpr (X == 1 || X == 2 || X == 3) {
    constexpr int ctrl = X == 1 ? 0xB1 : X == 2 ? 0x4E : 0x1B;  // [1032] [2301] [3210]
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
  } else if constexpr (X == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else {
    static_assert(X == 4, "lane distance");
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x104, 0xF, 0xF, false);  // row_shl:4
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    return (threadIdx.x & 4) ? dn : up;
  }
}

template <int X>
__device__ __forceinline__ uint64_t lane_xor(uint64_t v) {
  if constexpr (X <= 8) {
    return join(dpp_xor32<X>((uint32_t)v), dpp_xor32<X>((uint32_t)(v >> 32)));
  } else {  // across rows: through the LDS crossbar (no LDS memory is used)
    const int src = ((int)(threadIdx.x % kWave) ^ X) * 4;
    return join((uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)v),
                (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(v >> 32)));
  }
}

// One compare-exchange stage at element distance J within blocks of K; a block descends when
// element i + 16 flip has bit K clear (K = 32: the whole list descends unless flip).  One
// compare per pair: equal words are only absent ones (0), for which either order is right.
template <int K, int J>
__device__ __forceinline__ void stage(uint64_t (&v)[4], int q, int flip) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = r + 4 * q;
    const bool desc = K >= 32 ? !flip : ((i + 16 * flip) & K) == 0;
    if constexpr (J < 4) {  // partners in the same lane: registers r and r + J
      if (r & J) continue;
      const uint64_t a = v[r], b = v[r + J];
      const bool swap = (a < b) == desc;  // descending wants a >= b, ascending a <= b
      v[r] = swap ? b : a;
      v[r + J] = swap ? a : b;
    } else {  // partners in lane ^ (J / 4), the same register
      const bool want_hi = ((i & J) == 0) == desc;
      const uint64_t o = lane_xor<J / 4>(v[r]);
      v[r] = ((v[r] < o) == want_hi) ? o : v[r];
    }
  }
}

// Sorts the quad's 16 words, largest first (smallest first when flip).
__device__ __forceinline__ void sort16(uint64_t (&v)[4], int q, int flip) {
  stage<2, 1>(v, q, flip);
  stage<4, 2>(v, q, flip);
  stage<4, 1>(v, q, flip);
  stage<8, 4>(v, q, flip);
  stage<8, 2>(v, q, flip);
  stage<8, 1>(v, q, flip);
  stage<16, 8>(v, q, flip);
  stage<16, 4>(v, q, flip);
  stage<16, 2>(v, q, flip);
  stage<16, 1>(v, q, flip);
}

// The 16 largest of this quad's list and that of the quad DQ quads away (sorted in opposite
// directions), sorted ascending when flip, in both quads.
template <int DQ>
__device__ __forceinline__ void merge16(uint64_t (&v)[4], int q, int flip) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t o = lane_xor<4 * DQ>(v[r]);
    v[r] = v[r] < o ? o : v[r];
  }
  stage<32, 8>(v, q, flip);
  stage<32, 4>(v, q, flip);
  stage<32, 2>(v, q, flip);
  stage<32, 1>(v, q, flip);
}

// One compare-exchange stage over the lanes of the wave (one word per lane), blocks of K
// lanes descending when bit K of the lane is clear (the whole wave descends at K = 64).
template <int K, int J>
__device__ __forceinline__ uint64_t lane_stage(uint64_t x, int lane) {
  const bool desc = K >= kWave ? true : (lane & K) == 0;
  const bool want_hi = ((lane & J) == 0) == desc;
  const uint64_t o = lane_xor<J>(x);
  return ((x < o) == want_hi) ? o : x;
}

// The words of lanes 0..31, largest first by lane (lanes 32..63 likewise among themselves).
__device__ __forceinline__ uint64_t sort32(uint64_t x, int lane) {
  x = lane_stage<2, 1>(x, lane);
  x = lane_stage<4, 2>(x, lane);
  x = lane_stage<4, 1>(x, lane);
  x = lane_stage<8, 4>(x, lane);
  x = lane_stage<8, 2>(x, lane);
  x = lane_stage<8, 1>(x, lane);
  x = lane_stage<16, 8>(x, lane);
  x = lane_stage<16, 4>(x, lane);
  x = lane_stage<16, 2>(x, lane);
  x = lane_stage<16, 1>(x, lane);
  x = lane_stage<32, 16>(x, lane);
  x = lane_stage<32, 8>(x, lane);
  x = lane_stage<32, 4>(x, lane);
  x = lane_stage<32, 2>(x, lane);
  x = lane_stage<32, 1>(x, lane);
  return x;
}

// The wave's 64 words, largest first by lane.
__device__ __forceinline__ uint64_t sort64(uint64_t x, int lane) {
  x = sort32(x, lane);
  x = lane_stage<64, 32>(x, lane);
  x = lane_stage<64, 16>(x, lane);
  x = lane_stage<64, 8>(x, lane);
  x = lane_stage<64, 4>(x, lane);
  x = lane_stage<64, 2>(x, lane);
  x = lane_stage<64, 1>(x, lane);
  return x;
}

__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a < b ? b : a; }

}  // namespace bitonic

__host__ __device__ inline bool select_bitonic_supported(int32_t E, int32_t topk) {
  return E >= 1 && E <= 4 * kSelThreads && topk >= 1 && topk <= 16;
}

// One 256-thread workgroup, topk <= 16, E <= 1024.  idx_out and gates_out may be global or
// LDS addresses; every thread of the workgroup must call it.
__device__ __forceinline__ void select_topk_bitonic(const float* __restrict__ s_t,
                                                    const float* __restrict__ bias, int32_t E,
                                                    int32_t topk, int32_t renorm, float rscale,
                                                    int32_t* idx_out, float* gates_out) {
  using namespace bitonic;
  __shared__ float sc_of[4 * kSelThreads];       // unbiased score by expert
  __shared__ uint64_t best[kSelWaves][16];        // each wave's 16 largest words, descending
  __shared__ uint64_t qmax[kSelThreads / 4];      // the quads' largest words
  __shared__ uint64_t cand[kSelWaves][kWave];     // each wave's words at or above the bound
  __shared__ uint32_t ncand[kSelWaves];           // and their number
  __shared__ uint64_t top16[16];                  // the picks' words in slot order
  __shared__ float ranked[16];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave, q = lane & 3;
  const int quad = lane >> 2;

  float sc[4], c[4];
  bool ok[4];
  load_scores<4>(s_t, bias, E, sc, c, ok);
  uint64_t v[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = tid + kSelThreads * m;
    if (ok[m]) sc_of[e] = sc[m];
    v[m] = ok[m] ? join(~(uint32_t)e, score_key(c[m])) : 0ull;
  }
  // the quad's largest word
  uint64_t mx = max64(max64(v[0], v[1]), max64(v[2], v[3]));
  mx = max64(mx, lane_xor<1>(mx));
  mx = max64(mx, lane_xor<2>(mx));
  if (q == 0) qmax[wv * 16 + quad] = mx;
  __syncthreads();
  // the bound: the 16th largest quad maximum (every wave sorts the 64 of them itself)
  const uint64_t sm = sort64(qmax[lane], lane);
  const uint64_t bound = join((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sm, 15),
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(sm >> 32), 15));
  // the words at or above it (none of them absent unless the bound is 0): each wave packs
  // its own into cand[wave] in register-then-lane order
  uint32_t base = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const unsigned long long bal = __ballot(v[m] >= bound);
    const uint32_t off = base + (uint32_t)__builtin_amdgcn_mbcnt_hi(
                                    (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (v[m] >= bound && off < (uint32_t)kWave) cand[wv][off] = v[m];
    base += (uint32_t)__popcll(bal);
  }
  if (lane == 0) ncand[wv] = base;
  __syncthreads();
  const uint32_t n0 = ncand[0], n1 = n0 + ncand[1], n2 = n1 + ncand[2], n = n2 + ncand[3];
  if (n <= (uint32_t)kWave) {
    if (wv != 0) return;
    // lane l takes the l-th word of the four lists one after another
    const uint32_t l = (uint32_t)lane;
    const int src = (l >= n0) + (l >= n1) + (l >= n2);
    const uint32_t at = l - (src == 0 ? 0u : src == 1 ? n0 : src == 2 ? n1 : n2);
    const uint64_t x = l < n ? cand[src][at] : 0ull;
    const uint64_t t = n <= 32 ? sort32(x, lane) : sort64(x, lane);
    if (lane < 16) top16[lane] = t;
  } else {
    // too many words at the bound (ties, or quads with no expert): the full networks
    // a quad's list runs in the direction its next partner needs: bit l of the quad index
    // before the round with partner 2^l quads away
    sort16(v, q, quad & 1);
    merge16<1>(v, q, (quad >> 1) & 1);
    merge16<2>(v, q, (quad >> 2) & 1);
    merge16<4>(v, q, (quad >> 3) & 1);
    merge16<8>(v, q, 0);
    if (lane < 4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) best[wv][r + 4 * q] = v[r];
    }
    __syncthreads();
    if (wv != 0) return;
    // quads 0..3 take the lists of waves 0..3, odd ones reversed (ascending); other quads empty
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r + 4 * q;
      v[r] = quad < kSelWaves ? best[quad][(quad & 1) ? 15 - i : i] : 0ull;
    }
    merge16<1>(v, q, (quad >> 1) & 1);
    merge16<2>(v, q, 0);
    // slot i = element i of quad 0: lane i / 4, register i % 4
    if (lane < 4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) top16[r + 4 * q] = v[r];
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < topk) {
    const int e = (int)~(uint32_t)top16[lane];
    idx_out[lane] = e;
    ranked[lane] = sc_of[e];
  }
  __builtin_amdgcn_wave_barrier();
  // every lane forms the slot-order sum from its own copy of the picks' scores (one LDS read
  // of all sixteen, then the additions in order)
  float rk[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) rk[j] = ranked[j];  // entries past topk are not used
  float sum = 0.0f;
  if (renorm) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < topk) sum = sum + rk[j];
  }
  if (lane < topk) {
    float w = ranked[lane];
    if (renorm && sum > 0.0f) w = w / sum;
    gates_out[lane] = w * rscale;
  }
}

}  // namespace k3x
