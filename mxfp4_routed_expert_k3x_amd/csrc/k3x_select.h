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
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = tid + kSelThreads * m;
    sc[m] = e < E ? s_t[e] : 0.0f;
    c[m] = e < E ? sc[m] + (bias ? bias[e] : 0.0f) : 0.0f;
    key[m] = score_key(c[m]);
  }

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


}  // namespace k3x
