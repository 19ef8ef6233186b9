// Prefill-sized grouped GEMMs of the routed experts (many slots per expert).
//
// Sources: kimi-k3-in-c README, Part II section 4 "Reduction one: the experts already ship at
// half a byte" (MXFP4 weights taken straight from the nibbles: E2M1 value times 2^(scale -
// 127), low nibble = even element, scale byte 255 zeroes its group; nothing dequantized is
// written to memory) and section 9 "Picking 16 experts of 896" (routed-expert loop, SwiGLU
// with h rounded to bf16 before W2, slot-order combine).
//
// Slots are sorted by expert into tiles of at most 128 slots of one expert.  A workgroup
// (4 waves) computes one tile against a chunk of output rows:
//   - W1/W3 mode: 128 rows of h (each wave 16 + 16 rows of W1 and the same 32 rows of W3),
//     epilogue h = bf16(silu(g) * u);
//   - W2 mode: 256 rows of d (each wave 64 rows of W2).
// The packed weights go from HBM straight into registers as the MFMA A operand: lane
// (n = lane % 16, q = lane / 16) loads 16 bytes = one whole MX group (group 4 kb + q of row
// n) and converts it with the gfx950 scaled FP4 -> bf16 instruction, the group's power-of-two
// scale folded in (exact).  One 16-byte load feeds four bf16 MFMAs (16x16x32) that together
// cover 16 rows x 128 K.  The tile's activations (x rows by token, or h rows by slot) are the
// B operand: each 128-wide K block of all the tile's rows is staged in LDS (double buffered,
// rows padded by 16 bytes so the 16 lanes of one read hit distinct banks) and every B
// fragment is used by the wave's four row blocks.  The MFMA's K order is a permutation
// shared by A and B, so the product is unchanged; accumulation is fp32.
//
// Work is persistent: tile t belongs to die t % 8 (all its row chunks), so the tile's
// activation rows are fetched into one die's L2 and reused by every chunk; within a die the
// workgroups take (tile, chunk) items in turn.
#include "k3x_internal.h"

namespace k3x {
namespace {

constexpr int kTT = 128;            // slots per tile
constexpr int kNB = kTT / 16;       // 16-column MFMA blocks per tile
constexpr int kLdsRow = kKBlock + 8;  // bf16 per staged activation row (256 + 16 bytes)

struct PrefillArgs {
  const uint8_t* wa;  // W1 (W1/W3 mode) or W2, packed, expert 0
  const uint8_t* sa;
  const uint8_t* wb;  // W3, W1/W3 mode only
  const uint8_t* sb;
  int64_t st_wa, st_sa, st_wb, st_sb;
  int32_t K;          // H (W1/W3) or I (W2)
  int32_t rows;       // I (W1/W3) or H (W2)
  const uint16_t* act;  // x [T][H] by token (W1/W3) or h [slots][I] by slot (W2)
  int32_t topk;
  const uint8_t* ws;  // n_tiles at +8, tiles, perm
  size_t off_tiles, off_perm;
  void* out;          // h bf16 [slots][I] or d fp32 [slots][H]
};

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

template <bool kW13>
__global__ __launch_bounds__(256, 2) void gemm_prefill(PrefillArgs a) {
  __shared__ __align__(16) uint16_t xs[2][kTT][kLdsRow];
  __shared__ int s_arow[kTT];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane % 16;
  const int q = lane / 16;

  const int n_tiles = *reinterpret_cast<const int32_t*>(a.ws + 8);
  const int4* tiles = reinterpret_cast<const int4*>(a.ws + a.off_tiles);
  const int32_t* perm = reinterpret_cast<const int32_t*>(a.ws + a.off_perm);
  const int chunk_rows = kW13 ? 128 : 256;
  const int chunks = a.rows / chunk_rows;
  const int nk = a.K / kKBlock;
  const uint32_t wrow = (uint32_t)a.K / 2, srow = (uint32_t)a.K / kGroup;

  int die, rank, per_die;
  xcd_rank(die, rank, per_die);
  const int my_tiles = n_tiles > die ? (n_tiles - die + kNumXcd - 1) / kNumXcd : 0;
  const int items = my_tiles * chunks;

  for (int it = rank; it < items; it += per_die) {
    const int tile = die + kNumXcd * (it / chunks);
    const int chunk = it % chunks;
    const int4 tv = tiles[tile];
    const int e = tv.x, start = tv.y, m = tv.z;
    const int nb = (m + 15) / 16;

    for (int i = tid; i < kTT; i += blockDim.x) {
      int r = -1;
      if (i < m) {
        const int slot = perm[start + i];
        r = kW13 ? slot / a.topk : slot;
      }
      s_arow[i] = r;
    }
    __syncthreads();

    // A operand rows of this lane in the wave's four row blocks
    const uint8_t *wlo, *whi, *slo, *shi;
    uint32_t woff[4], soff[4];
    if (kW13) {
      wlo = a.wa + (size_t)e * a.st_wa;
      slo = a.sa + (size_t)e * a.st_sa;
      whi = a.wb + (size_t)e * a.st_wb;
      shi = a.sb + (size_t)e * a.st_sb;
    } else {
      wlo = whi = a.wa + (size_t)e * a.st_wa;
      slo = shi = a.sa + (size_t)e * a.st_sa;
    }
    const int r0 = chunk * chunk_rows + wave * (chunk_rows / 4);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = kW13 ? r0 + 16 * (rb & 1) + n : r0 + 16 * rb + n;
      woff[rb] = (uint32_t)row * wrow + 16u * (uint32_t)q;
      soff[rb] = (uint32_t)row * srow;
    }
    auto load_a = [&](int kb, uint4 (&w)[4], uint32_t (&sc)[4]) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const uint8_t* wb = rb < 2 ? wlo : whi;
        const uint8_t* sb = rb < 2 ? slo : shi;
        w[rb] = *reinterpret_cast<const uint4*>(wb + woff[rb] + 64u * (uint32_t)kb);
        sc[rb] = *reinterpret_cast<const uint32_t*>(sb + soff[rb] + 4u * (uint32_t)kb);
      }
    };
    // staging of one K block of the tile's activation rows: thread owns 16-byte chunk
    // (tid % 16) of rows tid / 16 + 16 p
    uint4 xr[kTT / 16];
    auto load_x = [&](int kb) {
#pragma unroll
      for (int p = 0; p < kTT / 16; ++p) {
        const int i = tid / 16 + 16 * p;
        const int r = s_arow[i];
        if (r >= 0)
          xr[p] = *reinterpret_cast<const uint4*>(a.act + (size_t)r * a.K + kKBlock * kb + 8 * (tid % 16));
      }
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int p = 0; p < kTT / 16; ++p) {
        const int i = tid / 16 + 16 * p;
        if (i < m) *reinterpret_cast<uint4*>(&xs[buf][i][8 * (tid % 16)]) = xr[p];
      }
    };

    f32x4 acc[4][kNB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int tb = 0; tb < kNB; ++tb) acc[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 wcur[4], wnxt[4];
    uint32_t scur[4], snxt[4];
    load_a(0, wcur, scur);
    load_x(0);
    store_x(0);
    __syncthreads();

    for (int kb = 0; kb < nk; ++kb) {
      const int buf = kb & 1;
      const bool more = kb + 1 < nk;
      if (more) {
        load_a(kb + 1, wnxt, snxt);
        load_x(kb + 1);
      }
      float scale[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) scale[rb] = e8m0_to_f32((scur[rb] >> (8 * q)) & 0xFFu);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 av[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) av[rb] = dequant8(dword_of(wcur[rb], s), scale[rb]);
#pragma unroll
        for (int tb = 0; tb < kNB; ++tb) {
          if (tb < nb) {
            const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(&xs[buf][16 * tb + n][32 * q + 8 * s]));
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) acc[rb][tb] = mfma16x16x32(av[rb], b, acc[rb][tb]);
          }
        }
      }
      if (more) {
        store_x(buf ^ 1);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          wcur[rb] = wnxt[rb];
          scur[rb] = snxt[rb];
        }
      }
      __syncthreads();
    }

    // epilogue: lane holds rows 4q..4q+3 of each row block for column 16 tb + n
#pragma unroll
    for (int tb = 0; tb < kNB; ++tb) {
      const int col = 16 * tb + n;
      if (tb < nb && col < m) {
        const int slot = perm[start + col];
        if (kW13) {
          uint16_t* h = static_cast<uint16_t*>(a.out);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            uint32_t hv[2];
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              uint32_t two = 0;
#pragma unroll
              for (int k2 = 0; k2 < 2; ++k2) {
                const float g = acc[rb][tb][i + k2];
                const float u = acc[rb + 2][tb][i + k2];
                const float ex = (float)exp(-(double)g);
                two |= f32_to_bf16_bits((g / (1.0f + ex)) * u) << (16 * k2);
              }
              hv[i / 2] = two;
            }
            const int row = r0 + 16 * rb + 4 * q;
            *reinterpret_cast<uint2*>(h + (size_t)slot * a.rows + row) = make_uint2(hv[0], hv[1]);
          }
        } else {
          float* d = static_cast<float*>(a.out);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int row = r0 + 16 * rb + 4 * q;
            *reinterpret_cast<float4*>(d + (size_t)slot * a.rows + row) =
                make_float4(acc[rb][tb][0], acc[rb][tb][1], acc[rb][tb][2], acc[rb][tb][3]);
          }
        }
      }
    }
    __syncthreads();  // s_arow and xs are rewritten by the next item
  }
}

int prefill_grid(const void* fn) {
  static int cached[2] = {0, 0};
  const int which = fn == reinterpret_cast<const void*>(&gemm_prefill<true>) ? 0 : 1;
  if (!cached[which]) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    cached[which] = per_cu;
  }
  return device_cu_count() * cached[which];
}

}  // namespace

int prefill_tile_tokens() { return kTT; }

hipError_t launch_prefill_gemms(const k3x_pool& p, const uint16_t* x, int32_t topk,
                                uint8_t* ws, const MoeLayout& L, hipStream_t s) {
  PrefillArgs a{};
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
  a.topk = topk;
  a.ws = ws;
  a.off_tiles = L.tiles;
  a.off_perm = L.perm;
  a.out = ws + L.h;
  hipError_t err = launch("w13_prefill", gemm_prefill<true>,
                          dim3(prefill_grid(reinterpret_cast<const void*>(&gemm_prefill<true>))),
                          dim3(256), 0, s, a);
  if (err != hipSuccess) return err;
  PrefillArgs b = a;
  b.wa = p.base[4];
  b.sa = p.base[5];
  b.wb = nullptr;
  b.sb = nullptr;
  b.st_wa = p.stride[4];
  b.st_sa = p.stride[5];
  b.K = p.I;
  b.rows = p.H;
  b.act = reinterpret_cast<const uint16_t*>(ws + L.h);
  b.out = ws + L.d;
  return launch("w2_prefill", gemm_prefill<false>,
                dim3(prefill_grid(reinterpret_cast<const void*>(&gemm_prefill<false>))),
                dim3(256), 0, s, b);
}

}  // namespace k3x
