// Routed-expert SwiGLU over MXFP4 weights (kimi-k3-in-c README, Part II section 4
// "Reduction one: the experts already ship at half a byte" for the weight format and the
// rule that nothing is dequantized to memory; section 9 "Picking 16 experts of 896" for the
// per-slot expert loop and the slot-order weighted combine).  The activation is SwiGLU with
// h rounded to bf16 before W2.
//
// Pipeline of one forward (all on the caller's stream):
//   1. moe_sort       slots (t, j) counted per expert, laid out expert by expert, and cut
//                     into tiles of at most `tile_tokens` slots of one expert
//   2. w13            per tile: g = W1 x, u = W3 x for 32 rows at a time, h = bf16(silu(g) u)
//   3. w2             per tile: d = W2 h for 64 rows at a time
//   4. combine        y[t] = sum_j gate[t][j] * d[t][j], slot order, invalid slots skipped
//
// The expert GEMMs run on bf16 MFMA (16x16x32, fp32 accumulate).  Packed weights stream from
// HBM straight into the MFMA A operand: each lane loads 16 bytes = 32 nibbles = one whole
// MX group of one row, and converts them with the gfx950 scaled FP4 -> bf16 conversion, the
// group's power-of-two scale folded in (exact).  Lane quarter q of a wave takes group
// 4 kb + q, so one 16-byte load per lane feeds four MFMAs that together cover 16 rows x 128
// K.  The activations (x or h) form the B operand; the MFMA's K order is a permutation shared
// by A and B, so the product is unchanged.
#include "k3x_internal.h"

namespace k3x {

MoeLayout moe_layout(int32_t E, int32_t H, int32_t I, int32_t T, int32_t topk) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  MoeLayout L{};
  const size_t slots = (size_t)T * topk;
  L.tile_tokens = 16;  // decode tiles: one 16-column MFMA block
  const size_t nonempty = slots < (size_t)E ? slots : (size_t)E;
  L.max_tiles = (int32_t)(nonempty + (slots + L.tile_tokens - 1) / L.tile_tokens + 1);
  size_t off = 0;
  L.drops = off;
  off = up(off + 16);
  L.offsets = off;
  off = up(off + sizeof(int32_t) * ((size_t)E + 1));
  L.tiles = off;
  off = up(off + sizeof(int32_t) * 4 * (size_t)L.max_tiles);
  L.perm = off;
  off = up(off + sizeof(int32_t) * (slots ? slots : 1));
  L.h = off;
  off = up(off + sizeof(uint16_t) * slots * (size_t)I);
  L.d = off;
  off = up(off + sizeof(float) * slots * (size_t)H);
  L.total = off;
  return L;
}

namespace {

// ---------------------------------------------------------------------------------------
// 1. Sort slots by expert (one workgroup; counting sort with LDS atomics).  Slot order
//    inside an expert is not fixed, and nothing downstream depends on it: every output
//    column of the MFMA is computed independently of the other columns.
// ---------------------------------------------------------------------------------------
constexpr int kSortThreads = 1024;

__global__ __launch_bounds__(kSortThreads) void moe_sort(const int32_t* __restrict__ idx,
                                                         int32_t n_slots, int32_t E,
                                                         int32_t tile_tokens,
                                                         uint8_t* __restrict__ ws,
                                                         size_t off_offsets, size_t off_tiles,
                                                         size_t off_perm) {
  extern __shared__ int32_t counts[];  // [E]
  __shared__ int32_t scan_c[kSortThreads];
  __shared__ int32_t scan_t[kSortThreads];
  __shared__ int32_t drop_cnt;
  const int tid = threadIdx.x;
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + off_offsets);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + off_tiles);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + off_perm);

  for (int e = tid; e < E; e += kSortThreads) counts[e] = 0;
  if (tid == 0) drop_cnt = 0;
  __syncthreads();
  for (int p = tid; p < n_slots; p += kSortThreads) {
    const int e = idx[p];
    if (e >= 0 && e < E)
      atomicAdd(&counts[e], 1);
    else
      atomicAdd(&drop_cnt, 1);
  }
  __syncthreads();

  const int per = (E + kSortThreads - 1) / kSortThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int csum = 0, tsum = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e];
    csum += c;
    tsum += (c + tile_tokens - 1) / tile_tokens;
  }
  scan_c[tid] = csum;
  scan_t[tid] = tsum;
  __syncthreads();
  for (int o = 1; o < kSortThreads; o <<= 1) {
    const int vc = tid >= o ? scan_c[tid - o] : 0;
    const int vt = tid >= o ? scan_t[tid - o] : 0;
    __syncthreads();
    scan_c[tid] += vc;
    scan_t[tid] += vt;
    __syncthreads();
  }
  int bc = scan_c[tid] - csum;
  int bt = scan_t[tid] - tsum;
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e];
    offsets[e] = bc;
    const int nt = (c + tile_tokens - 1) / tile_tokens;
    for (int i = 0; i < nt; ++i) {
      int4 tv;
      tv.x = e;
      tv.y = bc + i * tile_tokens;
      tv.z = min(tile_tokens, c - i * tile_tokens);
      tv.w = 0;
      reinterpret_cast<int4*>(tiles)[bt + i] = tv;
    }
    counts[e] = bc;  // becomes the scatter cursor
    bc += c;
    bt += nt;
  }
  if (tid == kSortThreads - 1) {
    offsets[E] = scan_c[kSortThreads - 1];
    *reinterpret_cast<int64_t*>(ws) = (int64_t)drop_cnt;
    *reinterpret_cast<int32_t*>(ws + 8) = scan_t[kSortThreads - 1];
  }
  __syncthreads();
  for (int p = tid; p < n_slots; p += kSortThreads) {
    const int e = idx[p];
    if (e >= 0 && e < E) perm[atomicAdd(&counts[e], 1)] = p;
  }
}

// ---------------------------------------------------------------------------------------
// Shared pieces of the expert GEMMs
// ---------------------------------------------------------------------------------------
struct GemmArgs {
  const uint8_t* wa;   // first weight tensor (W1 or W2) packed, expert 0
  const uint8_t* sa;   // its scales
  const uint8_t* wb;   // second weight tensor (W3) packed, or null
  const uint8_t* sb;   // its scales
  int64_t st_wa, st_sa, st_wb, st_sb;  // per-expert byte strides
  int32_t K;           // reduction length (H for W1/W3, I for W2)
  int32_t rows;        // output rows per expert (I for W1/W3, H for W2)
  const uint16_t* act; // B operand rows: x [T][H] (by token) or h [slots][I] (by slot)
  int32_t act_by_token;  // 1: row = slot / topk (x); 0: row = slot (h)
  int32_t topk;
  const uint8_t* ws;   // workspace: n_tiles at +8, tiles, perm
  size_t off_tiles, off_perm;
  void* out;           // h (bf16 [slots][I]) or d (fp32 [slots][H])
};

// Load one K block (128 K) of the A operand for one 16-row block: this lane's 16 packed
// bytes (group 4 kb + q of row `row`) and the group's scale as a float.
struct AFrag {
  uint4 q;
  float scale;
};

__device__ __forceinline__ AFrag load_a(const uint8_t* __restrict__ wrow,
                                        const uint8_t* __restrict__ srow, int grp) {
  AFrag f;
  f.q = *reinterpret_cast<const uint4*>(wrow + (size_t)grp * 16);
  f.scale = e8m0_to_f32(srow[grp]);
  return f;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------------------
// 2/3. Decode-sized grouped GEMM: tiles of at most 16 slots.  Work item = one wave, 4
// row blocks of 16 (W1/W3 mode: W1 rows r0..r0+31 and W3 rows r0..r0+31; W2 mode: W2 rows
// r0..r0+63), the full K.  The B operand comes straight from global memory (the tile's
// activation rows are few and cache-resident).  Items are split over the 8 dies in
// contiguous ranges and dealt to waves so that every workgroup gets a share.
// ---------------------------------------------------------------------------------------
template <bool kSwiGLU>
__global__ __launch_bounds__(256) void gemm_decode(GemmArgs a) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int n = lane % 16;  // B column / A row within a 16-row block
  const int q = lane / 16;  // lane quarter: which group of the K block
  const int32_t n_tiles = *reinterpret_cast<const int32_t*>(a.ws + 8);
  const int4* tiles = reinterpret_cast<const int4*>(a.ws + a.off_tiles);
  const int32_t* perm = reinterpret_cast<const int32_t*>(a.ws + a.off_perm);
  const int rows_per_item = kSwiGLU ? 32 : 64;
  const int items_per_tile = a.rows / rows_per_item;
  const int items = n_tiles * items_per_tile;

  int die, rank, per_die;
  xcd_rank(die, rank, per_die);
  const int chunk = (items + kNumXcd - 1) / kNumXcd;
  const int lo = die * chunk;
  const int hi = min(items, lo + chunk);
  const int wave_rank = wave * per_die + rank;
  const int waves_per_die = per_die * (blockDim.x / kWave);
  const int nk = a.K / kKBlock;
  const size_t wrow_bytes = (size_t)a.K / 2;
  const size_t srow_bytes = (size_t)a.K / kGroup;

  for (int it = lo + wave_rank; it < hi; it += waves_per_die) {
    const int tile = it / items_per_tile;
    const int r0 = (it % items_per_tile) * rows_per_item;
    const int4 tv = tiles[tile];
    const int e = tv.x, start = tv.y, m = tv.z;

    // B column n of this tile
    const bool valid = n < m;
    const int slot = valid ? perm[start + n] : 0;
    const int arow = a.act_by_token ? slot / a.topk : slot;
    const uint16_t* brow = a.act + (size_t)arow * a.K;

    // A rows of the 4 row blocks
    const uint8_t* wp[4];
    const uint8_t* sp[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      int row;
      const uint8_t *wbase, *sbase;
      if (kSwiGLU) {
        row = r0 + 16 * (rb & 1) + n;
        wbase = (rb < 2) ? a.wa + (size_t)e * a.st_wa : a.wb + (size_t)e * a.st_wb;
        sbase = (rb < 2) ? a.sa + (size_t)e * a.st_sa : a.sb + (size_t)e * a.st_sb;
      } else {
        row = r0 + 16 * rb + n;
        wbase = a.wa + (size_t)e * a.st_wa;
        sbase = a.sa + (size_t)e * a.st_sa;
      }
      wp[rb] = wbase + (size_t)row * wrow_bytes;
      sp[rb] = sbase + (size_t)row * srow_bytes;
    }

    f32x4 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    AFrag cur[4];
    uint4 xb[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) cur[rb] = load_a(wp[rb], sp[rb], q);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xb[s] = valid ? *reinterpret_cast<const uint4*>(brow + 32 * q + 8 * s) : make_uint4(0, 0, 0, 0);

    for (int kb = 0; kb < nk; ++kb) {
      AFrag nxt[4];
      uint4 xn[4];
      const bool more = kb + 1 < nk;
      if (more) {
        const int g = 4 * (kb + 1) + q;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) nxt[rb] = load_a(wp[rb], sp[rb], g);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xn[s] = valid ? *reinterpret_cast<const uint4*>(brow + 128 * (kb + 1) + 32 * q + 8 * s)
                        : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 b = as_bf16x8(xb[s]);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb] = mfma16x16x32(dequant8(dword_of(cur[rb].q, s), cur[rb].scale), b, acc[rb]);
      }
      if (more) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) cur[rb] = nxt[rb];
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[s] = xn[s];
      }
    }

    // epilogue: lane holds rows 4q..4q+3 of each row block, column n
    if (valid) {
      if (kSwiGLU) {
        uint16_t* h = static_cast<uint16_t*>(a.out);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          uint32_t packed[2];
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            uint32_t two = 0;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
              const float g = acc[rb][i + k2];
              const float u = acc[rb + 2][i + k2];
              const float v = (g / (1.0f + expf(-g))) * u;
              two |= f32_to_bf16_bits(v) << (16 * k2);
            }
            packed[i / 2] = two;
          }
          const int row = r0 + 16 * rb + 4 * q;
          *reinterpret_cast<uint2*>(h + (size_t)slot * a.rows + row) = make_uint2(packed[0], packed[1]);
        }
      } else {
        float* d = static_cast<float*>(a.out);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int row = r0 + 16 * rb + 4 * q;
          *reinterpret_cast<float4*>(d + (size_t)slot * a.rows + row) =
              make_float4(acc[rb][0], acc[rb][1], acc[rb][2], acc[rb][3]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// 4. Combine: y[t][r] = sum_j gates[t][j] * d[t*topk + j][r], slots in order, slots whose
// expert id is invalid skipped.  One thread per 4 consecutive rows.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_combine(const float* __restrict__ d,
                                                   const int32_t* __restrict__ idx,
                                                   const float* __restrict__ gates,
                                                   int32_t T, int32_t topk, int32_t H,
                                                   int32_t E, float* __restrict__ y) {
  const int per_tok = H / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * per_tok) return;
  const int t = (int)(i / per_tok);
  const int r = (int)(i % per_tok) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < topk; ++j) {
    const int e = idx[(size_t)t * topk + j];
    if (e < 0 || e >= E) continue;
    const float g = gates[(size_t)t * topk + j];
    const float4 v = *reinterpret_cast<const float4*>(d + ((size_t)t * topk + j) * H + r);
    acc.x = acc.x + g * v.x;
    acc.y = acc.y + g * v.y;
    acc.z = acc.z + g * v.z;
    acc.w = acc.w + g * v.w;
  }
  *reinterpret_cast<float4*>(y + (size_t)t * H + r) = acc;
}

}  // namespace

hipError_t launch_moe(const k3x_pool& p, const uint16_t* x, int32_t T, const int32_t* idx,
                      const float* gates, int32_t topk, float* y, uint8_t* ws,
                      const MoeLayout& L, hipStream_t s) {
  const int n_slots = T * topk;
  const size_t sort_lds = sizeof(int32_t) * (size_t)p.E;
  {
    LaunchTimer lt("moe_sort", s);
    hipLaunchKernelGGL(moe_sort, dim3(1), dim3(kSortThreads), sort_lds, s, idx, n_slots, p.E,
                       L.tile_tokens, ws, L.offsets, L.tiles, L.perm);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || T == 0) return err;

  const int grid = device_cu_count() * 2;  // two 4-wave workgroups per CU; multiple of 8

  GemmArgs a13{};
  a13.wa = p.base[0];
  a13.sa = p.base[1];
  a13.wb = p.base[2];
  a13.sb = p.base[3];
  a13.st_wa = p.stride[0];
  a13.st_sa = p.stride[1];
  a13.st_wb = p.stride[2];
  a13.st_sb = p.stride[3];
  a13.K = p.H;
  a13.rows = p.I;
  a13.act = x;
  a13.act_by_token = 1;
  a13.topk = topk;
  a13.ws = ws;
  a13.off_tiles = L.tiles;
  a13.off_perm = L.perm;
  a13.out = ws + L.h;
  {
    LaunchTimer lt("w13_decode", s);
    hipLaunchKernelGGL(gemm_decode<true>, dim3(grid), dim3(256), 0, s, a13);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;

  GemmArgs a2 = a13;
  a2.wa = p.base[4];
  a2.sa = p.base[5];
  a2.wb = nullptr;
  a2.sb = nullptr;
  a2.st_wa = p.stride[4];
  a2.st_sa = p.stride[5];
  a2.K = p.I;
  a2.rows = p.H;
  a2.act = reinterpret_cast<const uint16_t*>(ws + L.h);
  a2.act_by_token = 0;
  a2.out = ws + L.d;
  {
    LaunchTimer lt("w2_decode", s);
    hipLaunchKernelGGL(gemm_decode<false>, dim3(grid), dim3(256), 0, s, a2);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;

  const int64_t threads = (int64_t)T * (p.H / 4);
  {
    LaunchTimer lt("moe_combine", s);
    hipLaunchKernelGGL(moe_combine, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float*>(ws + L.d), idx, gates, T, topk, p.H, p.E,
                       y);
  }
  return hipGetLastError();
}

}  // namespace k3x
