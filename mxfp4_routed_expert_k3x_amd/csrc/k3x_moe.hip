// Routed-expert SwiGLU over MXFP4 weights (kimi-k3-in-c README, Part II section 4
// "Reduction one: the experts already ship at half a byte" for the weight format and the
// rule that nothing is dequantized to memory; section 9 "Picking 16 experts of 896" for the
// per-slot expert loop and the slot-order weighted combine).  The activation is SwiGLU with
// h rounded to bf16 before W2.
//
// Pipeline of one forward (all on the caller's stream):
//   1. moe_sort   (T > 1 only) slots (t, j) counted per expert, laid out expert by expert,
//                 cut into tiles of one expert; counts drops.  Batches of 8192 slots or more
//                 take the split sort (count per slice, one scan, scatter per slice).
//   2. w13        per tile and 32 rows: g = W1 x, u = W3 x, h = bf16(silu(g) * u)
//   3. w2         per tile and 64 rows: d = W2 h
//   4. combine    y[t] = sum_j gate[t][j] * d[t][j] in slot order, invalid slots skipped
//
// The expert GEMMs run on bf16 MFMA (16x16x32, fp32 accumulate).  Packed weights stream from
// HBM straight into the MFMA A operand: each lane loads 16 bytes = 32 nibbles = one whole
// MX group of one row, and converts them with the gfx950 scaled FP4 -> bf16 conversion, the
// group's power-of-two scale folded in (exact).  Lane quarter q of a wave takes group
// 4 kb + q, so one 16-byte load per lane feeds four MFMAs that together cover 16 rows x 128
// K.  The activations (x or h) form the B operand; the MFMA's K order is a permutation shared
// by A and B, so the product is unchanged.  The four waves of a workgroup split K in four
// contiguous ranges and their partial sums are added in a fixed order, (p0 + p1) + (p2 + p3),
// which keeps every serial fp32 chain short.
#include "k3x_internal.h"

namespace k3x {

// Large batches sort in three launches over kSortParts slices of the slots (count per slice,
// one scan, scatter per slice); smaller ones in one workgroup.
constexpr int kSortParts = 64;
constexpr int kSortSplitMin = 8192;

MoeLayout moe_layout(int32_t E, int32_t H, int32_t I, int32_t T, int32_t topk) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  MoeLayout L{};
  const size_t slots = (size_t)T * topk;
  // decode-sized batches: tiles of one 16-column MFMA block; prefill: tiles of 128 slots
  L.tile_tokens = use_prefill(E, H, I, T, topk) ? prefill_tile_tokens() : 16;
  const size_t nonempty = slots < (size_t)E ? slots : (size_t)E;
  L.max_tiles = (int32_t)(nonempty + (slots + L.tile_tokens - 1) / L.tile_tokens + 1);
  size_t off = 0;
  L.drops = off;
  off = up(off + 64);  // drop count, tile count, the tile classes' ends
  L.offsets = off;
  off = up(off + sizeof(int32_t) * ((size_t)E + 1));
  L.tiles = off;
  off = up(off + sizeof(int32_t) * 4 * (size_t)L.max_tiles);
  L.perm = off;
  off = up(off + sizeof(int32_t) * (slots ? slots : 1));
  L.inv = off;
  off = up(off + sizeof(int32_t) * (slots ? slots : 1));
  L.h = off;
  off = up(off + sizeof(uint16_t) * slots * (size_t)I);
  L.d = off;
  off = up(off + sizeof(float) * slots * (size_t)H);
  L.sort_n = slots >= (size_t)kSortSplitMin ? kSortParts : 0;
  L.sort_parts = off;
  off = up(off + sizeof(int32_t) * (size_t)L.sort_n * ((size_t)E + 1));
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

// Tiles are written class by class: class k holds the tiles of 16 k + 1 .. 16 k + 16 slots
// (the number of 16-column MFMA blocks they need, minus one), each class in expert order.  The
// header of the workspace gives the tile count at byte 8 and, from byte 12, the end of each
// class in the tile array (kTileClasses ints), so the sorted-tile kernels can run every class
// with a loop compiled for its width.
constexpr int kTileClasses = kMaxTileClasses;

__device__ __forceinline__ int tile_class(int size) { return min((size + 15) / 16, kTileClasses) - 1; }

// Workgroup-wide inclusive scans (kSortThreads threads) of the slot count csum and the
// per-class tile counts kc[] of each thread's experts; returns, in csum and kc[], the
// exclusive prefixes, in tot[] the workgroup totals (tot[0] slots, tot[1 + k] tiles of class k).
__device__ void scan_tiles(int32_t (&sc)[1 + kTileClasses][kSortThreads], int& csum,
                           int (&kc)[kTileClasses], int (&tot)[1 + kTileClasses]) {
  const int tid = threadIdx.x;
  sc[0][tid] = csum;
#pragma unroll
  for (int k = 0; k < kTileClasses; ++k) sc[1 + k][tid] = kc[k];
  __syncthreads();
  for (int o = 1; o < kSortThreads; o <<= 1) {
    int v[1 + kTileClasses];
#pragma unroll
    for (int k = 0; k <= kTileClasses; ++k) v[k] = tid >= o ? sc[k][tid - o] : 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k <= kTileClasses; ++k) sc[k][tid] += v[k];
    __syncthreads();
  }
  csum = sc[0][tid] - csum;
#pragma unroll
  for (int k = 0; k < kTileClasses; ++k) kc[k] = sc[1 + k][tid] - kc[k];
#pragma unroll
  for (int k = 0; k <= kTileClasses; ++k) tot[k] = sc[k][kSortThreads - 1];
}

// The tiles of one expert (c slots from position bc) at the cursors of their classes.
__device__ __forceinline__ void emit_expert_tiles(int4* tiles, int e, int bc, int c, int tt,
                                                  int (&cur)[kTileClasses]) {
  const int nt = (c + tt - 1) / tt;
  for (int i = 0; i < nt; ++i) {
    int4 tv;
    tv.x = e;
    tv.y = bc + i * tt;
    tv.z = min(tt, c - i * tt);
    tv.w = 0;
    const int k = tile_class(tv.z);
#pragma unroll
    for (int j = 0; j < kTileClasses; ++j)
      if (j == k) tiles[cur[j]++] = tv;
  }
}

// Per-thread tile counts by class of experts with the given slot count.
__device__ __forceinline__ void count_expert_tiles(int c, int tt, int (&kc)[kTileClasses]) {
  const int nt = (c + tt - 1) / tt;
  for (int i = 0; i < nt; ++i) {
    const int k = tile_class(min(tt, c - i * tt));
#pragma unroll
    for (int j = 0; j < kTileClasses; ++j) kc[j] += j == k;
  }
}

// Writes the header's tile count and class ends (thread 0).
__device__ __forceinline__ void write_tile_header(uint8_t* ws, const int (&tot)[1 + kTileClasses]) {
  int32_t* h = reinterpret_cast<int32_t*>(ws + 8);
  int end = 0;
#pragma unroll
  for (int k = 0; k < kTileClasses; ++k) {
    end += tot[1 + k];
    h[1 + k] = end;
  }
  h[0] = end;
}

struct SortArgs {
  const int32_t* idx;
  int32_t T, topk, E, tile_tokens;
  uint8_t* ws;
  size_t off_offsets, off_tiles, off_perm, off_inv;
};

__global__ __launch_bounds__(kSortThreads) void moe_sort(SortArgs a) {
  extern __shared__ int32_t counts[];  // [E]
  __shared__ int32_t scan[1 + kTileClasses][kSortThreads];
  __shared__ int32_t drop_cnt;
  const int tid = threadIdx.x;
  const int n_slots = a.T * a.topk;
  const int E = a.E;
  int32_t* offsets = reinterpret_cast<int32_t*>(a.ws + a.off_offsets);
  int32_t* tiles = reinterpret_cast<int32_t*>(a.ws + a.off_tiles);
  int32_t* perm = reinterpret_cast<int32_t*>(a.ws + a.off_perm);
  int32_t* inv = reinterpret_cast<int32_t*>(a.ws + a.off_inv);

  for (int e = tid; e < E; e += kSortThreads) counts[e] = 0;
  if (tid == 0) drop_cnt = 0;
  __syncthreads();
  for (int p = tid; p < n_slots; p += kSortThreads) {
    const int e = a.idx[p];
    if (e >= 0 && e < E)
      atomicAdd(&counts[e], 1);
    else
      atomicAdd(&drop_cnt, 1);
  }
  __syncthreads();

  const int per = (E + kSortThreads - 1) / kSortThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int csum = 0;
  int kc[kTileClasses] = {};
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e];
    csum += c;
    count_expert_tiles(c, a.tile_tokens, kc);
  }
  int tot[1 + kTileClasses];
  scan_tiles(scan, csum, kc, tot);
  // class k's tiles start after all tiles of the classes before it
  int cur[kTileClasses];
  int base = 0;
#pragma unroll
  for (int k = 0; k < kTileClasses; ++k) {
    cur[k] = base + kc[k];
    base += tot[1 + k];
  }
  int bc = csum;
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e];
    offsets[e] = bc;
    emit_expert_tiles(reinterpret_cast<int4*>(tiles), e, bc, c, a.tile_tokens, cur);
    counts[e] = bc;  // becomes the scatter cursor
    bc += c;
  }
  if (tid == kSortThreads - 1) {
    offsets[E] = tot[0];
    *reinterpret_cast<int64_t*>(a.ws) = (int64_t)drop_cnt;
    write_tile_header(a.ws, tot);
  }
  __syncthreads();
  for (int p = tid; p < n_slots; p += kSortThreads) {
    const int e = a.idx[p];
    int pos = -1;
    if (e >= 0 && e < E) {
      pos = atomicAdd(&counts[e], 1);
      perm[pos] = p;
    }
    inv[p] = pos;
  }
}

// Split sort for large batches.  Slice g of the slots (kSortParts slices) is counted by
// workgroup g into parts[g][e]; one workgroup then forms the expert totals, offsets and tiles
// as moe_sort does and turns parts[g][e] into the first position of slice g's slots of expert
// e; workgroup g finally scatters its slice from those cursors.  No workgroup waits on
// another inside a launch.
constexpr int kSplitThreads = 256;

struct SplitArgs {
  const int32_t* idx;
  int32_t n_slots, E, tile_tokens;
  uint8_t* ws;
  size_t off_offsets, off_tiles, off_perm, off_inv, off_parts;
};

__device__ __forceinline__ void slice_of(int n_slots, int& p0, int& p1) {
  const int chunk = (n_slots + kSortParts - 1) / kSortParts;
  p0 = min(n_slots, (int)blockIdx.x * chunk);
  p1 = min(n_slots, p0 + chunk);
}

__global__ __launch_bounds__(kSplitThreads) void sort_count(SplitArgs a) {
  extern __shared__ int32_t cnt[];  // [E]
  __shared__ int32_t drops;
  int32_t* parts = reinterpret_cast<int32_t*>(a.ws + a.off_parts);
  for (int e = threadIdx.x; e < a.E; e += kSplitThreads) cnt[e] = 0;
  if (threadIdx.x == 0) drops = 0;
  __syncthreads();
  int p0, p1;
  slice_of(a.n_slots, p0, p1);
  for (int p = p0 + threadIdx.x; p < p1; p += kSplitThreads) {
    const int e = a.idx[p];
    if (e >= 0 && e < a.E)
      atomicAdd(&cnt[e], 1);
    else
      atomicAdd(&drops, 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kSplitThreads) parts[(size_t)blockIdx.x * a.E + e] = cnt[e];
  if (threadIdx.x == 0) parts[(size_t)kSortParts * a.E + blockIdx.x] = drops;
}

__global__ __launch_bounds__(kSortThreads) void sort_scan(SplitArgs a) {
  __shared__ int32_t scan[1 + kTileClasses][kSortThreads];
  const int tid = threadIdx.x;
  const int E = a.E;
  int32_t* offsets = reinterpret_cast<int32_t*>(a.ws + a.off_offsets);
  int32_t* tiles = reinterpret_cast<int32_t*>(a.ws + a.off_tiles);
  int32_t* parts = reinterpret_cast<int32_t*>(a.ws + a.off_parts);
  const int per = (E + kSortThreads - 1) / kSortThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  auto total_of = [&](int e) {
    int c = 0;
#pragma unroll 16
    for (int g = 0; g < kSortParts; ++g) c += parts[(size_t)g * E + e];
    return c;
  };
  int csum = 0;
  int kc[kTileClasses] = {};
  for (int e = e0; e < e1; ++e) {
    const int c = total_of(e);
    csum += c;
    count_expert_tiles(c, a.tile_tokens, kc);
  }
  int tot[1 + kTileClasses];
  scan_tiles(scan, csum, kc, tot);
  int cur[kTileClasses];
  int base = 0;
#pragma unroll
  for (int k = 0; k < kTileClasses; ++k) {
    cur[k] = base + kc[k];
    base += tot[1 + k];
  }
  int bc = csum;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = bc;
    int run = bc;
#pragma unroll 16
    for (int g = 0; g < kSortParts; ++g) {  // slice g's first position among expert e's slots
      const int c = parts[(size_t)g * E + e];
      parts[(size_t)g * E + e] = run;
      run += c;
    }
    const int c = run - bc;
    emit_expert_tiles(reinterpret_cast<int4*>(tiles), e, bc, c, a.tile_tokens, cur);
    bc += c;
  }
  if (tid == kSortThreads - 1) {
    offsets[E] = tot[0];
    int64_t dr = 0;
    for (int g = 0; g < kSortParts; ++g) dr += parts[(size_t)kSortParts * E + g];
    *reinterpret_cast<int64_t*>(a.ws) = dr;
    write_tile_header(a.ws, tot);
  }
}

__global__ __launch_bounds__(kSplitThreads) void sort_scatter(SplitArgs a) {
  extern __shared__ int32_t cur[];  // [E]
  int32_t* perm = reinterpret_cast<int32_t*>(a.ws + a.off_perm);
  int32_t* inv = reinterpret_cast<int32_t*>(a.ws + a.off_inv);
  const int32_t* parts = reinterpret_cast<const int32_t*>(a.ws + a.off_parts);
  for (int e = threadIdx.x; e < a.E; e += kSplitThreads) cur[e] = parts[(size_t)blockIdx.x * a.E + e];
  __syncthreads();
  int p0, p1;
  slice_of(a.n_slots, p0, p1);
  for (int p = p0 + threadIdx.x; p < p1; p += kSplitThreads) {
    const int e = a.idx[p];
    int pos = -1;
    if (e >= 0 && e < a.E) {
      pos = atomicAdd(&cur[e], 1);
      perm[pos] = p;
    }
    inv[p] = pos;
  }
}

// ---------------------------------------------------------------------------------------
// Decode-sized grouped GEMM
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
  const int32_t* idx;  // [T][topk]
  const float* gates;  // [T][topk]
  int32_t T, topk, E;
  int32_t implicit_tiles;  // 1 (T == 1): tile j is slot j, no sort ran
  uint8_t* ws;         // workspace
  size_t off_tiles, off_perm;
  void* out;           // h (bf16 [slots][I]) or d (fp32 [slots][H])
  int32_t gact;        // k3x_activation of the W1/W3 epilogue
  float b1, b2;        // SiTU-GLU caps
};

// One K block (128 K) of operands for one lane: the packed bytes of 4 row blocks (group
// 4 kb + q of this lane's row), their 4 scale dwords (scales of groups 4 kb .. 4 kb + 3),
// and the 4 B fragments (8 activations each) of this lane's column.
struct Stage {
  uint4 w[4];
  uint32_t sc[4];
  uint4 x[4];
};

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// Operand addresses of one lane: two uniform expert bases (W1/W3 mode: W1 for row blocks
// 0-1 and W3 for 2-3; W2 mode: both W2) plus 32-bit per-lane offsets, so the bases live in
// scalar registers.
struct Addr {
  const uint8_t* wlo;  // packed base of row blocks 0-1
  const uint8_t* whi;  // packed base of row blocks 2-3
  const uint8_t* slo;  // scale base of row blocks 0-1
  const uint8_t* shi;  // scale base of row blocks 2-3
  uint32_t woff[4];    // byte offset of this lane's row in each row block (+ 16 q)
  uint32_t soff[4];    // byte offset of this lane's scale row in each row block
  const uint16_t* brow;
};

__device__ __forceinline__ void load_stage(Stage& st, const Addr& ad, bool valid, int kb, int q) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const uint8_t* wb = rb < 2 ? ad.wlo : ad.whi;
    const uint8_t* sb = rb < 2 ? ad.slo : ad.shi;
    st.w[rb] = *reinterpret_cast<const uint4*>(wb + ad.woff[rb] + (uint32_t)kb * 64u);
    st.sc[rb] = *reinterpret_cast<const uint32_t*>(sb + ad.soff[rb] + (uint32_t)kb * 4u);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
    st.x[s] = valid ? *reinterpret_cast<const uint4*>(ad.brow + kKBlock * kb + 32 * q + 8 * s)
                    : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void compute_stage(const Stage& st, f32x4 (&acc)[4], int q) {
  float scale[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) scale[rb] = e8m0_to_f32((st.sc[rb] >> (8 * q)) & 0xFFu);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8 b = as_bf16x8(st.x[s]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      acc[rb] = mfma16x16x32(dequant8(dword_of(st.w[rb], s), scale[rb]), b, acc[rb]);
  }
}

__device__ __forceinline__ bool expert_ok(int e, int E) { return e >= 0 && e < E; }

// Work item = (tile, row chunk): W1/W3 mode covers W1 rows r0..r0+31 and W3 rows r0..r0+31
// (row blocks 0,1 of W1 and 2,3 of W3); W2 mode covers W2 rows r0..r0+63.  Items are split
// over the 8 dies in contiguous ranges (a die's workgroups then share the tiles' activation
// rows in its L2) and strided over the die's workgroups.
template <bool kSwiGLU>
__global__ __launch_bounds__(256) void gemm_decode(GemmArgs a) {
  __shared__ f32x4 part[4][4][kWave];  // [wave][row block][lane] partial sums
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int n = lane % 16;  // B column / A row within a 16-row block
  const int q = lane / 16;  // lane quarter: which group of the K block
  int n_tiles;
  if (a.implicit_tiles) {
    n_tiles = a.T * a.topk;
    if (kSwiGLU && blockIdx.x == 0) {
      // upkeep of the sortless path (T == 1): the drop count
      if (threadIdx.x == 0) {
        int bad = 0;
        for (int j = 0; j < n_tiles; ++j) bad += expert_ok(a.idx[j], a.E) ? 0 : 1;
        *reinterpret_cast<int64_t*>(a.ws) = bad;
      }
    }
  } else {
    n_tiles = *reinterpret_cast<const int32_t*>(a.ws + 8);
  }
  const int4* tiles = reinterpret_cast<const int4*>(a.ws + a.off_tiles);
  const int32_t* perm = reinterpret_cast<const int32_t*>(a.ws + a.off_perm);
  const int rows_per_item = kSwiGLU ? 32 : 64;
  const int items_per_tile = a.rows / rows_per_item;
  const int items = n_tiles * items_per_tile;
  const int nk = a.K / kKBlock;
  const int kb0 = (wave * nk) / 4;
  const int kb1 = ((wave + 1) * nk) / 4;
  const size_t wrow_bytes = (size_t)a.K / 2;
  const size_t srow_bytes = (size_t)a.K / kGroup;

  int die, rank, per_die;
  xcd_rank(die, rank, per_die);
  const int chunk = (items + kNumXcd - 1) / kNumXcd;
  const int lo = die * chunk;
  const int hi = min(items, lo + chunk);

  for (int it = lo + rank; it < hi; it += per_die) {
    const int tile = it / items_per_tile;
    const int r0 = (it % items_per_tile) * rows_per_item;
    int e, start, m;
    if (a.implicit_tiles) {
      e = a.idx[tile];
      start = tile;
      m = 1;
      if (!expert_ok(e, a.E)) continue;  // a dropped slot (uniform across the workgroup)
    } else {
      const int4 tv = tiles[tile];
      e = tv.x;
      start = tv.y;
      m = tv.z;
    }

    const bool valid = n < m;
    const int slot = valid ? (a.implicit_tiles ? start + n : perm[start + n]) : 0;
    const int arow = a.act_by_token ? slot / a.topk : slot;

    Addr ad;
    ad.brow = a.act + (size_t)arow * a.K;
    if (kSwiGLU) {
      ad.wlo = a.wa + (size_t)e * a.st_wa;
      ad.whi = a.wb + (size_t)e * a.st_wb;
      ad.slo = a.sa + (size_t)e * a.st_sa;
      ad.shi = a.sb + (size_t)e * a.st_sb;
    } else {
      ad.wlo = ad.whi = a.wa + (size_t)e * a.st_wa;
      ad.slo = ad.shi = a.sa + (size_t)e * a.st_sa;
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = kSwiGLU ? r0 + 16 * (rb & 1) + n : r0 + 16 * rb + n;
      ad.woff[rb] = (uint32_t)(row * wrow_bytes) + 16u * (uint32_t)q;
      ad.soff[rb] = (uint32_t)(row * srow_bytes);
    }

    f32x4 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K range of this wave, loads issued one K block ahead of the MFMAs; two named stages
    // alternate so that no register copy waits on a load still in flight
    Stage s0, s1;
    if (kb0 < kb1) load_stage(s0, ad, valid, kb0, q);
    for (int kb = kb0; kb < kb1; kb += 2) {
      if (kb + 1 < kb1) load_stage(s1, ad, valid, kb + 1, q);
      compute_stage(s0, acc, q);
      if (kb + 1 >= kb1) break;
      if (kb + 2 < kb1) load_stage(s0, ad, valid, kb + 2, q);
      compute_stage(s1, acc, q);
    }

#pragma unroll
    for (int rb = 0; rb < 4; ++rb) part[wave][rb][lane] = acc[rb];
    __syncthreads();

    if (kSwiGLU) {
      if (wave < 2 && valid) {
        // lane holds rows 4q..4q+3 of row block `wave`, column n
        const int rb = wave;
        const f32x4 g = (part[0][rb][lane] + part[1][rb][lane]) + (part[2][rb][lane] + part[3][rb][lane]);
        const f32x4 u = (part[0][rb + 2][lane] + part[1][rb + 2][lane]) +
                        (part[2][rb + 2][lane] + part[3][rb + 2][lane]);
        uint32_t hv[2];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          uint32_t two = 0;
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const float gi = g[i + k2];
            const float v = a.gact == K3X_ACT_SITU ? situ_fast(gi, u[i + k2], a.b1, a.b2)
                                                   : (gi / (1.0f + expf(-gi))) * u[i + k2];
            two |= f32_to_bf16_bits(v) << (16 * k2);
          }
          hv[i / 2] = two;
        }
        uint16_t* h = static_cast<uint16_t*>(a.out);
        const int row = r0 + 16 * rb + 4 * q;
        *reinterpret_cast<uint2*>(h + (size_t)slot * a.rows + row) = make_uint2(hv[0], hv[1]);
      }
    } else {
      const int rb = wave;
      if (valid) {
        const f32x4 d = (part[0][rb][lane] + part[1][rb][lane]) + (part[2][rb][lane] + part[3][rb][lane]);
        float* dout = static_cast<float*>(a.out);
        const int row = r0 + 16 * rb + 4 * q;
        *reinterpret_cast<float4*>(dout + (size_t)slot * a.rows + row) = make_float4(d[0], d[1], d[2], d[3]);
      }
    }
    __syncthreads();  // part[] is reused by the next item
  }
}

// ---------------------------------------------------------------------------------------
// 4. Combine: y[t][r] = sum_j gates[t][j] * d[t*topk + j][r], slots in order, slots whose
// expert id is invalid skipped (a token without a valid slot gets 0).  Grid (row blocks, T):
// each thread owns 4 consecutive rows; the slot loop is unrolled 16 at a time so the
// independent loads of d overlap.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_combine(const float* __restrict__ d,
                                                   const int32_t* __restrict__ idx,
                                                   const float* __restrict__ gates,
                                                   const int32_t* __restrict__ inv,
                                                   int32_t topk, int32_t H, int32_t E,
                                                   float* __restrict__ y) {
  const int t = blockIdx.y;
  const int r = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (r >= H) return;
  const int32_t* it = idx + (size_t)t * topk;
  const float* gt = gates + (size_t)t * topk;
  const int32_t* pt = inv ? inv + (size_t)t * topk : nullptr;  // d rows by sorted position
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < topk; j0 += 16) {
    float4 v[16];
    float g[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int j = j0 + jj;
      const bool ok = j < topk && expert_ok(it[j], E);
      g[jj] = ok ? gt[j] : 0.0f;
      const size_t row = pt ? (size_t)(ok ? pt[j] : 0) : (size_t)t * topk + j;
      if (ok) {  // each d row is read once: non-temporal
        const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(d + row * H + r));
        v[jj] = make_float4(q[0], q[1], q[2], q[3]);
      } else {
        v[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      if (j0 + jj >= topk || !expert_ok(it[j0 + jj], E)) continue;
      acc.x = acc.x + g[jj] * v[jj].x;
      acc.y = acc.y + g[jj] * v[jj].y;
      acc.z = acc.z + g[jj] * v[jj].z;
      acc.w = acc.w + g[jj] * v[jj].w;
    }
  }
  *reinterpret_cast<float4*>(y + (size_t)t * H + r) = acc;
}

}  // namespace

hipError_t launch_moe(const k3x_pool& p, const uint16_t* x, int32_t T, const int32_t* idx,
                      const float* gates, int32_t topk, float* y, uint8_t* ws,
                      const MoeLayout& L, hipStream_t s) {
  if (p.contract && T > 0) return launch_contract(p, x, idx, gates, topk, y, ws, s);
  if (decode_exact_supported(p, T, topk))
    return launch_decode_exact(p, x, idx, gates, topk, y, ws, s);
  hipError_t err;
  const bool implicit = (T == 1);
  if (!implicit) {
    SortArgs sa{};
    sa.idx = idx;
    sa.T = T;
    sa.topk = topk;
    sa.E = p.E;
    sa.tile_tokens = L.tile_tokens;
    sa.ws = ws;
    sa.off_offsets = L.offsets;
    sa.off_tiles = L.tiles;
    sa.off_perm = L.perm;
    sa.off_inv = L.inv;
    const size_t sort_lds = sizeof(int32_t) * (size_t)p.E;
    if (L.sort_n) {
      SplitArgs b{idx, T * topk, p.E, L.tile_tokens, ws, L.offsets, L.tiles, L.perm, L.inv,
                  L.sort_parts};
      err = launch("sort_count", sort_count, dim3(kSortParts), dim3(kSplitThreads),
                   (uint32_t)sort_lds, s, b);
      if (err == hipSuccess)
        err = launch("sort_scan", sort_scan, dim3(1), dim3(kSortThreads), 0, s, b);
      if (err == hipSuccess)
        err = launch("sort_scatter", sort_scatter, dim3(kSortParts), dim3(kSplitThreads),
                     (uint32_t)sort_lds, s, b);
      if (err != hipSuccess) return err;
    } else {
      err = launch("moe_sort", moe_sort, dim3(1), dim3(kSortThreads), (uint32_t)sort_lds, s, sa);
      if (err != hipSuccess || T == 0) return err;
    }
  }

  if (L.tile_tokens > 16) {
    err = launch_prefill_gemms(p, x, T, topk, ws, L, s);
    if (err != hipSuccess) return err;
    return launch("moe_combine", moe_combine, dim3((p.H / 4 + 255) / 256, T), dim3(256), 0, s,
                  reinterpret_cast<const float*>(ws + L.d), idx, gates,
                  reinterpret_cast<const int32_t*>(ws + L.inv), topk, p.H, p.E, y);
  }

  // persistent grids: two 4-wave workgroups per CU (the occupancy the registers allow)
  const int max_grid = device_cu_count() * 2;

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
  a13.idx = idx;
  a13.gates = gates;
  a13.T = T;
  a13.topk = topk;
  a13.E = p.E;
  a13.implicit_tiles = implicit ? 1 : 0;
  a13.ws = ws;
  a13.off_tiles = L.tiles;
  a13.off_perm = L.perm;
  a13.out = ws + L.h;
  a13.gact = p.act;
  a13.b1 = p.b1;
  a13.b2 = p.b2;
  const int64_t max_tiles = implicit ? (int64_t)topk : (int64_t)L.max_tiles;
  auto grid_for = [&](int64_t items) {
    int64_t g = (items + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (g > max_grid) g = max_grid;
    return (int)(g < kNumXcd ? kNumXcd : g);
  };
  err = launch("w13_grouped", gemm_decode<true>, dim3(grid_for(max_tiles * (p.I / 32))),
               dim3(256), 0, s, a13);
  if (err != hipSuccess) return err;

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
  err = launch("w2_grouped", gemm_decode<false>, dim3(grid_for(max_tiles * (p.H / 64))),
               dim3(256), 0, s, a2);
  if (err != hipSuccess) return err;
  return launch("moe_combine", moe_combine, dim3((p.H / 4 + 255) / 256, T), dim3(256), 0, s,
                reinterpret_cast<const float*>(ws + L.d), idx, gates, nullptr, topk, p.H, p.E, y);
}

}  // namespace k3x
