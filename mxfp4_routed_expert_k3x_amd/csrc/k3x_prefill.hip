// Grouped GEMMs of the routed experts for batches of two or more tokens (prefill, and small
// decode batches, where they stream lightly shared experts' weights fastest).
//
// Sources: kimi-k3-in-c README, Part II section 4 "Reduction one: the experts already ship at
// half a byte" (MXFP4 weights taken straight from the nibbles: E2M1 value times 2^(scale -
// 127), low nibble = even element, scale byte 255 zeroes its group; nothing dequantized is
// written to memory) and section 9 "Picking 16 experts of 896" (routed-expert loop, SwiGLU
// with h rounded to bf16 before W2, slot-order combine).
//
// Slots are sorted by expert into tiles of at most 96 slots of one expert.  An item is one
// tile against a chunk of output rows, computed by one workgroup of 8 waves (2 per SIMD):
//   - W1/W3 mode: 256 rows of h (each wave 32 rows of W1 and the same 32 rows of W3),
//     epilogue h = bf16(silu(g) * u), or of SiTU-GLU when the pool asks for it;
//   - W2 mode: 512 rows of d (each wave 64 rows of W2).
// h and d are stored by sorted position (row = the slot's index in the sorted order), so W2
// reads its tile's h rows contiguously and the combine gathers d through the inverse order.
//
// The packed weights go from HBM straight into registers as the MFMA A operand: lane
// (n = lane % 16, q = lane / 16) loads 16 bytes = one whole MX group (group 4 kb + q of row
// n) and converts it with the gfx950 scaled FP4 -> bf16 instruction, the group's power-of-two
// scale folded in (exact).  One 16-byte load feeds four bf16 MFMAs (16x16x32) that together
// cover 16 rows x 128 K.  Weights run two K blocks ahead of the MFMAs in a ring of three
// register sets.  The item's scale rows are copied into LDS once per item (direct-to-LDS
// loads), and each K block's four scales are decoded from there before the barrier that
// starts the block.  The tile's activations (x rows by token, or h rows by position) are the B
// operand: each 128-wide K block of the tile's rows is staged in LDS one block ahead (double
// buffered, rows padded by 16 bytes so the 16 lanes of one read hit distinct banks) and every
// B fragment is used by the wave's four row blocks.  The MFMA's K order is a permutation
// shared by A and B, so the product is unchanged; accumulation is fp32.
//
// Work is persistent: tile t belongs to die t % 8 (all its row chunks), so the tile's
// activation rows are fetched into one die's L2 and reused by every chunk; within a die the
// workgroups take (tile, chunk) items in turn.  Items are pipelined: the next item's routing
// rows are fetched during the current item's K loop, and its first activation and weight
// blocks are in flight while the current item's epilogue runs.
#include <atomic>

#include "k3x_internal.h"

namespace k3x {
namespace {

constexpr int kTT = 96;                         // slots per tile
constexpr int kWaves = 8;
constexpr int kRB = 4;                          // 16-row weight blocks per wave
constexpr int kThreads = kWave * kWaves;
constexpr int kLdsRow = kKBlock + 8;            // bf16 per staged activation row (256 + 16 bytes)
constexpr int kXRowsPerPass = kThreads / 16;    // rows staged per pass (16 threads per row)
constexpr int kXPass = (kTT + kXRowsPerPass - 1) / kXRowsPerPass;  // staged pieces per thread
constexpr int kXRows = kXPass * kXRowsPerPass;  // staged rows (>= kTT)
constexpr int kMaxScaleRow = 128;               // scale bytes per weight row (K <= 4096)
constexpr int kScaleRows = kWaves * 16 * kRB;   // weight rows of one item (W1 + W3, or W2)

struct PrefillArgs {
  const uint8_t* wa;  // W1 (W1/W3 mode) or W2, packed, expert 0
  const uint8_t* sa;
  const uint8_t* wb;  // W3, W1/W3 mode only
  const uint8_t* sb;
  int64_t st_wa, st_sa, st_wb, st_sb;
  int32_t K;          // H (W1/W3) or I (W2)
  int32_t rows;       // I (W1/W3) or H (W2)
  const uint16_t* act;  // x [T][H] by token (W1/W3) or h [positions][I] (W2)
  uint32_t act_bytes;
  int32_t topk;
  void* out;          // h bf16 [positions][I] or d fp32 [positions][H]
  int32_t gact;       // k3x_activation of the W1/W3 epilogue
  float b1, b2;       // SiTU-GLU caps
};

// output rows of one item: W1/W3 mode 32 h rows per wave (32 W1 + 32 W3 rows), W2 mode 64
// d rows per wave
template <bool kW13>
constexpr int item_rows() { return kWaves * 16 * (kW13 ? kRB / 2 : kRB); }

// Raw buffer loads: the base and size live in four scalar registers, each lane supplies one
// 32-bit offset and the part of the offset shared by the wave is a scalar register.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// silu(g) * u for the prefill epilogue.  The hardware exponential and reciprocal are within
// a few ulp of the correctly rounded float values; the bf16 rounding of h that follows is
// where this can differ from the reference, in rare ties, well inside the output tolerance.
__device__ __forceinline__ float swiglu_fast(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// The sort's outputs are separate read-only, non-aliasing arguments, so the tile records
// come in through scalar loads (their own counter) and never wait behind operand loads.
template <bool kW13>
__global__ __launch_bounds__(kThreads, 1) void gemm_prefill(PrefillArgs a, const int32_t* __restrict__ n_tiles_p,
                                                            const int4* __restrict__ tiles,
                                                            const int32_t* __restrict__ perm) {
  __shared__ __align__(16) uint16_t xs[2][kXRows][kLdsRow];
  // the item's scale rows, copied once per item: W1/W3 mode W1 rows then W3 rows, W2 mode
  // the W2 rows, each K / 32 bytes
  __shared__ __align__(16) uint8_t ss[kScaleRows * kMaxScaleRow];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane % 16;
  const int q = lane / 16;
  const int xc = tid % 16;  // 16-byte piece of a staged row segment
  const int xr = tid / 16;  // staged rows xr + kXRowsPerPass * p

  const int n_tiles = *n_tiles_p;
  constexpr int kRows = item_rows<kW13>();
  const int chunks = a.rows / kRows;
  const int nk = a.K / kKBlock;
  const uint32_t wrow = (uint32_t)a.K / 2, srow = (uint32_t)a.K / kGroup;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.act, a.act_bytes);
  const uint32_t wbytes = (uint32_t)a.rows * wrow;
  // per-lane part of the weight addresses; the row block's base is uniform
  const uint32_t wl = (uint32_t)n * wrow + 16u * (uint32_t)q;
  // this lane's scale bytes in LDS: row block rb at sbase + rb_off(rb), group 4 kb + q
  const uint32_t sbase = (uint32_t)(wave * (kRows / kWaves) + n) * srow + (uint32_t)q;

  int die, rank, per_die;
  xcd_rank(die, rank, per_die);
  const int my_tiles = n_tiles > die ? (n_tiles - die + kNumXcd - 1) / kNumXcd : 0;
  const int items = my_tiles * chunks;
  int it = rank;
  if (it >= items) return;

  // ---- item state: expert, first position, slot count, first output row of this wave ----
  int e, start, m, r0;
  uint32_t xoff[kXPass];  // byte offset of this thread's staged activation rows
  __amdgpu_buffer_rsrc_t wlo, whi;
  // tile and routing rows of the next item, fetched one item ahead (W1/W3 mode: slot ids)
  int ne = 0, nstart = 0, nm = 1, nchunk = 0;
  int32_t nslot[kXPass];

  auto fetch_tile = [&](int item, int& te, int& tstart, int& tm, int& tchunk) __attribute__((always_inline)) {
    const int4 tv = tiles[die + kNumXcd * (item / chunks)];
    te = tv.x;
    tstart = tv.y;
    tm = tv.z;
    tchunk = item % chunks;
  };
  auto fetch_rows = [&](int tstart, int tm, int32_t (&slot)[kXPass]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < kXPass; ++p) {
      // rows past the tile repeat its last row (the LDS holds kXRows rows)
      const int i = min(xr + kXRowsPerPass * p, tm - 1);
      slot[p] = kW13 ? perm[tstart + i] : tstart + i;
    }
  };
  auto enter = [&](int te, int tstart, int tm, int tchunk, const int32_t (&slot)[kXPass]) __attribute__((always_inline)) {
    e = __builtin_amdgcn_readfirstlane(te);
    start = __builtin_amdgcn_readfirstlane(tstart);
    m = __builtin_amdgcn_readfirstlane(tm);
    r0 = __builtin_amdgcn_readfirstlane(tchunk * kRows + wave * (kRows / kWaves));
#pragma unroll
    for (int p = 0; p < kXPass; ++p) {
      const uint32_t r = kW13 ? (uint32_t)slot[p] / (uint32_t)a.topk : (uint32_t)slot[p];
      xoff[p] = 2u * (r * (uint32_t)a.K) + 16u * (uint32_t)xc;
    }
    wlo = make_rsrc(a.wa + (size_t)e * a.st_wa, wbytes);
    whi = kW13 ? make_rsrc(a.wb + (size_t)e * a.st_wb, wbytes) : wlo;
  };

  // ---- operand staging ----
  // Weight blocks run two K blocks ahead in a ring of three register sets (block kb in set
  // kb % 3), activation blocks one block ahead in two sets.  Each step issues its activation
  // loads before its weight loads; scheduling barriers keep that order, so the
  // memory-counter wait that the store of activation block kb + 1 needs at the end of step kb
  // covers only loads issued before it (weights up to block kb + 1, which step kb + 1 needs
  // anyway), never the weight block kb + 2 issued in the same step.
  auto load_x = [&](int kb, uint4 (&xv)[kXPass]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < kXPass; ++p) xv[p] = buf_load16(xrs, xoff[p], (uint32_t)(2 * kKBlock * kb));
    __builtin_amdgcn_sched_barrier(0);
  };
  auto store_x = [&](int buf, const uint4 (&xv)[kXPass]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < kXPass; ++p)
      *reinterpret_cast<uint4*>(&xs[buf][xr + kXRowsPerPass * p][8 * xc]) = xv[p];
  };
  auto load_w = [&](int kb, uint4 (&w)[kRB]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const uint32_t row = (uint32_t)(kW13 ? r0 + 16 * (rb % (kRB / 2)) : r0 + 16 * rb);
      w[rb] = buf_load16(rb < kRB / 2 ? wlo : whi, wl, row * wrow + 64u * (uint32_t)kb);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Scale rows of an item: contiguous in each scale tensor (the item's rows are
  // consecutive), copied global -> LDS with the 16-byte direct-to-LDS load (lane i lands at
  // base + 16 i; no registers).  W1/W3 mode: W1 rows at 0, W3 rows at half the buffer; W2
  // mode: the W2 rows.  Pieces past a region's end repeat its last piece into the unused
  // part of the region.  Done once per item; the compiler orders it before the next LDS
  // access with a full memory-counter wait.
  auto copy_scales = [&]() __attribute__((always_inline)) {
    const uint32_t item_row0 = (uint32_t)__builtin_amdgcn_readfirstlane(r0 - wave * (kRows / kWaves));
    constexpr int kChunk = kWave;  // 16-byte pieces per instruction
    if (kW13) {
      const int pieces = (int)(kScaleRows / 2 * srow / 16);
      const uint8_t* g1 = a.sa + (size_t)e * a.st_sa + (size_t)item_row0 * srow;
      const uint8_t* g3 = a.sb + (size_t)e * a.st_sb + (size_t)item_row0 * srow;
#pragma unroll
      for (int j = 0; j < kScaleRows / 2 * kMaxScaleRow / 16 / kChunk / kWaves; ++j) {
        const int chunk = j * kWaves + wave;
        const int gsrc = min(chunk * kChunk + lane, pieces - 1);
        __builtin_amdgcn_global_load_lds(g1 + 16 * gsrc, &ss[chunk * kChunk * 16], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(g3 + 16 * gsrc, &ss[kScaleRows / 2 * kMaxScaleRow + chunk * kChunk * 16], 16, 0, 0);
      }
    } else {
      const int pieces = (int)(kScaleRows * srow / 16);
      const uint8_t* g2 = a.sa + (size_t)e * a.st_sa + (size_t)item_row0 * srow;
#pragma unroll
      for (int j = 0; j < kScaleRows * kMaxScaleRow / 16 / kChunk / kWaves; ++j) {
        const int chunk = j * kWaves + wave;
        const int gsrc = min(chunk * kChunk + lane, pieces - 1);
        __builtin_amdgcn_global_load_lds(g2 + 16 * gsrc, &ss[chunk * kChunk * 16], 16, 0, 0);
      }
    }
  };
  // LDS byte offset of row block rb's scale row for this lane (relative to sbase)
  auto rb_off = [&](int rb) __attribute__((always_inline)) {
    return kW13 ? (uint32_t)((rb / (kRB / 2)) * (kScaleRows / 2 * kMaxScaleRow)) + (uint32_t)(16 * (rb % (kRB / 2))) * srow
                : (uint32_t)(16 * rb) * srow;
  };

  uint4 x0[kXPass], x1[kXPass];
  uint4 w0[kRB], w1[kRB], w2[kRB];
  {
    int te, ts, tm, tc;
    int32_t slot[kXPass];
    fetch_tile(it, te, ts, tm, tc);
    fetch_rows(ts, tm, slot);
    enter(te, ts, tm, tc, slot);
  }
  load_x(0, x0);
  load_w(0, w0);
  load_w(min(1, nk - 1), w1);
  copy_scales();

  // accumulators of the widest tile; a tile of NB column blocks uses the first NB
  f32x4 acc[kRB][kTT / 16];

  // One tile of nb column blocks (nb <= NB = kTT / 16).  Column blocks past nb skip their
  // MFMAs with a uniform branch; their LDS reads stay (stale rows, never stored), so no
  // branch ever separates a load from its wait.
  constexpr int NB = kTT / 16;
  auto kloop = [&](int nb) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) acc[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the scales of K block kb, decoded before the barrier that starts it (the item's scale
    // rows do not change while its K loop runs)
    float scl[kRB];
    auto read_scales = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) scl[rb] = e8m0_to_f32(ss[sbase + rb_off(rb) + 4u * (uint32_t)kb]);
    };
    auto compute = [&](int kb, const uint4 (&w)[kRB]) __attribute__((always_inline)) {
      const int buf = kb & 1;
      float scale[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) scale[rb] = scl[rb];
      // B fragments in (s, tb) order, read two fragments ahead of the MFMAs that use them
      const uint16_t* xb = &xs[buf][n][32 * q];
      auto read_b = [&](int f) __attribute__((always_inline)) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(xb + (16 * (f % NB)) * kLdsRow + 8 * (f / NB)));
      };
      constexpr int kF = 4 * NB;
      bf16x8 bq[3];
      bq[0] = read_b(0);
      if (kF > 1) bq[1] = read_b(1);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 av[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) av[rb] = dequant8(dword_of(w[rb], s), scale[rb]);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          const int f = s * NB + tb;
          if (f + 2 < kF) bq[(f + 2) % 3] = read_b(f + 2);
          if (tb < nb) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) acc[rb][tb] = mfma16x16x32(av[rb], bq[f % 3], acc[rb][tb]);
          }
        }
      }
    };

    // one K block: loads for later blocks, MFMAs, the next activation block into LDS, and
    // one barrier.  The body has no branches, so the compiler's memory-counter waits stay
    // exact (the last blocks re-read block nk - 1 instead of skipping the loads).
    // step kb: load activation block kb + 1 into xn and weight block kb + 2 into wn, MFMAs on
    // wc (block kb), then activation block kb + 1 into LDS
    auto step = [&](int kb, const uint4 (&wc)[kRB], uint4 (&xn)[kXPass], uint4 (&wn)[kRB]) __attribute__((always_inline)) {
      load_x(min(kb + 1, nk - 1), xn);
      load_w(min(kb + 2, nk - 1), wn);
      compute(kb, wc);
      store_x((kb + 1) & 1, xn);
      read_scales(min(kb + 1, nk - 1));
      __syncthreads();
    };

    store_x(0, x0);
    __syncthreads();
    // after the barrier: the item's scale rows were copied into LDS by all waves
    read_scales(0);
    // the first six steps are peeled so that the loop is only entered in the steady state
    // (the compiler then keeps every wait in the loop down to the block it needs)
    int kb = 0;
    if (nk >= 6) {
      step(0, w0, x1, w2);
      step(1, w1, x0, w0);
      step(2, w2, x1, w1);
      step(3, w0, x0, w2);
      step(4, w1, x1, w0);
      step(5, w2, x0, w1);
      for (kb = 6; kb + 6 <= nk; kb += 6) {
        step(kb, w0, x1, w2);
        step(kb + 1, w1, x0, w0);
        step(kb + 2, w2, x1, w1);
        step(kb + 3, w0, x0, w2);
        step(kb + 4, w1, x1, w0);
        step(kb + 5, w2, x0, w1);
      }
    }
    // remaining 0..5 blocks (the ring sets follow kb % 3, the activation sets kb % 2)
    if (kb < nk) step(kb, w0, x1, w2);
    if (kb + 1 < nk) step(kb + 1, w1, x0, w0);
    if (kb + 2 < nk) step(kb + 2, w2, x1, w1);
    if (kb + 3 < nk) step(kb + 3, w0, x0, w2);
    if (kb + 4 < nk) step(kb + 4, w1, x1, w0);
  };

  // epilogue: lane holds rows 4q..4q+3 of each row block for column 16 tb + n
  auto epilogue = [&](int cstart, int cm, int cr0) __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const int col = 16 * tb + n;
      if (col < cm) {
        const size_t pos = (size_t)(cstart + col);
        if (kW13) {
          uint16_t* h = static_cast<uint16_t*>(a.out) + pos * a.rows + cr0 + 4 * q;
#pragma unroll
          for (int rb = 0; rb < kRB / 2; ++rb) {
            uint32_t hv[2];
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const float g0 = acc[rb][tb][i], u0 = acc[rb + kRB / 2][tb][i];
              const float g1 = acc[rb][tb][i + 1], u1 = acc[rb + kRB / 2][tb][i + 1];
              const bool situ = a.gact == K3X_ACT_SITU;
              const float h0 = situ ? situ_fast(g0, u0, a.b1, a.b2) : swiglu_fast(g0, u0);
              const float h1 = situ ? situ_fast(g1, u1, a.b1, a.b2) : swiglu_fast(g1, u1);
              hv[i / 2] = f32_to_bf16_bits(h0) | (f32_to_bf16_bits(h1) << 16);
            }
            *reinterpret_cast<uint2*>(h + 16 * rb) = make_uint2(hv[0], hv[1]);
          }
        } else {
          float* d = static_cast<float*>(a.out) + pos * a.rows + cr0 + 4 * q;
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            *reinterpret_cast<float4*>(d + 16 * rb) =
                make_float4(acc[rb][tb][0], acc[rb][tb][1], acc[rb][tb][2], acc[rb][tb][3]);
        }
      }
    }
  };

  for (;;) {
    const int nit = it + per_die;
    const bool more = nit < items;
    if (more) {
      fetch_tile(nit, ne, nstart, nm, nchunk);
      fetch_rows(nstart, nm, nslot);
    }
    const int nb = (m + 15) / 16;
    kloop(nb);
    // the next item's first blocks go out before this item's epilogue
    const int cstart = start, cm = m, cr0 = r0;
    if (more) {
      enter(ne, nstart, nm, nchunk, nslot);
      load_x(0, x0);
      load_w(0, w0);
      load_w(min(1, nk - 1), w1);
      // every wave finished the last K block (barrier) before the scales are replaced; the
      // next item's first barrier publishes them
      copy_scales();
    }
    epilogue(cstart, cm, cr0);
    if (!more) break;
    it = nit;
  }
}

// Workgroups per CU of each mode, cached once for every device (a property of the kernel and
// the architecture); concurrent first calls store the same value.
int prefill_grid(const void* fn) {
  static std::atomic<int> cached[2] = {{0}, {0}};
  const int which = fn == reinterpret_cast<const void*>(&gemm_prefill<true>) ? 0 : 1;
  int per_cu = cached[which].load(std::memory_order_relaxed);
  if (!per_cu) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    cached[which].store(per_cu, std::memory_order_relaxed);
  }
  return device_cu_count() * per_cu;
}

}  // namespace

int prefill_tile_tokens() { return kTT; }

hipError_t launch_prefill_gemms(const k3x_pool& p, const uint16_t* x, int32_t T, int32_t topk,
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
  a.act_bytes = (uint32_t)((size_t)T * p.H * 2);
  a.topk = topk;
  a.out = ws + L.h;
  a.gact = p.act;
  a.b1 = p.b1;
  a.b2 = p.b2;
  const int32_t* n_tiles = reinterpret_cast<const int32_t*>(ws + 8);
  const int4* tiles = reinterpret_cast<const int4*>(ws + L.tiles);
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + L.perm);
  hipError_t err = launch("w13_prefill", gemm_prefill<true>,
                          dim3(prefill_grid(reinterpret_cast<const void*>(&gemm_prefill<true>))),
                          dim3(kThreads), 0, s, a, n_tiles, tiles, perm);
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
  b.act_bytes = (uint32_t)((size_t)T * topk * p.I * 2);
  b.out = ws + L.d;
  return launch("w2_prefill", gemm_prefill<false>,
                dim3(prefill_grid(reinterpret_cast<const void*>(&gemm_prefill<false>))),
                dim3(kThreads), 0, s, b, n_tiles, tiles, perm);
}

}  // namespace k3x
