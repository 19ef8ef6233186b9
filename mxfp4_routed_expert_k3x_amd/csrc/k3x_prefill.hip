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
// tile against a chunk of output rows, computed by one workgroup of 8 waves, one workgroup per
// CU (two waves per SIMD); the eight waves share each staged activation block, so a CU copies
// every activation block once per item for twice the weight rows of a 4-wave workgroup:
//   - W1/W3 mode: 256 rows of h (each wave 32 rows of W1 and the same 32 rows of W3),
//     epilogue h = bf16(silu(g) * u), or of SiTU-GLU when the pool asks for it;
//   - W2 mode: 512 rows of d (each wave 64 rows of W2).
// h and d are stored by sorted position (row = the slot's index in the sorted order), so W2
// reads its tile's h rows contiguously and the combine gathers d through the inverse order.
//
// Weights (the MFMA A operand) go from HBM straight into registers: lane (n = lane % 16, q =
// lane / 16) loads 16 bytes = one whole MX group (group 4 kb + q of row n) and converts it
// with the gfx950 scaled FP4 -> bf16 instruction, the group's power-of-two scale folded in
// (exact).  One 16-byte load feeds four bf16 MFMAs (16x16x32) that together cover 16 rows x
// 128 K.  Weights are requested two K blocks ahead in a ring of three register sets.
//
// Activations (the B operand: x rows by token, or h rows by position) are copied from memory
// into LDS by the buffer unit itself (16 bytes per lane, no registers), one 128-wide K block
// ahead, into two stages.  A staged row is 256 bytes in 16 pieces of 16 bytes; piece c of row
// r is stored at position c ^ (r % 16), so the 16 lanes that read one B fragment (16 rows,
// the same piece) hit 16 different bank groups.  The MFMA's K order is a permutation shared
// by A and B, so the product is unchanged; accumulation is fp32 over the whole K.  The item's
// scale rows are copied into LDS once per item the same way.
//
// Each K block ends with one wait + barrier: every wave waits for its own copies into the
// next stage (the copies were issued before the block's weight requests, so the wait leaves
// those in flight) and for its LDS reads of the current stage, then all eight waves meet.
// Within a block each B fragment is read two fragments before its MFMAs and the scale bytes
// one block ahead, so no MFMA waits for an LDS read issued just before it.
//
// Work is persistent: tile t belongs to die t % 8 (all its row chunks), so the tile's
// activation rows are fetched into one die's L2 and reused by every chunk; within a die the
// workgroups take (tile, chunk) items in turn.  The next item's first activation block, scale
// rows and weight blocks are requested before the current item's epilogue runs.
#include <atomic>
#include <type_traits>

#include "k3x_internal.h"

namespace k3x {
namespace {

constexpr int kTT = 96;                        // slots per tile
constexpr int kWaves = 8;                      // waves per workgroup; one workgroup per CU
constexpr int kThreads = kWave * kWaves;
constexpr int kRB = 4;                         // 16-row weight blocks per wave
constexpr int kXRow = 2 * kKBlock;             // bytes of one staged activation row (128 bf16)
constexpr int kXStage = kTT * kXRow;           // bytes of one activation stage
constexpr int kMaxScaleRow = 128;              // scale bytes per weight row (K <= 4096)
constexpr int kItemWRows = kWaves * 16 * kRB;  // weight rows of one item (W1 + W3, or W2)

typedef __attribute__((address_space(3))) void lds_void;

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

// Raw buffer accesses: the base and size live in four scalar registers, each lane supplies one
// 32-bit offset and the part of the offset shared by the wave is a scalar register.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 16 bytes per lane from memory into LDS: lane i's bytes land at lds + 16 i (lds is the same
// for the whole wave).
__device__ __forceinline__ void buf_copy16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                               uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// Waits until at most N of this wave's vector memory operations are outstanding and all its
// LDS operations are done, then meets the workgroup's other waves.  One asm statement with a
// memory clobber, so the compiler moves no memory access across either part.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  // the same wait as a builtin first, so that the compiler's own wait tracking knows it and
  // adds no wait of its own for the LDS copies it retires
  static_assert(N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4));
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
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

// Two floats rounded to bf16 (nearest, ties to even) and packed, a in the low half: one
// gfx950 conversion instruction for the pair.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 r = __builtin_convertvector(f2{a, b}, b2);
  return __builtin_bit_cast(uint32_t, r);
}

template <int N>
using ic = std::integral_constant<int, N>;

// The sort's outputs are separate read-only, non-aliasing arguments, so the tile records
// come in through scalar loads (their own counter) and never wait behind operand loads.
// header: [0] tile count, [1 + k] end of tile class k in the tile array (the sort writes the
// tiles class by class; class k needs k + 1 column blocks).
template <bool kW13>
__global__ __launch_bounds__(kThreads, 1) void gemm_prefill(PrefillArgs a, const int32_t* __restrict__ header,
                                                            const int4* __restrict__ tiles,
                                                            const int32_t* __restrict__ perm) {
  // two activation stages (24 KB each) and the item's scale rows (64 KB): 112 KB of the CU's
  // 160, with the epilogue's slices 122 KB (W1/W3) or 146 KB (W2)
  __shared__ __align__(16) uint8_t xs0[kXStage];
  __shared__ __align__(16) uint8_t xs1[kXStage];
  __shared__ __align__(16) uint8_t ss[kItemWRows * kMaxScaleRow];
  // The epilogue turns each wave's outputs of one column block around in a slice of its own
  // (no barrier), so that a store covers whole runs of rows of a position: W1/W3 16
  // positions x 32 h rows (bf16, rows padded to 40), W2 16 positions x 64 d rows (fp32,
  // rows padded to 68; 34 KB).  The padding spreads the writes of the 16 positions over the
  // banks.
  constexpr int kTrRowH = 40;
  constexpr int kTrRow = 68;
  __shared__ __align__(16) float xt[kW13 ? kWaves * 16 * kTrRowH / 2 : kWaves * 16 * kTrRow];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane % 16;
  const int q = lane / 16;

  constexpr int kRows = item_rows<kW13>();
  const int chunks = a.rows / kRows;
  const int nk = a.K / kKBlock;  // a multiple of 4 (K is a multiple of 512)
  const uint32_t wrow = (uint32_t)a.K / 2, srow = (uint32_t)a.K / kGroup;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.act, a.act_bytes);
  const uint32_t wbytes = (uint32_t)a.rows * wrow;
  // per-lane part of the weight addresses; the row block's base is uniform
  const uint32_t wl = (uint32_t)n * wrow + 16u * (uint32_t)q;
  // B fragment of MFMA step s: row n of the column block, the piece of K slice 32 q + 8 s,
  // at its swizzled position
  uint32_t bo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) bo[s] = (uint32_t)n * kXRow + 16u * (uint32_t)((4 * q + s) ^ n);
  // the activation rows this lane copies: row 16 j + xr of a stage (j = a column block of the
  // wave's copies), whose data piece (lane % 16) ^ xr it brings to position lane % 16
  const int xr = 4 * (wave % 4) + lane / 16;
  // the stage's 4 NBT row quads are dealt round-robin: waves 0..3 copy quad wave % 4 of the
  // even column blocks, waves 4..7 of the odd ones
  const int wh = __builtin_amdgcn_readfirstlane(wave / 4);
  const uint32_t xpiece = 16u * (uint32_t)((lane % 16) ^ xr);
  // this lane's scale bytes in LDS (group 4 kb + q of row block rb at sa[rb] + 4 kb): W1/W3
  // mode the 128 W1 rows in the first half of ss, the 128 W3 rows in the second; W2 mode the
  // 256 W2 rows; K / 32 bytes per row
  uint32_t sa[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const uint32_t region = kW13 && rb >= 2 ? (uint32_t)(kItemWRows / 2 * kMaxScaleRow) : 0u;
    const uint32_t row = kW13 ? (uint32_t)(32 * wave + 16 * (rb % 2)) : (uint32_t)(64 * wave + 16 * rb);
    sa[rb] = region + (row + (uint32_t)n) * srow + (uint32_t)q;
  }

  // Items: this die's tiles (tile t belongs to die t % 8), in the sort's class order, each
  // against every row chunk; item i is local tile i / chunks, chunk i % chunks.  The
  // workgroups of a die take items rank, rank + per_die, ...
  int die, rank, per_die;
  xcd_rank(die, rank, per_die);
  auto local_tiles = [&](int global_end) __attribute__((always_inline)) {
    return global_end > die ? (global_end - die + kNumXcd - 1) / kNumXcd : 0;
  };
  int it = rank;

  // Every item of tile class NBT - 1 (NBT column blocks) from `it` on, below item `hi`: one
  // persistent loop compiled for that width.
  auto run_class = [&](auto nbc, int hi) __attribute__((always_inline)) {
    constexpr int NBT = decltype(nbc)::value;
    if (it >= hi) return;

    // ---- item state: expert, first position, slot count, first row of the entered item,
    // and the next item's registers, set up before its first requests go out during the
    // entered item's last two K steps ----
    int e, start, m, r0;
    constexpr int kNC = (NBT + 1) / 2;  // copies per wave and stage
    auto jc = [&](int c) __attribute__((always_inline)) { return 2 * c + wh; };  // their column blocks
    uint32_t xo[kNC];  // byte offset of this lane's copied activation row of copy c
    __amdgpu_buffer_rsrc_t wlo, whi;
    int ne = 0, nstart = 0, nm = 1, nchunk = 0, nr0 = 0;
    int32_t nslot[kNC];
    uint32_t nxo[kNC];
    __amdgpu_buffer_rsrc_t nwlo, nwhi;

    auto fetch_tile = [&](int item, int& te, int& tstart, int& tm, int& tchunk) __attribute__((always_inline)) {
      const int4 tv = tiles[die + kNumXcd * (item / chunks)];
      te = __builtin_amdgcn_readfirstlane(tv.x);
      tstart = __builtin_amdgcn_readfirstlane(tv.y);
      tm = __builtin_amdgcn_readfirstlane(tv.z);
      tchunk = item % chunks;
    };
    auto fetch_rows = [&](int tstart, int tm, int32_t (&slot)[kNC]) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < kNC; ++c) {
        // rows past the tile repeat its last row
        const int i = min(16 * min(jc(c), NBT - 1) + xr, tm - 1);
        slot[c] = kW13 ? perm[tstart + i] : tstart + i;
      }
    };
    // first row and weight descriptors of an item
    auto item_rsrc = [&](int te, int tchunk, int& tr0, __amdgpu_buffer_rsrc_t& tlo,
                         __amdgpu_buffer_rsrc_t& thi) __attribute__((always_inline)) {
      tr0 = __builtin_amdgcn_readfirstlane(tchunk * kRows);
      tlo = make_rsrc(a.wa + (size_t)te * a.st_wa, wbytes);
      thi = kW13 ? make_rsrc(a.wb + (size_t)te * a.st_wb, wbytes) : tlo;
    };
    // offsets of this lane's activation copies of an item
    auto item_xo = [&](const int32_t (&slot)[kNC], uint32_t (&txo)[kNC]) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < kNC; ++c) {
        const uint32_t r = kW13 ? (uint32_t)slot[c] / (uint32_t)a.topk : (uint32_t)slot[c];
        // a copy into the unused column block NBT (odd NBT, waves 4..7) reads out of range:
        // the buffer unit then fetches nothing
        txo[c] = jc(c) < NBT ? 2u * (r * (uint32_t)a.K) + xpiece : 0x80000000u;
      }
    };

    // Activation block kb (this wave's row quads) into a stage.  With an odd NBT the last copy
    // of waves 4..7 targets column block NBT, which no MFMA reads (a stage holds six); its
    // offset is out of the buffer's range, so it fetches nothing.
    auto copy_x = [&](uint8_t* stage, int kb, const uint32_t (&txo)[kNC]) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < kNC; ++c)
        buf_copy16_lds(xrs, stage + (16 * jc(c) + 4 * (wave % 4)) * kXRow, txo[c], (uint32_t)(kXRow * kb));
    };
    // weight rows of this wave: W1/W3 mode row blocks 0, 1 of W1 and the same of W3
    auto load_w1 = [&](const __amdgpu_buffer_rsrc_t& tlo, const __amdgpu_buffer_rsrc_t& thi, int tr0, int kb,
                       int rb, uint4 (&w)[kRB]) __attribute__((always_inline)) {
      const uint32_t row = (uint32_t)(kW13 ? tr0 + 32 * wave + 16 * (rb % 2) : tr0 + 64 * wave + 16 * rb);
      w[rb] = buf_load16(kW13 && rb >= 2 ? thi : tlo, wl, row * wrow + 64u * (uint32_t)kb);
    };
    // Scale rows of an item: contiguous in each scale tensor (the item's rows are
    // consecutive), copied into ss with the buffer-to-LDS copy; pieces past a region's end
    // repeat its last piece into the unused part of the region (W1/W3 mode: two regions of
    // 16 KB, W2 mode one of 32 KB).
    auto copy_scales = [&](int te, int tr0) __attribute__((always_inline)) {
      const int pieces = (int)((kW13 ? kItemWRows / 2 : kItemWRows) * srow / 16);
      constexpr int kPer = (kW13 ? kItemWRows / 2 : kItemWRows) * kMaxScaleRow / 16 / kWave / kWaves;
      const uint32_t src = (uint32_t)tr0 * srow;
      const __amdgpu_buffer_rsrc_t s1 = make_rsrc(a.sa + (size_t)te * a.st_sa, (uint32_t)a.rows * srow);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int chunk = j * kWaves + wave;
        const uint32_t piece = (uint32_t)min(chunk * kWave + lane, pieces - 1);
        buf_copy16_lds(s1, &ss[chunk * kWave * 16], src + 16u * piece, 0);
      }
      if (kW13) {
        const __amdgpu_buffer_rsrc_t s3 = make_rsrc(a.sb + (size_t)te * a.st_sb, (uint32_t)a.rows * srow);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int chunk = j * kWaves + wave;
          const uint32_t piece = (uint32_t)min(chunk * kWave + lane, pieces - 1);
          buf_copy16_lds(s3, &ss[kItemWRows / 2 * kMaxScaleRow + chunk * kWave * 16], src + 16u * piece, 0);
        }
      }
    };

    // four weight sets: block kb lives in set kb % 4, and as K is a multiple of four blocks
    // every item starts in set 0, so its first two blocks can be requested during the
    // previous item's last two steps
    uint4 w0[kRB], w1[kRB], w2[kRB], w3[kRB];
    f32x4 acc[kRB][NBT];
    // Scale bytes of K block kb for this lane's four row blocks, and their conversion to the
    // power-of-two factors.
    auto read_scales = [&](int kb, uint32_t (&sb)[kRB]) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sb[rb] = ss[sa[rb] + 4u * (uint32_t)kb];
    };
    auto to_scales = [&](const uint32_t (&sb)[kRB], float (&sc)[kRB]) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sc[rb] = e8m0_to_f32(sb[rb]);
    };

    // MFMAs of one K block: per MFMA step s the four A operands are converted, then for each
    // column block one B fragment (read two fragments ahead) meets the four A operands.
    auto compute = [&](const uint4 (&w)[kRB], const float (&scale)[kRB], const uint8_t* stage,
                       auto&& request) __attribute__((always_inline)) {
      auto read_b = [&](int f) __attribute__((always_inline)) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(stage + (f % NBT) * 16 * kXRow + bo[f / NBT]));
      };
      constexpr int kF = 4 * NBT;
      bf16x8 bq[3];
      bq[0] = read_b(0);
      bq[1] = read_b(1);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 av[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) av[rb] = dequant8(dword_of(w[rb], s), scale[rb]);
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
          const int f = s * NBT + tb;
          if (f + 2 < kF) bq[(f + 2) % 3] = read_b(f + 2);
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) acc[rb][tb] = mfma16x16x32(av[rb], bq[f % 3], acc[rb][tb]);
          if (tb == 0) request(s);
        }
      }
      // keep that order: the first two B reads; per MFMA step its conversions, then per B
      // fragment the read two ahead and its four MFMAs (the groups count exactly these
      // instructions: the scale bytes are read and converted outside this region)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // conversions
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
          if (s * NBT + tb + 2 < kF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMAs
          if (tb == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // weight request
        }
      }
    };
    // Step kb (kb < nk - 2): copy activation block kb + 1 into the other stage, read the scale
    // bytes of block kb + 1, MFMAs of block kb with the four requests of weight block kb + 2
    // spread over them (one after the first MFMA group of each MFMA step: issued together at
    // the start they held the wave up behind the copies); then wait for the copy (all but the
    // four weight requests) and for this wave's LDS reads, meet at the barrier, and convert
    // the scale bytes read for the next step.  The empty asm keeps the conversion after the
    // barrier: moved up next to the reads, it made every step wait for them before its first
    // MFMA.
    uint32_t sbn[kRB];
    float sc[kRB];
    auto step = [&](int kb, uint8_t* cur, uint8_t* nxt, const uint4 (&wc)[kRB], uint4 (&wn)[kRB])
        __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      copy_x(nxt, kb + 1, xo);
      __builtin_amdgcn_sched_barrier(0);
      read_scales(kb + 1, sbn);
      __builtin_amdgcn_sched_barrier(0);
      compute(wc, sc, cur, [&](int rb) __attribute__((always_inline)) { load_w1(wlo, whi, r0, kb + 2, rb, wn); });
      __builtin_amdgcn_sched_barrier(0);
      wait_then_barrier<kRB>();
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) asm volatile("" : "+v"(sbn[rb]));
      to_scales(sbn, sc);
    };
    // Step nk - 2: as a step, but the weight requests are the next item's block 0 (set 0).
    auto step_penultimate = [&](int kb, uint8_t* cur, uint8_t* nxt, const uint4 (&wc)[kRB], uint4 (&wn)[kRB])
        __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      copy_x(nxt, kb + 1, xo);
      __builtin_amdgcn_sched_barrier(0);
      read_scales(kb + 1, sbn);
      __builtin_amdgcn_sched_barrier(0);
      compute(wc, sc, cur, [&](int rb) __attribute__((always_inline)) { load_w1(nwlo, nwhi, nr0, 0, rb, wn); });
      __builtin_amdgcn_sched_barrier(0);
      wait_then_barrier<kRB>();
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) asm volatile("" : "+v"(sbn[rb]));
      to_scales(sbn, sc);
    };
    // Step nk - 1: every wave has read the scale rows and stage 0 (barrier of step nk - 2), so
    // the next item's activation block 0 and scale rows are copied in while this block's
    // MFMAs run, with its weight block 1 (set 1) requested among them; the wait then covers
    // everything but those four requests, so the next item can start after the epilogue.
    auto step_last = [&](uint8_t* cur, uint8_t* nxt, const uint4 (&wc)[kRB], uint4 (&wn)[kRB])
        __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      copy_x(nxt, 0, nxo);
      copy_scales(ne, nr0);
      __builtin_amdgcn_sched_barrier(0);
      compute(wc, sc, cur, [&](int rb) __attribute__((always_inline)) { load_w1(nwlo, nwhi, nr0, 1, rb, wn); });
      __builtin_amdgcn_sched_barrier(0);
      wait_then_barrier<kRB>();
    };
    // The K loop: the stage (kb % 2) and the weight set (kb % 4) are fixed in each step of a
    // four-step body (nk is a multiple of 4); the last body's last two steps request the next
    // item's first blocks.  The next item's registers are set up before those two steps (the
    // entered item's own when it is the last: its blocks are then re-read and not used).
    auto kloop = [&](bool more) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) acc[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
      read_scales(0, sbn);
      to_scales(sbn, sc);
      int kb = 0;
      for (; kb + 4 < nk; kb += 4) {
        step(kb, xs0, xs1, w0, w2);
        step(kb + 1, xs1, xs0, w1, w3);
        step(kb + 2, xs0, xs1, w2, w0);
        step(kb + 3, xs1, xs0, w3, w1);
      }
      // the next item's rows (W1/W3 mode loads them from the sort's order) two steps ahead of
      // their use, so that they hold no registers through the rest of the loop
      if (more) fetch_rows(nstart, nm, nslot);
      step(kb, xs0, xs1, w0, w2);
      step(kb + 1, xs1, xs0, w1, w3);
      if (more) {
        item_rsrc(ne, nchunk, nr0, nwlo, nwhi);
        item_xo(nslot, nxo);
      } else {
        ne = e;
        nr0 = r0;
        nwlo = wlo;
        nwhi = whi;
        for (int c = 0; c < kNC; ++c) nxo[c] = xo[c];
      }
      step_penultimate(kb + 2, xs0, xs1, w2, w0);
      step_last(xs1, xs0, w3, w1);
    };
    // epilogue: lane holds rows 4q..4q+3 of each row block for column 16 tb + n.  W1/W3 mode
    // picks the activation once per item, so the branch-free body lets the compiler overlap
    // the evaluations of the item's h values.
    auto epilogue_h = [&](int cstart, int cm, int cr0, auto situ_c) __attribute__((always_inline)) {
      constexpr bool situ = decltype(situ_c)::value;
#pragma unroll
      for (int tb = 0; tb < NBT; ++tb) {
        uint32_t hv[kRB / 2][2];
#pragma unroll
        for (int rb = 0; rb < kRB / 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float g0 = acc[rb][tb][i], u0 = acc[rb + kRB / 2][tb][i];
            const float g1 = acc[rb][tb][i + 1], u1 = acc[rb + kRB / 2][tb][i + 1];
            const float h0 = situ ? situ_fast(g0, u0, a.b1, a.b2) : swiglu_fast(g0, u0);
            const float h1 = situ ? situ_fast(g1, u1, a.b1, a.b2) : swiglu_fast(g1, u1);
            hv[rb][i / 2] = pack_bf16x2_rne(h0, h1);
          }
        // one 16-byte store per lane: 8 rows of a position, 64 bytes per position
        uint16_t* tw = reinterpret_cast<uint16_t*>(xt) + wave * 16 * kTrRowH;
#pragma unroll
        for (int rb = 0; rb < kRB / 2; ++rb)
          *reinterpret_cast<uint2*>(tw + n * kTrRowH + 16 * rb + 4 * q) = make_uint2(hv[rb][0], hv[rb][1]);
        const int p = lane / 4;
        const uint4 v = *reinterpret_cast<const uint4*>(tw + p * kTrRowH + 8 * (lane % 4));
        const int col = 16 * tb + p;
        if (col < cm)
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + (size_t)(cstart + col) * a.rows + cr0 +
                                    32 * wave + 8 * (lane % 4)) = v;
      }
    };
    auto epilogue = [&](int cstart, int cm, int cr0) __attribute__((always_inline)) {
      if constexpr (kW13) {
        if (a.gact == K3X_ACT_SITU)
          epilogue_h(cstart, cm, cr0, std::true_type{});
        else
          epilogue_h(cstart, cm, cr0, std::false_type{});
      } else {
        // each store covers 4 positions x 64 rows (256 bytes each)
        float* tw = xt + wave * 16 * kTrRow;
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            *reinterpret_cast<f32x4*>(tw + n * kTrRow + 16 * rb + 4 * q) = acc[rb][tb];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int p = 4 * j + lane / 16;
            const f32x4 v = *reinterpret_cast<const f32x4*>(tw + p * kTrRow + 4 * (lane % 16));
            const int col = 16 * tb + p;
            if (col < cm)
              // non-temporal: the d rows are read once, by the combine, long after the cache
              // has turned over
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(a.out) +
                                                                      (size_t)(cstart + col) * a.rows + cr0 +
                                                                      64 * wave + 4 * (lane % 16)));
          }
        }
      }
    };

    // the class's first item: its first requests (activation block 0 and the scale rows, the
    // oldest, then weight blocks 0 and 1), and the wait for the copies
    {
      int tchunk;
      int32_t slot[kNC];
      fetch_tile(it, e, start, m, tchunk);
      fetch_rows(start, m, slot);
      item_rsrc(e, tchunk, r0, wlo, whi);
      item_xo(slot, xo);
      copy_x(xs0, 0, xo);
      copy_scales(e, r0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) load_w1(wlo, whi, r0, 0, rb, w0);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) load_w1(wlo, whi, r0, 1, rb, w1);
      __builtin_amdgcn_sched_barrier(0);
      wait_then_barrier<2 * kRB>();
    }
    for (;;) {
      const int nit = it + per_die;
      const bool more = nit < hi;
      if (more) fetch_tile(nit, ne, nstart, nm, nchunk);
      // activation block 0 and the scale rows of this item are in LDS for every wave; the
      // K loop ends with the next item's block 0 and scale rows in LDS and its first weight
      // blocks requested
      kloop(more);
      epilogue(start, m, r0);
      it = nit;
      if (!more) break;
      e = ne;
      start = nstart;
      m = nm;
      r0 = nr0;
      for (int c = 0; c < kNC; ++c) xo[c] = nxo[c];
      wlo = nwlo;
      whi = nwhi;
    }
  };
  run_class(ic<1>{}, local_tiles(header[1]) * chunks);
  run_class(ic<2>{}, local_tiles(header[2]) * chunks);
  run_class(ic<3>{}, local_tiles(header[3]) * chunks);
  run_class(ic<4>{}, local_tiles(header[4]) * chunks);
  run_class(ic<5>{}, local_tiles(header[5]) * chunks);
  run_class(ic<6>{}, local_tiles(header[6]) * chunks);
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
  const int32_t* header = reinterpret_cast<const int32_t*>(ws + 8);
  const int4* tiles = reinterpret_cast<const int4*>(ws + L.tiles);
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + L.perm);
  hipError_t err = launch("w13_prefill", gemm_prefill<true>,
                          dim3(prefill_grid(reinterpret_cast<const void*>(&gemm_prefill<true>))),
                          dim3(kThreads), 0, s, a, header, tiles, perm);
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
                dim3(kThreads), 0, s, b, header, tiles, perm);
}

}  // namespace k3x
