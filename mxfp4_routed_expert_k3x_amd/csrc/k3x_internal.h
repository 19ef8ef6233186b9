// Internal declarations of the k3x HIP library (gfx950 only).
//
// Nothing here is shared with the CPU oracle: conversions, decoders and reductions below
// are this library's own.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/k3x.h"

namespace k3x {

// ---------------------------------------------------------------------------------------
// Vector types used by the gfx950 builtins
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 32;   // MX group along K
constexpr int kKBlock = 128; // K per main-loop step: 4 groups, one per lane quarter
constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

// ---------------------------------------------------------------------------------------
// bf16 <-> f32
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Round-to-nearest-even narrowing of a float to bf16 bits.  NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------------------
// MXFP4 decode: one E8M0 byte -> the float 2^(s-127); byte 255 -> 0 (zeroes the group).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  // s in 1..254 is a normal float exponent field; s = 0 gives 2^-127 (subnormal)
  const float v = s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
  return s == 255u ? 0.0f : v;
}

// Eight consecutive E2M1 elements (the four bytes of one dword, low nibble = even element)
// times a power-of-two scale, as eight bf16 in element order.  The products are exact and
// normal for scale bytes 2..252 (0.5 * 2^-125 = 2^-126 is the smallest, 6 * 2^125 the largest).
__device__ __forceinline__ bf16x8 dequant8(uint32_t dw, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// tanh for the GEMM epilogues (h is rounded to bf16 right after): the odd series to x^7 for
// |x| < 1/8 (next term below 2e-10), else (1 - e) / (1 + e) with e = exp(-2|x|) from the
// hardware exponential; the sign is copied back.
__device__ __forceinline__ float tanh_fast(float x) {
  const float ax = fabsf(x);
  const float x2 = x * x;
  const float p =
      ax * (1.0f + x2 * (-1.0f / 3.0f + x2 * (2.0f / 15.0f + x2 * (-17.0f / 315.0f))));
  const float e = __expf(-2.0f * ax);
  const float q = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
  return copysignf(ax < 0.125f ? p : q, x);
}

// SiTU-GLU for the GEMM epilogues: (b1 tanh(g / b1) sigmoid(g)) * (b2 tanh(u / b2)), the
// sigmoid on the uncapped gate (kimi-k3-in-c README, Part II section 9, the activation
// listing), with the hardware exponential and reciprocal.
__device__ __forceinline__ float situ_fast(float g, float u, float b1, float b2) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  const float a = b1 * tanh_fast(__fdividef(g, b1)) * sg;
  return a * (b2 * tanh_fast(__fdividef(u, b2)));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// XCD-aware placement: workgroups are dealt to the 8 dies round-robin, so workgroup b runs
// on die b % 8.  Returns this workgroup's die and its rank among the die's workgroups.
__device__ __forceinline__ void xcd_rank(int& die, int& rank, int& per_die) {
  die = blockIdx.x % kNumXcd;
  rank = blockIdx.x / kNumXcd;
  per_die = gridDim.x / kNumXcd;  // grids are launched as a multiple of 8
}

// ---------------------------------------------------------------------------------------
// Workspace layout of k3x_moe_forward (byte offsets; every region 256-byte aligned)
// ---------------------------------------------------------------------------------------
// Tile classes of the sort: class k holds the tiles of 16 k + 1 .. 16 k + 16 slots.
constexpr int kMaxTileClasses = 6;

struct MoeLayout {
  size_t drops;       // int64 drop counter, int32 n_tiles at +8, int32 end of each tile class
                      // [kMaxTileClasses] at +12 (64 bytes)
  size_t offsets;     // int32 [E + 1] start of each expert's slots in perm
  size_t tiles;       // int32 [max_tiles][4] = expert, first slot in perm, count, pad
  size_t perm;        // int32 [T * topk] slot ids (t * topk + j) grouped by expert
  size_t inv;         // int32 [T * topk] position of each slot in perm, -1 if dropped
  size_t h;           // bf16 [T * topk][I]
  size_t d;           // fp32 [T * topk][H]
  size_t sort_parts;  // int32 [sort_n][E] per-part expert counts (then cursors) + [sort_n] drops
  size_t total;
  int32_t max_tiles;
  int32_t tile_tokens;
  int32_t sort_n;     // parts of the split sort (0: one workgroup sorts everything)
};

MoeLayout moe_layout(int32_t E, int32_t H, int32_t I, int32_t T, int32_t topk);

// ---------------------------------------------------------------------------------------
// Pool handle
// ---------------------------------------------------------------------------------------
}  // namespace k3x

struct k3x_pool {
  int32_t E, H, I;
  const uint8_t* base[6];
  int64_t stride[6];
  int32_t act;   // k3x_activation
  float b1, b2;  // SiTU-GLU caps
  int32_t contract;  // 1: the floating point contract's arithmetic (k3x_contract.hip)
};

namespace k3x {

// ---------------------------------------------------------------------------------------
// Launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------------------
hipError_t launch_route(const k3x_router_desc& r, const uint16_t* x, int32_t T, int32_t* idx,
                        float* gates, float* scores, hipStream_t s);
// The sigmoid scores alone (fp32 [T][E]).
hipError_t launch_route_scores(const k3x_router_desc& r, const uint16_t* x, int32_t T,
                               float* scores, hipStream_t s);
// One token's scores with the hidden-state update and RMSNorm before the router folded in:
// x_next = bf16(x + y_prev) (skipped when y_prev is NULL; x_next may then be NULL too), xn =
// the RMSNorm of that (unit weight, eps), scores = the router's scores of xn; all three equal
// those of launch_residual_rmsnorm (or launch_rmsnorm) followed by launch_route_scores, bit for
// bit.  x_next must not overlap x (other workgroups still read x while workgroup 0 writes it).
bool route_scores_residual_supported(const k3x_router_desc& r, int32_t T);
hipError_t launch_route_scores_residual(const k3x_router_desc& r, const uint16_t* x,
                                        const float* y_prev, float eps, uint16_t* x_next,
                                        uint16_t* xn, float* scores, hipStream_t s);
// The selection alone, on scores fp32 [T][E] already computed.
hipError_t launch_route_select(const k3x_router_desc& r, int32_t T, const float* scores,
                               int32_t* idx, float* gates, hipStream_t s);

hipError_t launch_moe(const k3x_pool& p, const uint16_t* x, int32_t T, const int32_t* idx,
                      const float* gates, int32_t topk, float* y, uint8_t* ws,
                      const MoeLayout& L, hipStream_t s);

// One token in the floating point contract's arithmetic (k3x_contract.hip).
bool contract_supported(const k3x_pool& p, int32_t T, int32_t topk);
size_t contract_ws(const k3x_pool& p, int32_t topk, size_t* off_h, size_t* off_d);
hipError_t launch_contract(const k3x_pool& p, const uint16_t* x, const int32_t* idx,
                           const float* gates, int32_t topk, float* y, uint8_t* ws,
                           hipStream_t s);

// Single-token decode in the reference arithmetic order (k3x_decode.hip).
bool decode_exact_supported(const k3x_pool& p, int32_t T, int32_t topk);
size_t decode_exact_ws(const k3x_pool& p, int32_t topk, size_t* off_h);
hipError_t launch_decode_exact(const k3x_pool& p, const uint16_t* x, const int32_t* idx,
                               const float* gates, int32_t topk, float* y, uint8_t* ws,
                               hipStream_t s);
// Router and single-token decode in three launches: route_scores, then W1/W3 with the
// selection run by every workgroup (no separate selection launch), then W2 + combine.  Its
// picks, gates and y equal launch_route followed by launch_decode_exact, bit for bit.
bool decode_routed_supported(const k3x_router_desc& r, const k3x_pool& p, int32_t T);
hipError_t launch_decode_routed(const k3x_router_desc& r, const k3x_pool& p, const uint16_t* x,
                                float* scores, int32_t* idx, float* gates, float* y, uint8_t* ws,
                                hipStream_t s);
// The same with the residual update and RMSNorm folded into the scores launch
// (launch_route_scores_residual); the experts read xn.
bool decode_routed_residual_supported(const k3x_router_desc& r, const k3x_pool& p, int32_t T);
hipError_t launch_decode_routed_residual(const k3x_router_desc& r, const k3x_pool& p,
                                         const uint16_t* x, const float* y_prev, float eps,
                                         uint16_t* x_next, uint16_t* xn, float* scores,
                                         int32_t* idx, float* gates, float* y, uint8_t* ws,
                                         hipStream_t s);
// Latent MoE block (k3x_dense.hip): workspace layout and launcher.
struct LatentLayout {
  size_t scores;  // router scores fp32 [T][E]
  size_t idx;     // int32 [T][topk]
  size_t gates;   // fp32 [T][topk]
  size_t z;       // bf16 [T][L] latent input of the routed experts
  size_t acc;     // fp32 [T][L] their aggregate
  size_t s;       // bf16 [T][S] shared experts' activation
  size_t moe;     // the routed experts' workspace
};
LatentLayout latent_layout(const k3x_latent_desc& d, const k3x_pool& p, int32_t E, int32_t T,
                           int32_t topk);
hipError_t launch_latent(const k3x_latent_desc& d, const k3x_pool& p, const k3x_router_desc& r,
                         const uint16_t* x, int32_t T, float* out, uint8_t* ws,
                         const LatentLayout& L, const MoeLayout& ML, hipStream_t s);

// Prefill-sized grouped GEMMs (k3x_prefill.hip): expert tiles of up to 128 slots.
int prefill_tile_tokens();
hipError_t launch_prefill_gemms(const k3x_pool& p, const uint16_t* x, int32_t T, int32_t topk, uint8_t* ws,
                                const MoeLayout& L, hipStream_t s);

// True when the sorted-tile kernels take the batch: two or more tokens, hidden and inter
// multiples of 512, K <= 4096 and 32-bit row offsets.
inline bool use_prefill(int32_t E, int32_t H, int32_t I, int32_t T, int32_t topk) {
  // Tiles of 96 slots; items of 256 h rows (W1/W3) or 512 d rows (W2); the item's scale rows
  // (K / 32 bytes each, K <= 4096) fit in LDS.  (They also stream the weights of lightly
  // shared experts faster than the 16-slot tiles.)  A single token takes the exact decode
  // path before this is asked.
  (void)E;
  const int64_t slots = (int64_t)T * topk;
  return T >= 2 && H % 512 == 0 && I % 512 == 0 && H <= 4096 && I <= 4096 &&
         slots * (int64_t)(H > I ? H : I) < ((int64_t)1 << 31);
}

hipError_t launch_rmsnorm(const uint16_t* x, int32_t T, int32_t H, float eps, uint16_t* out,
                          hipStream_t s);

hipError_t launch_residual(uint16_t* x, const float* y, int32_t T, int32_t H, hipStream_t s);
// x_out <- bf16(x + y) and out <- rmsnorm(x_out); x_out may be x, out overlaps neither.
hipError_t launch_residual_rmsnorm(const uint16_t* x, const float* y, int32_t T, int32_t H,
                                   float eps, uint16_t* x_out, uint16_t* out, hipStream_t s);

int device_cu_count();

// Records a message as the calling thread's last error (k3x_last_error) and returns st.
k3x_status fail_status(k3x_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// The same for a HIP error: "where: <HIP error string>", K3X_E_HIP.
k3x_status hip_status(hipError_t e, const char* where);

// When a profiler is attached to the calling thread and has room, reserves the next record
// for kernel `name` and returns its start/stop events.
bool profiler_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Enqueues one kernel.  With a profiler attached the launch carries the record's events,
// which the runtime stamps at the start and end of that dispatch itself.
template <typename F, typename... Args>
inline hipError_t launch(const char* name, F kernel, dim3 grid, dim3 block, uint32_t shm,
                         hipStream_t s, Args... args) {
  hipEvent_t start, stop;
  if (profiler_events(name, &start, &stop))
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, start, stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
  return hipGetLastError();
}

}  // namespace k3x
