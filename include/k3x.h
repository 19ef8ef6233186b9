/*
 * k3x -- routed-expert SwiGLU over MXFP4-packed weights, with a sigmoid + correction-bias
 * top-k router, for AMD Instinct MI355X (gfx950).  Plain C ABI.
 *
 * What is computed (sources: the kimi-k3-in-c README, Part II; the Kimi K3 artifact audit):
 *
 *   router (README section 9 "Picking 16 experts of 896"):
 *     l[t][e] = x[t] . Wr[e]                        (double sum, rounded to float)
 *     s[t][e] = sigmoid(l[t][e])                    (unbiased score)
 *     c[t][e] = s[t][e] + bias[e]                   (selection score; bias steers selection only)
 *     idx[t]  = the topk experts of largest c, picked one at a time; equal c -> lower e first
 *     gates   = s of the chosen experts, divided by their float sum when renorm != 0 and the
 *               sum is > 0, then times routed_scale
 *
 *   expert forward (README section 4 "Reduction one: the experts already ship at half a
 *   byte", and the routed-expert loop of section 9), for every token t and slot j with
 *   e = idx[t][j]:
 *     g = W1_e . x[t],  u = W3_e . x[t]             (W1_e, W3_e: [I][H] MXFP4)
 *     h = bf16_rne(silu(g) * u)                     (silu(g) = g / (1 + exp(-g)), fp32)
 *     d = W2_e . h                                  (W2_e: [H][I] MXFP4)
 *     y[t] = sum_j gates[t][j] * d                  (fp32, slot order)
 *
 *   MXFP4 weight (README section 4; audit section 4.3): element c of row r is
 *   E2M1[nibble] * 2^(scale - 127); the nibble of even c is the low nibble of byte c/2 and
 *   the nibble of odd c is its high nibble; one E8M0 scale byte per 32 consecutive elements
 *   along K; scale byte 255 zeroes its group.  E2M1 = {0, .5, 1, 1.5, 2, 3, 4, 6} with a
 *   sign bit (bit 3).
 *
 * Memory and threading conventions (all calls):
 *  - Every tensor pointer is a DEVICE pointer unless stated; the library never allocates,
 *    frees or copies caller memory, and never allocates device memory in a forward call.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  Device work is
 *    enqueued asynchronously on it; host-detectable errors return at once and enqueue nothing.
 *  - A pool is immutable after creation; concurrent calls on different streams are safe
 *    when each has its own workspace and outputs.
 *  - No exception crosses this ABI.  k3x_last_error() gives a thread-local message about the
 *    latest failing call on the calling thread.
 */
#ifndef K3X_H
#define K3X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum k3x_status {
  K3X_OK = 0,
  K3X_E_INVALID_ARG = -1, /* NULL pointer, negative size, topk out of range, ...          */
  K3X_E_UNSUPPORTED = -2, /* a shape, group size or alignment the library does not support */
  K3X_E_WORKSPACE = -3,   /* workspace missing, misaligned or smaller than required        */
  K3X_E_HIP = -4,         /* a HIP launch or runtime error (message in k3x_last_error)    */
  K3X_E_DROPS = -5        /* k3x_fetch_drops: at least one slot named an invalid expert    */
} k3x_status;

/* Static description of a status code. */
const char *k3x_status_str(k3x_status s);

/* Thread-local text of the latest error raised on this thread ("" if none). */
const char *k3x_last_error(void);

/* ------------------------------------------------------------------------------------------
 * Expert pool: the borrowed device tensors of one MoE layer's routed experts.
 * Layout per expert (audit section 4.3): w1_packed, w3_packed u8 [inter][hidden/2];
 * w1_scale, w3_scale u8 [inter][hidden/32]; w2_packed u8 [hidden][inter/2];
 * w2_scale u8 [hidden][inter/32]; all row-major.  Expert e of tensor k starts at
 * base_k + e * stride_bytes[k]; stride 0 means dense (the tensor's own size).
 * Tensor order in stride_bytes: w1_packed, w1_scale, w3_packed, w3_scale, w2_packed, w2_scale.
 * ---------------------------------------------------------------------------------------- */
/* The gated activation between W1/W3 and W2 (h is rounded to bf16 after it):
 * K3X_ACT_SWIGLU: silu(g) * u.
 * K3X_ACT_SITU:   SiTU-GLU, the engine's own routed-expert activation (README Part II
 *                 section 9, the activation listing): (b1 tanh(g / b1) sigmoid(g)) *
 *                 (b2 tanh(u / b2)), the sigmoid on the uncapped gate; the checkpoint's caps
 *                 are b1 = 4, b2 = 25, so |h| <= 100. */
typedef enum { K3X_ACT_SWIGLU = 0, K3X_ACT_SITU = 1 } k3x_activation;

typedef struct k3x_pool_desc {
  int32_t n_experts; /* 1..8192                                                    */
  int32_t hidden;    /* H: multiple of 128 (e.g. 3584)                              */
  int32_t inter;     /* I: multiple of 128 (e.g. 3072)                              */
  int32_t group;     /* must be 32                                                  */
  const void *w1_packed, *w1_scale, *w3_packed, *w3_scale, *w2_packed, *w2_scale;
  int64_t stride_bytes[6];
  int32_t activation; /* k3x_activation; 0 (a zeroed desc) is SwiGLU               */
  float situ_b1;      /* K3X_ACT_SITU: gate cap, finite and > 0 (4.0 in the checkpoint) */
  float situ_b2;      /* K3X_ACT_SITU: up cap, finite and > 0 (25.0 in the checkpoint)  */
  int32_t contract;   /* 0: the routed path's arithmetic (per-group fp32 sums, h in bf16);
                         1: the floating point contract of README Part II sections 4 and 5
                         (per row, groups summed in sequence in double, each the sequential
                         double sum of its products times its scale, one rounding to float;
                         h kept in fp32) -- one token per call only                       */
} k3x_pool_desc;

typedef struct k3x_pool k3x_pool;

/* Validates d and creates a host-side handle in *out.  Refuses (K3X_E_UNSUPPORTED)
 * group != 32, hidden or inter not a multiple of 128, packed pointers or strides not
 * 16-byte aligned, and a contract pool with hidden or inter above 4096; refuses
 * (K3X_E_INVALID_ARG) NULL pointers, n_experts out of range, strides smaller than the dense
 * tensor size, an unknown activation, contract not 0 or 1 and, for SiTU-GLU, caps that are
 * not finite and positive.  Allocates host memory only; the device
 * tensors are borrowed and must outlive the pool.  Scale bytes are read as given: bytes
 * 2..252 give finite, normal weights for every E2M1 code (6 * 2^125 is the largest); 255
 * zeroes a group; 0, 1, 253 and 254 are outside the range the library promises to reproduce
 * exactly (253 and 254 overflow float for the larger codes, 0 and 1 give subnormal weights). */
k3x_status k3x_expert_pool_create(const k3x_pool_desc *d, k3x_pool **out);

/* Frees the handle only (never the borrowed tensors).  NULL is a no-op. */
void k3x_expert_pool_destroy(k3x_pool *p);

/* ------------------------------------------------------------------------------------------
 * Router (README section 9).
 * ---------------------------------------------------------------------------------------- */
typedef struct k3x_router_desc {
  const void *weight; /* bf16 [n_experts][hidden], row-major, 16-byte aligned          */
  const float *bias;  /* fp32 [n_experts] correction bias, or NULL for none             */
  int32_t n_experts;  /* 1..4096                                                        */
  int32_t hidden;     /* multiple of 8, <= 16384                                        */
  int32_t topk;       /* 1..n_experts                                                   */
  int32_t renorm;     /* nonzero: divide the gates by their sum when the sum is > 0     */
  float routed_scale; /* gates are multiplied by this last                              */
} k3x_router_desc;

/* Bytes of device workspace k3x_route_topk needs for T tokens (0 if r is invalid). */
size_t k3x_route_workspace_size(const k3x_router_desc *r, int32_t T);

/* Routes T tokens.  x_bf16: bf16 [T][hidden] (16-byte aligned).  Outputs idx_out int32
 * [T][topk] in selection order (descending selection score, equal scores -> lower expert
 * first) and gates_out fp32 [T][topk].  ws: device workspace of at least
 * k3x_route_workspace_size bytes, 256-byte aligned.  T = 0 enqueues nothing.
 * The logits are summed in double in a fixed order and the sigmoid is evaluated in double
 * and rounded once to float, so the selection is reproducible bit for bit. */
k3x_status k3x_route_topk(const k3x_router_desc *r, const void *x_bf16, int32_t T,
                          int32_t *idx_out, float *gates_out, void *ws, size_t ws_bytes,
                          void *stream);

/* ------------------------------------------------------------------------------------------
 * Expert forward (README sections 4 and 9).
 * ---------------------------------------------------------------------------------------- */

/* Bytes of device workspace k3x_moe_forward needs for T tokens with topk slots each
 * (0 if the arguments are invalid).  It holds the drop counter, the expert-sorted slot
 * list, h (bf16 [T*topk][inter]) and the per-slot expert outputs (fp32 [T*topk][hidden]). */
size_t k3x_moe_workspace_size(const k3x_pool *p, int32_t T, int32_t topk);

/* y[t] = sum_j gates[t][j] * W2_e(bf16(silu(W1_e x[t]) * (W3_e x[t]))), e = idx[t][j].
 * x_bf16: bf16 [T][hidden], 16-byte aligned; idx int32 [T][topk]; gates fp32 [T][topk];
 * y fp32 [T][hidden], overwritten (not accumulated).  topk in 1..64.  Duplicate experts
 * within a token are allowed (slots are independent).  A slot whose expert id lies outside
 * [0, n_experts) contributes 0 and is counted in the workspace's drop counter, which each
 * call resets; read it with k3x_fetch_drops.  T = 0 only resets the counter.  A contract pool
 * (k3x_pool_desc.contract = 1) takes T <= 1 and returns K3X_E_UNSUPPORTED for more; its y
 * follows the contract's arithmetic, with h in fp32 instead of bf16. */
k3x_status k3x_moe_forward(const k3x_pool *p, const void *x_bf16, int32_t T, const int32_t *idx,
                           const float *gates, int32_t topk, float *y, void *ws,
                           size_t ws_bytes, void *stream);

/* Router and experts in one call (README Part II section 9: route, then the experts of the
 * picks): the same idx_out, gates_out and y, bit for bit, as k3x_route_topk followed by
 * k3x_moe_forward on them.  Requires r->n_experts == p->E, r->hidden == p->H, topk <= 64
 * (K3X_E_INVALID_ARG / K3X_E_UNSUPPORTED otherwise); one workspace serves both steps.
 * x_bf16 bf16 [T][hidden]; idx_out int32 [T][topk], gates_out fp32
 * [T][topk], y fp32 [T][hidden] (all written); ws: at least k3x_route_moe_workspace_size
 * bytes, 256-byte aligned, its start is the experts' workspace (k3x_fetch_drops(ws) reads
 * the drop count).  T = 0 routes nothing and only resets the drop counter (x, idx_out,
 * gates_out and y may then be NULL). */
size_t k3x_route_moe_workspace_size(const k3x_router_desc *r, const k3x_pool *p, int32_t T);
k3x_status k3x_route_moe_forward(const k3x_router_desc *r, const k3x_pool *p, const void *x_bf16,
                                 int32_t T, int32_t *idx_out, float *gates_out, float *y,
                                 void *ws, size_t ws_bytes, void *stream);

/* The previous layer's residual update and this layer's RMSNorm (README section 5, "Kernels
 * with a floating point contract"), then the router and the experts (README Part II section
 * 9), in one call:
 *   x_next = bf16_rne(float(x) + y_prev)       (when y_prev != NULL; else x_next = x, unwritten)
 *   xn     = RMSNorm(x_next), unit weight, eps (as k3x_rmsnorm_bf16)
 *   idx_out, gates_out, y = k3x_route_moe_forward on xn.
 * All four outputs equal those of k3x_residual_add_rmsnorm_bf16 (or k3x_rmsnorm_bf16 when
 * y_prev is NULL) followed by k3x_route_moe_forward, bit for bit.  At one token, when the
 * single-token decode applies, the update and the norm run inside the router's scores launch
 * (three launches per layer instead of four).
 * x bf16 [T][hidden] (read only); y_prev fp32 [T][hidden] or NULL (the first layer);
 * x_next bf16 [T][hidden] (written when y_prev != NULL, may be NULL otherwise); xn bf16
 * [T][hidden] (written: the router's and experts' input, for a caller that also needs it);
 * idx_out, gates_out, y, ws, ws_bytes as k3x_route_moe_forward (same workspace size).  y may
 * be y_prev: a chain of layers can pass one y buffer and swap two x buffers.  x_next must not
 * overlap x, y_prev or xn, and xn must not overlap x, y_prev or y (K3X_E_INVALID_ARG); all
 * pointers 16-byte aligned, hidden a multiple of 8 and <= 16384 (K3X_E_UNSUPPORTED).  Other
 * errors as k3x_route_moe_forward; T = 0 only resets the drop counter. */
k3x_status k3x_residual_route_moe_forward(const k3x_router_desc *r, const k3x_pool *p,
                                          const void *x_bf16, const float *y_prev, float eps,
                                          void *x_next_bf16, void *xn_bf16, int32_t T,
                                          int32_t *idx_out, float *gates_out, float *y, void *ws,
                                          size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): k3x_moe_forward with its workspace in a
 * scratch array built into the library instead of a caller's buffer.  Each GPU the library
 * runs on holds its own K3X_NOALLOC_SCRATCH_BYTES (32 MiB) of it from module load until the
 * process ends; the call itself allocates nothing, host or device.  Arguments as
 * k3x_moe_forward (the calling thread's current device must be that of the stream and the
 * pointers).  drops_out: NULL, or a DEVICE int64 that receives this call's drop count
 * (copied on the stream after the forward).  Refuses (K3X_E_UNSUPPORTED) a call whose
 * workspace, k3x_moe_workspace_size(p, T, topk), exceeds the scratch (at the K3 shape, hidden
 * 3584 and inter 3072, up to T = 102 at topk 16), and enqueues nothing then.  Every call on one GPU
 * uses that GPU's one scratch, which keeps the last call's contents: calls that overlap in
 * time on one GPU (other streams or threads) race and must be serialised by the caller. */
#define K3X_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
k3x_status k3x_moe_forward_noalloc(const k3x_pool *p, const void *x_bf16, int32_t T,
                                   const int32_t *idx, const float *gates, int32_t topk, float *y,
                                   int64_t *drops_out, void *stream);

/* Waits for stream, then stores in *n the number of dropped slots of the latest
 * k3x_moe_forward that used ws.  Returns K3X_E_DROPS when *n > 0 (the run must be treated
 * as invalid), K3X_OK when 0.  n is a host pointer. */
k3x_status k3x_fetch_drops(const void *ws, int64_t *n, void *stream);

/* ------------------------------------------------------------------------------------------
 * Hidden-state helpers for chaining layers (README section 5 "Kernels with a floating point
 * contract"): RMSNorm with unit weight and a double sum of squares, eps inside the square
 * root, and the residual update.
 * ---------------------------------------------------------------------------------------- */

/* out[t] = bf16_rne(x[t] * inv_t), inv_t = (float)(1 / sqrt(sum_h x[t][h]^2 / H + eps)),
 * the sum taken in double in a fixed order.  x, out: bf16 [T][H] (16-byte aligned; may
 * alias); H a multiple of 8, <= 16384. */
k3x_status k3x_rmsnorm_bf16(const void *x, int32_t T, int32_t H, float eps, void *out,
                            void *stream);

/* x[t][h] <- bf16_rne(float(x[t][h]) + y[t][h]).  x bf16 [T][H], y fp32 [T][H]; H a
 * multiple of 8. */
k3x_status k3x_residual_add_bf16(void *x, const float *y, int32_t T, int32_t H, void *stream);

/* The residual update of one layer fused with the RMSNorm that starts the next:
 * x[t][h] <- bf16_rne(float(x[t][h]) + y[t][h]), then out[t] <- RMSNorm(x[t]) exactly as
 * k3x_rmsnorm_bf16 computes it (same summation order), so the results equal those of
 * k3x_residual_add_bf16 followed by k3x_rmsnorm_bf16 bit for bit, in one launch.
 * x bf16 [T][H] (updated in place), y fp32 [T][H], out bf16 [T][H]; all 16-byte aligned;
 * out must not overlap x or y (K3X_E_INVALID_ARG); H a multiple of 8, <= 16384
 * (K3X_E_UNSUPPORTED). */
k3x_status k3x_residual_add_rmsnorm_bf16(void *x, const float *y, int32_t T, int32_t H,
                                         float eps, void *out, void *stream);

/* ------------------------------------------------------------------------------------------
 * Latent MoE block (README Part II section 9, the k3_moe listing): the routed experts inside
 * the block that wraps them.  Per token:
 *   1. route on the full width D (router desc with hidden = D);
 *   2. z = bf16(down . x);
 *   3. acc = the routed experts on z (pool with hidden = L, the latent), as k3x_moe_forward;
 *   4. a = bf16 RMSNorm of the AGGREGATE acc with norm_weight (latent_norm != 0; the sum of
 *      squares in double in a fixed order, (acc * inv) * w), or a = bf16(acc);
 *   5. out = up . a;
 *   6. out += sh2 . s, s = bf16(act(sh1 . x, sh3 . x)): the shared experts on the ORIGINAL x,
 *      added unweighted (act = shared_activation with the caps).
 * Dense products are bf16 x bf16, exact in double and summed in double in a fixed order, then
 * rounded once to float (the floating point contract's bf16 matmul, README Part II section 5);
 * the path is sized for decode batches (larger ones read the dense weights once per 8 tokens).
 * ---------------------------------------------------------------------------------------- */
typedef struct k3x_latent_desc {
  int32_t hidden;           /* D: multiple of 512, <= 8192 (7168 in the checkpoint)        */
  int32_t shared_inter;     /* S = n_shared * inter: multiple of 512, L + S <= 9728 (6144) */
  const void *down;         /* bf16 [L][D], L = the routed pool's hidden                    */
  const void *up;           /* bf16 [D][L]                                                  */
  const void *sh1, *sh3;    /* bf16 [S][D]: gate and up rows of the shared experts          */
  const void *sh2;          /* bf16 [D][S]                                                  */
  int32_t latent_norm;      /* nonzero: RMSNorm of the aggregate (the checkpoint: 1)        */
  const float *norm_weight; /* fp32 [L], or NULL for weight 1                               */
  float eps;                /* RMSNorm eps, >= 0                                            */
  int32_t shared_activation; /* k3x_activation of the shared experts                        */
  float situ_b1, situ_b2;   /* K3X_ACT_SITU caps of the shared experts                      */
} k3x_latent_desc;

/* Bytes of device workspace k3x_latent_forward needs (0 if the arguments are invalid). */
size_t k3x_latent_workspace_size(const k3x_latent_desc *d, const k3x_pool *p,
                                 const k3x_router_desc *r, int32_t T);

/* Runs the block on T tokens.  x_bf16 bf16 [T][D] -> out fp32 [T][D] (overwritten); all device
 * pointers 16-byte aligned; ws: at least k3x_latent_workspace_size bytes, 256-byte aligned.
 * Refuses (K3X_E_INVALID_ARG) NULL weights or mismatched widths (router hidden != D, pool
 * hidden != L) and (K3X_E_UNSUPPORTED) D, L or S not multiples of 512 or above 8192, or
 * L + S above 9728 (the K3 block: 3584 + 6144), or topk above 64.  Dropped
 * routed slots are counted in the workspace as for k3x_moe_forward (k3x_fetch_drops on
 * ws + offs[5] of k3x_latent_ws_layout).  T = 0 only resets that counter. */
k3x_status k3x_latent_forward(const k3x_latent_desc *d, const k3x_pool *p,
                              const k3x_router_desc *r, const void *x_bf16, int32_t T,
                              float *out, void *ws, size_t ws_bytes, void *stream);

/* Byte offsets, inside the block's workspace for T tokens, of its intermediates (256-byte
 * aligned), readable once k3x_latent_forward has completed on its stream:
 *   offs[0] idx int32 [T][topk]   offs[1] gates fp32 [T][topk]   offs[2] z bf16 [T][L]
 *   offs[3] acc fp32 [T][L] (the aggregate of the routed experts)
 *   offs[4] s bf16 [T][S] (the shared experts' activation)
 *   offs[5] the routed experts' workspace (its drop counter first, read by k3x_fetch_drops).
 * Returns K3X_OK, or the error k3x_latent_forward would return for these arguments. */
k3x_status k3x_latent_ws_layout(const k3x_latent_desc *d, const k3x_pool *p,
                                const k3x_router_desc *r, int32_t T, size_t offs[6]);

/* ------------------------------------------------------------------------------------------
 * Expert arena: pools larger than HBM (README Part II section 12 "An LRU cache for the
 * experts", section 13 "How big should that cache be? Ask the trace").  n_slots experts are
 * resident in an HBM arena; the rest stay in a backing store in pinned host memory and are
 * copied in on demand.  A slot holds an expert, or is EMPTY, or INFLIGHT; a miss takes the
 * lowest EMPTY slot, else the least recently used slot that is not in flight, pinned or held
 * by the same batch (recency: one tick per request).  A batch reserves serially, copies its
 * misses in the backing store's offset order, then publishes them.  Host-side state; use an
 * arena from one host thread and one stream.
 * ---------------------------------------------------------------------------------------- */
typedef struct k3x_arena k3x_arena;

typedef struct k3x_arena_desc {
  int32_t n_slots;            /* experts resident at once, 1..8192                          */
  int32_t n_layers;           /* the backing store holds n_layers * n_experts experts       */
  int32_t n_experts;          /* per layer                                                  */
  int32_t hidden, inter, group; /* as k3x_pool_desc (group 32)                              */
  const void *host[6];        /* backing store, PINNED host memory (hipHostMalloc): tensor k
                                 (w1_packed, w1_scale, w3_packed, w3_scale, w2_packed,
                                 w2_scale) of expert (l, e) at host[k] + (l * n_experts + e)
                                 * host_stride[k]; when the six are back to back with one
                                 stride, an expert is one copy, else six                    */
  int64_t host_stride[6];     /* bytes, 0 = the tensor's dense size                         */
  int32_t max_slots_per_call; /* T * topk bound of k3x_arena_moe_forward                    */
  int32_t activation;         /* as k3x_pool_desc                                           */
  float situ_b1, situ_b2;
} k3x_arena_desc;

/* Bytes of one expert's six tensors (17,547,264 at hidden 3584, inter 3072); 0 if invalid. */
size_t k3x_expert_bytes(int32_t hidden, int32_t inter);

/* Allocates the arena: n_slots * (k3x_expert_bytes rounded up to 256) bytes of device memory,
 * pinned host and device buffers of max_slots_per_call ids, and a pool over the slots.
 * Refuses NULL backing pointers, strides below the dense sizes or sizes out of range
 * (K3X_E_INVALID_ARG), shapes a pool refuses (K3X_E_UNSUPPORTED); K3X_E_HIP when the device
 * allocation fails (k3x_arena_last_error says why).  The backing store is borrowed. */
k3x_status k3x_arena_create(const k3x_arena_desc *d, k3x_arena **out);
void k3x_arena_destroy(k3x_arena *a);
const char *k3x_arena_last_error(void);

/* The pool whose experts are the arena's slots (owned by the arena). */
const k3x_pool *k3x_arena_pool(const k3x_arena *a);

/* Makes experts[0..n) of one layer resident (host int32 ids; ids outside [0, n_experts) are
 * skipped) and writes slots_out[j] (host int32): the slot of experts[j], or -1 when none
 * could be given (every slot in flight, pinned or held by this batch).  An id repeated in
 * the batch shares its first request's slot.  The copies are enqueued on stream (ordered
 * before any later work on it); *hits and *misses (host, may be NULL) count this call. */
k3x_status k3x_arena_getmany(k3x_arena *a, int32_t layer, const int32_t *experts, int32_t n,
                             int32_t *slots_out, int32_t *hits, int32_t *misses, void *stream);

/* Pins a resident expert: its slot is never evicted (K3X_E_INVALID_ARG if not resident). */
k3x_status k3x_arena_pin(k3x_arena *a, int32_t layer, int32_t expert);

/* Totals since creation: requests that hit, requests that missed, bytes copied in. */
k3x_status k3x_arena_stats(const k3x_arena *a, int64_t *hits, int64_t *misses, int64_t *bytes);

/* The expert forward of one layer through the arena: copies idx (device int32 [T][topk]) to
 * the host (this waits for the stream), makes the call's distinct experts resident in slot
 * order (token-major), writes the slot ids to the device and runs k3x_moe_forward on the
 * arena's pool.  The result equals k3x_moe_forward on a pool holding the layer's experts,
 * bit for bit.  Experts that got no slot are dropped (k3x_fetch_drops on ws counts them).
 * T * topk <= max_slots_per_call (else K3X_E_UNSUPPORTED); ws as k3x_moe_forward on
 * k3x_arena_pool.  Waits for the stream again before returning. */
k3x_status k3x_arena_moe_forward(k3x_arena *a, int32_t layer, const void *x_bf16, int32_t T,
                                 const int32_t *idx, const float *gates, int32_t topk, float *y,
                                 void *ws, size_t ws_bytes, int32_t *hits, int32_t *misses,
                                 void *stream);

/* Trace replay (host only): the hits of a replacement rule with cap slots over trace[0..n)
 * (keys, one request each).  K3X_CACHE_LRU is the arena's own policy; K3X_CACHE_BELADY evicts
 * the key needed furthest ahead (a ceiling, not a policy); K3X_CACHE_PIN_LRU is LRU with the
 * keys pinned[0..n_pinned) never evicted once resident. */
typedef enum { K3X_CACHE_LRU = 0, K3X_CACHE_BELADY = 1, K3X_CACHE_PIN_LRU = 2 } k3x_cache_policy;
k3x_status k3x_cache_replay(const int64_t *trace, int64_t n, int32_t cap, int32_t policy,
                            const int64_t *pinned, int32_t n_pinned, int64_t *hits);

/* The arena's policy over batches without a device: batch b is keys[batch_start[b] ..
 * batch_start[b + 1]); slots_out[j] is the slot given to keys[j] (-1: none). */
k3x_status k3x_cache_replay_batches(const int64_t *keys, const int64_t *batch_start,
                                    int64_t n_batches, int32_t cap, int32_t *slots_out);

/* ------------------------------------------------------------------------------------------
 * Kernel timing (instrumentation only; the work done is unchanged).  While a profiler is
 * attached to the calling thread, every kernel the library enqueues from that thread is
 * bracketed by two HIP events recorded on the same stream, up to the profiler's capacity.
 * ---------------------------------------------------------------------------------------- */
typedef struct k3x_profiler k3x_profiler;

/* Creates a profiler able to record `capacity` (1..1<<20) kernel launches.  Creates 2 *
 * capacity HIP events on the current device. */
k3x_status k3x_profiler_create(int32_t capacity, k3x_profiler **out);

/* Destroys the events and the handle (detaches it first if attached).  NULL is a no-op. */
void k3x_profiler_destroy(k3x_profiler *p);

/* Attaches p to the calling thread (NULL detaches).  One profiler per thread at a time. */
k3x_status k3x_profiler_attach(k3x_profiler *p);

/* Forgets the recorded launches (the events are reused). */
k3x_status k3x_profiler_reset(k3x_profiler *p);

/* Number of launches recorded since the last reset (at most the capacity). */
int32_t k3x_profiler_count(const k3x_profiler *p);

/* Waits for launch i's stop event, then returns its kernel name (a static string) and its
 * duration in milliseconds.  name and ms are host pointers. */
k3x_status k3x_profiler_read(k3x_profiler *p, int32_t i, const char **name, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* K3X_H */
