// C ABI of the k3x library: argument validation, workspace layout and dispatch.
// The operations are defined in include/k3x.h (with their sources on the pages).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include <cmath>

#include "k3x_internal.h"

namespace {

thread_local char g_last_error[512] = "";

k3x_status fail(k3x_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

k3x_status hip_fail(hipError_t e, const char* where) {
  return fail(K3X_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

namespace k3x {

k3x_status fail_status(k3x_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

k3x_status hip_status(hipError_t e, const char* where) { return hip_fail(e, where); }

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return (n + kNumXcd - 1) / kNumXcd * kNumXcd;
}

}  // namespace k3x

extern "C" {

const char* k3x_status_str(k3x_status s) {
  switch (s) {
    case K3X_OK: return "ok";
    case K3X_E_INVALID_ARG: return "invalid argument";
    case K3X_E_UNSUPPORTED: return "unsupported shape, group size or alignment";
    case K3X_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case K3X_E_HIP: return "HIP launch or runtime error";
    case K3X_E_DROPS: return "slots with invalid expert ids were dropped";
  }
  return "unknown status";
}

const char* k3x_last_error(void) { return g_last_error; }

k3x_status k3x_expert_pool_create(const k3x_pool_desc* d, k3x_pool** out) {
  if (!d || !out) return fail(K3X_E_INVALID_ARG, "pool_create: NULL desc or out");
  *out = nullptr;
  if (d->n_experts < 1 || d->n_experts > 8192)
    return fail(K3X_E_INVALID_ARG, "pool_create: n_experts %d not in 1..8192", d->n_experts);
  if (d->group != 32) return fail(K3X_E_UNSUPPORTED, "pool_create: group %d != 32", d->group);
  if (d->hidden <= 0 || d->inter <= 0)
    return fail(K3X_E_INVALID_ARG, "pool_create: hidden %d / inter %d", d->hidden, d->inter);
  if (d->hidden % 128 || d->inter % 128)
    return fail(K3X_E_UNSUPPORTED, "pool_create: hidden %d and inter %d must be multiples of 128",
                d->hidden, d->inter);
  if (d->hidden > 65536 || d->inter > 65536)
    return fail(K3X_E_UNSUPPORTED, "pool_create: hidden/inter above 65536");
  if (d->activation != K3X_ACT_SWIGLU && d->activation != K3X_ACT_SITU)
    return fail(K3X_E_INVALID_ARG, "pool_create: unknown activation %d", d->activation);
  if (d->activation == K3X_ACT_SITU &&
      !(std::isfinite(d->situ_b1) && std::isfinite(d->situ_b2) && d->situ_b1 > 0.0f &&
        d->situ_b2 > 0.0f))
    return fail(K3X_E_INVALID_ARG, "pool_create: SiTU caps %g, %g must be finite and > 0",
                (double)d->situ_b1, (double)d->situ_b2);
  if (d->contract != 0 && d->contract != 1)
    return fail(K3X_E_INVALID_ARG, "pool_create: contract %d is neither 0 nor 1", d->contract);
  if (d->contract && (d->hidden > 4096 || d->inter > 4096))
    return fail(K3X_E_UNSUPPORTED, "pool_create: the contract arithmetic takes hidden and inter <= 4096");
  const void* ptrs[6] = {d->w1_packed, d->w1_scale, d->w3_packed, d->w3_scale, d->w2_packed, d->w2_scale};
  const int64_t H = d->hidden, I = d->inter;
  const int64_t dense[6] = {I * H / 2, I * H / 32, I * H / 2, I * H / 32, H * I / 2, H * I / 32};
  k3x_pool* p = new (std::nothrow) k3x_pool;
  if (!p) return fail(K3X_E_INVALID_ARG, "pool_create: out of host memory");
  p->E = d->n_experts;
  p->H = d->hidden;
  p->I = d->inter;
  p->act = d->activation;
  p->b1 = d->activation == K3X_ACT_SITU ? d->situ_b1 : 0.0f;
  p->b2 = d->activation == K3X_ACT_SITU ? d->situ_b2 : 0.0f;
  p->contract = d->contract;
  for (int k = 0; k < 6; ++k) {
    if (!ptrs[k]) {
      delete p;
      return fail(K3X_E_INVALID_ARG, "pool_create: tensor %d is NULL", k);
    }
    const int64_t st = d->stride_bytes[k] ? d->stride_bytes[k] : dense[k];
    if (st < dense[k]) {
      delete p;
      return fail(K3X_E_INVALID_ARG, "pool_create: stride of tensor %d (%lld) below its size %lld", k,
                  (long long)st, (long long)dense[k]);
    }
    if (k % 2 == 0 && (!aligned(ptrs[k], 16) || st % 16)) {
      delete p;
      return fail(K3X_E_UNSUPPORTED, "pool_create: packed tensor %d not 16-byte aligned", k);
    }
    p->base[k] = static_cast<const uint8_t*>(ptrs[k]);
    p->stride[k] = st;
  }
  *out = p;
  g_last_error[0] = 0;
  return K3X_OK;
}

void k3x_expert_pool_destroy(k3x_pool* p) { delete p; }

static k3x_status check_router(const k3x_router_desc* r) {
  if (!r) return fail(K3X_E_INVALID_ARG, "router: NULL desc");
  if (!r->weight) return fail(K3X_E_INVALID_ARG, "router: NULL weight");
  if (r->n_experts < 1 || r->n_experts > 4096)
    return fail(K3X_E_INVALID_ARG, "router: n_experts %d not in 1..4096", r->n_experts);
  if (r->hidden <= 0 || r->hidden % 8 || r->hidden > 16384)
    return fail(K3X_E_UNSUPPORTED, "router: hidden %d must be a positive multiple of 8, <= 16384",
                r->hidden);
  if (r->topk < 1 || r->topk > r->n_experts)
    return fail(K3X_E_INVALID_ARG, "router: topk %d not in 1..%d", r->topk, r->n_experts);
  if (!aligned(r->weight, 16)) return fail(K3X_E_UNSUPPORTED, "router: weight not 16-byte aligned");
  return K3X_OK;
}

size_t k3x_route_workspace_size(const k3x_router_desc* r, int32_t T) {
  if (check_router(r) != K3X_OK || T < 0) return 0;
  const size_t b = sizeof(float) * (size_t)T * (size_t)r->n_experts;
  return b ? (b + 255) & ~(size_t)255 : 256;
}

k3x_status k3x_route_topk(const k3x_router_desc* r, const void* x_bf16, int32_t T,
                          int32_t* idx_out, float* gates_out, void* ws, size_t ws_bytes,
                          void* stream) {
  k3x_status st = check_router(r);
  if (st != K3X_OK) return st;
  if (T < 0) return fail(K3X_E_INVALID_ARG, "route_topk: T %d < 0", T);
  if (T == 0) return K3X_OK;
  if (!x_bf16 || !idx_out || !gates_out)
    return fail(K3X_E_INVALID_ARG, "route_topk: NULL x, idx or gates");
  if (!aligned(x_bf16, 16)) return fail(K3X_E_UNSUPPORTED, "route_topk: x not 16-byte aligned");
  const size_t need = k3x_route_workspace_size(r, T);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(K3X_E_WORKSPACE, "route_topk: workspace %zu bytes, need %zu (256-byte aligned)",
                ws_bytes, need);
  hipError_t e = k3x::launch_route(*r, static_cast<const uint16_t*>(x_bf16), T, idx_out,
                                   gates_out, static_cast<float*>(ws), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "route_topk");
  return K3X_OK;
}

size_t k3x_moe_workspace_size(const k3x_pool* p, int32_t T, int32_t topk) {
  if (!p || T < 0 || topk < 1 || topk > 64) return 0;
  if ((int64_t)T * topk > (int64_t)1 << 26) return 0;
  const size_t general = k3x::moe_layout(p->E, p->H, p->I, T, topk).total;
  size_t off_h, off_d;
  const size_t exact = k3x::decode_exact_ws(*p, topk, &off_h);
  size_t need = general > exact ? general : exact;
  if (p->contract) {
    const size_t c = k3x::contract_ws(*p, topk, &off_h, &off_d);
    need = need > c ? need : c;
  }
  return need;
}

k3x_status k3x_moe_forward(const k3x_pool* p, const void* x_bf16, int32_t T, const int32_t* idx,
                           const float* gates, int32_t topk, float* y, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!p) return fail(K3X_E_INVALID_ARG, "moe_forward: NULL pool");
  if (T < 0) return fail(K3X_E_INVALID_ARG, "moe_forward: T %d < 0", T);
  if (topk < 1 || topk > 64) return fail(K3X_E_INVALID_ARG, "moe_forward: topk %d not in 1..64", topk);
  if ((int64_t)T * topk > (int64_t)1 << 26)
    return fail(K3X_E_UNSUPPORTED, "moe_forward: T * topk above 2^26");
  if (p->contract && T > 1)
    return fail(K3X_E_UNSUPPORTED, "moe_forward: the contract arithmetic runs one token per call");
  const size_t need = k3x_moe_workspace_size(p, T, topk);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(K3X_E_WORKSPACE, "moe_forward: workspace %zu bytes, need %zu (256-byte aligned)",
                ws_bytes, need);
  if (T > 0) {
    if (!x_bf16 || !idx || !gates || !y)
      return fail(K3X_E_INVALID_ARG, "moe_forward: NULL x, idx, gates or y");
    if (!aligned(x_bf16, 16) || !aligned(y, 16))
      return fail(K3X_E_UNSUPPORTED, "moe_forward: x and y must be 16-byte aligned");
  }
  const k3x::MoeLayout L = k3x::moe_layout(p->E, p->H, p->I, T, topk);
  hipError_t e = k3x::launch_moe(*p, static_cast<const uint16_t*>(x_bf16), T, idx, gates, topk,
                                 y, static_cast<uint8_t*>(ws), L, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_forward");
  return K3X_OK;
}

static k3x_status check_latent(const k3x_latent_desc* d, const k3x_pool* p,
                               const k3x_router_desc* r, int32_t T) {
  if (!d || !p) return fail(K3X_E_INVALID_ARG, "latent: NULL desc or pool");
  k3x_status st = check_router(r);
  if (st != K3X_OK) return st;
  if (T < 0) return fail(K3X_E_INVALID_ARG, "latent: T %d < 0", T);
  if (!d->down || !d->up || !d->sh1 || !d->sh3 || !d->sh2)
    return fail(K3X_E_INVALID_ARG, "latent: NULL dense weight");
  if (r->hidden != d->hidden)
    return fail(K3X_E_INVALID_ARG, "latent: router hidden %d != block hidden %d", r->hidden,
                d->hidden);
  if (r->n_experts != p->E)
    return fail(K3X_E_INVALID_ARG, "latent: router experts %d != pool experts %d", r->n_experts,
                p->E);
  if (r->topk > 64) return fail(K3X_E_UNSUPPORTED, "latent: topk %d above 64", r->topk);
  const int32_t dims[3] = {d->hidden, p->H, d->shared_inter};
  const char* names[3] = {"hidden", "latent", "shared_inter"};
  for (int i = 0; i < 3; ++i)
    if (dims[i] <= 0 || dims[i] % 512 || dims[i] > 8192)
      return fail(K3X_E_UNSUPPORTED, "latent: %s %d must be a positive multiple of 512, <= 8192",
                  names[i], dims[i]);
  if (p->H + d->shared_inter > 9728)
    return fail(K3X_E_UNSUPPORTED, "latent: latent %d + shared_inter %d above 9728", p->H,
                d->shared_inter);
  if (!(d->eps >= 0.0f) || !std::isfinite(d->eps))
    return fail(K3X_E_INVALID_ARG, "latent: eps %g must be finite and >= 0", (double)d->eps);
  if (d->shared_activation != K3X_ACT_SWIGLU && d->shared_activation != K3X_ACT_SITU)
    return fail(K3X_E_INVALID_ARG, "latent: unknown shared activation %d", d->shared_activation);
  if (d->shared_activation == K3X_ACT_SITU &&
      !(std::isfinite(d->situ_b1) && std::isfinite(d->situ_b2) && d->situ_b1 > 0.0f &&
        d->situ_b2 > 0.0f))
    return fail(K3X_E_INVALID_ARG, "latent: SiTU caps %g, %g must be finite and > 0",
                (double)d->situ_b1, (double)d->situ_b2);
  const void* dense[5] = {d->down, d->up, d->sh1, d->sh3, d->sh2};
  for (int i = 0; i < 5; ++i)
    if (!aligned(dense[i], 16))
      return fail(K3X_E_UNSUPPORTED, "latent: dense weight %d not 16-byte aligned", i);
  if (d->norm_weight && !aligned(d->norm_weight, 16))
    return fail(K3X_E_UNSUPPORTED, "latent: norm weight not 16-byte aligned");
  if ((int64_t)T * r->topk > (int64_t)1 << 26)
    return fail(K3X_E_UNSUPPORTED, "latent: T * topk above 2^26");
  if (p->contract && T > 1)
    return fail(K3X_E_UNSUPPORTED, "latent: the contract arithmetic runs one token per call");
  return K3X_OK;
}

k3x_status k3x_latent_ws_layout(const k3x_latent_desc* d, const k3x_pool* p,
                                const k3x_router_desc* r, int32_t T, size_t offs[6]) {
  k3x_status st = check_latent(d, p, r, T);
  if (st != K3X_OK) return st;
  if (!offs) return fail(K3X_E_INVALID_ARG, "latent_ws_layout: NULL offs");
  const k3x::LatentLayout L = k3x::latent_layout(*d, *p, r->n_experts, T, r->topk);
  const size_t o[6] = {L.idx, L.gates, L.z, L.acc, L.s, L.moe};
  for (int i = 0; i < 6; ++i) offs[i] = o[i];
  return K3X_OK;
}

size_t k3x_latent_workspace_size(const k3x_latent_desc* d, const k3x_pool* p,
                                 const k3x_router_desc* r, int32_t T) {
  if (check_latent(d, p, r, T) != K3X_OK) return 0;
  const size_t moe = k3x_moe_workspace_size(p, T, r->topk);
  if (!moe) return 0;
  return k3x::latent_layout(*d, *p, r->n_experts, T, r->topk).moe + moe;
}

k3x_status k3x_latent_forward(const k3x_latent_desc* d, const k3x_pool* p,
                              const k3x_router_desc* r, const void* x_bf16, int32_t T,
                              float* out, void* ws, size_t ws_bytes, void* stream) {
  k3x_status st = check_latent(d, p, r, T);
  if (st != K3X_OK) return st;
  const size_t need = k3x_latent_workspace_size(d, p, r, T);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(K3X_E_WORKSPACE, "latent_forward: workspace %zu bytes, need %zu (256-byte aligned)",
                ws_bytes, need);
  if (T == 0) {
    // the routed experts' empty call resets their drop counter, as k3x_moe_forward does
    const k3x::LatentLayout L = k3x::latent_layout(*d, *p, r->n_experts, 0, r->topk);
    const k3x::MoeLayout ML = k3x::moe_layout(p->E, p->H, p->I, 0, r->topk);
    hipError_t e = k3x::launch_moe(*p, nullptr, 0, nullptr, nullptr, r->topk, nullptr,
                                   static_cast<uint8_t*>(ws) + L.moe, ML, (hipStream_t)stream);
    return e == hipSuccess ? K3X_OK : hip_fail(e, "latent_forward");
  }
  if (!x_bf16 || !out) return fail(K3X_E_INVALID_ARG, "latent_forward: NULL x or out");
  if (!aligned(x_bf16, 16) || !aligned(out, 16))
    return fail(K3X_E_UNSUPPORTED, "latent_forward: x and out must be 16-byte aligned");
  const k3x::LatentLayout L = k3x::latent_layout(*d, *p, r->n_experts, T, r->topk);
  const k3x::MoeLayout ML = k3x::moe_layout(p->E, p->H, p->I, T, r->topk);
  hipError_t e = k3x::launch_latent(*d, *p, *r, static_cast<const uint16_t*>(x_bf16), T, out,
                                    static_cast<uint8_t*>(ws), L, ML, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "latent_forward");
  return K3X_OK;
}

static k3x_status check_route_moe(const k3x_router_desc* r, const k3x_pool* p, int32_t T) {
  k3x_status st = check_router(r);
  if (st != K3X_OK) return st;
  if (!p) return fail(K3X_E_INVALID_ARG, "route_moe: NULL pool");
  if (r->n_experts != p->E)
    return fail(K3X_E_INVALID_ARG, "route_moe: router experts %d != pool experts %d",
                r->n_experts, p->E);
  if (r->hidden != p->H)
    return fail(K3X_E_INVALID_ARG, "route_moe: router hidden %d != pool hidden %d", r->hidden,
                p->H);
  if (r->topk > 64) return fail(K3X_E_UNSUPPORTED, "route_moe: topk %d above 64", r->topk);
  if (T < 0) return fail(K3X_E_INVALID_ARG, "route_moe: T %d < 0", T);
  if (p->contract && T > 1)
    return fail(K3X_E_UNSUPPORTED, "route_moe: the contract arithmetic runs one token per call");
  if ((int64_t)T * r->topk > (int64_t)1 << 26)
    return fail(K3X_E_UNSUPPORTED, "route_moe: T * topk above 2^26");
  return K3X_OK;
}

// Workspace of k3x_route_moe_forward: the experts' workspace first (its drop counter at 0),
// then the router's scores.
static size_t route_moe_scores_offset(const k3x_router_desc* r, const k3x_pool* p, int32_t T) {
  const size_t moe = k3x_moe_workspace_size(p, T, r->topk);
  return (moe + 255) & ~(size_t)255;
}

size_t k3x_route_moe_workspace_size(const k3x_router_desc* r, const k3x_pool* p, int32_t T) {
  if (check_route_moe(r, p, T) != K3X_OK) return 0;
  return route_moe_scores_offset(r, p, T) + k3x_route_workspace_size(r, T);
}

// Router and experts after the checks: the fused single-token decode when it applies, else
// the router's two launches and the experts' path for T tokens.
static hipError_t route_moe_run(const k3x_router_desc* r, const k3x_pool* p, const uint16_t* x,
                                int32_t T, int32_t* idx_out, float* gates_out, float* y,
                                uint8_t* w, hipStream_t s) {
  float* scores = reinterpret_cast<float*>(w + route_moe_scores_offset(r, p, T));
  if (!p->contract && k3x::decode_routed_supported(*r, *p, T))
    return k3x::launch_decode_routed(*r, *p, x, scores, idx_out, gates_out, y, w, s);
  hipError_t e = k3x::launch_route(*r, x, T, idx_out, gates_out, scores, s);
  if (e != hipSuccess) return e;
  const k3x::MoeLayout L = k3x::moe_layout(p->E, p->H, p->I, T, r->topk);
  return k3x::launch_moe(*p, x, T, idx_out, gates_out, r->topk, y, w, L, s);
}

k3x_status k3x_route_moe_forward(const k3x_router_desc* r, const k3x_pool* p, const void* x_bf16,
                                 int32_t T, int32_t* idx_out, float* gates_out, float* y,
                                 void* ws, size_t ws_bytes, void* stream) {
  k3x_status st = check_route_moe(r, p, T);
  if (st != K3X_OK) return st;
  const size_t need = k3x_route_moe_workspace_size(r, p, T);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(K3X_E_WORKSPACE, "route_moe_forward: workspace %zu bytes, need %zu (256-byte aligned)",
                ws_bytes, need);
  if (T == 0) {
    // nothing to route; the experts' empty call resets the drop counter, as k3x_moe_forward does
    const k3x::MoeLayout L = k3x::moe_layout(p->E, p->H, p->I, 0, r->topk);
    hipError_t e = k3x::launch_moe(*p, nullptr, 0, nullptr, nullptr, r->topk, nullptr,
                                   static_cast<uint8_t*>(ws), L, (hipStream_t)stream);
    return e == hipSuccess ? K3X_OK : hip_fail(e, "route_moe_forward");
  }
  if (!x_bf16 || !idx_out || !gates_out || !y)
    return fail(K3X_E_INVALID_ARG, "route_moe_forward: NULL x, idx, gates or y");
  if (!aligned(x_bf16, 16) || !aligned(y, 16))
    return fail(K3X_E_UNSUPPORTED, "route_moe_forward: x and y must be 16-byte aligned");
  hipError_t e = route_moe_run(r, p, static_cast<const uint16_t*>(x_bf16), T, idx_out, gates_out,
                               y, static_cast<uint8_t*>(ws), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "route_moe_forward");
  return K3X_OK;
}

static bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t ao = (uintptr_t)a, bo = (uintptr_t)b;
  return a && b && ao < bo + bn && bo < ao + an;
}

k3x_status k3x_residual_route_moe_forward(const k3x_router_desc* r, const k3x_pool* p,
                                          const void* x_bf16, const float* y_prev, float eps,
                                          void* x_next_bf16, void* xn_bf16, int32_t T,
                                          int32_t* idx_out, float* gates_out, float* y, void* ws,
                                          size_t ws_bytes, void* stream) {
  k3x_status st = check_route_moe(r, p, T);
  if (st != K3X_OK) return st;
  const int32_t H = p->H;
  if (H % 8 || H > 16384)
    return fail(K3X_E_UNSUPPORTED, "residual_route_moe: H %d must be a multiple of 8, <= 16384", H);
  const size_t need = k3x_route_moe_workspace_size(r, p, T);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(K3X_E_WORKSPACE,
                "residual_route_moe: workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes,
                need);
  if (T == 0) return k3x_route_moe_forward(r, p, nullptr, 0, nullptr, nullptr, nullptr, ws,
                                           ws_bytes, stream);
  if (!x_bf16 || !xn_bf16 || !idx_out || !gates_out || !y || (y_prev && !x_next_bf16))
    return fail(K3X_E_INVALID_ARG, "residual_route_moe: NULL x, x_next, xn, idx, gates or y");
  if (!aligned(x_bf16, 16) || !aligned(y_prev, 16) || !aligned(x_next_bf16, 16) ||
      !aligned(xn_bf16, 16) || !aligned(y, 16))
    return fail(K3X_E_UNSUPPORTED, "residual_route_moe: 16-byte alignment");
  const size_t xb = (size_t)T * H * 2, yb = (size_t)T * H * 4;
  void* x_next = y_prev ? x_next_bf16 : nullptr;
  if (overlaps(x_next, xb, x_bf16, xb) || overlaps(x_next, xb, y_prev, yb) ||
      overlaps(x_next, xb, xn_bf16, xb) || overlaps(xn_bf16, xb, x_bf16, xb) ||
      overlaps(xn_bf16, xb, y_prev, yb) || overlaps(xn_bf16, xb, y, yb))
    return fail(K3X_E_INVALID_ARG, "residual_route_moe: x_next or xn overlaps another operand");
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint16_t* xn = static_cast<uint16_t*>(xn_bf16);
  uint8_t* w = static_cast<uint8_t*>(ws);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (!p->contract && k3x::decode_routed_residual_supported(*r, *p, T)) {
    float* scores = reinterpret_cast<float*>(w + route_moe_scores_offset(r, p, T));
    e = k3x::launch_decode_routed_residual(*r, *p, x, y_prev, eps,
                                           static_cast<uint16_t*>(x_next), xn, scores, idx_out,
                                           gates_out, y, w, s);
  } else {
    e = y_prev ? k3x::launch_residual_rmsnorm(x, y_prev, T, H, eps,
                                              static_cast<uint16_t*>(x_next), xn, s)
               : k3x::launch_rmsnorm(x, T, H, eps, xn, s);
    if (e == hipSuccess) e = route_moe_run(r, p, xn, T, idx_out, gates_out, y, w, s);
  }
  if (e != hipSuccess) return hip_fail(e, "residual_route_moe");
  return K3X_OK;
}

k3x_status k3x_fetch_drops(const void* ws, int64_t* n, void* stream) {
  if (!ws || !n) return fail(K3X_E_INVALID_ARG, "fetch_drops: NULL ws or n");
  int64_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fetch_drops");
  *n = v;
  return v > 0 ? K3X_E_DROPS : K3X_OK;
}

k3x_status k3x_rmsnorm_bf16(const void* x, int32_t T, int32_t H, float eps, void* out,
                            void* stream) {
  if (T < 0 || H <= 0) return fail(K3X_E_INVALID_ARG, "rmsnorm: T %d, H %d", T, H);
  if (H % 8 || H > 16384) return fail(K3X_E_UNSUPPORTED, "rmsnorm: H %d must be a multiple of 8, <= 16384", H);
  if (T == 0) return K3X_OK;
  if (!x || !out) return fail(K3X_E_INVALID_ARG, "rmsnorm: NULL x or out");
  if (!aligned(x, 16) || !aligned(out, 16)) return fail(K3X_E_UNSUPPORTED, "rmsnorm: 16-byte alignment");
  hipError_t e = k3x::launch_rmsnorm(static_cast<const uint16_t*>(x), T, H, eps,
                                     static_cast<uint16_t*>(out), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rmsnorm");
  return K3X_OK;
}

k3x_status k3x_residual_add_bf16(void* x, const float* y, int32_t T, int32_t H, void* stream) {
  if (T < 0 || H <= 0) return fail(K3X_E_INVALID_ARG, "residual_add: T %d, H %d", T, H);
  if (H % 8) return fail(K3X_E_UNSUPPORTED, "residual_add: H %d must be a multiple of 8", H);
  if (T == 0) return K3X_OK;
  if (!x || !y) return fail(K3X_E_INVALID_ARG, "residual_add: NULL x or y");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(K3X_E_UNSUPPORTED, "residual_add: 16-byte alignment");
  hipError_t e = k3x::launch_residual(static_cast<uint16_t*>(x), y, T, H, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "residual_add");
  return K3X_OK;
}

k3x_status k3x_residual_add_rmsnorm_bf16(void* x, const float* y, int32_t T, int32_t H,
                                          float eps, void* out, void* stream) {
  if (T < 0 || H <= 0) return fail(K3X_E_INVALID_ARG, "residual_add_rmsnorm: T %d, H %d", T, H);
  if (H % 8 || H > 16384)
    return fail(K3X_E_UNSUPPORTED, "residual_add_rmsnorm: H %d must be a multiple of 8, <= 16384", H);
  if (T == 0) return K3X_OK;
  if (!x || !y || !out) return fail(K3X_E_INVALID_ARG, "residual_add_rmsnorm: NULL x, y or out");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(out, 16))
    return fail(K3X_E_UNSUPPORTED, "residual_add_rmsnorm: 16-byte alignment");
  const uintptr_t xb = (uintptr_t)T * (uintptr_t)H * 2, yb = (uintptr_t)T * (uintptr_t)H * 4;
  const uintptr_t xo = (uintptr_t)x, yo = (uintptr_t)y, oo = (uintptr_t)out;
  if ((oo < xo + xb && xo < oo + xb) || (oo < yo + yb && yo < oo + xb))
    return fail(K3X_E_INVALID_ARG, "residual_add_rmsnorm: out overlaps x or y");
  hipError_t e = k3x::launch_residual_rmsnorm(static_cast<const uint16_t*>(x), y, T, H, eps,
                                              static_cast<uint16_t*>(x),
                                              static_cast<uint16_t*>(out), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "residual_add_rmsnorm");
  return K3X_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Kernel timing
// ---------------------------------------------------------------------------------------
struct k3x_profiler {
  int32_t capacity = 0;
  int32_t n = 0;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
  const char** name = nullptr;
};

namespace {
thread_local k3x_profiler* g_prof = nullptr;
}

namespace k3x {

bool profiler_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  k3x_profiler* p = g_prof;
  if (!p || p->n >= p->capacity) return false;
  const int i = p->n++;
  p->name[i] = name;
  *start = p->start[i];
  *stop = p->stop[i];
  return true;
}

}  // namespace k3x

extern "C" {

k3x_status k3x_profiler_create(int32_t capacity, k3x_profiler** out) {
  if (!out || capacity < 1 || capacity > (1 << 20))
    return fail(K3X_E_INVALID_ARG, "profiler_create: capacity %d not in 1..2^20", capacity);
  *out = nullptr;
  k3x_profiler* p = new (std::nothrow) k3x_profiler;
  if (!p) return fail(K3X_E_INVALID_ARG, "profiler_create: out of host memory");
  p->start = new (std::nothrow) hipEvent_t[capacity]();
  p->stop = new (std::nothrow) hipEvent_t[capacity]();
  p->name = new (std::nothrow) const char*[capacity]();
  if (!p->start || !p->stop || !p->name) {
    k3x_profiler_destroy(p);
    return fail(K3X_E_INVALID_ARG, "profiler_create: out of host memory");
  }
  p->capacity = capacity;
  for (int i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&p->start[i]);
    if (e == hipSuccess) e = hipEventCreate(&p->stop[i]);
    if (e != hipSuccess) {
      k3x_profiler_destroy(p);
      return hip_fail(e, "profiler_create");
    }
  }
  *out = p;
  return K3X_OK;
}

void k3x_profiler_destroy(k3x_profiler* p) {
  if (!p) return;
  if (g_prof == p) g_prof = nullptr;
  for (int i = 0; i < p->capacity; ++i) {
    if (p->start && p->start[i]) (void)hipEventDestroy(p->start[i]);
    if (p->stop && p->stop[i]) (void)hipEventDestroy(p->stop[i]);
  }
  delete[] p->start;
  delete[] p->stop;
  delete[] p->name;
  delete p;
}

k3x_status k3x_profiler_attach(k3x_profiler* p) {
  g_prof = p;
  return K3X_OK;
}

k3x_status k3x_profiler_reset(k3x_profiler* p) {
  if (!p) return fail(K3X_E_INVALID_ARG, "profiler_reset: NULL");
  p->n = 0;
  return K3X_OK;
}

int32_t k3x_profiler_count(const k3x_profiler* p) { return p ? p->n : 0; }

k3x_status k3x_profiler_read(k3x_profiler* p, int32_t i, const char** name, float* ms) {
  if (!p || !name || !ms || i < 0 || i >= p->n)
    return fail(K3X_E_INVALID_ARG, "profiler_read: bad index %d", i);
  hipError_t e = hipEventSynchronize(p->stop[i]);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, p->start[i], p->stop[i]);
  if (e != hipSuccess) return hip_fail(e, "profiler_read");
  *name = p->name[i];
  return K3X_OK;
}

}  // extern "C"
