/*
 * k3x oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously ordered CPU implementation of the routed-expert hot path, used
 * only by the test suite, the smoke check and the bench's CPU-baseline leg to check the
 * HIP kernels.  The product path never calls it and shares no code, header, table or
 * constant with it.
 *
 * Sources (the pages describing the kimi-k3-in-c engine):
 *  - kimi-k3-in-c README, Part II section 4 "Reduction one: the experts already ship at half
 *    a byte": the E2M1 table, the E8M0 rule 2^(s-127) with byte 255 mapped to 0, low nibble =
 *    even element, y = W.x taken straight from the nibbles with one scale per group of 32.
 *  - same README, section 5 "Kernels with a floating point contract": RMSNorm with a double
 *    sum of squares and eps inside the square root; widening bf16 to f32 is a 16-bit shift;
 *    a fixed reduction order is part of the contract.
 *  - same README, section 9 "Picking 16 experts of 896": router logits as double dot
 *    products, sigmoid score, bias added for selection only, repeated strict-> argmax
 *    (lowest index wins ties), gates from the unbiased scores, renormalised when the sum
 *    is positive, times routed_scale; the slot-order weighted combine of expert outputs.
 *  - Kimi K3 artifact audit, section 4.3: the six packed/scale tensors of one expert.
 *
 * Readings taken where the pages leave a step open (each also listed in the design notes):
 *  - Activation: SwiGLU, h = silu(g) * u with silu(g) = g / (1 + E) in fp32, E the float
 *    exponential of -g taken as the float nearest to the exact value (evaluated in double
 *    and rounded once, so every conforming implementation gets the same E), and h rounded to
 *    bf16 (round to nearest even) before W2.
 *  - Optional activation SiTU-GLU, the engine's own (README Part II section 9, the routed-
 *    expert loop and its activation listing; default b1 = 4, b2 = 25 from the config
 *    header): a = b1 * T(g / b1) * s(g) with the sigmoid on the uncapped gate, v = b2 *
 *    T(u / b2), h = a * v, where T(q) is the float nearest to tanh(q) (evaluated in double,
 *    rounded once, as E above) and s(g) = 1 / (1 + E); quotients and products in fp32, left
 *    to right as the listing writes them.
 *  - Expert dot products: each group of 32 is summed sequentially in ACC, multiplied by its
 *    exact power-of-two scale, and the group partials are summed by a pairwise tree (zero
 *    padded to a power of two).  ACC = float is the verdict oracle; ACC = double is its
 *    self-check.  This file is compiled once per ACC.
 *  - Router logits and the RMSNorm sum of squares: double, in a fixed 64-way order.  The
 *    vector is cut into chunks of 8 elements; partial L (0..63) sums, in ascending order,
 *    the chunks whose index is L mod 64; then partial[L] += partial[L + s] for
 *    s = 32, 16, 8, 4, 2, 1.  Products of two bf16 values are exact in double, so only the
 *    order of additions matters, and it is fixed here.
 *  - Router sigmoid: computed in double from the float logit and rounded once to float.
 *  - The combine y = sum_j gate_j * d_j runs in ACC in slot order and is rounded at the end.
 *  - Latent MoE block (README Part II section 9, the k3_moe listing): every vector that enters
 *    a bf16 matrix is rounded to bf16 first (the input x, the latent z, the normalised
 *    aggregate, the shared experts' activation); the dense bf16 products follow the
 *    contract's bf16 matmul (README Part II section 5: products and sums in double, the
 *    result rounded once to float), with the double sum taken in the 64-way order above
 *    instead of the contract's four interleaved accumulators (the same reading as the router
 *    logits); the aggregate's RMSNorm sums squares in double in the 64-way order and scales as
 *    (x * inv) * w; the shared experts' output is added to the up-projection once, in fp32.
 *    Only the routed experts inside the block depend on ACC.
 *
 * Build: cc -O2 -ffp-contract=off -fno-fast-math -fopenmp, once with
 * -DORACLE_ACC=float -DORACLE_SFX=f32 -DORACLE_COMMON=1 and once with
 * -DORACLE_ACC=double -DORACLE_SFX=f64.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_ACC
#define ORACLE_ACC float
#endif
#ifndef ORACLE_SFX
#define ORACLE_SFX f32
#endif
#define ORACLE_CAT2(a, b) a##_##b
#define ORACLE_CAT(a, b) ORACLE_CAT2(a, b)
#define ORC(name) ORACLE_CAT(name, ORACLE_SFX)

typedef ORACLE_ACC acc_t;

int oracle_rmsnorm_w_f32(const float *x, int T, int n, const float *w, float eps, uint16_t *out);
int oracle_dense64_bf16(const uint16_t *W, const uint16_t *v, int64_t rows, int64_t K, float *y);
static float glu_one(float g, float u, int act, float b1, float b2);
int oracle_route(const uint16_t *x, int T, int H, const uint16_t *Wr, const float *bias, int E,
                 int topk, int renorm, float routed_scale, int32_t *idx, float *gates,
                 float *logits_out, float *scores_out);

/* ----------------------------------------------------------------------------------------
 * Tables and bit helpers (README section 4; section 5 for bf16 widening)
 * -------------------------------------------------------------------------------------- */

/* E2M1: sign, two exponent bits, one mantissa bit; the sixteen values as printed. */
static const float ORACLE_E2M1_TABLE[16] = {
    0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
    -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

static inline float e2m1_value(unsigned code) { return ORACLE_E2M1_TABLE[code & 15u]; }

/* E8M0 scale byte -> 2^(s-127); byte 255 (NaN in the OCP format) is taken as 0. */
static inline float e8m0_value(unsigned s) {
  return s == 255u ? 0.0f : ldexpf(1.0f, (int)s - 127);
}

/* Nibble of logical element c in a packed row: low nibble holds the even element. */
static inline unsigned nibble_at(const uint8_t *row, int64_t c) {
  const uint8_t b = row[c >> 1];
  return (c & 1) ? (unsigned)(b >> 4) : (unsigned)(b & 15u);
}

static inline float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* float -> bf16, round to nearest even; NaN stays a quiet NaN. */
static inline uint16_t float_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) return (uint16_t)((u >> 16) | 0x40u);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

#ifdef ORACLE_COMMON
/* Fixed 64-way double reduction of sum_i a[i]*b[i] over n elements (n % 8 == 0). */
static double sum64_products(const double *a, const double *b, int64_t n) {
  double part[64];
  const int64_t chunks = n / 8;
  for (int L = 0; L < 64; ++L) {
    double p = 0.0;
    for (int64_t c = L; c < chunks; c += 64)
      for (int j = 0; j < 8; ++j) p += a[8 * c + j] * b[8 * c + j];
    part[L] = p;
  }
  for (int s = 32; s >= 1; s >>= 1)
    for (int L = 0; L < s; ++L) part[L] = part[L] + part[L + s];
  return part[0];
}

float oracle_e2m1(int code) { return e2m1_value((unsigned)code); }
float oracle_e8m0(int s) { return e8m0_value((unsigned)s); }
float oracle_bf16_to_f32(uint16_t b) { return bf16_to_float(b); }
uint16_t oracle_f32_to_bf16(float f) { return float_to_bf16(f); }
void oracle_f32_to_bf16_n(const float *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16(x[i]);
}

double oracle_sum64(const double *a, const double *b, int64_t n) { return sum64_products(a, b, n); }

/* Threads of the oracle's OpenMP loops (the CPU baseline times one core and all of them);
 * the arithmetic of every output is the same for any count. */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_max_threads(void) { return omp_get_max_threads(); }

/* The contract's MXFP4 matmul in the listing's own order (README Part II section 4, the
 * MXFP4 matmul; section 5, "double, always"): per row, acc = 0 in double; groups in order; a
 * scale byte of 255 (NaN) skips its group; else part = the sequential double sum of the
 * group's products (exact in double) and acc += part * scale; y = (float)acc.
 * x fp32 [K]; packed u8 [rows][K/2] (low nibble = even element); scales u8 [rows][K/32]. */
void oracle_mxfp4_matvec_contract(const float *x, const uint8_t *packed, const uint8_t *scales,
                                  int64_t rows, int64_t K, float *y) {
  const int64_t ngroup = K / 32, rowbytes = K / 2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t *prow = packed + r * rowbytes;
    const uint8_t *srow = scales + r * ngroup;
    double acc = 0.0;
    for (int64_t g = 0; g < ngroup; ++g) {
      if (srow[g] == 255u) continue;
      double part = 0.0;
      for (int64_t c = 32 * g; c < 32 * g + 32; ++c)
        part += (double)x[c] * (double)e2m1_value(nibble_at(prow, c));
      acc += part * (double)e8m0_value(srow[g]);
    }
    y[r] = (float)acc;
  }
}

/* One routed expert in the contract's arithmetic: g, u by the matmul above on x (bf16 widened
 * exactly), h = act(g, u) kept in fp32 (not rounded to bf16), d = W2 . h by the same matmul.
 * h_out fp32 [I] may be NULL; d_out fp32 [H].  Returns -1 on bad arguments. */
int oracle_expert_forward_contract(const uint16_t *x, int64_t H, int64_t I, const uint8_t *w1p,
                                   const uint8_t *w1s, const uint8_t *w3p, const uint8_t *w3s,
                                   const uint8_t *w2p, const uint8_t *w2s, int act, float b1,
                                   float b2, float *h_out, float *d_out) {
  if (H <= 0 || I <= 0 || H % 32 || I % 32 || (act != 0 && act != 1)) return -1;
  float *xf = (float *)malloc(sizeof(float) * (size_t)H);
  float *g = (float *)malloc(sizeof(float) * (size_t)I);
  float *u = (float *)malloc(sizeof(float) * (size_t)I);
  float *h = (float *)malloc(sizeof(float) * (size_t)I);
  for (int64_t i = 0; i < H; ++i) xf[i] = bf16_to_float(x[i]);
  oracle_mxfp4_matvec_contract(xf, w1p, w1s, I, H, g);
  oracle_mxfp4_matvec_contract(xf, w3p, w3s, I, H, u);
  for (int64_t r = 0; r < I; ++r) h[r] = glu_one(g[r], u[r], act, b1, b2);
  oracle_mxfp4_matvec_contract(h, w2p, w2s, H, I, d_out);
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)I);
  free(xf);
  free(g);
  free(u);
  free(h);
  return 0;
}

/* The contract's bf16 matmul (README Part II section 5) in the fixed 64-way order:
 * y[r] = (float) sum64(W[r][k] * v[k]), W bf16 [rows][K], v bf16 [K], K % 8 == 0.  The
 * products of two bf16 values are exact in double.  Returns -1 on bad arguments. */
int oracle_dense64_bf16(const uint16_t *W, const uint16_t *v, int64_t rows, int64_t K, float *y) {
  if (rows < 0 || K <= 0 || K % 8) return -1;
  double *vd = (double *)malloc(sizeof(double) * (size_t)K);
  if (!vd) return -1;
  for (int64_t k = 0; k < K; ++k) vd[k] = (double)bf16_to_float(v[k]);
  int bad = 0;
#pragma omp parallel
  {
    double *wd = (double *)malloc(sizeof(double) * (size_t)K);
    if (!wd) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < K; ++k) wd[k] = (double)bf16_to_float(W[r * K + k]);
        y[r] = (float)sum64_products(wd, vd, K);
      }
      free(wd);
    }
  }
  free(vd);
  return bad ? -1 : 0;
}

/* --------------------------------------------------------------------------------------
 * Router (README section 9).  x bf16 [T][H], Wr bf16 [E][H], bias fp32 [E] or NULL.
 * Outputs idx [T][topk] in selection order and gates [T][topk]; optionally the float
 * logits and unbiased scores [T][E].  Returns 0, or -1 on bad arguments.
 * ------------------------------------------------------------------------------------ */
int oracle_route(const uint16_t *x, int T, int H, const uint16_t *Wr, const float *bias, int E,
                 int topk, int renorm, float routed_scale, int32_t *idx, float *gates,
                 float *logits_out, float *scores_out) {
  if (T < 0 || H <= 0 || H % 8 || E <= 0 || topk < 1 || topk > E) return -1;
  double *xd = (double *)malloc(sizeof(double) * (size_t)H);
  double *wd = (double *)malloc(sizeof(double) * (size_t)H);
  float *sc = (float *)malloc(sizeof(float) * (size_t)E);
  float *ch = (float *)malloc(sizeof(float) * (size_t)E);
  char *taken = (char *)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) xd[h] = (double)bf16_to_float(x[(size_t)t * H + h]);
    for (int e = 0; e < E; ++e) {
      for (int h = 0; h < H; ++h) wd[h] = (double)bf16_to_float(Wr[(size_t)e * H + h]);
      const float l = (float)sum64_products(xd, wd, H);
      sc[e] = (float)(1.0 / (1.0 + exp(-(double)l))); /* unbiased score */
      ch[e] = sc[e] + (bias ? bias[e] : 0.0f);        /* selection score */
      if (logits_out) logits_out[(size_t)t * E + e] = l;
      if (scores_out) scores_out[(size_t)t * E + e] = sc[e];
    }
    memset(taken, 0, (size_t)E);
    int32_t *it = idx + (size_t)t * topk;
    float *wt = gates + (size_t)t * topk;
    for (int j = 0; j < topk; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || ch[e] > ch[best])) best = e;
      taken[best] = 1;
      it[j] = best;
      wt[j] = sc[best];
    }
    if (renorm) {
      float s = 0.0f;
      for (int j = 0; j < topk; ++j) s += wt[j];
      if (s > 0.0f)
        for (int j = 0; j < topk; ++j) wt[j] /= s;
    }
    for (int j = 0; j < topk; ++j) wt[j] *= routed_scale;
  }
  free(xd);
  free(wd);
  free(sc);
  free(ch);
  free(taken);
  return 0;
}

/* RMSNorm with unit weight (README section 5): inv = (float)(1/sqrt(ss/H + (double)eps)),
 * ss the double sum of squares in the fixed 64-way order; out = bf16(x * inv). */
int oracle_rmsnorm_bf16(const uint16_t *x, int T, int H, float eps, uint16_t *out) {
  if (T < 0 || H <= 0 || H % 8) return -1;
  double *xd = (double *)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) xd[h] = (double)bf16_to_float(x[(size_t)t * H + h]);
    const double ss = sum64_products(xd, xd, H);
    const float inv = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
    for (int h = 0; h < H; ++h) {
      const float v = bf16_to_float(x[(size_t)t * H + h]) * inv * 1.0f;
      out[(size_t)t * H + h] = float_to_bf16(v);
    }
  }
  free(xd);
  return 0;
}

/* Weighted RMSNorm of fp32 rows (README section 5, the RMSNorm of the floating point
 * contract): ss = sum of squares in double in the fixed 64-way order, inv = (float)(1 /
 * sqrt(ss / n + eps)), out = bf16((x * inv) * w) (w NULL: weight 1).  n % 8 == 0. */
int oracle_rmsnorm_w_f32(const float *x, int T, int n, const float *w, float eps, uint16_t *out) {
  if (T < 0 || n <= 0 || n % 8) return -1;
  double *xd = (double *)malloc(sizeof(double) * (size_t)n);
  for (int t = 0; t < T; ++t) {
    const float *xt = x + (size_t)t * n;
    for (int h = 0; h < n; ++h) xd[h] = (double)xt[h];
    const double ss = sum64_products(xd, xd, n);
    const float inv = (float)(1.0 / sqrt(ss / (double)n + (double)eps));
    for (int h = 0; h < n; ++h) out[(size_t)t * n + h] = float_to_bf16(xt[h] * inv * (w ? w[h] : 1.0f));
  }
  free(xd);
  return 0;
}

/* Residual update of the hidden state: x <- bf16(float(x) + y). */
int oracle_residual_add_bf16(uint16_t *x, const float *y, int T, int H) {
  if (T < 0 || H <= 0) return -1;
  for (int64_t i = 0; i < (int64_t)T * H; ++i) x[i] = float_to_bf16(bf16_to_float(x[i]) + y[i]);
  return 0;
}
#endif /* ORACLE_COMMON */

/* ----------------------------------------------------------------------------------------
 * MXFP4 matrix-vector product (README section 4), ACC-templated.
 * y[r] = sum_g 2^(S[r][g]-127) * sum_{c in group g} x[c] * E2M1[nib(r, c)], r < rows.
 * packed u8 [rows][K/2], scales u8 [rows][K/32], K % 32 == 0.
 * -------------------------------------------------------------------------------------- */
void ORC(oracle_mxfp4_matvec)(const float *x, const uint8_t *packed, const uint8_t *scales,
                              int64_t rows, int64_t K, float *y) {
  const int64_t ngroup = K / 32;
  const int64_t rowbytes = K / 2;
  int64_t npad = 1;
  while (npad < ngroup) npad <<= 1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    acc_t *part = (acc_t *)calloc((size_t)npad, sizeof(acc_t));
    const uint8_t *prow = packed + r * rowbytes;
    const uint8_t *srow = scales + r * ngroup;
    for (int64_t g = 0; g < ngroup; ++g) {
      const unsigned s = srow[g];
      if (s == 255u) {
        part[g] = 0; /* a NaN scale zeroes the group */
        continue;
      }
      acc_t p = 0;
      for (int64_t c = 32 * g; c < 32 * g + 32; ++c)
        p += (acc_t)x[c] * (acc_t)e2m1_value(nibble_at(prow, c));
      part[g] = p * (acc_t)e8m0_value(s); /* exact power of two */
    }
    for (int64_t n = npad; n > 1; n >>= 1)
      for (int64_t i = 0; i < n / 2; ++i) part[i] = part[2 * i] + part[2 * i + 1];
    y[r] = (float)part[0];
    free(part);
  }
}

/* The gated activation of one (g, u) pair before h is rounded to bf16.  act 0: SwiGLU,
 * silu(g) * u with silu(g) = g / (1 + E), E the float nearest to exp(-g).  act 1: SiTU-GLU
 * with caps b1 (gate) and b2 (up): (b1 * T(g / b1) * s(g)) * (b2 * T(u / b2)), T(q) the float
 * nearest to tanh(q), s(g) = 1 / (1 + E). */
static float glu_one(float g, float u, int act, float b1, float b2) {
  const float ex = (float)exp(-(double)g);
  if (act == 1) {
    const float tg = (float)tanh((double)(g / b1));
    const float sg = 1.0f / (1.0f + ex);
    const float a = b1 * tg * sg;
    const float tu = (float)tanh((double)(u / b2));
    const float v = b2 * tu;
    return a * v;
  }
  const float silu = g / (1.0f + ex);
  return silu * u;
}

#ifdef ORACLE_COMMON
/* out[i] = the activation of (g[i], u[i]) in fp32 (before the bf16 rounding of h).
 * Returns -1 for an unknown act or, with act 1, caps that are not finite and positive. */
int oracle_glu(const float *g, const float *u, int64_t n, int act, float b1, float b2,
               float *out) {
  if (act != 0 && act != 1) return -1;
  if (act == 1 && !(b1 > 0.0f && b2 > 0.0f && isfinite(b1) && isfinite(b2))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = glu_one(g[i], u[i], act, b1, b2);
  return 0;
}
#endif

/* One routed expert on one activation: g = W1.x, u = W3.x, h = bf16(act(g, u)), d = W2.h
 * (act as in glu_one).
 * x bf16 [H]; h_out bf16 [I] (may be NULL); g_out/u_out fp32 [I] (may be NULL);
 * d_out fp32 [H]. */
void ORC(oracle_expert_forward_act)(const uint16_t *x, int64_t H, int64_t I, const uint8_t *w1p,
                                    const uint8_t *w1s, const uint8_t *w3p, const uint8_t *w3s,
                                    const uint8_t *w2p, const uint8_t *w2s, int act, float b1,
                                    float b2, uint16_t *h_out, float *g_out, float *u_out,
                                    float *d_out) {
  float *xf = (float *)malloc(sizeof(float) * (size_t)H);
  float *g = (float *)malloc(sizeof(float) * (size_t)I);
  float *u = (float *)malloc(sizeof(float) * (size_t)I);
  float *hf = (float *)malloc(sizeof(float) * (size_t)I);
  for (int64_t c = 0; c < H; ++c) xf[c] = bf16_to_float(x[c]);
  ORC(oracle_mxfp4_matvec)(xf, w1p, w1s, I, H, g);
  ORC(oracle_mxfp4_matvec)(xf, w3p, w3s, I, H, u);
  for (int64_t r = 0; r < I; ++r) {
    const uint16_t hb = float_to_bf16(glu_one(g[r], u[r], act, b1, b2));
    if (h_out) h_out[r] = hb;
    hf[r] = bf16_to_float(hb);
  }
  ORC(oracle_mxfp4_matvec)(hf, w2p, w2s, H, I, d_out);
  if (g_out) memcpy(g_out, g, sizeof(float) * (size_t)I);
  if (u_out) memcpy(u_out, u, sizeof(float) * (size_t)I);
  free(xf);
  free(g);
  free(u);
  free(hf);
}

/* The MXFP4 product of the matvec above for n vectors at once: xt fp32 [K][n] (vector t in
 * column t), yt fp32 [rows][n].  Output (r, t) is computed with exactly the operations
 * oracle_mxfp4_matvec performs for vector t alone (the same products, the same sequential
 * sum inside each group, the same scale, the same pairwise tree); the vectors only run side
 * by side in the innermost loops, so every weight is decoded once for all of them. */
static void ORC(mxfp4_matmat)(const float *xt, int64_t n, const uint8_t *packed,
                              const uint8_t *scales, int64_t rows, int64_t K, float *yt) {
  const int64_t ngroup = K / 32;
  const int64_t rowbytes = K / 2;
  int64_t npad = 1;
  while (npad < ngroup) npad <<= 1;
#pragma omp parallel
  {
    acc_t *part = (acc_t *)malloc(sizeof(acc_t) * (size_t)(npad * n)); /* [npad][n] */
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      const uint8_t *prow = packed + r * rowbytes;
      const uint8_t *srow = scales + r * ngroup;
      for (int64_t g = 0; g < npad; ++g) {
        acc_t *pg = part + g * n;
        for (int64_t t = 0; t < n; ++t) pg[t] = 0;
        if (g >= ngroup || srow[g] == 255u) continue; /* padding; a NaN scale zeroes the group */
        for (int64_t c = 32 * g; c < 32 * g + 32; ++c) {
          const acc_t w = (acc_t)e2m1_value(nibble_at(prow, c));
          const float *xc = xt + c * n;
#pragma omp simd
          for (int64_t t = 0; t < n; ++t) pg[t] += (acc_t)xc[t] * w;
        }
        const acc_t s = (acc_t)e8m0_value(srow[g]); /* exact power of two */
        for (int64_t t = 0; t < n; ++t) pg[t] = pg[t] * s;
      }
      for (int64_t m = npad; m > 1; m >>= 1)
        for (int64_t i = 0; i < m / 2; ++i)
          for (int64_t t = 0; t < n; ++t) part[i * n + t] = part[2 * i * n + t] + part[(2 * i + 1) * n + t];
      for (int64_t t = 0; t < n; ++t) yt[r * n + t] = (float)part[t];
    }
    free(part);
  }
}

/* One routed expert on n activations (an expert-major pass, as a prefill walks the experts
 * one by one): d_out[t] equals what oracle_expert_forward_act gives for x[t] alone, bit for
 * bit.  x bf16 [n][H]; d_out fp32 [n][H]. */
void ORC(oracle_expert_forward_many)(const uint16_t *x, int64_t n, int64_t H, int64_t I,
                                     const uint8_t *w1p, const uint8_t *w1s, const uint8_t *w3p,
                                     const uint8_t *w3s, const uint8_t *w2p, const uint8_t *w2s,
                                     int act, float b1, float b2, float *d_out) {
  if (n <= 0) return;
  float *xt = (float *)malloc(sizeof(float) * (size_t)(H * n));
  float *gt = (float *)malloc(sizeof(float) * (size_t)(I * n));
  float *ut = (float *)malloc(sizeof(float) * (size_t)(I * n));
  float *dt = (float *)malloc(sizeof(float) * (size_t)(H * n));
  for (int64_t t = 0; t < n; ++t)
    for (int64_t c = 0; c < H; ++c) xt[c * n + t] = bf16_to_float(x[t * H + c]);
  ORC(mxfp4_matmat)(xt, n, w1p, w1s, I, H, gt);
  ORC(mxfp4_matmat)(xt, n, w3p, w3s, I, H, ut);
  /* h = bf16(act(g, u)), widened back to fp32 for W2 (kept in gt) */
  for (int64_t i = 0; i < I * n; ++i) gt[i] = bf16_to_float(float_to_bf16(glu_one(gt[i], ut[i], act, b1, b2)));
  ORC(mxfp4_matmat)(gt, n, w2p, w2s, H, I, dt);
  for (int64_t t = 0; t < n; ++t)
    for (int64_t r = 0; r < H; ++r) d_out[t * H + r] = dt[r * n + t];
  free(xt);
  free(gt);
  free(ut);
  free(dt);
}

/* The SwiGLU expert (act 0). */
void ORC(oracle_expert_forward)(const uint16_t *x, int64_t H, int64_t I, const uint8_t *w1p,
                                const uint8_t *w1s, const uint8_t *w3p, const uint8_t *w3s,
                                const uint8_t *w2p, const uint8_t *w2s, uint16_t *h_out,
                                float *g_out, float *u_out, float *d_out) {
  ORC(oracle_expert_forward_act)(x, H, I, w1p, w1s, w3p, w3s, w2p, w2s, 0, 0.0f, 0.0f, h_out,
                                 g_out, u_out, d_out);
}

/* Slot-order weighted combine: y[t][r] = sum_j gates[t][j] * d[t][j][r] in ACC, j ascending,
 * rounded to float at the end; slots with valid[t][j] == 0 contribute nothing. */
void ORC(oracle_combine)(int64_t T, int64_t topk, int64_t H, const float *gates, const float *d,
                         const uint8_t *valid, float *y) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t r = 0; r < H; ++r) {
      acc_t a = 0;
      for (int64_t j = 0; j < topk; ++j) {
        if (valid && !valid[t * topk + j]) continue;
        a += (acc_t)gates[t * topk + j] * (acc_t)d[(t * topk + j) * H + r];
      }
      y[t * H + r] = (float)a;
    }
}

/* Whole MoE forward over a pool held in host memory (small cases).  Pool tensors are
 * [E][rows][cols] with the per-expert byte strides given (0 = dense).  An expert id outside
 * [0, E) is a dropped slot: it contributes 0 and is counted.  Returns the drop count. */
int64_t ORC(oracle_moe_forward_act)(int64_t E, int64_t H, int64_t I, const uint8_t *w1p,
                                    const uint8_t *w1s, const uint8_t *w3p, const uint8_t *w3s,
                                    const uint8_t *w2p, const uint8_t *w2s,
                                    const int64_t *strides, int act, float b1, float b2,
                                    int64_t T, const uint16_t *x, const int32_t *idx,
                                    const float *gates, int64_t topk, float *y) {
  const int64_t dflt[6] = {I * H / 2, I * H / 32, I * H / 2, I * H / 32, H * I / 2, H * I / 32};
  int64_t st[6];
  for (int i = 0; i < 6; ++i) st[i] = (strides && strides[i]) ? strides[i] : dflt[i];
  float *d = (float *)malloc(sizeof(float) * (size_t)(T * topk * H));
  uint8_t *valid = (uint8_t *)malloc((size_t)(T * topk));
  int64_t drops = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < topk; ++j) {
      const int64_t e = idx[t * topk + j];
      float *dj = d + (t * topk + j) * H;
      if (e < 0 || e >= E) {
        ++drops;
        valid[t * topk + j] = 0;
        memset(dj, 0, sizeof(float) * (size_t)H);
        continue;
      }
      valid[t * topk + j] = 1;
      ORC(oracle_expert_forward_act)(x + t * H, H, I, w1p + e * st[0], w1s + e * st[1],
                                     w3p + e * st[2], w3s + e * st[3], w2p + e * st[4],
                                     w2s + e * st[5], act, b1, b2, NULL, NULL, NULL, dj);
    }
  ORC(oracle_combine)(T, topk, H, gates, d, valid, y);
  free(d);
  free(valid);
  return drops;
}

/* The SwiGLU forward (act 0). */
int64_t ORC(oracle_moe_forward)(int64_t E, int64_t H, int64_t I, const uint8_t *w1p,
                                const uint8_t *w1s, const uint8_t *w3p, const uint8_t *w3s,
                                const uint8_t *w2p, const uint8_t *w2s, const int64_t *strides,
                                int64_t T, const uint16_t *x, const int32_t *idx,
                                const float *gates, int64_t topk, float *y) {
  return ORC(oracle_moe_forward_act)(E, H, I, w1p, w1s, w3p, w3s, w2p, w2s, strides, 0, 0.0f,
                                     0.0f, T, x, idx, gates, topk, y);
}

/* ----------------------------------------------------------------------------------------
 * Stable LatentMoE block (README Part II section 9, the k3_moe listing), T tokens:
 *   1. route on the full width D;  2. z = bf16(down . x), down bf16 [L][D];
 *   3. accL = routed experts on z (the MoE forward above, activation act with caps b1, b2);
 *   4. a = RMSNorm_w(accL) (norm_w fp32 [L], or skipped when norm_w is NULL: a = bf16(accL));
 *   5. o = up . a, up bf16 [D][L];
 *   6. shared experts on the ORIGINAL x, added unweighted: g = sh1 . x, u = sh3 . x (sh1, sh3
 *      bf16 [S][D]), s = bf16(act_sh(g, u)), out = o + sh2 . s (sh2 bf16 [D][S]).
 * Returns the number of dropped routed slots, or -1 on bad arguments.
 * ---------------------------------------------------------------------------------------- */
int64_t ORC(oracle_latent_block)(int64_t T, int64_t D, int64_t L, int64_t I, int64_t S,
                                 int64_t E, int64_t topk, const uint16_t *x, const uint16_t *Wr,
                                 const float *bias, int renorm, float rscale,
                                 const uint16_t *down, const uint16_t *up, const uint16_t *sh1,
                                 const uint16_t *sh3, const uint16_t *sh2, const float *norm_w,
                                 float eps, const uint8_t *w1p, const uint8_t *w1s,
                                 const uint8_t *w3p, const uint8_t *w3s, const uint8_t *w2p,
                                 const uint8_t *w2s, int act, float b1, float b2, int act_sh,
                                 float *out) {
  if (T < 0 || D <= 0 || L <= 0 || I <= 0 || S <= 0 || D % 8 || L % 32 || I % 32 || S % 8 ||
      E <= 0 || topk < 1 || topk > E)
    return -1;
  if (T == 0) return 0;
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * topk));
  float *gates = (float *)malloc(sizeof(float) * (size_t)(T * topk));
  uint16_t *z = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T * L));
  float *acc = (float *)malloc(sizeof(float) * (size_t)(T * L));
  uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T * L));
  const int64_t fmax = D > S ? (D > L ? D : L) : (S > L ? S : L);
  float *f = (float *)malloc(sizeof(float) * (size_t)fmax);
  float *g = (float *)malloc(sizeof(float) * (size_t)S);
  float *u = (float *)malloc(sizeof(float) * (size_t)S);
  uint16_t *sb = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)S);
  int64_t drops = -1;
  if (oracle_route(x, (int)T, (int)D, Wr, bias, (int)E, (int)topk, renorm, rscale, idx, gates,
                   NULL, NULL) != 0)
    goto done;
  for (int64_t t = 0; t < T; ++t) {
    if (oracle_dense64_bf16(down, x + t * D, L, D, f) != 0) {
      drops = -1;
      goto done;
    }
    for (int64_t i = 0; i < L; ++i) z[t * L + i] = float_to_bf16(f[i]);
  }
  drops = ORC(oracle_moe_forward_act)(E, L, I, w1p, w1s, w3p, w3s, w2p, w2s, NULL, act, b1, b2, T,
                                      z, idx, gates, topk, acc);
  if (norm_w) {
    oracle_rmsnorm_w_f32(acc, (int)T, (int)L, norm_w, eps, a);
  } else {
    for (int64_t i = 0; i < T * L; ++i) a[i] = float_to_bf16(acc[i]);
  }
  for (int64_t t = 0; t < T; ++t) {
    float *ot = out + t * D;
    if (oracle_dense64_bf16(up, a + t * L, D, L, ot) != 0 ||
        oracle_dense64_bf16(sh1, x + t * D, S, D, g) != 0 ||
        oracle_dense64_bf16(sh3, x + t * D, S, D, u) != 0) {
      drops = -1;
      goto done;
    }
    for (int64_t i = 0; i < S; ++i) sb[i] = float_to_bf16(glu_one(g[i], u[i], act_sh, b1, b2));
    if (oracle_dense64_bf16(sh2, sb, D, S, f) != 0) {
      drops = -1;
      goto done;
    }
    for (int64_t i = 0; i < D; ++i) ot[i] = ot[i] + f[i];
  }
done:
  free(idx);
  free(gates);
  free(z);
  free(acc);
  free(a);
  free(f);
  free(g);
  free(u);
  free(sb);
  return drops;
}
