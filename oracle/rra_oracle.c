/*
 * CPU oracle for the fused residual-add/RMSNorm/SiLU/RoPE/quant path.
 *
 * TEST INFRASTRUCTURE ONLY: the plain definition the HIP library is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it.  It shares nothing with rope_residual_add_amd/.
 *
 * Page abbreviations used in the citations below:
 *   [FUSION]  vLLM design page "Fusion torch.compile passes"
 *   [TUNING]  blog "Making vLLM fast: configuration, internals, and the places
 *             worth touching code", section "PagedAttention"
 *   [OFP8]    OCP 8-bit Floating Point Specification, E4M3 format
 *
 * Readings taken where the pages are silent are stated at each function.
 */
#include "rra_oracle.h"

#include <fenv.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ======================================================================= */
/* Codecs                                                                   */
/* ======================================================================= */

/* bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits; the upper half of an
 * IEEE binary32.  Largest finite value (2 - 2^-7) * 2^127. */
static const double kBf16Max = 3.3895313892515355e38;

/* Round a double to the nearest bf16, ties to even, overflow to infinity
 * (IEEE round-to-nearest-even semantics), NaN to a quiet NaN of the same sign.
 * Method: the representable neighbours of |v| are integer multiples of the
 * quantum 2^(E-7) of |v|'s binade E (clamped to the smallest normal binade,
 * which subnormals share); nearbyint() in the default rounding mode rounds
 * half to even. */
uint16_t orc_bf16_encode(double v) {
  const uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs(v);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  if (E < -126) E = -126;
  const double quantum = ldexp(1.0, E - 7);
  const double n = nearbyint(a / quantum);
  const double r = n * quantum;
  if (r > kBf16Max) return (uint16_t)(sign | 0x7F80u);
  const float f = (float)r; /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

double orc_bf16_decode(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

float orc_fp32_round(double v) { return (float)v; /* RNE in FE_TONEAREST */ }

/* IEEE 754 binary16 (fp16): 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * Normal values (1 + f/1024) * 2^(e-15) for exponent fields 1..30, subnormals
 * f * 2^-24 for field 0, infinities and NaNs for field 31; largest finite
 * value (2 - 2^-10) * 2^15 = 65504. */
static const double kF16Max = 65504.0;

/* Round a double to the nearest fp16, ties to even, overflow to infinity,
 * NaN to a quiet NaN of the same sign.  Same method as orc_bf16_encode: the
 * neighbours of |v| are integer multiples of the quantum 2^(E-10) of its
 * binade E, clamped to the smallest normal binade -14 (the subnormals' quantum
 * 2^-24). */
uint16_t orc_f16_encode(double v) {
  const uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
  const double a = fabs(v);
  if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  if (E < -14) E = -14;
  const double r = nearbyint(a / ldexp(1.0, E - 10)) * ldexp(1.0, E - 10);
  if (r > kF16Max) return (uint16_t)(sign | 0x7C00u);
  /* Encode the fp16 value r exactly. */
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
  frexp(r, &e);
  const int Er = e - 1; /* r in [2^Er, 2^(Er+1)), -14 <= Er <= 15 */
  const uint16_t frac = (uint16_t)((r / ldexp(1.0, Er) - 1.0) * 1024.0);
  return (uint16_t)(sign | (uint16_t)((Er + 15) << 10) | frac);
}

double orc_f16_decode(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double mag;
  if (e == 0x1F)
    mag = f ? NAN : INFINITY;
  else if (e == 0)
    mag = ldexp((double)f, -24);
  else
    mag = ldexp(1.0 + (double)f / 1024.0, e - 15);
  return s ? -mag : mag;
}

/* The 16-bit element types of the RoPE + KV-cache and padding ops. */
static double elem_decode(uint16_t h, int dtype) {
  return dtype == ORC_DT_F16 ? orc_f16_decode(h) : orc_bf16_decode(h);
}
static uint16_t elem_encode(double v, int dtype) {
  return dtype == ORC_DT_F16 ? orc_f16_encode(v) : orc_bf16_encode(v);
}

/* [OFP8] E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
 * Exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there is
 * no infinity, so S.1111.110 = 448 is the largest finite magnitude. */
double orc_e4m3fn_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return s ? -NAN : NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* The 127 non-negative finite E4M3 values, indexed by code 0x00..0x7E, in
 * increasing order (the encoding is monotonic in the code). */
static double g_e4m3_values[127];

__attribute__((constructor)) static void build_e4m3_table(void) {
  for (int c = 0; c < 127; ++c) g_e4m3_values[c] = orc_e4m3fn_decode((uint8_t)c);
}

/* Encode to E4M3 by search over the decoded value table: the nearest finite
 * value, ties to the even code (the code's last bit is the mantissa's last
 * bit), magnitudes at or above 448 saturate to 448 (reading: the quantizer
 * saturates rather than producing NaN), NaN maps to S.1111.111, and the sign
 * of zero is kept. */
uint8_t orc_e4m3fn_encode(double v) {
  const uint8_t sign = signbit(v) ? 0x80u : 0u;
  if (isnan(v)) return (uint8_t)(sign | 0x7Fu);
  const double a = fabs(v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  int lo = 0, hi = 126; /* invariant: table[lo] <= a < table[hi] */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (g_e4m3_values[mid] <= a)
      lo = mid;
    else
      hi = mid;
  }
  if (a == g_e4m3_values[lo]) return (uint8_t)(sign | lo);
  const double midpoint = 0.5 * (g_e4m3_values[lo] + g_e4m3_values[hi]); /* exact */
  int k;
  if (a < midpoint)
    k = lo;
  else if (a > midpoint)
    k = hi;
  else
    k = (lo % 2 == 0) ? lo : hi;
  return (uint8_t)(sign | k);
}

/* A second E4M3 encoder built a different way, used only to cross-check the
 * first: scale |v| by the quantum of its binade (2^(E-3), or 2^-9 below the
 * smallest normal binade 2^-6), round half to even with nearbyint(), clamp to
 * 448, then assemble the bit fields from frexp(). */
uint8_t orc_e4m3fn_encode_arith(double v) {
  const uint8_t sign = signbit(v) ? 0x80u : 0u;
  if (isnan(v)) return (uint8_t)(sign | 0x7Fu);
  double a = fabs(v);
  if (isinf(a)) return (uint8_t)(sign | 0x7Eu);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int E = e - 1;
  if (E < -6) E = -6;
  const double q = ldexp(1.0, E - 3);
  double r = nearbyint(a / q) * q;
  if (r > 448.0) r = 448.0;
  if (r < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(r * 512.0)); /* m * 2^-9 */
  int e2;
  const double f = frexp(r, &e2); /* r = f * 2^e2, f in [0.5, 1) */
  const int biased = (e2 - 1) + 7;
  const int m = (int)((2.0 * f - 1.0) * 8.0);
  return (uint8_t)(sign | (biased << 3) | m);
}

void orc_bf16_encode_f32_array(const float* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_encode((double)in[i]);
}

void orc_e4m3fn_encode_f32_array(const float* in, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3fn_encode((double)in[i]);
}

void orc_e4m3fn_decode_array(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3fn_decode(in[i]);
}

int64_t orc_e4m3fn_cross_check(uint64_t begin, uint64_t end) {
  int64_t bad = 0;
  const int64_t b = (int64_t)begin, n = (int64_t)end;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int64_t i = b; i < n; ++i) {
    const uint32_t u = (uint32_t)i;
    float f;
    memcpy(&f, &u, sizeof f);
    if (orc_e4m3fn_encode((double)f) != orc_e4m3fn_encode_arith((double)f)) ++bad;
  }
  return bad;
}

/* ======================================================================= */
/* Threading                                                                */
/* ======================================================================= */

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ======================================================================= */
/* Row building blocks                                                      */
/* ======================================================================= */

static int quant_args_ok(int mode, int group_size, int64_t H, int allow_none) {
  switch (mode) {
    case ORC_Q_NONE:
      return allow_none;
    case ORC_Q_STATIC:
    case ORC_Q_PER_TOKEN:
      return 1;
    case ORC_Q_PER_GROUP:
      return group_size > 0 && H % group_size == 0;
    default:
      return 0;
  }
}

/* RMSNorm of one row.  The pages name the op (rms_norm) without a formula;
 * the reading is the usual one: y_j = z_j / sqrt(mean_j(z_j^2) + eps) * w_j,
 * with eps inside the root and a multiplicative weight.
 * [FUSION] sections "RMSNorm + Quantization" and "MLA Dual RMSNorm". */
static void rms_norm_row(const double* z, const uint16_t* w, float eps, int64_t H, double* y,
                         int dtype) {
  double ss = 0.0;
  for (int64_t j = 0; j < H; ++j) ss += z[j] * z[j];
  const double rho = 1.0 / sqrt(ss / (double)H + (double)eps);
  for (int64_t j = 0; j < H; ++j) y[j] = z[j] * rho * elem_decode(w[j], dtype);
}

/* One scale from an amax: s = amax / 448 rounded to fp32 (448 is E4M3's
 * largest finite value).  Reading: no floor and no cap, so an all-zero slice
 * gets s = 0. */
static float dynamic_scale(double amax) { return orc_fp32_round(amax / 448.0); }

/* Code of one value for a stored fp32 scale s.  Reading: quantize with the
 * stored scale so that dequantization is decode(code) * s; s = 0 (all-zero
 * slice) gives +0 codes. */
static uint8_t quant_one(double y, float s) {
  if (s == 0.0f) return 0;
  return orc_e4m3fn_encode(y / (double)s);
}

/* FP8 quantization of one row y[0..H).  Static: the given per-tensor scale;
 * per-token: one dynamic scale per row; per-group: one dynamic scale per
 * contiguous slice of group_size elements, scales laid out [row, H/g].
 * [FUSION] sections "RMSNorm + Quantization" (static per-tensor, dynamic
 * per-token, dynamic per-token-group 128/64) and "SiLU+Mul + Quantization". */
static void quant_row(const double* y, int64_t H, int mode, int group_size, float static_scale,
                      uint8_t* out, float* scales_row) {
  if (mode == ORC_Q_STATIC) {
    for (int64_t j = 0; j < H; ++j) out[j] = quant_one(y[j], static_scale);
  } else if (mode == ORC_Q_PER_TOKEN) {
    double amax = 0.0;
    for (int64_t j = 0; j < H; ++j) amax = fmax(amax, fabs(y[j]));
    const float s = dynamic_scale(amax);
    scales_row[0] = s;
    for (int64_t j = 0; j < H; ++j) out[j] = quant_one(y[j], s);
  } else { /* ORC_Q_PER_GROUP */
    for (int64_t g0 = 0, k = 0; g0 < H; g0 += group_size, ++k) {
      double amax = 0.0;
      for (int64_t j = g0; j < g0 + group_size; ++j) amax = fmax(amax, fabs(y[j]));
      const float s = dynamic_scale(amax);
      scales_row[k] = s;
      for (int64_t j = g0; j < g0 + group_size; ++j) out[j] = quant_one(y[j], s);
    }
  }
}

static float* scales_row_ptr(float* scales, int mode, int group_size, int64_t H, int64_t t) {
  if (mode == ORC_Q_PER_TOKEN) return scales + t;
  if (mode == ORC_Q_PER_GROUP) return scales + t * (H / group_size);
  return NULL;
}

static int static_scale_ok(int mode, float s) {
  return mode != ORC_Q_STATIC || (isfinite(s) && s > 0.0f);
}

/* ======================================================================= */
/* Residual add + RMSNorm + FP8 quant                                       */
/* ======================================================================= */

/* Fused-add RMSNorm followed by FP8 quantization, one pass, no intermediate
 * tensor; the residual is overwritten with the sum.
 * [FUSION] section "RMSNorm + Quantization (fuse_norm_quant)": the two fused
 * variants are rms_norm(x) -> quant and fused_add_rms_norm(x, residual) ->
 * quant with the residual updated in place.
 * Readings: z = bf16(x + residual) is both the stored residual and the norm
 * input; y is never rounded before the single FP8 rounding. */
int orc_fused_add_rmsnorm_quant(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                                int64_t res_stride, const uint16_t* weight, float eps,
                                int quant_mode, int group_size, float static_scale,
                                uint8_t* out, int64_t out_stride, float* scales, int64_t T,
                                int64_t H) {
  if (T < 0 || H <= 0 || !quant_args_ok(quant_mode, group_size, H, 0)) return ORC_EARG;
  if (!static_scale_ok(quant_mode, static_scale)) return ORC_ECONTRACT;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* z = (double*)malloc((size_t)H * sizeof(double));
    double* y = (double*)malloc((size_t)H * sizeof(double));
    for (int64_t j = 0; j < H; ++j) {
      const double xv = orc_bf16_decode(x[t * x_stride + j]);
      if (residual) {
        /* the sum of two bf16 values is exact in double */
        const uint16_t zb = orc_bf16_encode(xv + orc_bf16_decode(residual[t * res_stride + j]));
        residual[t * res_stride + j] = zb;
        z[j] = orc_bf16_decode(zb);
      } else {
        z[j] = xv;
      }
    }
    rms_norm_row(z, weight, eps, H, y, ORC_DT_BF16);
    quant_row(y, H, quant_mode, group_size, static_scale, out + t * out_stride,
              scales_row_ptr(scales, quant_mode, group_size, H, t));
    free(z);
    free(y);
  }
  return ORC_OK;
}

/* The unfused composition the fusion replaces: fused_add_rms_norm writes the
 * residual and a bf16 normalized tensor, then a separate quant op reads that
 * bf16 tensor and derives its scale from it.  [FUSION] section "RMSNorm +
 * Quantization". */
int orc_unfused_add_rmsnorm_quant(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                                  int64_t res_stride, const uint16_t* weight, float eps,
                                  int quant_mode, int group_size, float static_scale,
                                  uint8_t* out, int64_t out_stride, float* scales, int64_t T,
                                  int64_t H) {
  if (T < 0 || H <= 0 || !quant_args_ok(quant_mode, group_size, H, 0)) return ORC_EARG;
  if (!static_scale_ok(quant_mode, static_scale)) return ORC_ECONTRACT;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* z = (double*)malloc((size_t)H * sizeof(double));
    double* y = (double*)malloc((size_t)H * sizeof(double));
    /* step 1: the residual add, stored */
    for (int64_t j = 0; j < H; ++j) {
      double v = orc_bf16_decode(x[t * x_stride + j]);
      if (residual) {
        const uint16_t zb = orc_bf16_encode(v + orc_bf16_decode(residual[t * res_stride + j]));
        residual[t * res_stride + j] = zb;
        v = orc_bf16_decode(zb);
      }
      z[j] = v;
    }
    /* step 2: rms_norm materializes a bf16 tensor */
    rms_norm_row(z, weight, eps, H, y, ORC_DT_BF16);
    for (int64_t j = 0; j < H; ++j) y[j] = orc_bf16_decode(orc_bf16_encode(y[j]));
    /* step 3: quant_fp8 of that tensor */
    quant_row(y, H, quant_mode, group_size, static_scale, out + t * out_stride,
              scales_row_ptr(scales, quant_mode, group_size, H, t));
    free(z);
    free(y);
  }
  return ORC_OK;
}

/* ======================================================================= */
/* SiLU-and-Mul + FP8 quant                                                 */
/* ======================================================================= */

/* silu(g) * u in double.  Reading: silu(x) = x * sigmoid(x) = x / (1 + e^-x);
 * the gate is the first half of the gate-up projection row and up the second.
 * [FUSION] section "SiLU+Mul + Quantization (fuse_act_quant)". */
static double silu_mul(double g, double u) { return g / (1.0 + exp(-g)) * u; }

/* silu_and_mul followed by FP8 quantization without materializing the
 * activation.  [FUSION] section "SiLU+Mul + Quantization": static per-tensor
 * and dynamic per-group (128/64) variants. */
int orc_silu_mul_quant(const uint16_t* in, int64_t in_stride, int quant_mode, int group_size,
                       float static_scale, uint8_t* out, int64_t out_stride, float* scales,
                       int64_t T, int64_t I) {
  if (T < 0 || I <= 0 || !quant_args_ok(quant_mode, group_size, I, 0)) return ORC_EARG;
  if (!static_scale_ok(quant_mode, static_scale)) return ORC_ECONTRACT;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* a = (double*)malloc((size_t)I * sizeof(double));
    const uint16_t* row = in + t * in_stride;
    for (int64_t j = 0; j < I; ++j)
      a[j] = silu_mul(orc_bf16_decode(row[j]), orc_bf16_decode(row[I + j]));
    quant_row(a, I, quant_mode, group_size, static_scale, out + t * out_stride,
              scales_row_ptr(scales, quant_mode, group_size, I, t));
    free(a);
  }
  return ORC_OK;
}

/* The unfused composition: silu_and_mul writes a bf16 activation tensor, the
 * quant op reads it back.  [FUSION] section "SiLU+Mul + Quantization". */
int orc_unfused_silu_mul_quant(const uint16_t* in, int64_t in_stride, int quant_mode,
                               int group_size, float static_scale, uint8_t* out,
                               int64_t out_stride, float* scales, int64_t T, int64_t I) {
  if (T < 0 || I <= 0 || !quant_args_ok(quant_mode, group_size, I, 0)) return ORC_EARG;
  if (!static_scale_ok(quant_mode, static_scale)) return ORC_ECONTRACT;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* a = (double*)malloc((size_t)I * sizeof(double));
    const uint16_t* row = in + t * in_stride;
    for (int64_t j = 0; j < I; ++j)
      a[j] = orc_bf16_decode(
          orc_bf16_encode(silu_mul(orc_bf16_decode(row[j]), orc_bf16_decode(row[I + j]))));
    quant_row(a, I, quant_mode, group_size, static_scale, out + t * out_stride,
              scales_row_ptr(scales, quant_mode, group_size, I, t));
    free(a);
  }
  return ORC_OK;
}

/* ======================================================================= */
/* RoPE + paged KV-cache write                                              */
/* ======================================================================= */

static int rope_args_ok(int64_t T, int Hq, int Hkv, int D, int rot_dim, int block_size,
                        int64_t num_blocks, int is_neox, int dtype) {
  return T >= 0 && Hq > 0 && Hkv > 0 && D > 0 && rot_dim > 0 && rot_dim % 2 == 0 &&
         rot_dim <= D && block_size > 0 && num_blocks > 0 && (is_neox == 0 || is_neox == 1) &&
         (dtype == ORC_DT_BF16 || dtype == ORC_DT_F16);
}

static int cmp_i64(const void* a, const void* b) {
  const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/* Data contract of the cache write: every position inside the rotary table,
 * every non-negative slot inside the cache, and no two tokens on one slot
 * (with duplicates several final cache states would be "correct"). */
static int rope_contract_ok(const int64_t* positions, int64_t max_pos,
                            const int64_t* slot_mapping, int64_t T, int block_size,
                            int64_t num_blocks) {
  const int64_t n_slots = (int64_t)block_size * num_blocks;
  int64_t* s = (int64_t*)malloc((size_t)(T > 0 ? T : 1) * sizeof(int64_t));
  int64_t n = 0;
  int ok = 1;
  for (int64_t t = 0; t < T && ok; ++t) {
    if (positions[t] < 0 || positions[t] >= max_pos) ok = 0;
    if (slot_mapping[t] >= n_slots) ok = 0;
    if (slot_mapping[t] >= 0) s[n++] = slot_mapping[t];
  }
  if (ok) {
    qsort(s, (size_t)n, sizeof(int64_t), cmp_i64);
    for (int64_t i = 1; i < n; ++i)
      if (s[i] == s[i - 1]) ok = 0;
  }
  free(s);
  return ok;
}

/* cos and sin of the rotation angles of one position.  Reading (the pages
 * give no RoPE formula): the RoFormer frequencies inv_i = theta^(-2i/rot_dim)
 * for i < rot_dim/2, angle = pos * inv_i, evaluated in double. */
static void rope_angles(int64_t pos, double theta, int rot_dim, double* c, double* s) {
  for (int i = 0; i < rot_dim / 2; ++i) {
    const double inv = pow(theta, -2.0 * (double)i / (double)rot_dim);
    const double ang = (double)pos * inv;
    c[i] = cos(ang);
    s[i] = sin(ang);
  }
}

/* Rotate one head of D values of element type dtype (each output rounded once
 * from double).  Pairs are (i, i + rot_dim/2) in the GPT-NeoX
 * layout and (2i, 2i+1) in the GPT-J layout; each pair (a, b) becomes
 * (a cos - b sin, b cos + a sin).  Dimensions at and past rot_dim pass
 * through.  The head is read completely before it is written, so out may
 * alias in. */
static void rotate_head(const uint16_t* in, uint16_t* out, const double* c, const double* s,
                        int D, int rot_dim, int is_neox, int dtype) {
  double* x = (double*)malloc((size_t)D * sizeof(double));
  uint16_t* keep = (uint16_t*)malloc((size_t)D * sizeof(uint16_t));
  for (int d = 0; d < D; ++d) {
    x[d] = elem_decode(in[d], dtype);
    keep[d] = in[d];
  }
  const int half = rot_dim / 2;
  for (int i = 0; i < half; ++i) {
    const int a = is_neox ? i : 2 * i;
    const int b = is_neox ? i + half : 2 * i + 1;
    out[a] = elem_encode(x[a] * c[i] - x[b] * s[i], dtype);
    out[b] = elem_encode(x[b] * c[i] + x[a] * s[i], dtype);
  }
  for (int d = rot_dim; d < D; ++d) out[d] = keep[d];
  free(x);
  free(keep);
}

/* Address of head h of a slot in a paged cache laid out
 * [num_blocks, block_size, Hkv, D].  [TUNING] section "PagedAttention": the
 * cache is cut into fixed-size blocks and a request's logical token positions
 * map to physical blocks through its block table.  Reading: the slot of a
 * token is block * block_size + offset, as the caller's slot mapping gives. */
static uint16_t* cache_head(uint16_t* cache, int64_t slot, int block_size, int Hkv, int D,
                            int h) {
  const int64_t blk = slot / block_size, off = slot % block_size;
  return cache + (((blk * block_size + off) * Hkv + h) * (int64_t)D);
}

/* Rotary embedding fused with the KV-cache scatter: rotated q is written to
 * q_out (which may alias q), rotated k and the unmodified v go straight into
 * the slot of each token; k is not written anywhere else, and tokens with a
 * negative slot (padding, a reading) write no cache.  q, k, v and the caches
 * hold one 16-bit element type, bf16 or fp16 (dtype): the fusion is listed
 * for both on ROCm in the [FUSION] support matrix.
 * [FUSION] section "RoPE + KV-Cache Update (fuse_rope_kvcache)". */
int orc_rope_kv_write(const int64_t* positions, const uint16_t* q, int64_t q_stride,
                      uint16_t* q_out, int64_t q_out_stride, const uint16_t* k,
                      int64_t k_stride, const uint16_t* v, int64_t v_stride, double theta,
                      int64_t max_pos, const int64_t* slot_mapping, uint16_t* key_cache,
                      uint16_t* value_cache, int64_t T, int Hq, int Hkv, int D, int rot_dim,
                      int block_size, int64_t num_blocks, int is_neox, int dtype) {
  if (!rope_args_ok(T, Hq, Hkv, D, rot_dim, block_size, num_blocks, is_neox, dtype))
    return ORC_EARG;
  if (!rope_contract_ok(positions, max_pos, slot_mapping, T, block_size, num_blocks))
    return ORC_ECONTRACT;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* c = (double*)malloc((size_t)rot_dim / 2 * sizeof(double));
    double* s = (double*)malloc((size_t)rot_dim / 2 * sizeof(double));
    rope_angles(positions[t], theta, rot_dim, c, s);
    for (int h = 0; h < Hq; ++h)
      rotate_head(q + t * q_stride + (int64_t)h * D, q_out + t * q_out_stride + (int64_t)h * D,
                  c, s, D, rot_dim, is_neox, dtype);
    const int64_t slot = slot_mapping[t];
    if (slot >= 0) {
      for (int h = 0; h < Hkv; ++h) {
        rotate_head(k + t * k_stride + (int64_t)h * D,
                    cache_head(key_cache, slot, block_size, Hkv, D, h), c, s, D, rot_dim,
                    is_neox, dtype);
        memcpy(cache_head(value_cache, slot, block_size, Hkv, D, h),
               v + t * v_stride + (int64_t)h * D, (size_t)D * sizeof(uint16_t));
      }
    }
    free(c);
    free(s);
  }
  return ORC_OK;
}

/* The unfused pair the fusion replaces: the rotary_embedding op writes
 * rotated q and k back as tensors, then the KV-cache update op re-reads k and
 * v and writes the slots.  [FUSION] section "RoPE + KV-Cache Update". */
int orc_unfused_rope_kv_write(const int64_t* positions, const uint16_t* q, int64_t q_stride,
                              uint16_t* q_out, int64_t q_out_stride, const uint16_t* k,
                              int64_t k_stride, uint16_t* k_out, const uint16_t* v,
                              int64_t v_stride, double theta, int64_t max_pos,
                              const int64_t* slot_mapping, uint16_t* key_cache,
                              uint16_t* value_cache, int64_t T, int Hq, int Hkv, int D,
                              int rot_dim, int block_size, int64_t num_blocks, int is_neox,
                              int dtype) {
  if (!rope_args_ok(T, Hq, Hkv, D, rot_dim, block_size, num_blocks, is_neox, dtype))
    return ORC_EARG;
  if (!rope_contract_ok(positions, max_pos, slot_mapping, T, block_size, num_blocks))
    return ORC_ECONTRACT;
  /* op 1: rotary embedding of q and k */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* c = (double*)malloc((size_t)rot_dim / 2 * sizeof(double));
    double* s = (double*)malloc((size_t)rot_dim / 2 * sizeof(double));
    rope_angles(positions[t], theta, rot_dim, c, s);
    for (int h = 0; h < Hq; ++h)
      rotate_head(q + t * q_stride + (int64_t)h * D, q_out + t * q_out_stride + (int64_t)h * D,
                  c, s, D, rot_dim, is_neox, dtype);
    for (int h = 0; h < Hkv; ++h)
      rotate_head(k + t * k_stride + (int64_t)h * D, k_out + (t * Hkv + h) * (int64_t)D, c, s,
                  D, rot_dim, is_neox, dtype);
    free(c);
    free(s);
  }
  /* op 2: KV-cache update from the materialized k and the input v */
  for (int64_t t = 0; t < T; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    for (int h = 0; h < Hkv; ++h) {
      memcpy(cache_head(key_cache, slot, block_size, Hkv, D, h),
             k_out + (t * Hkv + h) * (int64_t)D, (size_t)D * sizeof(uint16_t));
      memcpy(cache_head(value_cache, slot, block_size, Hkv, D, h),
             v + t * v_stride + (int64_t)h * D, (size_t)D * sizeof(uint16_t));
    }
  }
  return ORC_OK;
}

/* ======================================================================= */
/* MLA dual RMSNorm (+ FP8 quant of the q latent)                           */
/* ======================================================================= */

/* Normalize one row (no residual) and emit it as bf16 (mode NONE) or as FP8
 * codes with scales. */
static void norm_emit_row(const uint16_t* src, const uint16_t* w, float eps, int64_t H,
                          int mode, int group_size, void* dst, float* scales_row) {
  if (H <= 0) return;
  double* z = (double*)calloc((size_t)H, sizeof(double));
  double* y = (double*)calloc((size_t)H, sizeof(double));
  for (int64_t j = 0; j < H; ++j) z[j] = orc_bf16_decode(src[j]);
  rms_norm_row(z, w, eps, H, y, ORC_DT_BF16);
  if (mode == ORC_Q_NONE) {
    uint16_t* o = (uint16_t*)dst;
    for (int64_t j = 0; j < H; ++j) o[j] = orc_bf16_encode(y[j]);
  } else {
    quant_row(y, H, mode, group_size, 0.0f, (uint8_t*)dst, scales_row);
  }
  free(z);
  free(y);
}

static int dual_args_ok(int64_t T, int64_t Hq, int64_t Hkv, int mode, int group_size) {
  return T >= 0 && Hq > 0 && Hkv > 0 && mode != ORC_Q_STATIC &&
         quant_args_ok(mode, group_size, Hq, 1);
}

/* The paired q_a / kv_a RMSNorms of an MLA layer in one op, each with its own
 * weight and epsilon; optionally the q latent is FP8-quantized (per token or
 * per group) while the kv latent stays bf16.
 * [FUSION] section "MLA Dual RMSNorm (fuse_mla_dual_rms_norm)", including its
 * FP8 per-token-quant variant. */
int orc_dual_rmsnorm_quant(const uint16_t* q, int64_t q_stride, const uint16_t* q_w,
                           float eps_q, const uint16_t* kv, int64_t kv_stride,
                           const uint16_t* kv_w, float eps_kv, int q_quant_mode,
                           int group_size, void* q_out, int64_t q_out_stride, float* q_scales,
                           uint16_t* kv_out, int64_t kv_out_stride, int64_t T, int64_t Hq,
                           int64_t Hkv) {
  if (!dual_args_ok(T, Hq, Hkv, q_quant_mode, group_size)) return ORC_EARG;
  const size_t q_elem = q_quant_mode == ORC_Q_NONE ? sizeof(uint16_t) : sizeof(uint8_t);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    norm_emit_row(q + t * q_stride, q_w, eps_q, Hq, q_quant_mode, group_size,
                  (char*)q_out + (size_t)(t * q_out_stride) * q_elem,
                  scales_row_ptr(q_scales, q_quant_mode, group_size, Hq, t));
    norm_emit_row(kv + t * kv_stride, kv_w, eps_kv, Hkv, ORC_Q_NONE, 0,
                  kv_out + t * kv_out_stride, NULL);
  }
  return ORC_OK;
}

/* The unfused form: two separate norm calls.  When q is quantized the q side
 * is the single-row norm+dynamic-quant op (the residual-free case of
 * orc_fused_add_rmsnorm_quant) and kv is a plain rms_norm.
 * [FUSION] section "MLA Dual RMSNorm", both unfused listings. */
int orc_unfused_dual_rmsnorm_quant(const uint16_t* q, int64_t q_stride, const uint16_t* q_w,
                                   float eps_q, const uint16_t* kv, int64_t kv_stride,
                                   const uint16_t* kv_w, float eps_kv, int q_quant_mode,
                                   int group_size, void* q_out, int64_t q_out_stride,
                                   float* q_scales, uint16_t* kv_out, int64_t kv_out_stride,
                                   int64_t T, int64_t Hq, int64_t Hkv) {
  if (!dual_args_ok(T, Hq, Hkv, q_quant_mode, group_size)) return ORC_EARG;
  int rc;
  if (q_quant_mode == ORC_Q_NONE) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
      norm_emit_row(q + t * q_stride, q_w, eps_q, Hq, ORC_Q_NONE, 0,
                    (uint16_t*)q_out + t * q_out_stride, NULL);
    rc = ORC_OK;
  } else {
    rc = orc_fused_add_rmsnorm_quant(q, q_stride, NULL, 0, q_w, eps_q, q_quant_mode, group_size,
                                     0.0f, (uint8_t*)q_out, q_out_stride, q_scales, T, Hq);
  }
  if (rc != ORC_OK) return rc;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    norm_emit_row(kv + t * kv_stride, kv_w, eps_kv, Hkv, ORC_Q_NONE, 0,
                  kv_out + t * kv_out_stride, NULL);
  return ORC_OK;
}

/* ======================================================================= */
/* Next rows: QK norm + RoPE (+ KV write), RMSNorm + padding, MLA RoPE +    */
/* cache concat                                                             */
/* ======================================================================= */

/* Rotate one head held in double (y[0..D)) and round once to bf16.  Pairs as
 * in rotate_head; dimensions at and past rot_dim pass through (rounded). */
static void rotate_head_f64(const double* y, uint16_t* out, const double* c, const double* s,
                            int D, int rot_dim, int is_neox) {
  const int half = rot_dim / 2;
  for (int i = 0; i < half; ++i) {
    const int a = is_neox ? i : 2 * i;
    const int b = is_neox ? i + half : 2 * i + 1;
    out[a] = orc_bf16_encode(y[a] * c[i] - y[b] * s[i]);
    out[b] = orc_bf16_encode(y[b] * c[i] + y[a] * s[i]);
  }
  for (int d = rot_dim; d < D; ++d) out[d] = orc_bf16_encode(y[d]);
}

/* Per-head RMSNorm of one head of D values with a weight of D values, then
 * the rotation.  round_between = 1 rounds the normalized head to bf16 first,
 * as the unfused sequence materializes it; the fused op rounds once. */
static void norm_rope_head(const uint16_t* in, const uint16_t* w, float eps, int D,
                           const double* c, const double* s, int rot_dim, int is_neox,
                           int round_between, uint16_t* out) {
  double* z = (double*)calloc((size_t)D, sizeof(double));
  double* y = (double*)calloc((size_t)D, sizeof(double));
  for (int d = 0; d < D; ++d) z[d] = orc_bf16_decode(in[d]);
  rms_norm_row(z, w, eps, D, y, ORC_DT_BF16);
  if (round_between)
    for (int d = 0; d < D; ++d) y[d] = orc_bf16_decode(orc_bf16_encode(y[d]));
  rotate_head_f64(y, out, c, s, D, rot_dim, is_neox);
  free(z);
  free(y);
}

static int qknorm_args_ok(int64_t T, int Hq, int Hkv, int D, int rot_dim, int block_size,
                          int64_t num_blocks, int is_neox, int64_t qkv_stride) {
  return rope_args_ok(T, Hq, Hkv, D, rot_dim, block_size, num_blocks, is_neox, ORC_DT_BF16) &&
         qkv_stride >= (int64_t)(Hq + 2 * Hkv) * D;
}

static int qknorm_common(const int64_t* positions, uint16_t* qkv, int64_t qkv_stride,
                         const uint16_t* q_weight, const uint16_t* k_weight, float eps,
                         double theta, int64_t max_pos, const int64_t* slot_mapping,
                         uint16_t* key_cache, uint16_t* value_cache, int write_k, int64_t T,
                         int Hq, int Hkv, int D, int rot_dim, int block_size, int64_t num_blocks,
                         int is_neox, int round_between) {
  if (!qknorm_args_ok(T, Hq, Hkv, D, rot_dim, block_size, num_blocks, is_neox, qkv_stride))
    return ORC_EARG;
  const int with_cache = slot_mapping != NULL;
  if (with_cache && (!key_cache || !value_cache)) return ORC_EARG;
  if (!with_cache) {
    for (int64_t t = 0; t < T; ++t)
      if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ECONTRACT;
  } else if (!rope_contract_ok(positions, max_pos, slot_mapping, T, block_size, num_blocks)) {
    return ORC_ECONTRACT;
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* c = (double*)malloc((size_t)rot_dim / 2 * sizeof(double));
    double* s = (double*)malloc((size_t)rot_dim / 2 * sizeof(double));
    uint16_t* kr = (uint16_t*)malloc((size_t)D * sizeof(uint16_t));
    rope_angles(positions[t], theta, rot_dim, c, s);
    uint16_t* row = qkv + t * qkv_stride;
    uint16_t* k = row + (int64_t)Hq * D;
    const uint16_t* v = k + (int64_t)Hkv * D;
    for (int h = 0; h < Hq; ++h)
      norm_rope_head(row + (int64_t)h * D, q_weight, eps, D, c, s, rot_dim, is_neox,
                     round_between, row + (int64_t)h * D);
    const int64_t slot = with_cache ? slot_mapping[t] : -1;
    for (int h = 0; h < Hkv; ++h) {
      norm_rope_head(k + (int64_t)h * D, k_weight, eps, D, c, s, rot_dim, is_neox,
                     round_between, kr);
      if (slot >= 0) {
        memcpy(cache_head(key_cache, slot, block_size, Hkv, D, h), kr,
               (size_t)D * sizeof(uint16_t));
        memcpy(cache_head(value_cache, slot, block_size, Hkv, D, h), v + (int64_t)h * D,
               (size_t)D * sizeof(uint16_t));
      }
      if (write_k) memcpy(k + (int64_t)h * D, kr, (size_t)D * sizeof(uint16_t));
    }
    free(c);
    free(s);
    free(kr);
  }
  return ORC_OK;
}

/* QK norm + RoPE, optionally with the paged KV-cache write.
 * [FUSION] section "QK Norm + RoPE (enable_qk_norm_rope_fusion)": split the
 * packed qkv row, RMSNorm every q head and every k head (each with its own
 * weight), then the rotary embedding, as one op on qkv.  The q part of qkv is
 * overwritten in place.  The cache write continues it the way section
 * "RoPE + KV-Cache Update" continues plain RoPE (the fuse_qk_norm_rope_kvcache
 * flag is only named on the pages): with slot_mapping given, the rotated k
 * and the unchanged v go to the token's slot; write_k = 1 also writes the
 * rotated k back into qkv.  Readings: per-head RMSNorm over the D values of a
 * head, one weight of D values per q and per k shared by all heads, one eps;
 * one rounding of each output. */
int orc_qk_norm_rope_kv_write(const int64_t* positions, uint16_t* qkv, int64_t qkv_stride,
                              const uint16_t* q_weight, const uint16_t* k_weight, float eps,
                              double theta, int64_t max_pos, const int64_t* slot_mapping,
                              uint16_t* key_cache, uint16_t* value_cache, int write_k,
                              int64_t T, int Hq, int Hkv, int D, int rot_dim, int block_size,
                              int64_t num_blocks, int is_neox) {
  return qknorm_common(positions, qkv, qkv_stride, q_weight, k_weight, eps, theta, max_pos,
                       slot_mapping, key_cache, value_cache, write_k, T, Hq, Hkv, D, rot_dim,
                       block_size, num_blocks, is_neox, 0);
}

/* The unfused sequence of the same section: rms_norm materializes q_norm and
 * k_norm as bf16, then rotary_embedding (and the cache update) runs on them. */
int orc_unfused_qk_norm_rope_kv_write(const int64_t* positions, uint16_t* qkv,
                                      int64_t qkv_stride, const uint16_t* q_weight,
                                      const uint16_t* k_weight, float eps, double theta,
                                      int64_t max_pos, const int64_t* slot_mapping,
                                      uint16_t* key_cache, uint16_t* value_cache, int write_k,
                                      int64_t T, int Hq, int Hkv, int D, int rot_dim,
                                      int block_size, int64_t num_blocks, int is_neox) {
  return qknorm_common(positions, qkv, qkv_stride, q_weight, k_weight, eps, theta, max_pos,
                       slot_mapping, key_cache, value_cache, write_k, T, Hq, Hkv, D, rot_dim,
                       block_size, num_blocks, is_neox, 1);
}

/* Residual add + RMSNorm + padding.
 * [FUSION] section "RMSNorm + Padding (fuse_act_padding)": residual add and
 * RMSNorm, then padding of the hidden dimension to the width the next GEMM
 * wants, as one op (GPT-OSS, hidden 2880).  x, residual, weight and out share
 * one element type, bf16 or fp16 (dtype; the section's support matrix lists
 * FP16/BF16 on ROCm).  Readings: the normalized row is written in that type to
 * out[:, 0:H] and the pad columns out[:, H:H_pad] are +0;
 * the residual is updated in place as in "RMSNorm + Quantization"; H_pad is
 * the caller's choice (the pages do not give the multiple). */
int orc_fused_add_rmsnorm_pad(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                              int64_t res_stride, const uint16_t* weight, float eps,
                              uint16_t* out, int64_t out_stride, int64_t T, int64_t H,
                              int64_t H_pad, int dtype) {
  if (T < 0 || H <= 0 || H_pad < H || out_stride < H_pad) return ORC_EARG;
  if (dtype != ORC_DT_BF16 && dtype != ORC_DT_F16) return ORC_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* z = (double*)malloc((size_t)H * sizeof(double));
    double* y = (double*)malloc((size_t)H * sizeof(double));
    const uint16_t* xr = x + t * x_stride;
    for (int64_t j = 0; j < H; ++j) z[j] = elem_decode(xr[j], dtype);
    if (residual) {
      uint16_t* rr = residual + t * res_stride;
      for (int64_t j = 0; j < H; ++j) {
        rr[j] = elem_encode(z[j] + elem_decode(rr[j], dtype), dtype);
        z[j] = elem_decode(rr[j], dtype);
      }
    }
    rms_norm_row(z, weight, eps, H, y, dtype);
    uint16_t* o = out + t * out_stride;
    for (int64_t j = 0; j < H; ++j) o[j] = elem_encode(y[j], dtype);
    for (int64_t j = H; j < H_pad; ++j) o[j] = 0;
    free(z);
    free(y);
  }
  return ORC_OK;
}

/* MLA: RoPE of the rope parts of q and k, and the MLA cache write of the
 * concatenation [kv_c | rotated k_pe].  The fuse_rope_kvcache_cat_mla flag is
 * only named on the pages ([LEVELS]); the reading joins the MLA split of
 * [FUSION] section "MLA Dual RMSNorm" (kv_lora -> kv_c, k_pe) with the
 * RoPE + KV-cache fusion of section "RoPE + KV-Cache Update": q_pe (Hq heads
 * of rope_dim, head stride q_head_stride) is rotated in place, k_pe (one head
 * of rope_dim shared by all q heads) is rotated, and the cache row of the
 * token's slot, [num_blocks, block_size, kv_lora + rope_dim], receives kv_c
 * (a bit copy: it is already normalized) followed by the rotated k_pe.  Tokens
 * with a negative slot write no cache. */
int orc_mla_rope_kv_write(const int64_t* positions, uint16_t* q_pe, int64_t q_stride,
                          int64_t q_head_stride, const uint16_t* k_pe, int64_t k_pe_stride,
                          const uint16_t* kv_c, int64_t kv_c_stride, double theta,
                          int64_t max_pos, const int64_t* slot_mapping, uint16_t* kv_cache,
                          int64_t T, int Hq, int kv_lora, int rope_dim, int block_size,
                          int64_t num_blocks, int is_neox) {
  if (T < 0 || Hq <= 0 || kv_lora <= 0 || rope_dim <= 0 || rope_dim % 2 != 0 ||
      block_size <= 0 || num_blocks <= 0 || q_head_stride < rope_dim ||
      q_stride < (int64_t)(Hq - 1) * q_head_stride + rope_dim || (is_neox != 0 && is_neox != 1))
    return ORC_EARG;
  if (!rope_contract_ok(positions, max_pos, slot_mapping, T, block_size, num_blocks))
    return ORC_ECONTRACT;
  const int64_t row_w = (int64_t)kv_lora + rope_dim;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* c = (double*)malloc((size_t)rope_dim / 2 * sizeof(double));
    double* s = (double*)malloc((size_t)rope_dim / 2 * sizeof(double));
    rope_angles(positions[t], theta, rope_dim, c, s);
    for (int h = 0; h < Hq; ++h) {
      uint16_t* qh = q_pe + t * q_stride + (int64_t)h * q_head_stride;
      rotate_head(qh, qh, c, s, rope_dim, rope_dim, is_neox, ORC_DT_BF16);
    }
    const int64_t slot = slot_mapping[t];
    if (slot >= 0) {
      uint16_t* dst = kv_cache + slot * row_w;  /* [num_blocks, block_size] flattened */
      memcpy(dst, kv_c + t * kv_c_stride, (size_t)kv_lora * sizeof(uint16_t));
      rotate_head(k_pe + t * k_pe_stride, dst + kv_lora, c, s, rope_dim, rope_dim, is_neox,
                  ORC_DT_BF16);
    }
    free(c);
    free(s);
  }
  return ORC_OK;
}
