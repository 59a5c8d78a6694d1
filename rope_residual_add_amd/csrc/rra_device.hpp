// Device-side building blocks shared by the gfx950 kernels: 128-bit vector
// memory access, bf16 and OCP e4m3fn packing with the CDNA4 conversion
// instructions, and wavefront-64 reductions built from DPP row operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rra {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kWavesPerBlock = 4;  // 256-lane workgroups
constexpr int kBlock = kWave * kWavesPerBlock;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 bf16 or 16 fp8
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // 8 fp8
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---- wave -> work-item mapping ---------------------------------------------
// n / d for 0 <= n < 2^31 as a multiply-high (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994): with
// l = ceil(log2 d), magic = ceil(2^(31 + l) / d) and shift = 31 + l,
// (n * magic) >> shift equals n / d exactly, because magic * d exceeds
// 2^(31 + l) by less than d <= 2^l.  The host builds it (make_fast_div); in a
// kernel the operands are wave-uniform, so the division costs a few scalar
// instructions.
struct FastDiv {
  uint32_t d;
  uint32_t magic;
  uint32_t shift;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * f.magic) >> f.shift);
}

// The same constants with the shift, 31 + ceil(log2 d), recomputed from d (for
// kernels whose first argument words are too precious to carry it).
__device__ __forceinline__ FastDiv fast_div_of(uint32_t d, uint32_t magic) {
  const uint32_t l = d > 1u ? 32u - static_cast<uint32_t>(__clz(d - 1u)) : 0u;
  return FastDiv{d, magic, 31u + l};
}

// Workgroups are dispatched to the 8 XCDs (each with its own L2) in turn:
// workgroup x runs on XCD x % 8.  xcd_block() renumbers them so that runs of
// kXcdRun consecutive numbers share an XCD while the runs still go round the
// XCDs in order: x = 8 kXcdRun c + 8 s + k (XCD k, slot s < kXcdRun) becomes
// kXcdRun (8 c + k) + s.  The last, partial group of 8 kXcdRun workgroups
// keeps its numbers; the map is a bijection on [0, n).
constexpr uint32_t kXcds = 8;
constexpr uint32_t kXcdRun = 16;

// n is the grid size (gridDim.x, which a kernel may instead derive from its
// own arguments: the implicit argument that holds it is not preloaded).
__device__ __forceinline__ uint32_t xcd_block(uint32_t n) {
  const uint32_t x = blockIdx.x;
  const uint32_t full = n / (kXcds * kXcdRun) * (kXcds * kXcdRun);
  if (x >= full) return x;
  const uint32_t k = x % kXcds, s = x / kXcds;
  return (s / kXcdRun * kXcds + k) * kXcdRun + s % kXcdRun;
}

// ---- memory ---------------------------------------------------------------
// Streaming data is touched exactly once, so loads and stores of activations
// use the non-temporal hint; weights and tables use ordinary loads.

__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld_cached(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ f32x4 ld_f32x4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void st_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_stream(void* p, u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

// ---- bf16 ---------------------------------------------------------------
// A 32-bit word holds two bf16 values, element 2i in the low half.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two bf16, round-to-nearest-even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// IEEE binary16 halves of a packed word (exact widening to fp32).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2, w)[0]);
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2, w)[1]);
}

// Two fp32 -> two fp16, round-to-nearest-even, overflow to infinity.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// The 16-bit element types a kernel can be instantiated for: unpack the two
// halves of a 32-bit word to fp32 and pack two fp32 values back (RNE).
struct ElemBf16 {
  static __device__ __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};
struct ElemF16 {
  static __device__ __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
};

// ---- OCP e4m3fn -----------------------------------------------------------
// gfx950's v_cvt_pk_fp8_f32 converts to OCP e4m3fn with round-to-nearest-even:
// magnitudes up to 464 (the midpoint above 448, a tie that goes to the even
// code 448) give finite codes, larger ones give NaN (0x7F).  Saturating
// conversion clamps to +-448 first (v_med3_f32, which would turn a NaN into
// -448, so a NaN is passed through to the conversion as it is); a caller whose
// values are known to stay below 464 in magnitude (dynamic scales, where the
// largest |y / s| is 448 within a few ulps) skips the clamp.

__device__ __forceinline__ float clamp_e4m3(float v) {
  return __builtin_isnan(v) ? v : __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// Four fp32 -> four e4m3fn bytes, element 0 in the lowest byte; kClamp
// saturates to +-448 first.
template <bool kClamp = true>
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  if (kClamp) {
    a = clamp_e4m3(a);
    b = clamp_e4m3(b);
    c = clamp_e4m3(c);
    d = clamp_e4m3(d);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// ---- correctly rounded quantization ------------------------------------------
// A code is e4m3fn(q) of the exact quotient q = y / s.  Dynamic scales make
// exact ties common: y / s = 448 * t / m * (1 + d), where t and m (products of
// two bf16 values) often stand in a short ratio such as 3/8 that puts
// 448 * t / m exactly on an e4m3 rounding midpoint, and only the tiny offset d
// left by rounding s to fp32 decides the side.  An fp32 quotient cannot see d.
// So each value is bracketed: v_dn = fp32(t * f_dn) and v_up = fp32(t * f_up)
// with f_dn and f_up fp32 multipliers a little below and above rho / s, so
// that q lies strictly between v_dn and v_up.  Rounding to e4m3 is monotone,
// so where the two give the same code that code is e4m3fn(q).  Where they
// differ a rounding midpoint lies within about 2^-20 of q (an exact tie, or a
// near one, about 2.5e-4 of the codes at dynamic scales): q = (t * rho) / s is
// then recomputed in double (the quotient correctly rounded) and narrowed to
// fp32 with round-to-odd, after which the single hardware rounding to e4m3 is
// the correct rounding of q (fp32 keeps 20 more fraction bits than e4m3;
// round-to-odd makes the double rounding innocuous).  The bracket needs no
// special case for e4m3 subnormals, zeros or saturation: it holds wherever
// t * f is a normal fp32 number, and below that (|q| < 2^-126) every code is
// a zero of t's sign on both sides.

// double -> fp32 rounding to odd: truncate toward zero, set the last bit if
// anything was discarded.
__device__ __forceinline__ float f32_round_odd(double q) {
  const float v = static_cast<float>(q);  // to nearest even
  const double back = static_cast<double>(v);
  if (back == q) return v;
  uint32_t b = __float_as_uint(v);
  if (fabs(back) > fabs(q)) b -= 1u;  // rounded away from zero: step back
  return __uint_as_float(b | 1u);
}

// A quantization step: codes e4m3fn(t * rho / s).  f = fp32(rho) * rcp(s) is
// within 2.5 fp32 ulps (2^-21.6 relative) of rho / s, so f_dn = f (1 - 2^-20)
// and f_up = f (1 + 2^-20), each rounded once more, lie below and above it by
// more than 2^-21; after the final rounding of t * f (2^-24) the bracket still
// holds.  A scale that is not positive (s = 0 for an all-zero slice; NaN where
// rho is NaN, from a NaN or infinite value in the row) becomes s = 0, and such
// a slice gets +0 codes.  Where rho / s leaves the normal fp32 range (a row of
// values near the fp32 subnormal range, where rho or 448 / amax is huge) or s
// is itself subnormal (whose hardware reciprocal is not accurate), the bracket
// is made [0, inf]: the two codes then differ for every value (0 against NaN
// or 448), so every value takes the exact path.
struct QuantStep {
  float f_dn;
  float f_up;
  float s;
  double rho;
};

__device__ __forceinline__ QuantStep quant_step(double rho, float s) {
  if (!(s > 0.0f)) return QuantStep{0.0f, 0.0f, 0.0f, rho};
  const float f = static_cast<float>(rho) * __builtin_amdgcn_rcpf(s);
  // false for an infinite or NaN f too
  const bool in_range = f < 0x1p127f && f >= 0x1p-126f && s >= 0x1p-126f;
  if (!in_range) return QuantStep{0.0f, __builtin_inff(), s, rho};
  return QuantStep{f * (1.0f - 0x1p-20f), f * (1.0f + 0x1p-20f), s, rho};
}

// Eight codes from a bracket [f_dn, f_up] around the multiplier rho / s:
// c = e4m3fn(t[j] * f_dn) for j = 0..7 and d = c ^ e4m3fn(t[j] * f_up), so a
// nonzero byte of d flags a code the bracket leaves open.  kClamp = false when
// s is a dynamic scale (|t * rho / s| <= 448 within rounding; the conversion
// rounds up to 464 to 448 by itself).
struct Bracket8 {
  u32x2 c;
  u32x2 d;
};

template <bool kClamp>
__device__ __forceinline__ Bracket8 bracket8(const float t[8], float f_dn, float f_up) {
  float lo[8], hi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo[j] = t[j] * f_dn;
    hi[j] = t[j] * f_up;
  }
  const u32x2 c{pack_e4m3x4<kClamp>(lo[0], lo[1], lo[2], lo[3]),
                pack_e4m3x4<kClamp>(lo[4], lo[5], lo[6], lo[7])};
  return Bracket8{c, u32x2{c[0] ^ pack_e4m3x4<kClamp>(hi[0], hi[1], hi[2], hi[3]),
                           c[1] ^ pack_e4m3x4<kClamp>(hi[4], hi[5], hi[6], hi[7])}};
}

// The codes of a bracket with its open ones settled: each flagged code is
// recomputed from the exact quotient q = (t * rho) / s, correctly rounded in
// double: q0 = p * y with y the rounded reciprocal of s, then one correction
// with the residual p - q0 * s, which an fma gives exactly (Markstein's final
// division step), narrowed to fp32 with round-to-odd.  Taking p * (rho / s)
// instead can miss an exact midpoint by an ulp of the double, and the
// round-to-odd narrowing would then move a true tie off it.  The quotient
// takes t's sign: the correction cannot flip a nonzero q0, but for t = -0 the
// residual sum +0 + -0 is +0.  Requires s > 0.
template <bool kClamp>
__device__ __forceinline__ u32x2 settle8(const float t[8], const Bracket8& b, float f_dn, float s,
                                         double rho) {
  if ((b.d[0] | b.d[1]) == 0u) return b.c;
  float lo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lo[j] = t[j] * f_dn;
  const double sd = static_cast<double>(s);
  const double y = 1.0 / sd;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if ((((j < 4 ? b.d[0] : b.d[1]) >> (8 * (j & 3))) & 0xFFu) != 0u) {
      const double p = static_cast<double>(t[j]) * rho;
      const double q0 = p * y;
      lo[j] = copysignf(f32_round_odd(fma(fma(-q0, sd, p), y, q0)), t[j]);
    }
  }
  return u32x2{pack_e4m3x4<kClamp>(lo[0], lo[1], lo[2], lo[3]),
               pack_e4m3x4<kClamp>(lo[4], lo[5], lo[6], lo[7])};
}

// Eight codes e4m3fn(t[j] * rho / s) for a quantization step.
template <bool kClamp>
__device__ __forceinline__ u32x2 quant8(const float t[8], const QuantStep& qs) {
  if (!(qs.s > 0.0f)) return u32x2{0u, 0u};
  return settle8<kClamp>(t, bracket8<kClamp>(t, qs.f_dn, qs.f_up), qs.f_dn, qs.s, qs.rho);
}

// Dynamic scales before rho is known.  With s = fp32(m * rho / 448) for a
// slice of amax m * rho (m = max |t|), the multiplier is rho / s =
// 448 / (m (1 + e)), where e (|e| <= 2^-24 for a normal s) is the rounding of
// s; the row's rho cancels.  So f = fp32(448 * rcp(m)) (the hardware
// reciprocal is within 1 ulp) lies within 2^-21.6 of rho / s, the same
// distance as the multiplier of quant_step, and the same bracket f (1 -+ 2^-20)
// encloses every quotient of the slice.  Its codes can be formed while rho is
// still being computed; once rho is known, dyn_settle takes s and settles
// what the bracket leaves open.  Where m or f is not a normal fp32 number
// (an amax near the fp32 subnormal range; m = 0, infinite or NaN) the bracket
// is [0, inf] and every code is recomputed, as in quant_step.
struct DynStep {
  float f_dn;
  float f_up;
};

__device__ __forceinline__ DynStep dyn_step(float m) {
  const float f = 448.0f * __builtin_amdgcn_rcpf(m);
  const bool in_range = m >= 0x1p-126f && f < 0x1p127f && f >= 0x1p-126f;
  if (!in_range) return DynStep{0.0f, __builtin_inff()};
  return DynStep{f * (1.0f - 0x1p-20f), f * (1.0f + 0x1p-20f)};
}

// A slice's codes with a dynamic scale s, from its bracket (dyn_step(m)).  A
// scale that is not positive (an all-zero slice, or a row whose rho is 0 or
// NaN because it holds an infinite or NaN value) gives +0 codes; a scale that
// is not a normal fp32 number breaks the bound on e, so every code is then
// recomputed.
__device__ __forceinline__ u32x2 dyn_settle(const float t[8], Bracket8 b, const DynStep& ds,
                                            float s, double rho) {
  if (!(s > 0.0f)) return u32x2{0u, 0u};
  if (!(s >= 0x1p-126f && s < __builtin_inff())) b.d = u32x2{~0u, ~0u};
  return settle8<false>(t, b, ds.f_dn, s, rho);
}

// a / b correctly rounded, given r = 1/b correctly rounded: the product
// q0 = a * r, corrected once by its residual a - q0 * b, which an fma gives
// exactly (Markstein's final division step).  A non-finite q0 (a infinite) is
// returned as it is.
__device__ __forceinline__ double div_rn(double a, double b, double r) {
  const double q0 = a * r;
  return __builtin_isfinite(q0) ? fma(fma(-q0, b, a), r, q0) : q0;
}

// ---- wavefront reductions ---------------------------------------------------
// DPP moves within 16-lane rows: quad_perm [1,0,3,2] (0xB1), quad_perm
// [2,3,0,1] (0x4E), row_half_mirror (0x141), row_mirror (0x140); across rows:
// row_bcast:15 (0x142) and row_bcast:31 (0x143).  Every combining step adds
// the same two partials in both lanes of a pair, so all lanes of a segment end
// with bit-identical results (fp addition and max are commutative).
// The moves carry no "old" value: within-row patterns write every lane from a
// valid source, and the row-masked broadcasts leave the other rows undefined,
// which only the whole-wave reductions use and only through lane 63, whose sum
// never reads them.  (A zero "old" costs one extra move per step.)

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, kRowMask, 0xF, true));
}

// The max reductions take non-negative values only (amaxes of |x|), whose
// bit patterns order like unsigned integers: the cross-lane steps compare the
// bits with v_max_u32, which needs no NaN canonicalization (fmaxf adds one
// instruction per step) and takes the DPP move as an operand modifier.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), kCtrl, kRowMask, 0xF, true));
}

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t max_step(uint32_t u) {
  const uint32_t o = dpp_u32<kCtrl, kRowMask>(u);
  return u > o ? u : o;
}

// Max over each aligned group of 8 lanes (inputs >= 0), result in all 8.
__device__ __forceinline__ float max8(float v) {
  uint32_t u = __float_as_uint(v);
  u = max_step<0xB1>(u);
  u = max_step<0x4E>(u);
  u = max_step<0x141>(u);
  return __uint_as_float(u);
}

// Max over each 16-lane row (inputs >= 0), result in all 16.
__device__ __forceinline__ float max16(float v) {
  uint32_t u = __float_as_uint(max8(v));
  return __uint_as_float(max_step<0x140>(u));
}

__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

__device__ __forceinline__ float readlane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the whole wave; the result is wave-uniform (an SGPR).
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  v += dpp<0x142, 0xA>(v);  // rows 1, 3 += last lane of rows 0, 2
  v += dpp<0x143, 0xC>(v);  // rows 2, 3 += lane 31
  return readlane63(v);
}

// Sum of doubles over the whole wave, with the same DPP pattern applied to
// both 32-bit halves; wave-uniform result.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(u & 0xFFFFFFFFu), kCtrl, kRowMask, 0xF, true));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), kCtrl, kRowMask, 0xF, true));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Max over aligned groups of n lanes (n = 8 or 16) of doubles >= 0; result in
// every lane of the group.
template <int n>
__device__ __forceinline__ double group_max_f64(double v) {
  static_assert(n == 8 || n == 16, "group size");
  v = fmax(v, dpp_f64<0xB1>(v));
  v = fmax(v, dpp_f64<0x4E>(v));
  v = fmax(v, dpp_f64<0x141>(v));
  if (n == 16) v = fmax(v, dpp_f64<0x140>(v));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  v += dpp_f64<0x142, 0xA>(v);
  v += dpp_f64<0x143, 0xC>(v);
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), 63));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Sums of two rows' doubles at once, one value per lane of each: a (lanes
// 0-63) and b (lanes 0-63).  v_permlane32_swap exchanges the upper half of a
// with the lower half of b, so that one add leaves a's half sums in lanes
// 0-31 and b's in lanes 32-63; five DPP steps then finish each half (the last
// adds row 0 into row 1 and row 2 into row 3).  Lane 31 ends with the sum of
// a, lane 63 with the sum of b; other lanes hold partial sums.  Half the DPP
// work of two whole-wave reductions, in a fixed order.
__device__ __forceinline__ double pair_sum_f64(double a, double b) {
  const uint64_t ua = static_cast<uint64_t>(__double_as_longlong(a));
  const uint64_t ub = static_cast<uint64_t>(__double_as_longlong(b));
  const auto lo = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(ua),
                                                   static_cast<uint32_t>(ub), false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(ua >> 32),
                                                   static_cast<uint32_t>(ub >> 32), false, false);
  const double x = __longlong_as_double(
      static_cast<long long>((static_cast<uint64_t>(hi[0]) << 32) | lo[0]));
  const double y = __longlong_as_double(
      static_cast<long long>((static_cast<uint64_t>(hi[1]) << 32) | lo[1]));
  double v = x + y;
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  v += dpp_f64<0x142, 0xA>(v);
  return v;
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), lane));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Max over the whole wave (inputs >= 0); wave-uniform result.
__device__ __forceinline__ float wave_max(float v) {
  uint32_t u = __float_as_uint(max16(v));
  u = max_step<0x142, 0xA>(u);
  u = max_step<0x143, 0xC>(u);
  return readlane63(__uint_as_float(u));
}

// Index of this lane's wave inside its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Kernel arguments: gfx950 starts a wave with the first 14 dwords of its
// arguments in scalar registers (with the library's preload build flag); the
// rest are fetched by scalar loads, which the compiler issues where a value is
// first used, so an argument first used by a kernel's last stores costs a
// memory round trip at the end of the wave's chain.  args_ready(a, ...) makes
// the arguments resident at the point of the call: placed right after a
// kernel's first vector loads are issued, their fetch runs under those loads.
// The scheduler may still move ordinary loads across it; where it would hoist
// the wait above them, a __builtin_amdgcn_sched_barrier(0) before the call
// keeps the loads first.
template <typename V>
__device__ __forceinline__ void arg_ready(V v) {
  asm volatile("" ::"s"(v));
}

template <typename... A>
__device__ __forceinline__ void args_ready(A... a) {
  (arg_ready(a), ...);
}

// Dynamic scale from an amax given as m * rho (m >= 0 exact in fp32, rho in
// double): s = fp32(m * rho / 448), 448 being e4m3fn's largest finite value,
// computed as m * rho448 with rho448 = rho * (1/448) formed once per row.  The
// double product then differs from m * rho / 448 by at most two ulps, which
// moves the fp32 result only if it lies within 2^-51 of an fp32 rounding
// boundary.
__device__ __forceinline__ double rho_448(double rho) { return rho * (1.0 / 448.0); }

__device__ __forceinline__ float dynamic_scale(float m, double rho448) {
  return static_cast<float>(static_cast<double>(m) * rho448);
}

// 1/sqrt(x) in double for x > 0: the hardware estimate refined by two Newton
// steps y <- y + y/2 * (1 - x y^2), each roughly doubling the correct bits.
// x = +inf gives 0 (the steps alone would give inf * 0 = NaN).
__device__ __forceinline__ double rsqrt_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const double e = fma(-x * y, y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return __builtin_isinf(x) ? 0.0 : y;
}

}  // namespace rra
