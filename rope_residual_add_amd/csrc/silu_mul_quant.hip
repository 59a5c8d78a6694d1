// SiLU-and-Mul + FP8 quant for gfx950.
//
// Operation: vLLM design page "Fusion torch.compile passes", section
// "SiLU+Mul + Quantization (fuse_act_quant)": the gate-up activation
// silu(gate) * up followed by static or per-group FP8 quantization, without
// writing the activation to memory.
//
// Mapping: each wavefront owns one chunk of 512 output columns of one row
// (wave g of the launch: row g / chunks, chunk g % chunks, the division a
// multiply-high).  Lane l handles the chunk's vector l (8 columns) and loads
// the matching 16-byte vectors of the gate half and of the up half, so every
// load instruction of the wave reads 1 KiB of contiguous memory.  A group of
// 128 (64) outputs is 16 (8) consecutive lanes: the group amax is a DPP row
// reduction.  Measured at T = 8192, I = 14336: one vector per lane and 32-bit
// index arithmetic beat 2 or 4 vectors per lane (fewer, longer waves) by 3%;
// with the earlier 64-bit row division one vector per lane was 8% slower.
//
// Arithmetic budget: at the HBM roofline this kernel has about 25 VALU lane
// slots per output element on MI355X (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
// against 5 bytes of traffic per output element at 8 TB/s), and the loop
// already needs most of them.  A correctly rounded expf and fp32 divide would
// use more than that, so silu uses the hardware exp2 and reciprocal:
// silu(g) * u = (g * rcp(1 + exp2(-g * log2(e)))) * u, relative error ~1e-6,
// which moves an FP8 code only for values within that distance of a rounding
// midpoint.
#include "rra_device.hpp"
#include "rra_host.hpp"

namespace rra {

// silu(g) is formed before the product with u, so that a large u cannot
// meet an overflowed g * u (g = -100, u = 4e36: -inf * 0 = NaN, where
// silu(g) * u is about -1.5e-5).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

__device__ __forceinline__ void silu8(u32x4 g, u32x4 u, float a[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[2 * k] = silu_mul(bf16_lo(g[k]), bf16_lo(u[k]));
    a[2 * k + 1] = silu_mul(bf16_hi(g[k]), bf16_hi(u[k]));
  }
}

// The per-group path for a group whose activations leave the range of the
// fp32 path, in double: a = g / (1 + exp(-g)) * u from the bf16 inputs,
// s = fp32(max |a| / 448) (infinite where that exceeds fp32, as it rounds),
// and each code's quotient a / s narrowed to fp32 with round-to-odd before the
// one rounding to e4m3 (as the exact path of the norms).  Called by every lane
// of a group when its fp32 amax is below 2^-100 or infinite (NaN activations
// do not count towards it); a group with no nonzero product g * u keeps s = 0
// and gets +0 codes, as any slice whose scale is 0.
template <int kGroup>
__device__ __forceinline__ void double_group(u32x4 gv, u32x4 uv, float& s, float v[8]) {
  double a[8];
  bool nonzero = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double g0 = bf16_lo(gv[k]), g1 = bf16_hi(gv[k]);
    const double u0 = bf16_lo(uv[k]), u1 = bf16_hi(uv[k]);
    a[2 * k] = g0 / (1.0 + exp(-g0)) * u0;
    a[2 * k + 1] = g1 / (1.0 + exp(-g1)) * u1;
    nonzero |= (g0 != 0.0 && u0 != 0.0) || (g1 != 0.0 && u1 != 0.0);
  }
  double m = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmax(m, fabs(a[j]));
  m = group_max_f64<kGroup / 8>(m);
  const float nz = group_max_f64<kGroup / 8>(nonzero ? 1.0 : 0.0);
  if (nz == 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    return;
  }
  s = static_cast<float>(m / 448.0);
  const double sd = static_cast<double>(s);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = s > 0.0f ? f32_round_odd(a[j] / sd) : 0.0f;
}

// kMode RRA_Q_STATIC or RRA_Q_PER_GROUP with kGroup 64 or 128 (compile-time,
// so group indexing is a shift).  kFull: I is a whole number of chunks, so
// every vector index is in range and the bounds test is compiled out.
template <int kMode, int kGroup, bool kFull>
__global__ void __launch_bounds__(kBlock)
    silu_mul_quant_kernel(uint32_t chunks_d, uint32_t chunks_magic, uint32_t chunks_shift,
                          uint32_t T, int I, const uint16_t* __restrict__ in, int64_t in_stride,
                          uint8_t* __restrict__ out, int64_t out_stride,
                          float* __restrict__ scales, const float* __restrict__ static_scale) {
  static_assert(kMode == RRA_Q_STATIC || kGroup == 64 || kGroup == 128, "group size");
  // The launch shape leads the argument list as plain scalars, so that it is
  // preloaded into scalar registers with the first pointers.
  const FastDiv chunks{chunks_d, chunks_magic, chunks_shift};
  const uint32_t g = blockIdx.x * kWavesPerBlock + static_cast<uint32_t>(wave_id());
  const uint32_t row = fast_div(g, chunks);
  if (row >= T) return;  // whole waves; no barrier in this kernel
  const int lane = lane_id();
  const int idx = static_cast<int>(g - row * chunks.d) * kWave + lane;  // vector in the row
  const bool in_row = kFull || idx < (I >> 3);
  const uint16_t* gate = in + row * in_stride + idx * 8;

  u32x4 gv = u32x4{0u, 0u, 0u, 0u}, uv = u32x4{0u, 0u, 0u, 0u};
  if (in_row) {
    gv = ld_stream(gate);
    uv = ld_stream(gate + I);
  }
  float a[8];
  silu8(gv, uv, a);
  uint8_t* o = out + row * out_stride + idx * 8;
  if constexpr (kMode == RRA_Q_STATIC) {
    const float f = 1.0f / static_scale[0];
    if (in_row)
      st_stream(o, u32x2{pack_e4m3x4(a[0] * f, a[1] * f, a[2] * f, a[3] * f),
                         pack_e4m3x4(a[4] * f, a[5] * f, a[6] * f, a[7] * f)});
  } else {  // RRA_Q_PER_GROUP
    constexpr int kLanesPerGroup = kGroup / 8;
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(a[j]));
    m = kGroup == 128 ? max16(m) : max8(m);
    // s = amax / 448 and f = 1 / s with a multiply and the hardware
    // reciprocal: the activation itself carries ~1e-6 relative error, so
    // correctly rounded divisions would buy nothing here.
    float s = m * (1.0f / 448.0f);
    float f = s > 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = a[j] * f;
    // A group whose activations are all below 2^-100 (gates below about -88,
    // where exp overflows and the fp32 silu flushes to 0, or values near the
    // fp32 subnormal range), or whose largest one overflows fp32 (|silu(g) u|
    // above 3.4e38, or an infinite input), is redone in double from the bf16
    // inputs, unless every product g * u is exactly 0 (an all-zero group needs
    // nothing).
    if (__builtin_expect(!(m >= 0x1p-100f && m < __builtin_inff()), 0))
      double_group<kGroup>(gv, uv, s, v);
    if (in_row) {
      if ((lane & (kLanesPerGroup - 1)) == 0)
        scales[static_cast<int64_t>(row) * (I / kGroup) + idx / kLanesPerGroup] = s;
      // |a * f| <= 448 within rounding: no saturation needed
      st_stream(o, u32x2{pack_e4m3x4<false>(v[0], v[1], v[2], v[3]),
                         pack_e4m3x4<false>(v[4], v[5], v[6], v[7])});
    }
  }
}

// Arguments of one launch.
struct SiluLaunch {
  dim3 grid;
  hipStream_t st;
  const uint16_t* in;
  int64_t in_stride;
  const float* static_scale;
  uint8_t* out;
  int64_t out_stride;
  float* scales;
  uint32_t T;
  int I;
  FastDiv chunks;
};

template <bool kFull, int kMode, int kGroup>
static void launch_silu(const SiluLaunch& a) {
  hipLaunchKernelGGL((silu_mul_quant_kernel<kMode, kGroup, kFull>), a.grid, dim3(kBlock), 0,
                     a.st, a.chunks.d, a.chunks.magic, a.chunks.shift, a.T, a.I, a.in, a.in_stride,
                     a.out, a.out_stride, a.scales, a.static_scale);
}

template <bool kFull>
static void launch_silu_mode(const SiluLaunch& a, int mode, int group) {
  if (mode == RRA_Q_STATIC)
    launch_silu<kFull, RRA_Q_STATIC, 0>(a);
  else if (group == 64)
    launch_silu<kFull, RRA_Q_PER_GROUP, 64>(a);
  else
    launch_silu<kFull, RRA_Q_PER_GROUP, 128>(a);
}

}  // namespace rra

using namespace rra;

extern "C" int silu_mul_quant(const uint16_t* in, int64_t in_stride, int quant_mode,
                              int group_size, const float* static_scale, uint8_t* out,
                              int64_t out_stride, float* scales, int64_t T, int64_t I,
                              void* stream) {
  RRA_REQUIRE(T >= 0 && I > 0, RRA_ERR_SHAPE);
  RRA_REQUIRE(I % 8 == 0 && I <= (int64_t(1) << 30), RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(T == 0 || (in && out), RRA_ERR_NULL);  // empty tensors have no storage
  RRA_REQUIRE(in_stride >= 2 * I && out_stride >= I, RRA_ERR_SHAPE);
  switch (quant_mode) {
    case RRA_Q_STATIC:
      RRA_REQUIRE(static_scale, RRA_ERR_NULL);
      RRA_REQUIRE(aligned(static_scale, 4), RRA_ERR_ALIGN);
      break;
    case RRA_Q_PER_GROUP:
      RRA_REQUIRE(group_ok(group_size), RRA_ERR_UNSUPPORTED);
      RRA_REQUIRE(I % group_size == 0, RRA_ERR_SHAPE);
      RRA_REQUIRE(scales || T == 0, RRA_ERR_NULL);
      RRA_REQUIRE(aligned(scales, 4), RRA_ERR_ALIGN);
      break;
    default:
      return RRA_ERR_UNSUPPORTED;
  }
  RRA_REQUIRE(vec_ok(in, in_stride), RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(out, 8) && out_stride % 8 == 0, RRA_ERR_ALIGN);
  if (T == 0) return RRA_OK;

  // One wave per 512-column chunk of a row; the launch's wave index stays
  // below 2^31 (the multiply-high division's range).
  const int64_t chunks = ceil_div(I, 8 * kWave);
  RRA_REQUIRE(T <= 0x7FFFFFFF && T * chunks <= 0x7FFFFFFF - kWavesPerBlock,
              RRA_ERR_UNSUPPORTED);
  const int64_t blocks = ceil_div(T * chunks, kWavesPerBlock);
  const SiluLaunch a{dim3(static_cast<unsigned>(blocks)), as_stream(stream), in, in_stride,
                     static_scale, out, out_stride, scales, static_cast<uint32_t>(T),
                     static_cast<int>(I), make_fast_div(static_cast<uint32_t>(chunks))};
  if (I % (8 * kWave) == 0)
    launch_silu_mode<true>(a, quant_mode, group_size);
  else
    launch_silu_mode<false>(a, quant_mode, group_size);
  return launch_status();
}
