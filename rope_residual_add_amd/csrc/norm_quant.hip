// Residual add + RMSNorm + FP8 quant, and the MLA dual RMSNorm (+ FP8 quant
// of the q latent), for gfx950.
//
// Operations: vLLM design page "Fusion torch.compile passes", sections
// "RMSNorm + Quantization (fuse_norm_quant)" (rms_norm / fused_add_rms_norm
// followed by static, per-token or per-token-group FP8 quant, residual updated
// in place) and "MLA Dual RMSNorm (fuse_mla_dual_rms_norm)" (the q_a and kv_a
// norms in one launch; in the FP8 variant only q is quantized).
//
// Mapping: a row of H bf16 values is spread over the lanes of kW waves as
// 16-byte vectors: "row lane" rl = (wave within the row) * 64 + lane holds
// vectors rl, rl + 64 kW, rl + 128 kW, ... so every vector load of a wave
// reads 1 KiB of contiguous memory.  The row stays in VGPRs between the read
// and the write, so each element crosses HBM once in each direction.  Each
// wave reduces its share of the row statistics (sum of squares, amax) with
// DPP; with kW > 1 one LDS exchange and one barrier combine the kW partials in
// a fixed order, so every wave of the row sees bit-identical statistics.  A
// quantization group of 128 (64) columns is exactly 16 (8) consecutive lanes
// of one vector, so group amaxes are DPP row reductions with no exchange.
// Rows past the end are predicated off rather than returned from, so that
// every wave of a workgroup reaches the barrier.
//
// Statistics and scales are in double, and codes are rounded as the exact
// quotient would be (rra_device.hpp).  With a dynamic scale the row's rho
// cancels in y / s, so the codes are bracketed from the amaxes alone while rho
// is still being computed; after rho only the scales, a range check and the
// rare exact-quotient path remain (dyn_prepare, dyn_emit).
#include "rra_device.hpp"
#include "rra_host.hpp"

namespace rra {

// One row lane's share of a row: vector i covers columns (i * stride + rl) * 8.
// kFull: the row is exactly NV * stride vectors, so every index is in range
// and the per-vector bounds tests (which cost measurably in these short,
// latency-bound kernels) are compiled out.
template <int NV>
struct RowVecs {
  u32x4 v[NV];
};

template <int NV, bool kStream, bool kFull>
__device__ __forceinline__ void load_row(RowVecs<NV>& r, const uint16_t* base, int nvec, int rl,
                                         int stride, bool active) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = i * stride + rl;
    if (active && (kFull || idx < nvec))
      r.v[i] = kStream ? ld_stream(base + idx * 8) : ld_cached(base + idx * 8);
    else
      r.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int NV, bool kFull>
__device__ __forceinline__ void store_row(uint16_t* base, const RowVecs<NV>& r, int nvec, int rl,
                                         int stride) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = i * stride + rl;
    if (kFull || idx < nvec) st_stream(base + idx * 8, r.v[i]);
  }
}

// A row lane's share of t = z * w in fp32 (exact: 8-bit by 8-bit
// significands), which is all the output stage needs of z and w.
template <int NV>
struct RowT {
  float t[NV][8];
};

// One pass over this lane's vectors: t = z * w, the sum of z^2 in double
// (each z widened to double and squared by an fma: the sum keeps enough bits
// that the fp32 rounding of a scale derived from it is the one the plain
// definition gives) and, when wanted, max |t|.  E is the element type of z and
// w; t is exact in fp32 for bf16 (8 x 8 significand bits) and fp16 (11 x 11).
// Each vector has its own accumulator, so the dependent chain of double fmas
// is 8 long rather than 8 NV (the serial latency of a lone wave at decode
// sizes).
template <int NV, typename E = ElemBf16>
__device__ __forceinline__ void row_prepare(const RowVecs<NV>& z, const RowVecs<NV>& w,
                                            bool want_max, RowT<NV>& t, double& ss, float& m) {
  double acc[NV];
  m = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    acc[i] = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = E::lo(z.v[i][k]), b = E::hi(z.v[i][k]);
      const double ad = static_cast<double>(a), bd = static_cast<double>(b);
      acc[i] = fma(ad, ad, acc[i]);
      acc[i] = fma(bd, bd, acc[i]);
      t.t[i][2 * k] = a * E::lo(w.v[i][k]);
      t.t[i][2 * k + 1] = b * E::hi(w.v[i][k]);
    }
    if (want_max) {
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(t.t[i][j]));
    }
  }
  ss = acc[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) ss += acc[i];
}

// rho = 1/sqrt(ss / H + eps) of a row, in double, with ss / H correctly
// rounded from r = 1/H (itself correctly rounded): a product and one
// correction rather than a full division, which would lengthen the chain that
// every wave of the row waits on.
__device__ __forceinline__ double row_rho(double ss, double H, double r, float eps) {
  return rsqrt_f64(div_rn(ss, H, r) + static_cast<double>(eps));
}

// Combine the partials of the kW waves of a row: wave-level DPP reductions,
// then (kW > 1) an exchange through LDS slots [slot0, slot0 + kW).  Must be
// reached by every wave of the workgroup.
template <int kW>
__device__ __forceinline__ void row_reduce(double& ss, float& m, double* lds_ss, float* lds_m,
                                           int slot0, int wave_in_row) {
  ss = wave_sum_f64(ss);
  m = wave_max(m);
  if (kW > 1) {
    if (lane_id() == 0) {
      lds_ss[slot0 + wave_in_row] = ss;
      lds_m[slot0 + wave_in_row] = m;
    }
    __syncthreads();
    ss = lds_ss[slot0];
    m = lds_m[slot0];
#pragma unroll
    for (int j = 1; j < kW; ++j) {
      ss += lds_ss[slot0 + j];
      m = fmaxf(m, lds_m[slot0 + j]);
    }
  }
}

// The row's output from rho = 1/sqrt(ss / H + eps):
//   y = t * rho
// mode NONE writes y rounded to the element type E to out (uint16_t*); the
// static mode (E = bf16 inputs only) writes e4m3fn(y / s) to out (uint8_t*),
// rounded as the exact quotient would be (quant8).  The dynamic modes use
// dyn_prepare and dyn_emit: because rho > 0 is one number per row,
// max|y| = max|t| * rho, so the amax needs no second pass over y and the
// codes need no rho at all.
template <int NV, int kMode, bool kFull, typename E = ElemBf16>
__device__ __forceinline__ void rmsnorm_emit(const RowT<NV>& t, double rho, int nvec, int rl,
                                             int stride, float static_scale, void* out) {
  if constexpr (kMode == RRA_Q_NONE) {
    const float rho_f = static_cast<float>(rho);
    uint16_t* o = static_cast<uint16_t*>(out);
    // A row of values near the fp32 subnormal range (with eps = 0) can have a
    // rho beyond fp32: then y = t * rho is formed in double.
    const bool wide = !(rho_f < 0x1p127f);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = i * stride + rl;
      float y[8];
      if (!wide) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = t.t[i][k] * rho_f;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = static_cast<float>(static_cast<double>(t.t[i][k]) * rho);
      }
      const u32x4 packed{E::pack(y[0], y[1]), E::pack(y[2], y[3]), E::pack(y[4], y[5]),
                         E::pack(y[6], y[7])};
      if (kFull || idx < nvec) st_stream(o + idx * 8, packed);
    }
  } else {
    static_assert(kMode == RRA_Q_STATIC, "dynamic scales go through dyn_prepare / dyn_emit");
    uint8_t* o = static_cast<uint8_t*>(out);
    // |y / s| is unbounded, so codes saturate.
    const QuantStep qs = quant_step(rho, static_scale);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = i * stride + rl;
      if (kFull || idx < nvec) st_stream(o + idx * 8, quant8<true>(t.t[i], qs));
    }
  }
}

// Dynamic scales (per-token, per-group) in two halves.  dyn_prepare takes the
// amaxes (per-group slices their group's, a DPP max over the group's 16 or 8
// lanes, so every lane of the wave must be active; a per-token row the row's
// m_row) and, with kBrackets, forms a row lane's codes from them alone (rho
// cancels in y / s; see dyn_step).  It needs no rho, so it runs while rho is
// computed, or before the row's barrier.  dyn_emit then takes rho, forms and
// stores the scales, settles the codes the brackets leave open and stores the
// codes.  Held brackets cost 5 VGPRs per vector until the codes are stored;
// with three or more vectors per lane that drops the kernels below 8 waves per
// SIMD, so there (kBrackets = false) each vector's bracket is formed just
// before it is settled, still without a reciprocal of s on the way.
template <int NV, bool kBrackets>
struct DynCodes {
  Bracket8 b[kBrackets ? NV : 1];
  float m[NV];
};

// Whether a lane holds the brackets of all its nv vectors (up to two).
constexpr bool dyn_brackets(int nv) { return nv <= 2; }

template <int NV, int kMode, int kGroup, bool kBrackets>
__device__ __forceinline__ void dyn_prepare(const RowT<NV>& t, float m_row,
                                            DynCodes<NV, kBrackets>& dc) {
  static_assert(kMode == RRA_Q_PER_TOKEN || (kMode == RRA_Q_PER_GROUP &&
                                             (kGroup == 64 || kGroup == 128)), "mode");
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float m = m_row;
    if constexpr (kMode == RRA_Q_PER_GROUP) {
      m = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(t.t[i][j]));
      m = kGroup == 128 ? max16(m) : max8(m);
    }
    dc.m[i] = m;
    if constexpr (kBrackets) {
      const DynStep ds = dyn_step(m);
      dc.b[i] = bracket8<false>(t.t[i], ds.f_dn, ds.f_up);
    }
  }
}

template <int NV, int kMode, int kGroup, bool kFull, bool kBrackets>
__device__ __forceinline__ void dyn_emit(const RowT<NV>& t, const DynCodes<NV, kBrackets>& dc,
                                         double rho, int nvec, int rl, int stride, uint8_t* out,
                                         float* scale_row) {
  constexpr int kLanesPerGroup = kGroup / 8;
  const double rho448 = rho_448(rho);
  // A scale that is not positive (0 for an all-zero slice, NaN where rho is
  // NaN) is stored as +0.
  float s = 0.0f;
  if constexpr (kMode == RRA_Q_PER_TOKEN) {
    s = dynamic_scale(dc.m[0], rho448);
    s = s > 0.0f ? s : 0.0f;
    if (rl == 0) scale_row[0] = s;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = i * stride + rl;
    if constexpr (kMode == RRA_Q_PER_GROUP) {
      s = dynamic_scale(dc.m[i], rho448);
      s = s > 0.0f ? s : 0.0f;
    }
    if (kFull || idx < nvec) {
      if (kMode == RRA_Q_PER_GROUP && (lane_id() & (kLanesPerGroup - 1)) == 0)
        scale_row[idx / kLanesPerGroup] = s;
      const DynStep ds = dyn_step(dc.m[i]);
      Bracket8 b;
      if constexpr (kBrackets)
        b = dc.b[i];
      else
        b = bracket8<false>(t.t[i], ds.f_dn, ds.f_up);
      st_stream(out + idx * 8, dyn_settle(t.t[i], b, ds, s, rho));
    }
  }
}

// Waves per workgroup of the residual-add norm: four (kWavesPerBlock / kW
// rows per workgroup), or kW where a row spans more than four waves (the
// decode-size launches, one vector per lane: 8 waves for H = 4096).
constexpr int norm_block_waves(int kW) { return kW > kWavesPerBlock ? kW : kWavesPerBlock; }

// Residual add + RMSNorm + quant.  Workgroup = norm_block_waves(kW) waves =
// norm_block_waves(kW) / kW rows; each row lane holds NV vectors of x,
// residual and weight.
// kMode NONE writes the norm to out (uint16_t, element type E) and +0 to its
// columns [H, H_pad) (the padding variant); the quantizing modes write FP8
// codes (uint8_t) from bf16 inputs and take H_pad = H.
template <int NV, int kW, bool kResidual, int kMode, int kGroup, bool kFull,
          typename E = ElemBf16>
__device__ __forceinline__ void add_rmsnorm_body(const uint16_t* __restrict__ x, int64_t x_stride,
                                                 uint16_t* __restrict__ residual,
                                                 int64_t res_stride,
                                                 const uint16_t* __restrict__ weight, float eps,
                                                 const float* __restrict__ static_scale,
                                                 void* __restrict__ out, int64_t out_stride,
                                                 float* __restrict__ scales, int64_t T, int H,
                                                 int H_pad, double inv_h) {
  constexpr int kBlockWaves = norm_block_waves(kW);
  constexpr int kRowsPerBlock = kBlockWaves / kW;
  constexpr int kStride = kW * kWave;
  __shared__ double lds_ss[kBlockWaves];
  __shared__ float lds_m[kBlockWaves];
  const int wave = wave_id();
  const int wave_in_row = wave % kW;
  const int rl = wave_in_row * kWave + lane_id();
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave / kW;
  // With one row per workgroup the grid has exactly T blocks.
  const bool active = kRowsPerBlock == 1 || row < T;
  // With kFull the row width is known here, and H (past the preloaded
  // arguments) is not needed.
  constexpr int kWidth = NV * kStride * 8;
  const int nvec = kFull ? kWidth / 8 : H >> 3;

  RowVecs<NV> a, r, w;
  load_row<NV, true, kFull>(a, x + row * x_stride, nvec, rl, kStride, active);
  if (kResidual)
    load_row<NV, true, kFull>(r, residual + row * res_stride, nvec, rl, kStride, active);
  load_row<NV, false, kFull>(w, weight, nvec, rl, kStride, true);
  args_ready(out, out_stride, scales);
  if constexpr (!kFull || kMode == RRA_Q_NONE) args_ready(H, H_pad, inv_h);
  const float sscale = kMode == RRA_Q_STATIC ? static_scale[0] : 0.0f;
  if constexpr (kMode == RRA_Q_STATIC) arg_ready(sscale);

  if (kResidual) {
    // z = E(x + residual): fp32 carries at least 2p + 2 significand bits for
    // p = 8 (bf16) and p = 11 (fp16), so rounding the fp32 sum of two such
    // values to E gives the same value as rounding their exact sum.
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        a.v[i][k] = E::pack(E::lo(a.v[i][k]) + E::lo(r.v[i][k]),
                            E::hi(a.v[i][k]) + E::hi(r.v[i][k]));
    }
    if (active) store_row<NV, kFull>(residual + row * res_stride, a, nvec, rl, kStride);
  }

  RowT<NV> t;
  double ss;
  float m;
  row_prepare<NV, E>(a, w, kMode == RRA_Q_PER_TOKEN, t, ss, m);
  // Per-group codes need only this lane's groups: where they are held
  // (kBr) they are formed before the row's barrier; per-token codes, and the
  // amaxes of rows too wide to hold codes for, follow it.
  constexpr bool kDyn = kMode == RRA_Q_PER_TOKEN || kMode == RRA_Q_PER_GROUP;
  constexpr bool kBr = dyn_brackets(NV);
  DynCodes<NV, kBr> dc;
  if constexpr (kMode == RRA_Q_PER_GROUP && kBr) dyn_prepare<NV, kMode, kGroup, kBr>(t, 0.0f, dc);
  row_reduce<kW>(ss, m, lds_ss, lds_m, (wave / kW) * kW, wave_in_row);
  if (!active) return;
  if constexpr (kMode == RRA_Q_PER_TOKEN || (kMode == RRA_Q_PER_GROUP && !kBr))
    dyn_prepare<NV, kMode, kGroup, kBr>(t, m, dc);
  constexpr double kH = static_cast<double>(kWidth);
  const double rho = row_rho(ss, kFull ? kH : static_cast<double>(H), kFull ? 1.0 / kH : inv_h,
                             eps);

  if constexpr (kMode == RRA_Q_NONE) {
    uint16_t* o = static_cast<uint16_t*>(out) + row * out_stride;
    rmsnorm_emit<NV, RRA_Q_NONE, kFull, E>(t, rho, nvec, rl, kStride, 0.0f, o);
    for (int idx = nvec + rl; idx < (H_pad >> 3); idx += kStride)
      st_stream(o + idx * 8, u32x4{0u, 0u, 0u, 0u});
  } else if constexpr (kMode == RRA_Q_STATIC) {
    rmsnorm_emit<NV, kMode, kFull>(t, rho, nvec, rl, kStride, sscale,
                                   static_cast<uint8_t*>(out) + row * out_stride);
  } else {
    static_assert(kDyn, "mode");
    float* scale_row =
        kMode == RRA_Q_PER_TOKEN ? scales + row : scales + row * ((kFull ? kWidth : H) / kGroup);
    dyn_emit<NV, kMode, kGroup, kFull, kBr>(t, dc, rho, nvec, rl, kStride,
                                       static_cast<uint8_t*>(out) + row * out_stride, scale_row);
  }
}

// Two entry kernels over the same body, so that profiles tell the quantizing
// op from the padding op.  The rows, the weight, T (which bounds the row loads
// when a workgroup holds several rows) and eps are the first 14 argument
// dwords, which a wave starts with in registers.
template <int NV, int kW, bool kResidual, int kMode, int kGroup, bool kFull>
__global__ void __launch_bounds__(norm_block_waves(kW) * kWave)
    add_rmsnorm_quant_kernel(const uint16_t* __restrict__ x, int64_t x_stride,
                             uint16_t* __restrict__ residual, int64_t res_stride,
                             const uint16_t* __restrict__ weight, int64_t T, float eps,
                             const float* __restrict__ static_scale,
                             uint8_t* __restrict__ out, int64_t out_stride,
                             float* __restrict__ scales, int H, double inv_h) {
  add_rmsnorm_body<NV, kW, kResidual, kMode, kGroup, kFull>(x, x_stride, residual, res_stride,
                                                            weight, eps, static_scale, out,
                                                            out_stride, scales, T, H, H, inv_h);
}

template <int NV, int kW, bool kResidual, bool kFull, typename E>
__global__ void __launch_bounds__(norm_block_waves(kW) * kWave)
    add_rmsnorm_pad_kernel(const uint16_t* __restrict__ x, int64_t x_stride,
                           uint16_t* __restrict__ residual, int64_t res_stride,
                           const uint16_t* __restrict__ weight, int64_t T, float eps,
                           uint16_t* __restrict__ out, int64_t out_stride, int H, int H_pad,
                           double inv_h) {
  add_rmsnorm_body<NV, kW, kResidual, RRA_Q_NONE, 0, kFull, E>(x, x_stride, residual,
                                                               res_stride, weight, eps, nullptr,
                                                               out, out_stride, nullptr, T, H,
                                                               H_pad, inv_h);
}

// MLA dual RMSNorm: one wave per token handles both of its rows, the q latent
// (NVQ vectors per lane) and the kv latent (NVKV), so both row reductions are
// wave-local DPP reductions with no LDS exchange and no barrier (four tokens
// per workgroup; waves past T leave at once).  Measured on MI355X at the
// DeepSeek-V3 shape, this beats spreading a token over 2 or 4 waves at every
// T from 512 to 16384: the rows are short, and a barrier per token costs more
// than the extra vectors per lane.  The two rows share their statistics work:
// one paired reduction leaves q's sum of squares in lane 31 and kv's in lane
// 63, and one vector pass takes both mean squares and both rsqrts (each lane
// with its half's width and epsilon).  The row count, both rows and both
// weights are the first 14 argument dwords, which a wave starts with in
// registers, so the loads need no argument fetch; the widths and their
// reciprocals come last and are used only when they are not the compile-time
// ones of kFull.
// Waves per SIMD the one-wave kernel is held to: with all its waves resident
// in one round up to 8192 tokens, a ninth VGPR block would leave a second
// round.  Rows of up to four vectors per lane fit 64 VGPRs without spilling,
// except with a per-token scale (12 bytes of spill at the DeepSeek-V3 shape),
// which is left to the compiler.
constexpr int dual_min_waves(int nvq, int nvkv, int mode) {
  return nvq + nvkv <= 4 && mode != RRA_Q_PER_TOKEN ? 8 : 1;
}

template <int NVQ, int NVKV, int kMode, int kGroup, bool kFull>
__global__ void __launch_bounds__(kBlock)
    __attribute__((amdgpu_waves_per_eu(dual_min_waves(NVQ, NVKV, kMode))))
    dual_rmsnorm_quant_kernel(int64_t T, const uint16_t* __restrict__ q, int64_t q_stride,
                              const uint16_t* __restrict__ kv, int64_t kv_stride,
                              const uint16_t* __restrict__ q_w,
                              const uint16_t* __restrict__ kv_w, float eps_q, float eps_kv,
                              void* __restrict__ q_out, int64_t q_out_stride,
                              float* __restrict__ q_scales, uint16_t* __restrict__ kv_out,
                              int64_t kv_out_stride, int Hq, int Hkv, double inv_hq,
                              double inv_hkv) {
  const int rl = lane_id();
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_id();
  if (row >= T) return;
  const int nq = kFull ? NVQ * kWave : Hq >> 3, nkv = kFull ? NVKV * kWave : Hkv >> 3;

  // Every load of the token is issued before either row is touched, kv's
  // first (in-order returns then let kv's products start while q's vectors
  // are still in flight).
  RowVecs<NVQ> zq, wq;
  RowVecs<NVKV> zkv, wkv;
  load_row<NVKV, true, kFull>(zkv, kv + row * kv_stride, nkv, rl, kWave, true);
  load_row<NVKV, false, kFull>(wkv, kv_w, nkv, rl, kWave, true);
  load_row<NVQ, true, kFull>(zq, q + row * q_stride, nq, rl, kWave, true);
  load_row<NVQ, false, kFull>(wq, q_w, nq, rl, kWave, true);
  args_ready(eps_q, eps_kv, q_out, q_out_stride, q_scales, kv_out, kv_out_stride);
  if constexpr (!kFull) args_ready(Hq, Hkv, inv_hq, inv_hkv);

  RowT<NVKV> tkv;
  RowT<NVQ> tq;
  double ss_kv, ss_q;
  float m_kv, m_q;
  row_prepare(zkv, wkv, false, tkv, ss_kv, m_kv);
  row_prepare(zq, wq, kMode == RRA_Q_PER_TOKEN, tq, ss_q, m_q);

  // Lanes 0-31 finish with q's row, lanes 32-63 with kv's.  ms = ss / H is
  // taken correctly rounded from the rounded reciprocal of H (div_rn).  An
  // infinite ss (an infinite value in the row) keeps ms = inf, hence rho = 0.
  const double ss = pair_sum_f64(ss_q, ss_kv);
  const bool kv_half = rl >= 32;
  double h, r;
  if constexpr (kFull) {
    h = kv_half ? NVKV * 512.0 : NVQ * 512.0;
    r = kv_half ? 1.0 / (NVKV * 512.0) : 1.0 / (NVQ * 512.0);
  } else {
    h = static_cast<double>(kv_half ? Hkv : Hq);
    r = kv_half ? inv_hkv : inv_hq;
  }
  const double rho = rsqrt_f64(div_rn(ss, h, r) + static_cast<double>(kv_half ? eps_kv : eps_q));
  const double rho_q = readlane_f64(rho, 31), rho_kv = readlane_f64(rho, 63);
  // q's amaxes (and for short rows its codes) need no rho, but they follow
  // kv's output: formed before it, alongside the statistics, their live
  // values cost the DeepSeek-V3 shape two waves per SIMD, or spills when held
  // to eight.
  constexpr bool kBr = dyn_brackets(NVQ + NVKV);
  DynCodes<NVQ, kBr> dc;

  rmsnorm_emit<NVKV, RRA_Q_NONE, kFull>(tkv, rho_kv, nkv, rl, kWave, 0.0f,
                                        kv_out + row * kv_out_stride);
  if constexpr (kMode != RRA_Q_NONE)
    dyn_prepare<NVQ, kMode, kGroup, kBr>(tq, kMode == RRA_Q_PER_TOKEN ? wave_max(m_q) : 0.0f,
                                         dc);
  if constexpr (kMode == RRA_Q_NONE) {
    rmsnorm_emit<NVQ, kMode, kFull>(tq, rho_q, nq, rl, kWave, 0.0f,
                                    static_cast<uint16_t*>(q_out) + row * q_out_stride);
  } else {
    float* scale_row =
        kMode == RRA_Q_PER_TOKEN ? q_scales + row : q_scales + row * (nq * 8 / kGroup);
    dyn_emit<NVQ, kMode, kGroup, kFull, kBr>(tq, dc, rho_q, nq, rl, kWave,
                                        static_cast<uint8_t*>(q_out) + row * q_out_stride,
                                        scale_row);
  }
}

// MLA dual RMSNorm at decode sizes: one token per workgroup of NVQ + NVKV
// waves, each wave one 512-column vector of one row (waves 0 .. NVQ - 1 the q
// latent, the rest kv), so a wave's dependent chain covers one vector instead
// of the whole token.  Each wave reduces its partials with DPP; one LDS
// exchange and one barrier give every wave its row's sum of squares (and, for
// per-token scales, the q amax), combined in a fixed order.
template <int NVQ, int NVKV, int kMode, int kGroup, bool kFull>
__global__ void __launch_bounds__((NVQ + NVKV) * kWave)
    dual_rmsnorm_split_kernel(int64_t T, const uint16_t* __restrict__ q, int64_t q_stride,
                              const uint16_t* __restrict__ kv, int64_t kv_stride,
                              const uint16_t* __restrict__ q_w,
                              const uint16_t* __restrict__ kv_w, float eps_q, float eps_kv,
                              void* __restrict__ q_out, int64_t q_out_stride,
                              float* __restrict__ q_scales, uint16_t* __restrict__ kv_out,
                              int64_t kv_out_stride, int Hq, int Hkv, double inv_hq,
                              double inv_hkv) {
  constexpr int kW = NVQ + NVKV;
  __shared__ double lds_ss[kW];
  __shared__ float lds_m[kW];
  const int wave = wave_id(), lane = lane_id();
  const int64_t row = blockIdx.x;  // the grid has exactly T workgroups
  const bool is_q = wave < NVQ;    // wave-uniform
  const int rl = (is_q ? wave : wave - NVQ) * kWave + lane;  // this lane's vector of its row
  const int nq = kFull ? NVQ * kWave : Hq >> 3, nkv = kFull ? NVKV * kWave : Hkv >> 3;
  const int nvec = is_q ? nq : nkv;

  RowVecs<1> z, w;
  load_row<1, true, kFull>(z, is_q ? q + row * q_stride : kv + row * kv_stride, nvec, rl, kWave,
                           true);
  load_row<1, false, kFull>(w, is_q ? q_w : kv_w, nvec, rl, kWave, true);
  args_ready(eps_q, eps_kv, q_out, q_out_stride, q_scales, kv_out, kv_out_stride);
  if constexpr (!kFull) args_ready(inv_hq, inv_hkv);
  RowT<1> t;
  double ss;
  float m;
  row_prepare(z, w, kMode == RRA_Q_PER_TOKEN, t, ss, m);
  // Per-group codes are formed before the barrier (the kv wave forms some it
  // never stores, which costs it nothing it waits for).
  DynCodes<1, true> dc;
  if constexpr (kMode == RRA_Q_PER_GROUP) dyn_prepare<1, kMode, kGroup, true>(t, 0.0f, dc);
  ss = wave_sum_f64(ss);
  if (kMode == RRA_Q_PER_TOKEN) m = wave_max(m);
  if (lane == 0) {
    lds_ss[wave] = ss;
    lds_m[wave] = m;
  }
  __syncthreads();
  const int first = is_q ? 0 : NVQ, count = is_q ? NVQ : NVKV;
  ss = lds_ss[first];
  m = lds_m[first];
  for (int j = 1; j < count; ++j) {
    ss += lds_ss[first + j];
    m = fmaxf(m, lds_m[first + j]);
  }
  if constexpr (kMode == RRA_Q_PER_TOKEN) dyn_prepare<1, kMode, kGroup, true>(t, m, dc);
  double h, r;
  if constexpr (kFull) {
    h = is_q ? NVQ * 512.0 : NVKV * 512.0;
    r = is_q ? 1.0 / (NVQ * 512.0) : 1.0 / (NVKV * 512.0);
  } else {
    h = static_cast<double>(is_q ? Hq : Hkv);
    r = is_q ? inv_hq : inv_hkv;
  }
  const double rho = row_rho(ss, h, r, is_q ? eps_q : eps_kv);
  if (!is_q) {
    rmsnorm_emit<1, RRA_Q_NONE, kFull>(t, rho, nvec, rl, kWave, 0.0f,
                                       kv_out + row * kv_out_stride);
    return;
  }
  if constexpr (kMode == RRA_Q_NONE) {
    rmsnorm_emit<1, kMode, kFull>(t, rho, nvec, rl, kWave, 0.0f,
                                  static_cast<uint16_t*>(q_out) + row * q_out_stride);
  } else {
    float* scale_row =
        kMode == RRA_Q_PER_TOKEN ? q_scales + row : q_scales + row * (nq * 8 / kGroup);
    dyn_emit<1, kMode, kGroup, kFull, true>(t, dc, rho, nvec, rl, kWave,
                                      static_cast<uint8_t*>(q_out) + row * q_out_stride,
                                      scale_row);
  }
}

// Waves per row for the residual-add norm: enough that each lane holds at
// most two vectors of a row up to H = 4096 (four up to 8192).
inline int norm_waves_per_row(int64_t H) { return H <= 1024 ? 1 : (H <= 2048 ? 2 : 4); }

// Arguments of one residual-add norm launch.
struct NormLaunch {
  dim3 grid;
  hipStream_t st;
  const uint16_t* x;
  int64_t xs;
  uint16_t* res;
  int64_t rs;
  const uint16_t* w;
  float eps;
  const float* sscale;
  void* out;
  int64_t os;
  float* scales;
  int64_t T;
  int H, H_pad;
};

template <int N, int W, bool kResidual, bool kFull, int kMode, int kGroup>
static void launch_norm_quant(const NormLaunch& a) {
  hipLaunchKernelGGL((add_rmsnorm_quant_kernel<N, W, kResidual, kMode, kGroup, kFull>), a.grid,
                     dim3(norm_block_waves(W) * kWave), 0, a.st, a.x, a.xs, a.res, a.rs, a.w,
                     a.T, a.eps, a.sscale, static_cast<uint8_t*>(a.out), a.os, a.scales, a.H,
                     1.0 / static_cast<double>(a.H));
}

template <int N, int W, bool kResidual, bool kFull, typename E>
static void launch_norm_pad(const NormLaunch& a) {
  hipLaunchKernelGGL((add_rmsnorm_pad_kernel<N, W, kResidual, kFull, E>), a.grid,
                     dim3(norm_block_waves(W) * kWave), 0, a.st,
                     a.x, a.xs, a.res, a.rs, a.w, a.T, a.eps, static_cast<uint16_t*>(a.out),
                     a.os, a.H, a.H_pad, 1.0 / static_cast<double>(a.H));
}

// One (vectors per lane, waves per row) case: mode NONE launches the padding
// kernel (out in the element type dtype, columns [H, H_pad) zeroed), the
// quantizing modes the quant kernel for that mode and group size (bf16 in).
template <int N, int W, bool kResidual, bool kFull>
static void launch_norm_mode(const NormLaunch& a, int mode, int group, int dtype) {
  switch (mode) {
    case RRA_Q_NONE:
      if (dtype == RRA_F16)
        launch_norm_pad<N, W, kResidual, kFull, ElemF16>(a);
      else
        launch_norm_pad<N, W, kResidual, kFull, ElemBf16>(a);
      break;
    case RRA_Q_STATIC: launch_norm_quant<N, W, kResidual, kFull, RRA_Q_STATIC, 0>(a); break;
    case RRA_Q_PER_TOKEN: launch_norm_quant<N, W, kResidual, kFull, RRA_Q_PER_TOKEN, 0>(a); break;
    default:
      if (group == 64)
        launch_norm_quant<N, W, kResidual, kFull, RRA_Q_PER_GROUP, 64>(a);
      else
        launch_norm_quant<N, W, kResidual, kFull, RRA_Q_PER_GROUP, 128>(a);
  }
}

// The row fills the N * 64 * W vectors of a lane's share exactly, or not.
template <int N, int W, bool kResidual>
static void launch_norm_case(const NormLaunch& a, int mode, int group, int dtype) {
  if (a.H == N * 8 * kWave * W)
    launch_norm_mode<N, W, kResidual, true>(a, mode, group, dtype);
  else
    launch_norm_mode<N, W, kResidual, false>(a, mode, group, dtype);
}

// Up to this many rows, the residual-add norm runs one vector per lane (a row
// over up to 16 waves, one row per workgroup), which shortens each wave's
// chain of loads, double-precision statistics, scale and codes.  Above it,
// rows of up to 4096 columns take four waves with two vectors per lane.
// Measured on MI355X at H = 4096 (profiler medians, cold): the split shape is
// 0.1-0.16 us faster at T = 32 ... 512 and 3% faster at 1024, equal at 2048,
// 1% slower at 4096.
constexpr int64_t kNormSplitMaxT = 1024;

// (vectors per lane, waves per row) for a launch of T rows of width H.
inline void norm_shape(int64_t T, int64_t H, int& nv, int& kw) {
  if (T <= kNormSplitMaxT) {
    const int64_t need = ceil_div(H, 8 * kWave);  // waves at one vector per lane
    kw = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
    nv = 1;
  } else {
    kw = norm_waves_per_row(H);
    nv = static_cast<int>(ceil_div(H, 8 * kWave * kw));
  }
}

template <bool kResidual>
static int launch_add_rmsnorm(int64_t T, int H, int H_pad, hipStream_t st, const uint16_t* x,
                              int64_t xs, uint16_t* res, int64_t rs, const uint16_t* w, float eps,
                              int mode, int group, const float* sscale, void* out, int64_t os,
                              float* scales, int dtype) {
  int nv, kw;
  norm_shape(T, H, nv, kw);
  const int rows_per_block = norm_block_waves(kw) / kw;
  RRA_REQUIRE(ceil_div(T, rows_per_block) <= 0x7FFFFFFF, RRA_ERR_UNSUPPORTED);  // grid.x
  const NormLaunch a{dim3(static_cast<unsigned>(ceil_div(T, rows_per_block))),
                     st, x, xs, res, rs, w, eps, sscale, out, os, scales, T, H, H_pad};
#define RRA_NORM_CASE(N, W)                                   \
  if (nv == N && kw == W) {                                   \
    launch_norm_case<N, W, kResidual>(a, mode, group, dtype); \
    return launch_status();                                   \
  }
  RRA_NORM_CASE(1, 1)
  RRA_NORM_CASE(2, 1)
  RRA_NORM_CASE(1, 2)
  RRA_NORM_CASE(2, 2)
  RRA_NORM_CASE(1, 4)
  RRA_NORM_CASE(2, 4)
  RRA_NORM_CASE(3, 4)
  RRA_NORM_CASE(4, 4)
  RRA_NORM_CASE(1, 8)
  RRA_NORM_CASE(1, 16)
#undef RRA_NORM_CASE
  return RRA_ERR_UNSUPPORTED;
}

// Arguments of one MLA dual-norm launch.
struct DualLaunch {
  dim3 grid;
  hipStream_t st;
  const uint16_t* q;
  int64_t qs;
  const uint16_t* qw;
  float eps_q;
  const uint16_t* kv;
  int64_t kvs;
  const uint16_t* kvw;
  float eps_kv;
  void* q_out;
  int64_t qos;
  float* q_scales;
  uint16_t* kv_out;
  int64_t kvos;
  int64_t T;
  int Hq, Hkv;
};

// Up to this many tokens the MLA norm runs one wave per 512-column vector
// (dual_rmsnorm_split_kernel); above, one wave per token.  Measured on MI355X
// at the DeepSeek-V3 shape (profiler medians, cold): the split is 0.5 us
// (13-15%) faster at T = 32 ... 512 and 5% at 1024, equal at 2048, and 8-12%
// slower from 4096 (four times the waves, a barrier per token).
constexpr int64_t kDualSplitMaxT = 1024;

template <int A, int B, bool kFull, int kMode, int kGroup>
static void launch_dual(const DualLaunch& a) {
  if (a.T <= kDualSplitMaxT) {
    hipLaunchKernelGGL((dual_rmsnorm_split_kernel<A, B, kMode, kGroup, kFull>),
                       dim3(static_cast<unsigned>(a.T)), dim3((A + B) * kWave), 0, a.st, a.T,
                       a.q, a.qs, a.kv, a.kvs, a.qw, a.kvw, a.eps_q, a.eps_kv, a.q_out, a.qos,
                       a.q_scales, a.kv_out, a.kvos, a.Hq, a.Hkv,
                       1.0 / static_cast<double>(a.Hq), 1.0 / static_cast<double>(a.Hkv));
    return;
  }
  hipLaunchKernelGGL((dual_rmsnorm_quant_kernel<A, B, kMode, kGroup, kFull>), a.grid,
                     dim3(kBlock), 0,
                     a.st, a.T, a.q, a.qs, a.kv, a.kvs, a.qw, a.kvw, a.eps_q, a.eps_kv,
                     a.q_out, a.qos, a.q_scales, a.kv_out, a.kvos, a.Hq, a.Hkv,
                     1.0 / static_cast<double>(a.Hq), 1.0 / static_cast<double>(a.Hkv));
}

template <int A, int B, bool kFull>
static void launch_dual_mode(const DualLaunch& a, int mode, int group) {
  switch (mode) {
    case RRA_Q_NONE: launch_dual<A, B, kFull, RRA_Q_NONE, 0>(a); break;
    case RRA_Q_PER_TOKEN: launch_dual<A, B, kFull, RRA_Q_PER_TOKEN, 0>(a); break;
    default:
      if (group == 64)
        launch_dual<A, B, kFull, RRA_Q_PER_GROUP, 64>(a);
      else
        launch_dual<A, B, kFull, RRA_Q_PER_GROUP, 128>(a);
  }
}

// Both rows fill their A (B) vectors per lane exactly, or not.
template <int A, int B>
static void launch_dual_case(const DualLaunch& a, int mode, int group) {
  if (a.Hq == A * 8 * kWave && a.Hkv == B * 8 * kWave)
    launch_dual_mode<A, B, true>(a, mode, group);
  else
    launch_dual_mode<A, B, false>(a, mode, group);
}

}  // namespace rra

using namespace rra;

extern "C" int fused_add_rmsnorm_quant(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                                       int64_t residual_stride, const uint16_t* weight,
                                       float eps, int quant_mode, int group_size,
                                       const float* static_scale, uint8_t* out,
                                       int64_t out_stride, float* scales, int64_t T, int64_t H,
                                       void* stream) {
  RRA_REQUIRE(T >= 0 && H > 0, RRA_ERR_SHAPE);
  // Tensors of T rows may be NULL when T == 0 (an empty torch tensor has no storage).
  const bool rows_ok = T == 0 || (x && out);
  RRA_REQUIRE(rows_ok && weight, RRA_ERR_NULL);
  RRA_REQUIRE(x_stride >= H && out_stride >= H, RRA_ERR_SHAPE);
  RRA_REQUIRE(!residual || residual_stride >= H, RRA_ERR_SHAPE);
  RRA_REQUIRE(H % 8 == 0 && H <= 8192, RRA_ERR_UNSUPPORTED);
  switch (quant_mode) {
    case RRA_Q_STATIC:
      RRA_REQUIRE(static_scale, RRA_ERR_NULL);
      RRA_REQUIRE(aligned(static_scale, 4), RRA_ERR_ALIGN);
      break;
    case RRA_Q_PER_TOKEN:
      RRA_REQUIRE(scales || T == 0, RRA_ERR_NULL);
      break;
    case RRA_Q_PER_GROUP:
      RRA_REQUIRE(group_ok(group_size), RRA_ERR_UNSUPPORTED);
      RRA_REQUIRE(H % group_size == 0, RRA_ERR_SHAPE);
      RRA_REQUIRE(scales || T == 0, RRA_ERR_NULL);
      break;
    default:
      return RRA_ERR_UNSUPPORTED;
  }
  RRA_REQUIRE(vec_ok(x, x_stride) && aligned(weight, 16), RRA_ERR_ALIGN);
  RRA_REQUIRE(!residual || vec_ok(residual, residual_stride), RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(out, 8) && out_stride % 8 == 0, RRA_ERR_ALIGN);
  RRA_REQUIRE(!scales || aligned(scales, 4), RRA_ERR_ALIGN);
  if (T == 0) return RRA_OK;

  const int g = quant_mode == RRA_Q_PER_GROUP ? group_size : 0;
  const int h = static_cast<int>(H);
  if (residual)
    return launch_add_rmsnorm<true>(T, h, h, as_stream(stream), x, x_stride, residual,
                                    residual_stride, weight, eps, quant_mode, g, static_scale,
                                    out, out_stride, scales, RRA_BF16);
  return launch_add_rmsnorm<false>(T, h, h, as_stream(stream), x, x_stride, nullptr, 0, weight,
                                   eps, quant_mode, g, static_scale, out, out_stride, scales,
                                   RRA_BF16);
}

extern "C" int fused_add_rmsnorm_pad(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                                     int64_t residual_stride, const uint16_t* weight, float eps,
                                     uint16_t* out, int64_t out_stride, int64_t T, int64_t H,
                                     int64_t H_pad, int dtype, void* stream) {
  RRA_REQUIRE(T >= 0 && H > 0 && H_pad >= H, RRA_ERR_SHAPE);
  const bool rows_ok = T == 0 || (x && out);
  RRA_REQUIRE(rows_ok && weight, RRA_ERR_NULL);
  RRA_REQUIRE(x_stride >= H && out_stride >= H_pad, RRA_ERR_SHAPE);
  RRA_REQUIRE(!residual || residual_stride >= H, RRA_ERR_SHAPE);
  RRA_REQUIRE(H % 8 == 0 && H_pad % 8 == 0 && H <= 8192 && H_pad <= (int64_t(1) << 30),
              RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(dtype == RRA_BF16 || dtype == RRA_F16, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(vec_ok(x, x_stride) && aligned(weight, 16) && vec_ok(out, out_stride),
              RRA_ERR_ALIGN);
  RRA_REQUIRE(!residual || vec_ok(residual, residual_stride), RRA_ERR_ALIGN);
  if (T == 0) return RRA_OK;
  const int h = static_cast<int>(H), hp = static_cast<int>(H_pad);
  if (residual)
    return launch_add_rmsnorm<true>(T, h, hp, as_stream(stream), x, x_stride, residual,
                                    residual_stride, weight, eps, RRA_Q_NONE, 0, nullptr, out,
                                    out_stride, nullptr, dtype);
  return launch_add_rmsnorm<false>(T, h, hp, as_stream(stream), x, x_stride, nullptr, 0, weight,
                                   eps, RRA_Q_NONE, 0, nullptr, out, out_stride, nullptr, dtype);
}

extern "C" int dual_rmsnorm_quant(const uint16_t* q, int64_t q_stride, const uint16_t* q_weight,
                                  float eps_q, const uint16_t* kv, int64_t kv_stride,
                                  const uint16_t* kv_weight, float eps_kv, int q_quant_mode,
                                  int group_size, void* q_out, int64_t q_out_stride,
                                  float* q_scales, uint16_t* kv_out, int64_t kv_out_stride,
                                  int64_t T, int64_t Hq, int64_t Hkv, void* stream) {
  RRA_REQUIRE(T >= 0 && Hq > 0 && Hkv > 0, RRA_ERR_SHAPE);
  const bool rows_ok = T == 0 || (q && kv && q_out && kv_out);
  RRA_REQUIRE(rows_ok && q_weight && kv_weight, RRA_ERR_NULL);
  RRA_REQUIRE(q_stride >= Hq && kv_stride >= Hkv && q_out_stride >= Hq && kv_out_stride >= Hkv,
              RRA_ERR_SHAPE);
  RRA_REQUIRE(Hq % 8 == 0 && Hkv % 8 == 0 && Hq <= 2048 && Hkv <= 1024, RRA_ERR_UNSUPPORTED);
  switch (q_quant_mode) {
    case RRA_Q_NONE:
      RRA_REQUIRE(vec_ok(q_out, q_out_stride), RRA_ERR_ALIGN);
      break;
    case RRA_Q_PER_TOKEN:
      RRA_REQUIRE(q_scales || T == 0, RRA_ERR_NULL);
      RRA_REQUIRE(aligned(q_out, 8) && q_out_stride % 8 == 0, RRA_ERR_ALIGN);
      break;
    case RRA_Q_PER_GROUP:
      RRA_REQUIRE(group_ok(group_size), RRA_ERR_UNSUPPORTED);
      RRA_REQUIRE(Hq % group_size == 0, RRA_ERR_SHAPE);
      RRA_REQUIRE(q_scales || T == 0, RRA_ERR_NULL);
      RRA_REQUIRE(aligned(q_out, 8) && q_out_stride % 8 == 0, RRA_ERR_ALIGN);
      break;
    default:
      return RRA_ERR_UNSUPPORTED;
  }
  RRA_REQUIRE(vec_ok(q, q_stride) && vec_ok(kv, kv_stride) && vec_ok(kv_out, kv_out_stride),
              RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(q_weight, 16) && aligned(kv_weight, 16), RRA_ERR_ALIGN);
  RRA_REQUIRE(!q_scales || aligned(q_scales, 4), RRA_ERR_ALIGN);
  if (T == 0) return RRA_OK;

  RRA_REQUIRE(ceil_div(T, kWavesPerBlock) <= 0x7FFFFFFF, RRA_ERR_UNSUPPORTED);  // grid.x
  // One wave per token: NVQ = ceil(Hq / 512) and NVKV = ceil(Hkv / 512) vectors per lane.
  const int nvq = static_cast<int>(ceil_div(Hq, 8 * kWave));
  const int nvkv = static_cast<int>(ceil_div(Hkv, 8 * kWave));
  const DualLaunch a{dim3(static_cast<unsigned>(ceil_div(T, kWavesPerBlock))),
                     as_stream(stream), q, q_stride, q_weight, eps_q, kv, kv_stride, kv_weight,
                     eps_kv, q_out, q_out_stride, q_scales, kv_out, kv_out_stride, T,
                     static_cast<int>(Hq), static_cast<int>(Hkv)};
#define RRA_DUAL_CASE(A, B)                                \
  if (nvq == A && nvkv == B) {                             \
    launch_dual_case<A, B>(a, q_quant_mode, group_size);   \
    return launch_status();                                \
  }
  RRA_DUAL_CASE(1, 1)
  RRA_DUAL_CASE(2, 1)
  RRA_DUAL_CASE(3, 1)
  RRA_DUAL_CASE(4, 1)
  RRA_DUAL_CASE(1, 2)
  RRA_DUAL_CASE(2, 2)
  RRA_DUAL_CASE(3, 2)
  RRA_DUAL_CASE(4, 2)
#undef RRA_DUAL_CASE
  return RRA_ERR_UNSUPPORTED;
}
