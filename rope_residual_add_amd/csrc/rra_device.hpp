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

// ---- OCP e4m3fn -----------------------------------------------------------
// gfx950's v_cvt_pk_fp8_f32 converts to OCP e4m3fn with round-to-nearest-even.
// Inputs are clamped to the largest finite magnitude first (v_med3_f32), which
// gives the saturating behaviour for values that land just above 448.

__device__ __forceinline__ float clamp_e4m3(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// Four fp32 -> four e4m3fn bytes, element 0 in the lowest byte.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), w, true);
  return static_cast<uint32_t>(w);
}

// ---- wavefront reductions ---------------------------------------------------
// DPP moves within 16-lane rows: quad_perm [1,0,3,2] (0xB1), quad_perm
// [2,3,0,1] (0x4E), row_half_mirror (0x141), row_mirror (0x140); across rows:
// row_bcast:15 (0x142) and row_bcast:31 (0x143).  Every combining step adds
// the same two partials in both lanes of a pair, so all lanes of a segment end
// with bit-identical results (fp addition and max are commutative).

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}

// Max over each aligned group of 8 lanes, result in all 8.
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return v;
}

// Max over each 16-lane row, result in all 16.
__device__ __forceinline__ float max16(float v) {
  v = max8(v);
  return fmaxf(v, dpp<0x140>(v));
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

// Max over the whole wave (inputs >= 0); wave-uniform result.
__device__ __forceinline__ float wave_max(float v) {
  v = max16(v);
  v = fmaxf(v, dpp<0x142, 0xA>(v));
  v = fmaxf(v, dpp<0x143, 0xC>(v));
  return readlane63(v);
}

// Index of this lane's wave inside its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// 1/s for a quantization scale, with s = 0 (all-zero slice) mapped to 0 so
// that every code of the slice is +0.
__device__ __forceinline__ float inv_scale(float s) { return s > 0.0f ? 1.0f / s : 0.0f; }

}  // namespace rra
