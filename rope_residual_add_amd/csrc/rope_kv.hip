// Rotary embedding + paged KV-cache write for gfx950, and the fp32 cos/sin
// table it reads.
//
// Operation: vLLM design page "Fusion torch.compile passes", section
// "RoPE + KV-Cache Update (fuse_rope_kvcache)": rotary embedding and the
// KV-cache scatter as one kernel, so k and v are read once and the rotated k
// goes straight into the cache.  The cache is paged as in the PagedAttention
// section of "Making vLLM fast: configuration, internals, and the places worth
// touching code": fixed-size blocks, and every token carries the slot
// (block * block_size + offset) it writes.
//
// Mapping: four waves per token.  The token's work is cut into 16-byte units
// (rotation pairs of q and k heads, plain vectors of v) spread over the 256
// lanes so that each lane issues at most a few loads before its stores; see
// rope_kv_write_kernel.
#include "rra_device.hpp"
#include "rra_host.hpp"

namespace rra {

// Rotate 8 pairs: (a, b) -> (a c - b s, b c + a s), rounded to bf16.
__device__ __forceinline__ void rotate8(u32x4& lo, u32x4& hi, const float c[8],
                                        const float s[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a0 = bf16_lo(lo[k]), a1 = bf16_hi(lo[k]);
    const float b0 = bf16_lo(hi[k]), b1 = bf16_hi(hi[k]);
    lo[k] = pack_bf16x2(a0 * c[2 * k] - b0 * s[2 * k], a1 * c[2 * k + 1] - b1 * s[2 * k + 1]);
    hi[k] = pack_bf16x2(b0 * c[2 * k] + a0 * s[2 * k], b1 * c[2 * k + 1] + a1 * s[2 * k + 1]);
  }
}

// Work of one token, in units: a q unit or a k unit is 8 rotation pairs of one
// head (a 16-byte vector from each half of the head), a v unit is one 16-byte
// vector of v copied into the cache.  Units are numbered q first, then k,
// then v; row lane rl of the token's kW waves takes units rl, rl + 64 kW, ...
// A head has D/16 units and 64 kW is a multiple of D/16, so every q or k unit
// of a lane starts at the same column of its head: the lane reads its 8 cos
// and 8 sin values once.  Each lane reads a q unit before writing it back, so
// q_out may alias q.  kU units per lane are loaded before any is stored.
constexpr int kRopeUnitsPerPass = 2;

template <int D, int kW>
__global__ void __launch_bounds__(kBlock)
    rope_kv_write_kernel(const int64_t* __restrict__ positions, const uint16_t* q,
                         int64_t q_stride, uint16_t* q_out, int64_t q_out_stride,
                         const uint16_t* __restrict__ k, int64_t k_stride,
                         const uint16_t* __restrict__ v, int64_t v_stride,
                         const float* __restrict__ cos_sin,
                         const int64_t* __restrict__ slot_mapping,
                         uint16_t* __restrict__ key_cache, uint16_t* __restrict__ value_cache,
                         int64_t T, int Hq, int Hkv) {
  constexpr int kHalf = D / 2;
  constexpr int kUnitsPerHead = kHalf / 8;
  constexpr int kLanes = kW * kWave;
  constexpr int kTokensPerBlock = kWavesPerBlock / kW;
  constexpr int kU = kRopeUnitsPerPass;
  static_assert(kLanes % kUnitsPerHead == 0, "a lane must keep one column");
  const int wave = wave_id();
  const int rl = (wave % kW) * kWave + lane_id();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + wave / kW;
  if (t >= T) return;  // no barrier in this kernel

  const int64_t pos = positions[t];
  const int64_t slot = slot_mapping[t];
  const int col = (rl % kUnitsPerHead) * 8;
  const int uq = Hq * kUnitsPerHead;
  const int uk = slot >= 0 ? Hkv * kUnitsPerHead : 0;  // padding tokens: q only
  const int uv = slot >= 0 ? Hkv * (D / 8) : 0;
  const int total = uq + uk + uv;

  float c[8], s[8];
  {
    const float* cs = cos_sin + pos * D + col;
    const f32x4 c0 = ld_f32x4(cs), c1 = ld_f32x4(cs + 4);
    const f32x4 s0 = ld_f32x4(cs + kHalf), s1 = ld_f32x4(cs + kHalf + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = c0[j];
      c[4 + j] = c1[j];
      s[j] = s0[j];
      s[4 + j] = s1[j];
    }
  }
  const uint16_t* qt = q + t * q_stride;
  uint16_t* qo = q_out + t * q_out_stride;
  const uint16_t* kt = k + t * k_stride;
  const uint16_t* vt = v + t * v_stride;
  // The cache is [num_blocks, block_size, Hkv, D] and contiguous, so slot
  // block * block_size + offset starts at element slot * Hkv * D.
  uint16_t* kc = key_cache + (slot >= 0 ? slot : 0) * Hkv * D;
  uint16_t* vc = value_cache + (slot >= 0 ? slot : 0) * Hkv * D;

  for (int u0 = 0; u0 < total; u0 += kU * kLanes) {
    u32x4 lo[kU], hi[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * kLanes + rl;
      if (u < uq) {
        const uint16_t* p = qt + (u / kUnitsPerHead) * D + col;
        lo[j] = ld_stream(p);
        hi[j] = ld_stream(p + kHalf);
      } else if (u < uq + uk) {
        const uint16_t* p = kt + ((u - uq) / kUnitsPerHead) * D + col;
        lo[j] = ld_stream(p);
        hi[j] = ld_stream(p + kHalf);
      } else if (u < total) {
        lo[j] = ld_stream(vt + (u - uq - uk) * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * kLanes + rl;
      if (u < uq) {
        rotate8(lo[j], hi[j], c, s);
        uint16_t* p = qo + (u / kUnitsPerHead) * D + col;
        st_stream(p, lo[j]);
        st_stream(p + kHalf, hi[j]);
      } else if (u < uq + uk) {
        rotate8(lo[j], hi[j], c, s);
        uint16_t* p = kc + ((u - uq) / kUnitsPerHead) * D + col;
        st_stream(p, lo[j]);
        st_stream(p + kHalf, hi[j]);
      } else if (u < total) {
        st_stream(vc + (u - uq - uk) * 8, lo[j]);
      }
    }
  }
}

// cos_sin[p, i] = cos(p * theta^(-2i/rot_dim)), cos_sin[p, rot_dim/2 + i] = sin(...)
__global__ void __launch_bounds__(kBlock)
    rope_cos_sin_kernel(float* __restrict__ out, int64_t max_pos, int rot_dim, double theta) {
  const int half = rot_dim / 2;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= max_pos * half) return;
  const int64_t p = idx / half;
  const int i = static_cast<int>(idx - p * half);
  const double inv_freq = pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(rot_dim));
  const double angle = static_cast<double>(p) * inv_freq;
  double sn, cn;
  sincos(angle, &sn, &cn);
  out[p * rot_dim + i] = static_cast<float>(cn);
  out[p * rot_dim + half + i] = static_cast<float>(sn);
}

// Elementwise fp32 -> e4m3fn with the quantizing kernels' conversion.
__global__ void __launch_bounds__(kBlock)
    e4m3fn_encode_kernel(const float* __restrict__ in, uint8_t* __restrict__ out, int64_t n) {
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * 4;
  if (i4 + 4 <= n) {
    const f32x4 x = ld_f32x4(in + i4);
    *reinterpret_cast<uint32_t*>(out + i4) = pack_e4m3x4(x[0], x[1], x[2], x[3]);
  } else {
    for (int64_t j = i4; j < n; ++j) out[j] = static_cast<uint8_t>(pack_e4m3x4(in[j], 0, 0, 0));
  }
}

}  // namespace rra

using namespace rra;

extern "C" int rope_kv_write(const int64_t* positions, const uint16_t* q, int64_t q_stride,
                             uint16_t* q_out, int64_t q_out_stride, const uint16_t* k,
                             int64_t k_stride, const uint16_t* v, int64_t v_stride,
                             const float* cos_sin, int64_t max_pos,
                             const int64_t* slot_mapping, uint16_t* key_cache,
                             uint16_t* value_cache, int64_t T, int Hq, int Hkv, int D,
                             int rot_dim, int block_size, int64_t num_blocks, int is_neox,
                             void* stream) {
  RRA_REQUIRE(T >= 0 && Hq > 0 && Hkv > 0 && D > 0 && rot_dim > 0 && block_size > 0 &&
                  num_blocks > 0 && max_pos > 0,
              RRA_ERR_SHAPE);
  // Tensors of T tokens may be NULL when T == 0 (an empty torch tensor has no storage).
  const bool tokens_ok = T == 0 || (positions && q && q_out && k && v && slot_mapping);
  RRA_REQUIRE(tokens_ok && cos_sin && key_cache && value_cache, RRA_ERR_NULL);
  RRA_REQUIRE(q_stride >= int64_t(Hq) * D && q_out_stride >= int64_t(Hq) * D &&
                  k_stride >= int64_t(Hkv) * D && v_stride >= int64_t(Hkv) * D,
              RRA_ERR_SHAPE);
  RRA_REQUIRE(D == 64 || D == 128 || D == 256, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(rot_dim == D && is_neox == 1, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(vec_ok(q, q_stride) && vec_ok(q_out, q_out_stride) && vec_ok(k, k_stride) &&
                  vec_ok(v, v_stride),
              RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(key_cache, 16) && aligned(value_cache, 16) && aligned(cos_sin, 16),
              RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(positions, 8) && aligned(slot_mapping, 8), RRA_ERR_ALIGN);
  if (T == 0) return RRA_OK;

  // Four waves (256 lanes) per token: each lane carries at most a few units.
  constexpr int kW = 4;
  const dim3 grid(static_cast<unsigned>(ceil_div(T, kWavesPerBlock / kW)));
  RRA_REQUIRE(ceil_div(T, kWavesPerBlock / kW) <= 0x7FFFFFFF, RRA_ERR_UNSUPPORTED);
  const hipStream_t st = as_stream(stream);
#define RRA_ROPE_CASE(DD)                                                                     \
  case DD:                                                                                    \
    hipLaunchKernelGGL((rope_kv_write_kernel<DD, kW>), grid, dim3(kBlock), 0, st, positions,  \
                       q, q_stride, q_out, q_out_stride, k, k_stride, v, v_stride, cos_sin,   \
                       slot_mapping, key_cache, value_cache, T, Hq, Hkv);                     \
    break;
  switch (D) {
    RRA_ROPE_CASE(64)
    RRA_ROPE_CASE(128)
    RRA_ROPE_CASE(256)
    default:
      return RRA_ERR_UNSUPPORTED;
  }
#undef RRA_ROPE_CASE
  return launch_status();
}

extern "C" int rope_cos_sin_cache(float* cos_sin, int64_t max_pos, int rot_dim, double theta,
                                  void* stream) {
  RRA_REQUIRE(max_pos >= 0 && rot_dim > 0 && rot_dim % 2 == 0, RRA_ERR_SHAPE);
  RRA_REQUIRE(cos_sin, RRA_ERR_NULL);
  RRA_REQUIRE(rot_dim >= 16 && rot_dim <= 1024 && theta > 0.0, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(aligned(cos_sin, 16), RRA_ERR_ALIGN);
  if (max_pos == 0) return RRA_OK;
  const int64_t blocks = ceil_div(max_pos * (rot_dim / 2), kBlock);
  RRA_REQUIRE(blocks <= 0x7FFFFFFF, RRA_ERR_UNSUPPORTED);
  hipLaunchKernelGGL(rope_cos_sin_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     as_stream(stream), cos_sin, max_pos, rot_dim, theta);
  return launch_status();
}

extern "C" int rra_e4m3fn_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
  RRA_REQUIRE(n >= 0, RRA_ERR_SHAPE);
  RRA_REQUIRE(in && out, RRA_ERR_NULL);
  RRA_REQUIRE(aligned(in, 16) && aligned(out, 4), RRA_ERR_ALIGN);
  if (n == 0) return RRA_OK;
  const int64_t blocks = ceil_div(ceil_div(n, 4), kBlock);
  RRA_REQUIRE(blocks <= 0x7FFFFFFF, RRA_ERR_UNSUPPORTED);
  hipLaunchKernelGGL(e4m3fn_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     as_stream(stream), in, out, n);
  return launch_status();
}

extern "C" int rra_abi_version(void) { return RRA_ABI_VERSION; }

extern "C" const char* rra_status_string(int status) {
  switch (status) {
    case RRA_OK:
      return "ok";
    case RRA_ERR_NULL:
      return "a required pointer is NULL";
    case RRA_ERR_SHAPE:
      return "negative or inconsistent sizes or strides";
    case RRA_ERR_ALIGN:
      return "pointer or stride breaks the 16-byte vector alignment rules";
    case RRA_ERR_UNSUPPORTED:
      return "unsupported mode, size or layout";
    case RRA_ERR_LAUNCH:
      return "kernel launch failed";
    default:
      return "unknown status";
  }
}
