// Library-wide entry points: ABI version, status strings, and two diagnostic
// kernels that expose what the fused kernels are built from: the device FP8
// conversion, and the 16-byte streaming loads and stores as a plain copy that
// serves as the bandwidth yardstick for them.
#include "rra_device.hpp"
#include "rra_host.hpp"

namespace rra {

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

// V 16-byte vectors per lane, loaded and stored exactly as the fused kernels
// stream their activations: all V loads of a lane, then its V stores; each
// load or store instruction of a wave covers 1 KiB of contiguous memory.
template <int V>
__global__ void __launch_bounds__(kBlock)
    stream_copy_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n16) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kBlock * V + threadIdx.x;
  u32x4 r[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int64_t k = base + static_cast<int64_t>(i) * kBlock;
    if (k < n16) r[i] = ld_stream(src + k * 16);
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int64_t k = base + static_cast<int64_t>(i) * kBlock;
    if (k < n16) st_stream(dst + k * 16, r[i]);
  }
}

template <int V>
static int launch_copy(const void* src, void* dst, int64_t n16, hipStream_t st) {
  const int64_t blocks = ceil_div(n16, int64_t(kBlock) * V);
  RRA_REQUIRE(blocks <= 0x7FFFFFFF, RRA_ERR_UNSUPPORTED);
  hipLaunchKernelGGL(stream_copy_kernel<V>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     st, static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), n16);
  return launch_status();
}

}  // namespace rra

using namespace rra;

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

extern "C" int rra_stream_copy(const void* src, void* dst, int64_t nbytes, int vectors_per_lane,
                               void* stream) {
  RRA_REQUIRE(nbytes >= 0, RRA_ERR_SHAPE);
  RRA_REQUIRE(nbytes == 0 || (src && dst), RRA_ERR_NULL);
  RRA_REQUIRE(nbytes % 16 == 0 && aligned(src, 16) && aligned(dst, 16), RRA_ERR_ALIGN);
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  RRA_REQUIRE(nbytes == 0 || s + nbytes <= d || d + nbytes <= s, RRA_ERR_SHAPE);
  const int v = vectors_per_lane;
  RRA_REQUIRE(v == 1 || v == 2 || v == 4 || v == 8, RRA_ERR_UNSUPPORTED);
  if (nbytes == 0) return RRA_OK;
  const hipStream_t st = as_stream(stream);
  switch (v) {
    case 1: return launch_copy<1>(src, dst, nbytes / 16, st);
    case 2: return launch_copy<2>(src, dst, nbytes / 16, st);
    case 4: return launch_copy<4>(src, dst, nbytes / 16, st);
    default: return launch_copy<8>(src, dst, nbytes / 16, st);
  }
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
