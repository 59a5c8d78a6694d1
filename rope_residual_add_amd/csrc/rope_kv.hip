// Rotary embedding + paged KV-cache write for gfx950, its QK-norm and MLA
// variants, and the fp32 cos/sin table they read.
//
// Operations (vLLM design page "Fusion torch.compile passes"):
// - "RoPE + KV-Cache Update (fuse_rope_kvcache)": rotary embedding and the
//   KV-cache scatter as one kernel, so k and v are read once and the rotated k
//   goes straight into the cache.
// - "QK Norm + RoPE": per-head RMSNorm of q and k, then the rotary embedding,
//   on the packed qkv row; here optionally followed by the same cache write.
// - The MLA cache layout of section "MLA Dual RMSNorm" (kv_lora split into the
//   normalized kv_c and the rope part k_pe): rotate q_pe and k_pe and write
//   [kv_c | rotated k_pe] into the token's cache row.
// The cache is paged as in the PagedAttention section of "Making vLLM fast:
// configuration, internals, and the places worth touching code": fixed-size
// blocks, and every token carries the slot (block * block_size + offset) it
// writes.
//
// Mapping: W waves per token, as many as the token's units need at one unit
// per lane (at most 32; beyond that each lane takes kU > 1 units per pass),
// in ordinary four-wave workgroups: wave g of the launch is wave g % W of
// token g / W, so a token may straddle workgroups (the kernels have no
// barriers).  Each lane issues all its loads before its stores.  Measured at
// the Llama-3-8B attention shape (384 units): one unit per lane on six waves
// beats two units per lane on four waves by 3%, while workgroups of six waves
// (one token each) lose that gain, and fewer, fuller waves are slower still.
// A rotation unit depends on the pairing:
//   GPT-NeoX pairs (i, i + D/2): 8 pairs, the 16-byte vectors at columns 8c
//     and D/2 + 8c of a head;
//   GPT-J pairs (2i, 2i + 1): 4 pairs, the one 16-byte vector at columns 8c,
//     so that the 64 lanes of a load or store instruction cover whole, adjacent
//     cache lines of each head instead of every other 16 bytes of them;
// a copy unit moves v (or the MLA kv_c) without rotating it.  Unit c of a
// head reads entries kPairs*c .. kPairs*(c + 1) - 1 of the cos and of the sin
// half of a table row.  A head has D/16 (NeoX) or D/8 (GPT-J) rotation units,
// which divides the 64 lanes of a wave, so all rotation units of a lane share
// one c: the lane reads its cos and sin values once per token.
#include "rra_device.hpp"
#include "rra_host.hpp"

#include <type_traits>

namespace rra {

constexpr int kRopeMaxWaves = 32;                 // waves per token at most
constexpr int kRopeMaxHeads = 1 << 16;            // head counts accepted (unit indices fit int)
constexpr int64_t kRopeMaxStride8 = 0xFFFFFFFF;   // token strides / 8 passed as 32 bits
constexpr int kRopeMaxUnitsPerPass = 4;           // units a lane loads before storing

// Most units per lane and pass: 4 two-vector (NeoX) or 8 one-vector (GPT-J)
// rotation units.  A launch uses fewer only when one pass covers a token.
constexpr int rope_max_units(bool neox) {
  return neox ? kRopeMaxUnitsPerPass : 2 * kRopeMaxUnitsPerPass;
}

// Token t and row lane rl (0 .. W*64 - 1) of this lane, for W = tw.d waves per
// token and T tokens (launches stay below 2^31 waves, in ceil(T W / 4)
// workgroups).  The waves of one token span neighbouring workgroups (up to
// W/4 + 1 of them); xcd_block keeps neighbours on one XCD except across its
// 16-workgroup runs, so a token's table row, position and slot are fetched
// into one L2.
__device__ __forceinline__ void token_lane(const FastDiv& tw, uint32_t T, int64_t& t, int& rl) {
  const uint32_t blocks = (T * tw.d + kWavesPerBlock - 1) / kWavesPerBlock;
  const uint32_t gw = xcd_block(blocks) * kWavesPerBlock + static_cast<uint32_t>(wave_id());
  const uint32_t tt = fast_div(gw, tw);
  t = tt;
  rl = static_cast<int>(gw - tt * tw.d) * kWave + lane_id();
}

// Geometry of a rotation unit inside a head of D values (see the mapping
// above): kPerHead units per head, kPairs rotation pairs per unit, and for
// NeoX a second vector kHi columns after the first.
template <int D, bool kNeox>
struct RotUnit {
  static constexpr int kPerHead = kNeox ? D / 16 : D / 8;
  static constexpr int kPairs = kNeox ? 8 : 4;
  static constexpr int kHi = D / 2;  // NeoX only
  static __device__ __forceinline__ int lo(int c) { return c * 8; }
};

// The kPairs cos and sin values of rotation unit c at one position.
template <int D, bool kNeox>
__device__ __forceinline__ void unit_cos_sin(const float* row, int c, float cs[8], float sn[8]) {
  constexpr int P = RotUnit<D, kNeox>::kPairs;
  const float* p = row + c * P;
#pragma unroll
  for (int h = 0; h < P / 4; ++h) {
    const f32x4 c4 = ld_f32x4(p + 4 * h), s4 = ld_f32x4(p + D / 2 + 4 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cs[4 * h + j] = c4[j];
      sn[4 * h + j] = s4[j];
    }
  }
}

// Rotate the pairs of a unit, (a, b) -> (a cos - b sin, b cos + a sin).
// NeoX: 16 fp32 values x[0..8) (first vector) and x[8..16) (second), pair k
// = (x[k], x[8 + k]).  GPT-J: 8 values x[0..8), pair k = (x[2k], x[2k + 1]).
template <bool kNeox>
__device__ __forceinline__ void rotate_unit(float x[16], const float cs[8], const float sn[8]) {
  if (kNeox) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float a = x[k], b = x[8 + k];
      x[k] = a * cs[k] - b * sn[k];
      x[8 + k] = b * cs[k] + a * sn[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = x[2 * k], b = x[2 * k + 1];
      x[2 * k] = a * cs[k] - b * sn[k];
      x[2 * k + 1] = b * cs[k] + a * sn[k];
    }
  }
}

// One or two 16-byte vectors of 8 elements each (element type E) <-> fp32.
template <typename E = ElemBf16>
__device__ __forceinline__ void unpack8(u32x4 v, float x[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = E::lo(v[k]);
    x[2 * k + 1] = E::hi(v[k]);
  }
}

template <typename E = ElemBf16>
__device__ __forceinline__ u32x4 pack8(const float x[8]) {
  return u32x4{E::pack(x[0], x[1]), E::pack(x[2], x[3]), E::pack(x[4], x[5]),
               E::pack(x[6], x[7])};
}

template <typename E = ElemBf16>
__device__ __forceinline__ void unpack16(u32x4 lo, u32x4 hi, float x[16]) {
  unpack8<E>(lo, x);
  unpack8<E>(hi, x + 8);
}

template <typename E = ElemBf16>
__device__ __forceinline__ void pack16(const float x[16], u32x4& lo, u32x4& hi) {
  lo = pack8<E>(x);
  hi = pack8<E>(x + 8);
}

// Rotate a unit held as its packed vector(s); GPT-J units leave hi untouched.
template <bool kNeox, typename E = ElemBf16>
__device__ __forceinline__ void rotate_packed(u32x4& lo, u32x4& hi, const float cs[8],
                                              const float sn[8]) {
  float x[16];
  unpack8<E>(lo, x);
  if (kNeox) unpack8<E>(hi, x + 8);
  rotate_unit<kNeox>(x, cs, sn);
  lo = pack8<E>(x);
  if (kNeox) hi = pack8<E>(x + 8);
}

// Sum over aligned groups of n lanes (n = 4, 8, 16 or 32), result in every
// lane of the group.  Executed by all lanes of the wave.
template <int n>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(n == 4 || n == 8 || n == 16 || n == 32, "group size");
  v += dpp<0xB1>(v);  // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  if (n >= 8) v += dpp<0x141>(v);  // row_half_mirror
  if (n >= 16) v += dpp<0x140>(v);  // row_mirror
  if (n >= 32)  // lane ^ 16 within each 32-lane half (ds_swizzle bit mode, xor mask 16)
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (0x10 << 10) | 0x1F));
  return v;
}

// ---- RoPE + paged KV write ------------------------------------------------------
// Units of one token: q units, then k units, then v units, all of the rotation
// unit's geometry (kUnitsPerHead per head); q and k units are rotated, v units
// copied.  Row lane rl takes units rl, rl + 256, ...  A lane issues its loads
// before it needs the token's position or slot: the loads depend on t alone
// (a lane past the last unit re-reads the token's first q vector and discards
// it, and a padding token's k and v are read but not stored), so they leave
// before the table row and the slot arrive.  Each lane reads a q unit before
// writing it back, so q_out may alias q.  E is the element type of q, k, v and
// the caches (bf16 or fp16).
// The token's position and slot head the kernel's longest chains (the
// position, then its table row; the slot, then every cache store), so their
// loads leave first, ahead of the row loads, and the arguments they and the
// row loads need fill the 14 argument dwords a wave starts with in registers:
// the divider without its shift (fast_div_of), the head counts packed as
// (Hq - 1) | (Hkv - 1) << 16, and the q and k token strides in units of 8
// elements.  The remaining arguments are fetched while the row loads leave.
template <int D, bool kNeox, int kU, typename E>
__global__ void __launch_bounds__(kBlock)
    rope_kv_write_kernel(uint32_t tw_d, uint32_t tw_magic, uint32_t T, uint32_t heads,
                         const int64_t* __restrict__ positions,
                         const int64_t* __restrict__ slot_mapping, const uint16_t* q,
                         const uint16_t* __restrict__ k, uint32_t q_stride8, uint32_t k_stride8,
                         const float* __restrict__ cos_sin, const uint16_t* __restrict__ v,
                         int64_t v_stride, uint16_t* q_out, int64_t q_out_stride,
                         uint16_t* __restrict__ key_cache, uint16_t* __restrict__ value_cache) {
  const FastDiv tw = fast_div_of(tw_d, tw_magic);
  const int Hq = static_cast<int>(heads & 0xFFFFu) + 1, Hkv = static_cast<int>(heads >> 16) + 1;
  const int64_t q_stride = int64_t(q_stride8) * 8, k_stride = int64_t(k_stride8) * 8;
  using U = RotUnit<D, kNeox>;
  constexpr int kUnitsPerHead = U::kPerHead;
  static_assert(kWave % kUnitsPerHead == 0, "a lane must keep one column");
  int64_t t;
  int rl;
  token_lane(tw, T, t, rl);
  if (t >= T) return;  // whole waves; no barrier in this kernel
  const int64_t pos = positions[t];
  const int64_t slot = slot_mapping[t];
  // A compiler barrier (no instruction) keeps both loads above the row loads;
  // without it they are placed next to their first use.
  asm volatile("" ::: "memory");
  const int lanes = static_cast<int>(tw.d) * kWave;

  const int c = rl % kUnitsPerHead;
  const int lo_off = U::lo(c), hi_off = lo_off + U::kHi;
  const int uq = Hq * kUnitsPerHead;
  const int ukv = Hkv * kUnitsPerHead;
  const int total = uq + 2 * ukv;
  const uint16_t* qt = q + t * q_stride;
  const uint16_t* kt = k + t * k_stride;

  float cs[8], sn[8];
  for (int u0 = 0; u0 < total; u0 += kU * lanes) {
    u32x4 lo[kU], hi[kU];
    // q and k first: their addresses use only preloaded arguments.
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      if (u < uq + ukv) {
        const uint16_t* p = u < uq ? qt + (u / kUnitsPerHead) * D
                                   : kt + ((u - uq) / kUnitsPerHead) * D;
        lo[j] = ld_stream(p + lo_off);
        if (kNeox) hi[j] = ld_stream(p + hi_off);
      }
    }
    // The other arguments, fetched while the row loads leave, then the table
    // row and v.
    args_ready(cos_sin, v, v_stride, q_out, q_out_stride, key_cache, value_cache);
    if (u0 == 0) unit_cos_sin<D, kNeox>(cos_sin + pos * D, c, cs, sn);
    const uint16_t* vt = v + t * v_stride;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      if (u >= uq + ukv) {
        const uint16_t* p = u < total ? vt + ((u - uq - ukv) / kUnitsPerHead) * D : qt;
        lo[j] = ld_stream(p + lo_off);
        if (kNeox) hi[j] = ld_stream(p + hi_off);
      }
    }
    // The cache is [num_blocks, block_size, Hkv, D] and contiguous, so slot
    // block * block_size + offset starts at element slot * Hkv * D.
    const int64_t cache_row = (slot >= 0 ? slot : 0) * Hkv * D;
    uint16_t* qo = q_out + t * q_out_stride;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      uint16_t* p;
      if (u < uq) {
        rotate_packed<kNeox, E>(lo[j], hi[j], cs, sn);
        p = qo + (u / kUnitsPerHead) * D;
      } else if (u < total && slot >= 0) {  // padding tokens: q only
        const bool is_k = u < uq + ukv;
        if (is_k) rotate_packed<kNeox, E>(lo[j], hi[j], cs, sn);
        p = (is_k ? key_cache : value_cache) + cache_row +
            ((u - (is_k ? uq : uq + ukv)) / kUnitsPerHead) * D;
      } else {
        continue;
      }
      st_stream(p + lo_off, lo[j]);
      if (kNeox) st_stream(p + hi_off, hi[j]);
    }
    if (kU < rope_max_units(kNeox)) break;  // fewer than the most units per lane: one pass
  }
}

// ---- QK norm + RoPE (+ paged KV write) ------------------------------------------
// qkv row = [q: Hq heads | k: Hkv heads | v: Hkv heads] of D values.  Units as
// in rope_kv_write_kernel (q, then k, then v, all of the rotation unit's
// geometry); k units are present when k is written back or cached, v units
// when there is a cache.  A head's units sit on consecutive lanes of one wave,
// so its sum of squares is a DPP group sum; every lane runs the group sums
// (lanes without a q or k unit add zeros).  As in rope_kv_write_kernel the
// loads leave before the position, slot and weights are needed, the position
// and slot loads leave first, and the first 14 argument dwords hold what those
// loads need (the divider without its shift, the head counts packed as
// (Hq - 1) | (Hkv - 1) << 16, the position and slot pointers, the row, its
// stride, eps and write_k).  The norm and the rotation are applied in fp32 and
// rounded once to bf16.
template <int D, bool kNeox, int kU>
__global__ void __launch_bounds__(kBlock)
    qk_norm_rope_kv_kernel(uint32_t tw_d, uint32_t tw_magic, uint32_t T, uint32_t heads,
                           const int64_t* __restrict__ positions,
                           const int64_t* __restrict__ slot_mapping, uint16_t* qkv,
                           int64_t qkv_stride, float eps, int write_k,
                           const uint16_t* __restrict__ q_weight,
                           const uint16_t* __restrict__ k_weight,
                           const float* __restrict__ cos_sin, uint16_t* __restrict__ key_cache,
                           uint16_t* __restrict__ value_cache) {
  const FastDiv tw = fast_div_of(tw_d, tw_magic);
  const int Hq = static_cast<int>(heads & 0xFFFFu) + 1, Hkv = static_cast<int>(heads >> 16) + 1;
  using U = RotUnit<D, kNeox>;
  constexpr int kUnitsPerHead = U::kPerHead;
  constexpr int kVals = kNeox ? 16 : 8;  // values of a rotation unit
  static_assert(kWave % kUnitsPerHead == 0, "a lane must keep one column");
  int64_t t;
  int rl;
  token_lane(tw, T, t, rl);
  if (t >= T) return;  // whole waves; no barrier in this kernel
  const bool cached = slot_mapping != nullptr;
  const int64_t pos = positions[t];
  const int64_t slot = cached ? slot_mapping[t] : -1;
  // A compiler barrier (no instruction) keeps both loads above the row loads.
  asm volatile("" ::: "memory");
  const int lanes = static_cast<int>(tw.d) * kWave;

  const int c = rl % kUnitsPerHead;
  const int lo_off = U::lo(c), hi_off = lo_off + U::kHi;
  const int uq = Hq * kUnitsPerHead;
  const int uk = (cached || write_k) ? Hkv * kUnitsPerHead : 0;
  const int uv = cached ? Hkv * kUnitsPerHead : 0;
  const int total = uq + uk + uv;
  uint16_t* row = qkv + t * qkv_stride;
  uint16_t* kt = row + Hq * D;
  const uint16_t* vt = kt + Hkv * D;
  const float inv_d = 1.0f / static_cast<float>(D);

  float cs[8], sn[8];
  // This lane's q and k weight columns (the same in every head), packed.  With
  // one unit per lane only the weight of that unit's kind is loaded (kept in wq).
  u32x4 wq[2], wk[2];
  for (int u0 = 0; u0 < total; u0 += kU * lanes) {
    u32x4 lo[kU], hi[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      const uint16_t* p = u < uq          ? row + (u / kUnitsPerHead) * D
                          : u < uq + uk   ? kt + ((u - uq) / kUnitsPerHead) * D
                          : u < total     ? vt + ((u - uq - uk) / kUnitsPerHead) * D
                                          : row;
      lo[j] = ld_stream(p + lo_off);
      if (kNeox) hi[j] = ld_stream(p + hi_off);
    }
    // The remaining arguments, fetched under the row loads (the scheduling
    // barrier keeps the loads above the wait).
    __builtin_amdgcn_sched_barrier(0);
    args_ready(q_weight, k_weight, cos_sin, key_cache, value_cache);
    if (u0 == 0) {
      unit_cos_sin<D, kNeox>(cos_sin + pos * D, c, cs, sn);
      const uint16_t* w0 = (kU == 1 && rl >= uq) ? k_weight : q_weight;
      wq[0] = ld_cached(w0 + lo_off);
      if (kNeox) wq[1] = ld_cached(w0 + hi_off);
      if (kU > 1) {
        wk[0] = ld_cached(k_weight + lo_off);
        if (kNeox) wk[1] = ld_cached(k_weight + hi_off);
      }
    }
    const int64_t cache_row = (slot >= 0 ? slot : 0) * Hkv * D;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      const bool is_q = u < uq, is_k = !is_q && u < uq + uk;
      float x[16];
      unpack8(lo[j], x);
      if (kNeox) unpack8(hi[j], x + 8);
      float ss = 0.0f;
      if (is_q || is_k) {
#pragma unroll
        for (int e = 0; e < kVals; ++e) ss = fmaf(x[e], x[e], ss);
      }
      ss = group_sum<kUnitsPerHead>(ss);  // all lanes: groups are q-, k-, v-only or idle
      const float ms = ss * inv_d + eps;
      float rho = __builtin_amdgcn_rsqf(ms);
      // A head whose mean square (plus eps) lies outside [2^-100, 2^100) is
      // normalized from rescaled values, with the inverse scale folded into
      // x * rho:
      //  - below 2^-100 (eps ~ 0 and values below about 1e-15, whose squares
      //    lose bits or flush in fp32), from x * 2^100, with eps * 2^200
      //    (finite: eps is then below 2^-100 itself);
      //  - from 2^100 up, where the fp32 sum of squares may overflow (values
      //    above about 1e18 for D = 128, which would give rho = 0 and zero
      //    outputs), from x * 2^-100, with eps * 2^-200, which flushes to 0
      //    against a mean square of at least 2^-100 there.
      // The branch is wave-uniform, so every lane of each group takes part in
      // the second reduction.
      const bool rescale = (is_q || is_k) && !(ms >= 0x1p-100f && ms < 0x1p100f);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(rescale) != 0, 0)) {
        const float sc = ms < 1.0f ? 0x1p100f : 0x1p-100f;
        float ss2 = 0.0f;
        if (rescale) {
#pragma unroll
          for (int e = 0; e < kVals; ++e) {
            x[e] *= sc;
            ss2 = fmaf(x[e], x[e], ss2);
          }
        }
        ss2 = group_sum<kUnitsPerHead>(ss2);
        if (rescale) rho = __builtin_amdgcn_rsqf(ss2 * inv_d + (eps * sc) * sc);
      }
      if (is_q || is_k) {
        float w[16];
        const bool use_q = kU == 1 || is_q;
        unpack8(use_q ? wq[0] : wk[0], w);
        if (kNeox) unpack8(use_q ? wq[1] : wk[1], w + 8);
#pragma unroll
        for (int e = 0; e < kVals; ++e) x[e] = x[e] * rho * w[e];
        rotate_unit<kNeox>(x, cs, sn);
        const u32x4 a = pack8(x);
        const u32x4 b = kNeox ? pack8(x + 8) : a;
        if (is_q) {
          uint16_t* p = row + (u / kUnitsPerHead) * D;
          st_stream(p + lo_off, a);
          if (kNeox) st_stream(p + hi_off, b);
        } else {
          const int h = (u - uq) / kUnitsPerHead;
          if (slot >= 0) {
            uint16_t* p = key_cache + cache_row + h * D;
            st_stream(p + lo_off, a);
            if (kNeox) st_stream(p + hi_off, b);
          }
          if (write_k) {
            st_stream(kt + h * D + lo_off, a);
            if (kNeox) st_stream(kt + h * D + hi_off, b);
          }
        }
      } else if (u < total && slot >= 0) {  // v: a bit copy into the cache
        uint16_t* p = value_cache + cache_row + ((u - uq - uk) / kUnitsPerHead) * D;
        st_stream(p + lo_off, lo[j]);
        if (kNeox) st_stream(p + hi_off, hi[j]);
      }
    }
    if (kU < rope_max_units(kNeox)) break;  // fewer than the most units per lane: one pass
  }
}

// ---- MLA: q_pe / k_pe RoPE + [kv_c | k_pe] cache write ----------------------------
// Units of one token: the q_pe rotation units of Hq heads (head stride
// q_head_stride), then the k_pe rotation units, then kv_c vectors copied into
// the cache row (one vector each).  The cache is [num_blocks, block_size,
// kv_lora + R].  As in rope_kv_write_kernel the loads depend on t alone: they
// leave before the position and slot are needed (a padding token's k_pe and
// kv_c are read but not stored; a lane past the last unit re-reads the
// token's first kv_c vector), the position and slot loads leave first, and the
// first 14 argument dwords hold what those loads and q_pe's need (the divider
// without its shift, the position and slot pointers, q_pe and its token and
// head strides in units of 8 elements).
template <int R, bool kNeox, int kU>
__global__ void __launch_bounds__(kBlock)
    mla_rope_kv_kernel(uint32_t tw_d, uint32_t tw_magic, uint32_t T, int Hq, int kv_lora,
                       const int64_t* __restrict__ positions,
                       const int64_t* __restrict__ slot_mapping, uint16_t* q_pe,
                       uint32_t q_stride8, uint32_t q_head_stride8,
                       const uint16_t* __restrict__ k_pe, int64_t k_pe_stride,
                       const uint16_t* __restrict__ kv_c, int64_t kv_c_stride,
                       const float* __restrict__ cos_sin, uint16_t* __restrict__ kv_cache) {
  const FastDiv tw = fast_div_of(tw_d, tw_magic);
  const int64_t q_stride = int64_t(q_stride8) * 8, q_head_stride = int64_t(q_head_stride8) * 8;
  using U = RotUnit<R, kNeox>;
  constexpr int kUnitsPerHead = U::kPerHead;
  static_assert(kWave % kUnitsPerHead == 0, "a lane must keep one column");
  int64_t t;
  int rl;
  token_lane(tw, T, t, rl);
  if (t >= T) return;  // whole waves; no barrier in this kernel
  const int64_t pos = positions[t];
  const int64_t slot = slot_mapping[t];
  // A compiler barrier (no instruction) keeps both loads above the row loads.
  asm volatile("" ::: "memory");
  const int lanes = static_cast<int>(tw.d) * kWave;

  const int c = rl % kUnitsPerHead;
  const int lo_off = U::lo(c), hi_off = lo_off + U::kHi;
  const int uq = Hq * kUnitsPerHead;
  const int ur = uq + kUnitsPerHead;  // rotation units (q_pe and k_pe)
  const int total = ur + kv_lora / 8;
  uint16_t* qt = q_pe + t * q_stride;

  float cs[8], sn[8];
  for (int u0 = 0; u0 < total; u0 += kU * lanes) {
    u32x4 lo[kU], hi[kU];
    // q_pe first: its addresses use only preloaded arguments.
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      if (u < uq) {
        const uint16_t* p = qt + (u / kUnitsPerHead) * q_head_stride;
        lo[j] = ld_stream(p + lo_off);
        if (kNeox) hi[j] = ld_stream(p + hi_off);
      }
    }
    // The remaining arguments, fetched under the q_pe loads (the scheduling
    // barrier keeps those loads above the wait), then the table row, k_pe and
    // kv_c.
    __builtin_amdgcn_sched_barrier(0);
    args_ready(k_pe, k_pe_stride, kv_c, kv_c_stride, cos_sin, kv_cache);
    if (u0 == 0) unit_cos_sin<R, kNeox>(cos_sin + pos * R, c, cs, sn);
    const uint16_t* kt = k_pe + t * k_pe_stride;
    const uint16_t* ct = kv_c + t * kv_c_stride;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      if (u >= uq) {
        const uint16_t* pl;
        const uint16_t* ph;
        if (u < ur) {
          pl = kt + lo_off;
          ph = kt + hi_off;
        } else {
          pl = ct + (u < total ? (u - ur) * 8 : 0);
          ph = pl;  // a copy unit has one vector
        }
        lo[j] = ld_stream(pl);
        if (kNeox) hi[j] = ld_stream(ph);
      }
    }
    uint16_t* dst = kv_cache + (slot >= 0 ? slot : 0) * static_cast<int64_t>(kv_lora + R);
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int u = u0 + j * lanes + rl;
      if (u < uq) {
        rotate_packed<kNeox>(lo[j], hi[j], cs, sn);
        uint16_t* p = qt + (u / kUnitsPerHead) * q_head_stride;
        st_stream(p + lo_off, lo[j]);
        if (kNeox) st_stream(p + hi_off, hi[j]);
      } else if (u < total && slot >= 0) {  // padding tokens: q_pe only
        if (u < ur) {
          rotate_packed<kNeox>(lo[j], hi[j], cs, sn);
          st_stream(dst + kv_lora + lo_off, lo[j]);
          if (kNeox) st_stream(dst + kv_lora + hi_off, hi[j]);
        } else {
          st_stream(dst + (u - ur) * 8, lo[j]);
        }
      }
    }
    if (kU < rope_max_units(kNeox)) break;  // fewer than the most units per lane: one pass
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

// Rotation units per head under the two pairings (RotUnit::kPerHead).
inline int64_t rot_units_per_head(int D, int is_neox) { return is_neox ? D / 16 : D / 8; }

// Launch shape for tokens of `units` units each: ku units per lane per pass,
// the fewest that fit the units on kRopeMaxWaves waves (at most 4 two-vector
// NeoX or 8 one-vector GPT-J units; beyond that the lanes loop over passes),
// and the fewest waves per token that hold the units at ku per lane.
struct RopeLaunch {
  int ku;
  FastDiv tw;  // waves per token
};

inline RopeLaunch rope_launch(int64_t units, int is_neox) {
  const int64_t cap = rope_max_units(is_neox);
  int64_t ku = ceil_div(units, int64_t(kRopeMaxWaves) * kWave);
  ku = ku < 1 ? 1 : (ku > cap ? cap : ku);
  int64_t w = ceil_div(ceil_div(units, ku), kWave);
  w = w < 1 ? 1 : (w > kRopeMaxWaves ? kRopeMaxWaves : w);
  return RopeLaunch{static_cast<int>(ku), make_fast_div(static_cast<uint32_t>(w))};
}

// Workgroups for T tokens of shape.tw.d waves; 0 when the launch's wave count
// would reach 2^31 (the multiply-high division covers smaller ones).
inline int64_t rope_blocks(int64_t T, const RopeLaunch& shape) {
  if (T > (int64_t(1) << 31)) return 0;
  const int64_t waves = T * shape.tw.d;
  if (waves > 0x7FFFFFFF - kWavesPerBlock) return 0;
  return ceil_div(waves, kWavesPerBlock);
}

// Calls f(std::integral_constant<int, k>()) with k = ku clamped to [1, kMax],
// instantiating the launches for 1 .. kMax only.
template <int kMax, typename F>
static void with_units_per_pass(int ku, F&& f) {
  if constexpr (kMax > 1) {
    if (ku >= kMax) {
      f(std::integral_constant<int, kMax>());
      return;
    }
    with_units_per_pass<kMax - 1>(ku, f);
  } else {
    f(std::integral_constant<int, 1>());
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
                             int dtype, void* stream) {
  RRA_REQUIRE(T >= 0 && Hq > 0 && Hkv > 0 && D > 0 && rot_dim > 0 && block_size > 0 &&
                  num_blocks > 0 && max_pos > 0,
              RRA_ERR_SHAPE);
  RRA_REQUIRE(Hq <= kRopeMaxHeads && Hkv <= kRopeMaxHeads, RRA_ERR_UNSUPPORTED);
  // Tensors of T tokens may be NULL when T == 0 (an empty torch tensor has no storage).
  const bool tokens_ok = T == 0 || (positions && q && q_out && k && v && slot_mapping);
  RRA_REQUIRE(tokens_ok && cos_sin && key_cache && value_cache, RRA_ERR_NULL);
  RRA_REQUIRE(q_stride >= int64_t(Hq) * D && q_out_stride >= int64_t(Hq) * D &&
                  k_stride >= int64_t(Hkv) * D && v_stride >= int64_t(Hkv) * D,
              RRA_ERR_SHAPE);
  RRA_REQUIRE(D == 64 || D == 128 || D == 256, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(rot_dim == D && (is_neox == 0 || is_neox == 1), RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(dtype == RRA_BF16 || dtype == RRA_F16, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(vec_ok(q, q_stride) && vec_ok(q_out, q_out_stride) && vec_ok(k, k_stride) &&
                  vec_ok(v, v_stride),
              RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(key_cache, 16) && aligned(value_cache, 16) && aligned(cos_sin, 16),
              RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(positions, 8) && aligned(slot_mapping, 8), RRA_ERR_ALIGN);
  // The kernel takes the q and k token strides as 32-bit counts of 8 elements.
  RRA_REQUIRE(q_stride / 8 <= kRopeMaxStride8 && k_stride / 8 <= kRopeMaxStride8,
              RRA_ERR_UNSUPPORTED);
  if (T == 0) return RRA_OK;
  const hipStream_t st = as_stream(stream);
  const RopeLaunch shape =
      rope_launch(int64_t(Hq + 2 * Hkv) * rot_units_per_head(D, is_neox), is_neox);
  const int64_t blocks = rope_blocks(T, shape);
  RRA_REQUIRE(blocks > 0, RRA_ERR_UNSUPPORTED);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kBlock);
  const uint32_t T32 = static_cast<uint32_t>(T);  // below 2^31: rope_blocks refuses larger T
  const uint32_t heads = static_cast<uint32_t>(Hq - 1) | static_cast<uint32_t>(Hkv - 1) << 16;
  const uint32_t q_stride8 = static_cast<uint32_t>(q_stride / 8);
  const uint32_t k_stride8 = static_cast<uint32_t>(k_stride / 8);
#define RRA_ROPE_CASE(DD, NEOX, DT, EL)                                                        \
  if (D == DD && is_neox == NEOX && dtype == DT) {                                             \
    with_units_per_pass<rope_max_units(NEOX)>(shape.ku, [&](auto units) {                      \
      hipLaunchKernelGGL((rope_kv_write_kernel<DD, NEOX, decltype(units)::value, EL>), grid,   \
                         block, 0, st, shape.tw.d, shape.tw.magic, T32, heads, positions,      \
                         slot_mapping, q, k, q_stride8, k_stride8, cos_sin, v, v_stride,       \
                         q_out, q_out_stride, key_cache, value_cache);                         \
    });                                                                                        \
    return launch_status();                                                                    \
  }
  RRA_ROPE_CASE(64, 1, RRA_BF16, ElemBf16)
  RRA_ROPE_CASE(128, 1, RRA_BF16, ElemBf16)
  RRA_ROPE_CASE(256, 1, RRA_BF16, ElemBf16)
  RRA_ROPE_CASE(64, 0, RRA_BF16, ElemBf16)
  RRA_ROPE_CASE(128, 0, RRA_BF16, ElemBf16)
  RRA_ROPE_CASE(256, 0, RRA_BF16, ElemBf16)
  RRA_ROPE_CASE(64, 1, RRA_F16, ElemF16)
  RRA_ROPE_CASE(128, 1, RRA_F16, ElemF16)
  RRA_ROPE_CASE(256, 1, RRA_F16, ElemF16)
  RRA_ROPE_CASE(64, 0, RRA_F16, ElemF16)
  RRA_ROPE_CASE(128, 0, RRA_F16, ElemF16)
  RRA_ROPE_CASE(256, 0, RRA_F16, ElemF16)
#undef RRA_ROPE_CASE
  return RRA_ERR_UNSUPPORTED;
}

extern "C" int qk_norm_rope_kv_write(const int64_t* positions, uint16_t* qkv, int64_t qkv_stride,
                                     const uint16_t* q_weight, const uint16_t* k_weight,
                                     float eps, const float* cos_sin, int64_t max_pos,
                                     const int64_t* slot_mapping, uint16_t* key_cache,
                                     uint16_t* value_cache, int write_k, int64_t T, int Hq,
                                     int Hkv, int D, int rot_dim, int block_size,
                                     int64_t num_blocks, int is_neox, void* stream) {
  RRA_REQUIRE(T >= 0 && Hq > 0 && Hkv > 0 && D > 0 && rot_dim > 0 && max_pos > 0,
              RRA_ERR_SHAPE);
  RRA_REQUIRE(Hq <= kRopeMaxHeads && Hkv <= kRopeMaxHeads, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(qkv_stride >= int64_t(Hq + 2 * Hkv) * D, RRA_ERR_SHAPE);
  const bool tokens_ok = T == 0 || (positions && qkv);
  RRA_REQUIRE(tokens_ok && q_weight && k_weight && cos_sin, RRA_ERR_NULL);
  const bool with_cache = slot_mapping != nullptr;
  if (with_cache) {
    RRA_REQUIRE(key_cache && value_cache, RRA_ERR_NULL);
    RRA_REQUIRE(block_size > 0 && num_blocks > 0, RRA_ERR_SHAPE);
    RRA_REQUIRE(aligned(key_cache, 16) && aligned(value_cache, 16), RRA_ERR_ALIGN);
    RRA_REQUIRE(aligned(slot_mapping, 8), RRA_ERR_ALIGN);
  }
  // Without a cache, k's result has only qkv to go to.
  RRA_REQUIRE(with_cache || write_k, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(D == 64 || D == 128 || D == 256, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(rot_dim == D && (is_neox == 0 || is_neox == 1), RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(vec_ok(qkv, qkv_stride) && aligned(q_weight, 16) && aligned(k_weight, 16) &&
                  aligned(cos_sin, 16) && aligned(positions, 8),
              RRA_ERR_ALIGN);
  if (T == 0) return RRA_OK;
  const hipStream_t st = as_stream(stream);
  const RopeLaunch shape = rope_launch(
      int64_t(Hq + Hkv + (slot_mapping ? Hkv : 0)) * rot_units_per_head(D, is_neox), is_neox);
  const int64_t blocks = rope_blocks(T, shape);
  RRA_REQUIRE(blocks > 0, RRA_ERR_UNSUPPORTED);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kBlock);
  const uint32_t T32 = static_cast<uint32_t>(T);  // below 2^31: rope_blocks refuses larger T
  const uint32_t heads = static_cast<uint32_t>(Hq - 1) | static_cast<uint32_t>(Hkv - 1) << 16;
#define RRA_QKN_CASE(DD, NEOX)                                                                 \
  if (D == DD && is_neox == NEOX) {                                                            \
    with_units_per_pass<rope_max_units(NEOX)>(shape.ku, [&](auto units) {                      \
      hipLaunchKernelGGL((qk_norm_rope_kv_kernel<DD, NEOX, decltype(units)::value>), grid,     \
                         block, 0, st, shape.tw.d, shape.tw.magic, T32, heads, positions,      \
                         slot_mapping, qkv, qkv_stride, eps, write_k, q_weight, k_weight,      \
                         cos_sin, key_cache, value_cache);                                     \
    });                                                                                        \
    return launch_status();                                                                    \
  }
  RRA_QKN_CASE(64, 1)
  RRA_QKN_CASE(128, 1)
  RRA_QKN_CASE(256, 1)
  RRA_QKN_CASE(64, 0)
  RRA_QKN_CASE(128, 0)
  RRA_QKN_CASE(256, 0)
#undef RRA_QKN_CASE
  return RRA_ERR_UNSUPPORTED;
}

extern "C" int mla_rope_kv_write(const int64_t* positions, uint16_t* q_pe, int64_t q_stride,
                                 int64_t q_head_stride, const uint16_t* k_pe,
                                 int64_t k_pe_stride, const uint16_t* kv_c, int64_t kv_c_stride,
                                 const float* cos_sin, int64_t max_pos,
                                 const int64_t* slot_mapping, uint16_t* kv_cache, int64_t T,
                                 int Hq, int kv_lora, int rope_dim, int block_size,
                                 int64_t num_blocks, int is_neox, void* stream) {
  RRA_REQUIRE(T >= 0 && Hq > 0 && kv_lora > 0 && rope_dim > 0 && block_size > 0 &&
                  num_blocks > 0 && max_pos > 0,
              RRA_ERR_SHAPE);
  RRA_REQUIRE(Hq <= kRopeMaxHeads && kv_lora <= (1 << 24), RRA_ERR_UNSUPPORTED);
  // q_stride >= (Hq - 1) * q_head_stride + rope_dim, written so nothing overflows
  RRA_REQUIRE(q_head_stride >= rope_dim && q_stride >= rope_dim &&
                  (Hq == 1 || q_head_stride <= (q_stride - rope_dim) / (Hq - 1)) &&
                  k_pe_stride >= rope_dim && kv_c_stride >= kv_lora,
              RRA_ERR_SHAPE);
  const bool tokens_ok = T == 0 || (positions && q_pe && k_pe && kv_c && slot_mapping);
  RRA_REQUIRE(tokens_ok && cos_sin && kv_cache, RRA_ERR_NULL);
  RRA_REQUIRE(rope_dim == 64 || rope_dim == 128, RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(kv_lora % 8 == 0 && (is_neox == 0 || is_neox == 1), RRA_ERR_UNSUPPORTED);
  RRA_REQUIRE(vec_ok(q_pe, q_stride) && q_head_stride % 8 == 0 && vec_ok(k_pe, k_pe_stride) &&
                  vec_ok(kv_c, kv_c_stride),
              RRA_ERR_ALIGN);
  RRA_REQUIRE(aligned(kv_cache, 16) && aligned(cos_sin, 16) && aligned(positions, 8) &&
                  aligned(slot_mapping, 8),
              RRA_ERR_ALIGN);
  // The kernel takes the q_pe strides as 32-bit counts of 8 elements.
  RRA_REQUIRE(q_stride / 8 <= kRopeMaxStride8 && q_head_stride / 8 <= kRopeMaxStride8,
              RRA_ERR_UNSUPPORTED);
  if (T == 0) return RRA_OK;
  const hipStream_t st = as_stream(stream);
  const RopeLaunch shape = rope_launch(
      int64_t(Hq + 1) * rot_units_per_head(rope_dim, is_neox) + kv_lora / 8, is_neox);
  const int64_t blocks = rope_blocks(T, shape);
  RRA_REQUIRE(blocks > 0, RRA_ERR_UNSUPPORTED);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kBlock);
  const uint32_t T32 = static_cast<uint32_t>(T);  // below 2^31: rope_blocks refuses larger T
  const uint32_t q_stride8 = static_cast<uint32_t>(q_stride / 8);
  const uint32_t q_head_stride8 = static_cast<uint32_t>(q_head_stride / 8);
#define RRA_MLA_CASE(RR, NEOX)                                                                 \
  if (rope_dim == RR && is_neox == NEOX) {                                                     \
    with_units_per_pass<rope_max_units(NEOX)>(shape.ku, [&](auto units) {                      \
      hipLaunchKernelGGL((mla_rope_kv_kernel<RR, NEOX, decltype(units)::value>), grid, block,  \
                         0, st, shape.tw.d, shape.tw.magic, T32, Hq, kv_lora, positions,       \
                         slot_mapping, q_pe, q_stride8, q_head_stride8, k_pe, k_pe_stride,     \
                         kv_c, kv_c_stride, cos_sin, kv_cache);                                \
    });                                                                                        \
    return launch_status();                                                                    \
  }
  RRA_MLA_CASE(64, 0)
  RRA_MLA_CASE(64, 1)
  RRA_MLA_CASE(128, 0)
  RRA_MLA_CASE(128, 1)
#undef RRA_MLA_CASE
  return RRA_ERR_UNSUPPORTED;
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
