/*
 * rra.h - C ABI of the fused residual-add / RMSNorm / SiLU / RoPE / FP8-quant
 * kernels for AMD Instinct MI355X (gfx950).
 *
 * The operations are the fused patterns described on the vLLM design page
 * "Fusion torch.compile passes"; each entry point below names the section that
 * defines it.  Every entry point is a plain C function taking raw device
 * pointers, element strides and sizes.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Types: bf16 tensors are passed as uint16_t bit patterns; FP8 outputs are
 *   OCP e4m3fn bytes (largest finite value 448, round-to-nearest-even,
 *   saturating); scales are fp32; token indices are int64.  Entry points with
 *   a `dtype` argument (enum rra_dtype) take bf16 or IEEE fp16 tensors, also
 *   as uint16_t bit patterns; the same alignment rules apply to both.
 * - Layout: 2-D tensors are row-major [T, width] with an arbitrary row stride
 *   (in elements) and contiguous rows, so column slices ("split" views of a
 *   wider projection) are valid inputs.
 * - Alignment: every bf16 pointer must be 16-byte aligned and every bf16 row
 *   stride a multiple of 8 elements; FP8 outputs 8-byte aligned with strides a
 *   multiple of 8; scale pointers 4-byte aligned.
 * - Ownership: the caller allocates and owns every buffer.  The library
 *   allocates nothing, keeps no mutable state, never synchronizes, and only
 *   enqueues work on `stream` (a hipStream_t; NULL = the null stream).  Calls
 *   are therefore reentrant and may be captured into a HIP graph.
 * - Sizes: a launch covers T with at most 2^31 - 1 workgroups (one row per
 *   workgroup for the residual-add norms, four tokens per workgroup for the
 *   MLA norm) and, where waves are numbered across the launch, fewer than 2^31
 *   waves (SiLU: one wave per 512 outputs of a row; the RoPE family: one wave
 *   per 64 rotation or copy units of a token); a larger T returns
 *   RRA_ERR_UNSUPPORTED.
 * - Errors: each function returns RRA_OK (0) or a negative rra_status.  All
 *   argument checks run on the host before anything is launched, so an error
 *   return means nothing was enqueued.  T == 0 returns RRA_OK without a launch;
 *   with T == 0, pointers to tensors that have T rows (or T tokens) may be NULL,
 *   while weights, static scales, tables and caches must still be given.
 *   RRA_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).
 * - Device-data contract (not checked: checking would need a host sync):
 *   a static scale is finite and > 0; positions lie in [0, max_pos);
 *   non-negative slots lie below num_blocks * block_size and are pairwise
 *   distinct; in the quantizing norms each product z * weight stays below the
 *   fp32 maximum (~3.4e38) in magnitude.  Breaking it gives unspecified
 *   outputs (no memory is written outside the documented output ranges except
 *   through an out-of-range slot or position, which is undefined behaviour).
 * - Non-finite inputs propagate as IEEE arithmetic does, with these readings
 *   of the dynamic scales: a NaN (or an infinity) in a normalized row makes
 *   rho NaN (or 0) and every value of the row NaN or +-0, so each dynamic
 *   scale of that row is 0 and its codes are +0; any slice whose scale comes
 *   out 0 gets +0 codes; NaN activations (SiLU) are left out of their group's
 *   amax and code as NaN; an infinite activation makes its group's scale
 *   infinite and the group's finite values code as +-0; a static scale
 *   saturates infinities to +-448 and keeps NaN.  The sign bit of a NaN
 *   result is unspecified.
 */
#ifndef RRA_H
#define RRA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 6: rope_kv_write (q, k) and mla_rope_kv_write (q_pe) refuse token strides
 * of 2^35 elements or more. */
#define RRA_ABI_VERSION 6

enum rra_status {
  RRA_OK = 0,
  RRA_ERR_NULL = -1,        /* a required pointer is NULL */
  RRA_ERR_SHAPE = -2,       /* negative or inconsistent sizes */
  RRA_ERR_ALIGN = -3,       /* pointer or stride breaks the alignment rules */
  RRA_ERR_UNSUPPORTED = -4, /* valid but not implemented (mode, size, layout) */
  RRA_ERR_LAUNCH = -5       /* the kernel launch failed */
};

enum rra_quant_mode {
  RRA_Q_NONE = 0,      /* no quantization: bf16 output */
  RRA_Q_STATIC = 1,    /* one per-tensor scale given by the caller */
  RRA_Q_PER_TOKEN = 2, /* scale[t] = amax over the row / 448 */
  RRA_Q_PER_GROUP = 3  /* scale[t, k] = amax over columns [k*g, (k+1)*g) / 448 */
};

/* 16-bit element types selectable through a `dtype` argument. */
enum rra_dtype {
  RRA_BF16 = 0, /* bfloat16 */
  RRA_F16 = 1   /* IEEE 754 binary16; results round to nearest even, overflow to inf */
};

/* Version of this ABI (RRA_ABI_VERSION of the built library). */
int rra_abi_version(void);

/* Static description of a status code; never NULL. */
const char* rra_status_string(int status);

/*
 * Residual add + RMSNorm + FP8 quant.
 * Section "RMSNorm + Quantization (fuse_norm_quant)": rms_norm(x) -> quant and
 * fused_add_rms_norm(x, residual) -> quant as one kernel, with the residual
 * updated in place and no full-precision intermediate in memory.
 *
 *   z      = bf16(x + residual)           (z = x when residual is NULL)
 *   residual <- z                         (in place, when residual != NULL)
 *   y      = z / sqrt(mean(z^2) + eps) * weight
 *   out    = e4m3fn(y / s)
 * with s = *static_scale (RRA_Q_STATIC), s = fp32(amax(|y| over the row)/448)
 * written to scales[t] (RRA_Q_PER_TOKEN), or one such scale per contiguous
 * group of group_size columns written to scales[t * (H / group_size) + k]
 * (RRA_Q_PER_GROUP).  A zero amax gives s = 0 and all-zero codes.
 *
 * x          [T, H] bf16, row stride x_stride.
 * residual   [T, H] bf16, row stride residual_stride, read and overwritten; or
 *            NULL for plain RMSNorm + quant.
 * weight     [H] bf16, contiguous.
 * quant_mode RRA_Q_STATIC, RRA_Q_PER_TOKEN or RRA_Q_PER_GROUP.
 * group_size 64 or 128 with RRA_Q_PER_GROUP (H % group_size == 0), else 0.
 * static_scale  device pointer to one fp32 scale (RRA_Q_STATIC only).
 * out        [T, H] e4m3fn, row stride out_stride.
 * scales     [T] or [T, H/group_size] fp32 contiguous; NULL for RRA_Q_STATIC.
 * Limits: H % 8 == 0 and 8 <= H <= 8192.
 */
int fused_add_rmsnorm_quant(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                            int64_t residual_stride, const uint16_t* weight, float eps,
                            int quant_mode, int group_size, const float* static_scale,
                            uint8_t* out, int64_t out_stride, float* scales, int64_t T,
                            int64_t H, void* stream);

/*
 * SiLU-and-Mul + FP8 quant.
 * Section "SiLU+Mul + Quantization (fuse_act_quant)": the gate-up activation
 * silu_and_mul followed by quantization without materializing the activation.
 *
 *   a[t, j] = silu(in[t, j]) * in[t, I + j],   silu(g) = g / (1 + exp(-g))
 *   out     = e4m3fn(a / s)
 * with s = *static_scale (RRA_Q_STATIC) or one scale per group of group_size
 * columns, s = fp32(amax/448), written to scales[t * (I / group_size) + k]
 * (RRA_Q_PER_GROUP).
 *
 * Activations whose magnitude exceeds the fp32 range (silu(g) * u beyond
 * ~3.4e38, which bf16 inputs allow) are finite values: a group holding one is
 * taken in double, and its scale is the fp32 rounding of amax/448 (infinite
 * where that exceeds fp32, so that the group's codes are +-0).
 *
 * in     [T, 2I] bf16 (gate half, then up half), row stride in_stride.
 * out    [T, I] e4m3fn, row stride out_stride.
 * scales [T, I/group_size] fp32 contiguous; NULL for RRA_Q_STATIC.
 * Limits: I % 8 == 0; group_size 64 or 128 dividing I.
 */
int silu_mul_quant(const uint16_t* in, int64_t in_stride, int quant_mode, int group_size,
                   const float* static_scale, uint8_t* out, int64_t out_stride,
                   float* scales, int64_t T, int64_t I, void* stream);

/*
 * Rotary cos/sin table used by rope_kv_write.
 * cos_sin[p, i] = cos(p * theta^(-2i/rot_dim)) and
 * cos_sin[p, rot_dim/2 + i] = sin(same angle), for p < max_pos and
 * i < rot_dim/2, evaluated in double precision and rounded to fp32.
 * cos_sin: [max_pos, rot_dim] fp32, contiguous, 16-byte aligned.
 * Limits: rot_dim even, 16 <= rot_dim <= 1024; theta > 0.
 */
int rope_cos_sin_cache(float* cos_sin, int64_t max_pos, int rot_dim, double theta,
                       void* stream);

/*
 * Rotary embedding + paged KV-cache write.
 * Section "RoPE + KV-Cache Update (fuse_rope_kvcache)": the rotary embedding
 * and the KV-cache scatter in one kernel, so k and v are read once and k is
 * never written back.  The cache is paged as in the PagedAttention section of
 * "Making vLLM fast: configuration, internals, and the places worth touching
 * code": fixed-size blocks addressed through a per-token slot.
 *
 * For token t at position p = positions[t], every q head and k head of D
 * values is rotated pairwise, (a, b) -> (a cos - b sin, b cos + a sin), with
 * pairs (i, i + rot_dim/2) (GPT-NeoX layout, is_neox = 1) or (2i, 2i + 1)
 * (GPT-J layout, is_neox = 0), and the angles of row p of cos_sin.  Rotated
 * q goes to q_out (q_out may equal q: in-place).  With
 * s = slot_mapping[t] >= 0, rotated k goes to key_cache[s / block_size,
 * s % block_size, :, :] and v, unchanged, to value_cache at the same place.
 * Tokens with s < 0 (padding) write no cache.  Nothing else is written.
 *
 * The rotation runs in fp32 and each rotated value is rounded once to the
 * element type dtype (RRA_BF16 or RRA_F16; the section's support matrix lists
 * the fusion for FP16 and BF16 on ROCm), which q, q_out, k, v and both caches
 * share.
 *
 * positions    [T] int64.
 * q            [T, Hq, D] dtype, token stride q_stride, heads contiguous.
 * q_out        [T, Hq, D] dtype, token stride q_out_stride (may alias q).
 * k, v         [T, Hkv, D] dtype, token strides k_stride, v_stride.
 * cos_sin      [max_pos, rot_dim] fp32 (see rope_cos_sin_cache).
 * slot_mapping [T] int64.
 * key_cache, value_cache [num_blocks, block_size, Hkv, D] dtype, contiguous.
 * Limits: D in {64, 128, 256}; rot_dim == D; is_neox 1 (GPT-NeoX pairs
 * (i, i + D/2)) or 0 (GPT-J pairs (2i, 2i + 1)); 1 <= Hq, Hkv <= 65536;
 * q_stride and k_stride below 2^35 elements; block_size >= 1; dtype RRA_BF16
 * or RRA_F16 (else RRA_ERR_UNSUPPORTED).
 */
int rope_kv_write(const int64_t* positions, const uint16_t* q, int64_t q_stride,
                  uint16_t* q_out, int64_t q_out_stride, const uint16_t* k, int64_t k_stride,
                  const uint16_t* v, int64_t v_stride, const float* cos_sin, int64_t max_pos,
                  const int64_t* slot_mapping, uint16_t* key_cache, uint16_t* value_cache,
                  int64_t T, int Hq, int Hkv, int D, int rot_dim, int block_size,
                  int64_t num_blocks, int is_neox, int dtype, void* stream);

/*
 * MLA dual RMSNorm (+ FP8 quant of the q latent).
 * Section "MLA Dual RMSNorm (fuse_mla_dual_rms_norm)": the paired q_a and kv_a
 * RMSNorms of an MLA layer in one launch, each with its own weight and
 * epsilon; in the FP8 variant only the q latent is quantized and kv stays
 * bf16.
 *
 *   q_out  = RMSNorm(q; q_weight, eps_q)   as bf16 (RRA_Q_NONE) or e4m3fn
 *            codes with per-token or per-group scales in q_scales
 *   kv_out = RMSNorm(kv; kv_weight, eps_kv) as bf16
 *
 * q        [T, Hq] bf16, row stride q_stride;  kv [T, Hkv], row stride kv_stride.
 * q_out    [T, Hq] bf16 (RRA_Q_NONE) or e4m3fn, row stride q_out_stride.
 * q_scales [T] or [T, Hq/group_size] fp32 contiguous; NULL for RRA_Q_NONE.
 * kv_out   [T, Hkv] bf16, row stride kv_out_stride.
 * Limits: q_quant_mode NONE, PER_TOKEN or PER_GROUP (64/128 dividing Hq);
 * Hq and Hkv multiples of 8 with Hq <= 2048 and Hkv <= 1024.
 */
int dual_rmsnorm_quant(const uint16_t* q, int64_t q_stride, const uint16_t* q_weight,
                       float eps_q, const uint16_t* kv, int64_t kv_stride,
                       const uint16_t* kv_weight, float eps_kv, int q_quant_mode,
                       int group_size, void* q_out, int64_t q_out_stride, float* q_scales,
                       uint16_t* kv_out, int64_t kv_out_stride, int64_t T, int64_t Hq,
                       int64_t Hkv, void* stream);

/*
 * QK norm + RoPE (+ paged KV-cache write).
 * Section "QK Norm + RoPE (enable_qk_norm_rope_fusion)": split the packed qkv
 * row, RMSNorm each q head and each k head over its D values, then the rotary
 * embedding, as one op on qkv.  The cache write continues it as section
 * "RoPE + KV-Cache Update" continues plain RoPE (the pages only name that
 * flag, fuse_qk_norm_rope_kvcache).
 *
 *   q_h <- rope(q_h / sqrt(mean(q_h^2) + eps) * q_weight)   for every q head
 *   k_h  = rope(k_h / sqrt(mean(k_h^2) + eps) * k_weight)   for every k head
 * computed in fp32 and rounded once to bf16, for heads of any finite
 * magnitude (a head whose fp32 mean square falls outside [2^-100, 2^100) is
 * normalized from values rescaled by 2^100 or 2^-100).  q is overwritten in
 * place in qkv.  With slot_mapping != NULL, token t with s = slot_mapping[t] >= 0
 * writes k_h and the unchanged v_h to key_cache / value_cache[s / block_size,
 * s % block_size, h, :] (layout and slot rules as rope_kv_write).  write_k = 1
 * also writes k_h back into qkv, for every token, with or without a slot.
 * With write_k = 0, qkv's k heads keep their input values, and the k result of
 * a padding token (slot < 0) goes nowhere.  Without a cache (slot_mapping ==
 * NULL) write_k must be 1: write_k = 0 there returns RRA_ERR_UNSUPPORTED,
 * since k's result would be dropped for every token.
 *
 * qkv          [T, (Hq + 2 Hkv) D] bf16: q heads, then k heads, then v heads;
 *              row stride qkv_stride; read and written.
 * q_weight, k_weight  [D] bf16 each.
 * cos_sin      [max_pos, D] fp32 (see rope_cos_sin_cache).
 * slot_mapping [T] int64 or NULL (no cache write; caches may then be NULL).
 * Limits: D in {64, 128, 256}; rot_dim == D; is_neox 1 (pairs (i, i + D/2))
 * or 0 (pairs (2i, 2i + 1)); 1 <= Hq, Hkv <= 65536.
 */
int qk_norm_rope_kv_write(const int64_t* positions, uint16_t* qkv, int64_t qkv_stride,
                          const uint16_t* q_weight, const uint16_t* k_weight, float eps,
                          const float* cos_sin, int64_t max_pos, const int64_t* slot_mapping,
                          uint16_t* key_cache, uint16_t* value_cache, int write_k, int64_t T,
                          int Hq, int Hkv, int D, int rot_dim, int block_size,
                          int64_t num_blocks, int is_neox, void* stream);

/*
 * Residual add + RMSNorm + padding.
 * Section "RMSNorm + Padding (fuse_act_padding)": residual add and RMSNorm,
 * then the hidden dimension padded to the width the next GEMM expects
 * (GPT-OSS: 2880), as one op.
 *
 *   z = E(x + residual); residual <- z (in place; z = x if residual NULL)
 *   out[t, 0:H]     = E(z / sqrt(mean(z^2) + eps) * weight)
 *   out[t, H:H_pad] = +0
 * where E() rounds to the element type dtype (RRA_BF16 or RRA_F16, which the
 * section's support matrix lists for this fusion on ROCm), nearest even.
 *
 * x [T, H], residual [T, H] (or NULL), out [T, H_pad] dtype with row strides;
 * weight [H] dtype.  H_pad is the caller's padded width.
 * Limits: H % 8 == 0, H <= 8192; H_pad % 8 == 0, H_pad >= H; dtype RRA_BF16
 * or RRA_F16 (else RRA_ERR_UNSUPPORTED).
 */
int fused_add_rmsnorm_pad(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                          int64_t residual_stride, const uint16_t* weight, float eps,
                          uint16_t* out, int64_t out_stride, int64_t T, int64_t H, int64_t H_pad,
                          int dtype, void* stream);

/*
 * MLA RoPE + cache concat.
 * The MLA split of section "MLA Dual RMSNorm" (kv_lora -> kv_c, k_pe) joined
 * with the cache write of section "RoPE + KV-Cache Update" (the pages only
 * name this flag, fuse_rope_kvcache_cat_mla): the rope parts of q and k are
 * rotated, and each token's cache row receives [kv_c | rotated k_pe].
 *
 *   q_pe[t, h, :] <- rope(q_pe[t, h, :])   for the Hq heads (in place)
 *   kv_cache[s / block_size, s % block_size, 0:kv_lora]       = kv_c[t]
 *   kv_cache[s / block_size, s % block_size, kv_lora:+rope_dim] = rope(k_pe[t])
 * for s = slot_mapping[t] >= 0 (tokens with s < 0 write no cache).
 *
 * q_pe      rope part of head 0 of token 0; head h of token t starts at
 *           q_pe + t * q_stride + h * q_head_stride (e.g. q + nope_dim in a
 *           [T, Hq, nope_dim + rope_dim] q); read and written.
 * k_pe      [T, rope_dim] bf16, row stride k_pe_stride (one head shared by all q heads).
 * kv_c      [T, kv_lora] bf16 (already normalized), row stride kv_c_stride.
 * cos_sin   [max_pos, rope_dim] fp32 (see rope_cos_sin_cache).
 * kv_cache  [num_blocks, block_size, kv_lora + rope_dim] bf16, contiguous.
 * Limits: rope_dim in {64, 128}; kv_lora % 8 == 0, kv_lora <= 2^24;
 * q_head_stride % 8 == 0; q_stride and q_head_stride below 2^35 elements;
 * 1 <= Hq <= 65536;
 * is_neox 0 (GPT-J pairs, as DeepSeek) or 1.
 */
int mla_rope_kv_write(const int64_t* positions, uint16_t* q_pe, int64_t q_stride,
                      int64_t q_head_stride, const uint16_t* k_pe, int64_t k_pe_stride,
                      const uint16_t* kv_c, int64_t kv_c_stride, const float* cos_sin,
                      int64_t max_pos, const int64_t* slot_mapping, uint16_t* kv_cache,
                      int64_t T, int Hq, int kv_lora, int rope_dim, int block_size,
                      int64_t num_blocks, int is_neox, void* stream);

/*
 * Diagnostic: out[i] = e4m3fn(in[i]) for n fp32 values, using the same device
 * conversion every quantizing kernel above uses (round-to-nearest-even,
 * saturating to +-448).  NaN inputs give unspecified codes.
 * in: [n] fp32, 16-byte aligned; out: [n] bytes, 4-byte aligned.
 */
int rra_e4m3fn_encode(const float* in, uint8_t* out, int64_t n, void* stream);

/*
 * Diagnostic: dst[0:nbytes) = src[0:nbytes), vectors_per_lane 16-byte vectors
 * per lane (1, 2, 4 or 8: all of a lane's loads, then its stores), loaded and
 * stored with the same streaming cache policy as the fused kernels'
 * activations.  It is the bandwidth yardstick the fused kernels are measured
 * against (a copy of the same number of bytes; the fastest vectors_per_lane
 * differs with the size).
 * src, dst: device pointers, 16-byte aligned; nbytes % 16 == 0 (else
 * RRA_ERR_ALIGN); the two ranges must not overlap (else RRA_ERR_SHAPE);
 * another vectors_per_lane gives RRA_ERR_UNSUPPORTED.  nbytes == 0 launches
 * nothing.
 */
int rra_stream_copy(const void* src, void* dst, int64_t nbytes, int vectors_per_lane,
                    void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RRA_H */
