/*
 * CPU oracle for the fused residual-add/RMSNorm/SiLU/RoPE/quant path.
 *
 * TEST INFRASTRUCTURE ONLY.  This code is the plain, slow, obviously correct
 * definition that the HIP library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or constant with the HIP library under
 * rope_residual_add_amd/, and it includes no HIP or torch header.
 *
 * Arithmetic: every intermediate is an IEEE double; each output is rounded
 * exactly once (bf16 round-to-nearest-even, fp32 round-to-nearest-even for
 * scales, OCP e4m3fn round-to-nearest-even with saturation to +-448 for fp8
 * codes).  Build with -ffp-contract=off -fno-fast-math.  Rows are processed by
 * one thread each in a fixed order, so results do not depend on thread count.
 *
 * Sources of each definition are cited per function in rra_oracle.c.  The
 * pages the method comes from are:
 *   [FUSION]  vLLM design page "Fusion torch.compile passes"
 *   [TUNING]  blog "Making vLLM fast: configuration, internals, and the places
 *             worth touching code" (section on PagedAttention)
 *   [LEVELS]  blog "vLLM optimization levels explained: -O0 to -O3" (the
 *             fusion flag names only)
 *   [OFP8]    OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding
 * Where the pages leave a step open, the reading taken is stated at the
 * function.
 */
#ifndef RRA_ORACLE_H
#define RRA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Oracle status codes (the oracle's own; not the library's). */
#define ORC_OK 0
#define ORC_EARG (-1)      /* malformed arguments: shape, mode, group size */
#define ORC_ECONTRACT (-2) /* data contract violated: position or slot out of
                              range, duplicate slot, bad static scale */

/* Quantization modes understood by the oracle. */
#define ORC_Q_NONE 0      /* no quantization: bf16 output */
#define ORC_Q_STATIC 1    /* one given per-tensor scale */
#define ORC_Q_PER_TOKEN 2 /* scale = row amax / 448 */
#define ORC_Q_PER_GROUP 3 /* scale = amax of each contiguous group / 448 */

/* 16-bit element types of the RoPE + KV-cache path. */
#define ORC_DT_BF16 0
#define ORC_DT_F16 1 /* IEEE binary16 */

/* ---- codecs ------------------------------------------------------------ */
uint16_t orc_bf16_encode(double v);
double orc_bf16_decode(uint16_t h);
uint16_t orc_f16_encode(double v); /* round-to-nearest-even, overflow to inf */
double orc_f16_decode(uint16_t h);
uint8_t orc_e4m3fn_encode(double v);       /* table + binary search */
uint8_t orc_e4m3fn_encode_arith(double v); /* independent: frexp + rint */
double orc_e4m3fn_decode(uint8_t c);
float orc_fp32_round(double v);

void orc_bf16_encode_f32_array(const float* in, uint16_t* out, int64_t n);
void orc_e4m3fn_encode_f32_array(const float* in, uint8_t* out, int64_t n);
void orc_e4m3fn_decode_array(const uint8_t* in, double* out, int64_t n);
/* Number of fp32 bit patterns in [begin, end) on which the two e4m3fn
 * encoders disagree. */
int64_t orc_e4m3fn_cross_check(uint64_t begin, uint64_t end);

/* ---- threading (rows are split across OpenMP threads) ------------------- */
void orc_set_threads(int n);
int orc_get_threads(void);

/* ---- fused ops -------------------------------------------------------- */
/* residual may be NULL (plain RMSNorm + quant).  static_scale is used in
 * STATIC mode only.  scales: [T] for PER_TOKEN, [T, H/g] for PER_GROUP,
 * unused otherwise.  All strides are in elements. */
int orc_fused_add_rmsnorm_quant(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                                int64_t res_stride, const uint16_t* weight, float eps,
                                int quant_mode, int group_size, float static_scale,
                                uint8_t* out, int64_t out_stride, float* scales, int64_t T,
                                int64_t H);

int orc_silu_mul_quant(const uint16_t* in, int64_t in_stride, int quant_mode, int group_size,
                       float static_scale, uint8_t* out, int64_t out_stride, float* scales,
                       int64_t T, int64_t I);

int orc_rope_kv_write(const int64_t* positions, const uint16_t* q, int64_t q_stride,
                      uint16_t* q_out, int64_t q_out_stride, const uint16_t* k,
                      int64_t k_stride, const uint16_t* v, int64_t v_stride, double theta,
                      int64_t max_pos, const int64_t* slot_mapping, uint16_t* key_cache,
                      uint16_t* value_cache, int64_t T, int Hq, int Hkv, int D, int rot_dim,
                      int block_size, int64_t num_blocks, int is_neox, int dtype);

/* q_quant_mode NONE writes bf16 into q_out (as uint16_t), otherwise e4m3fn
 * codes (as uint8_t). */
int orc_dual_rmsnorm_quant(const uint16_t* q, int64_t q_stride, const uint16_t* q_w,
                           float eps_q, const uint16_t* kv, int64_t kv_stride,
                           const uint16_t* kv_w, float eps_kv, int q_quant_mode,
                           int group_size, void* q_out, int64_t q_out_stride, float* q_scales,
                           uint16_t* kv_out, int64_t kv_out_stride, int64_t T, int64_t Hq,
                           int64_t Hkv);

/* ---- unfused compositions (what the fusions replace) -------------------- */
int orc_unfused_add_rmsnorm_quant(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                                  int64_t res_stride, const uint16_t* weight, float eps,
                                  int quant_mode, int group_size, float static_scale,
                                  uint8_t* out, int64_t out_stride, float* scales, int64_t T,
                                  int64_t H);

int orc_unfused_silu_mul_quant(const uint16_t* in, int64_t in_stride, int quant_mode,
                               int group_size, float static_scale, uint8_t* out,
                               int64_t out_stride, float* scales, int64_t T, int64_t I);

int orc_unfused_dual_rmsnorm_quant(const uint16_t* q, int64_t q_stride, const uint16_t* q_w,
                                   float eps_q, const uint16_t* kv, int64_t kv_stride,
                                   const uint16_t* kv_w, float eps_kv, int q_quant_mode,
                                   int group_size, void* q_out, int64_t q_out_stride,
                                   float* q_scales, uint16_t* kv_out, int64_t kv_out_stride,
                                   int64_t T, int64_t Hq, int64_t Hkv);

/* Unfused RoPE + KV-cache update: rotary embedding writes rotated q and k as
 * bf16 tensors (k_out: [T, Hkv, D] contiguous), then a separate cache-update
 * step copies k_out and v into the paged caches. */
int orc_unfused_rope_kv_write(const int64_t* positions, const uint16_t* q, int64_t q_stride,
                              uint16_t* q_out, int64_t q_out_stride, const uint16_t* k,
                              int64_t k_stride, uint16_t* k_out, const uint16_t* v,
                              int64_t v_stride, double theta, int64_t max_pos,
                              const int64_t* slot_mapping, uint16_t* key_cache,
                              uint16_t* value_cache, int64_t T, int Hq, int Hkv, int D,
                              int rot_dim, int block_size, int64_t num_blocks, int is_neox,
                              int dtype);

/* ---- next rows ---------------------------------------------------------- */
/* qkv: [T, (Hq + 2 Hkv) D], row stride qkv_stride; the q part (and with
 * write_k the k part) is overwritten.  slot_mapping NULL: no cache write. */
int orc_qk_norm_rope_kv_write(const int64_t* positions, uint16_t* qkv, int64_t qkv_stride,
                              const uint16_t* q_weight, const uint16_t* k_weight, float eps,
                              double theta, int64_t max_pos, const int64_t* slot_mapping,
                              uint16_t* key_cache, uint16_t* value_cache, int write_k,
                              int64_t T, int Hq, int Hkv, int D, int rot_dim, int block_size,
                              int64_t num_blocks, int is_neox);
int orc_unfused_qk_norm_rope_kv_write(const int64_t* positions, uint16_t* qkv,
                                      int64_t qkv_stride, const uint16_t* q_weight,
                                      const uint16_t* k_weight, float eps, double theta,
                                      int64_t max_pos, const int64_t* slot_mapping,
                                      uint16_t* key_cache, uint16_t* value_cache, int write_k,
                                      int64_t T, int Hq, int Hkv, int D, int rot_dim,
                                      int block_size, int64_t num_blocks, int is_neox);

/* out: [T, H_pad] bf16; columns H..H_pad are written as +0. */
int orc_fused_add_rmsnorm_pad(const uint16_t* x, int64_t x_stride, uint16_t* residual,
                              int64_t res_stride, const uint16_t* weight, float eps,
                              uint16_t* out, int64_t out_stride, int64_t T, int64_t H,
                              int64_t H_pad, int dtype);

/* q_pe: Hq heads of rope_dim at head stride q_head_stride inside rows of
 * q_stride, rotated in place; kv_cache: [num_blocks, block_size,
 * kv_lora + rope_dim]. */
int orc_mla_rope_kv_write(const int64_t* positions, uint16_t* q_pe, int64_t q_stride,
                          int64_t q_head_stride, const uint16_t* k_pe, int64_t k_pe_stride,
                          const uint16_t* kv_c, int64_t kv_c_stride, double theta,
                          int64_t max_pos, const int64_t* slot_mapping, uint16_t* kv_cache,
                          int64_t T, int Hq, int kv_lora, int rope_dim, int block_size,
                          int64_t num_blocks, int is_neox);

#ifdef __cplusplus
}
#endif
#endif
