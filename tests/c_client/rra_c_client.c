/*
 * rra_c_client.c - a plain C11 caller of the rra.h C ABI, with no Python and no
 * torch.  It runs the four step entry points (fused_add_rmsnorm_quant,
 * silu_mul_quant, rope_kv_write, dual_rmsnorm_quant), the three further ones
 * (qk_norm_rope_kv_write, fused_add_rmsnorm_pad, mla_rope_kv_write) and
 * rope_cos_sin_cache on inputs read from raw files, and writes their outputs
 * back as raw files.  A GPU test runs it beside the Python binding on the same
 * inputs and requires byte-identical outputs.  Test infrastructure: nothing in
 * the library uses it.
 *
 * Usage: rra_c_client DIR
 *   DIR/shapes.txt holds 36 whitespace-separated integers:
 *     T_norm H_norm  T_silu I_silu  T_rope Hq Hkv D num_blocks block_size
 *     max_pos theta  T_mla Hq_mla Hkv_mla
 *     T_qk Hq_qk Hkv_qk D_qk num_blocks_qk block_size_qk max_pos_qk theta_qk
 *     T_pad H H_pad
 *     T_mr Hq_mr nope rope_dim kv_lora num_blocks_mr block_size_mr max_pos_mr
 *     theta_mr is_neox_mr
 *   Inputs (little-endian, row-major, contiguous): norm_x, norm_res, norm_w,
 *   silu_in, rope_q, rope_k, rope_v, rope_pos, rope_slot, rope_kc, rope_vc,
 *   mla_q, mla_kv, mla_qw, mla_kvw, qk_qkv, qk_qw, qk_kw, qk_pos, qk_slot,
 *   qk_kc, qk_vc, pad_x, pad_res, pad_w, mr_q, mr_kpe, mr_kvc, mr_pos,
 *   mr_slot, mr_cache (each NAME.bin).
 *   Outputs: out_norm_codes, out_norm_scales, out_norm_res, out_silu_codes,
 *   out_silu_scales, out_rope_cos_sin, out_rope_q, out_rope_kc, out_rope_vc,
 *   out_mla_q, out_mla_qs, out_mla_kv, out_qk_qkv, out_qk_kc, out_qk_vc,
 *   out_pad, out_pad_res, out_mr_q, out_mr_cache (each NAME.bin).
 * It also checks that a few invalid calls return the documented statuses
 * without launching.  Exit status 0 on success; on any failure it prints the
 * call and its status string and exits 1.
 *
 * Workloads (the fused patterns of the vLLM page "Fusion torch.compile
 * passes", one call each): the residual-add norm with per-token scales (eps
 * 1e-5), SiLU-and-Mul with group-128 scales, GPT-NeoX RoPE with the paged KV
 * write (q rotated in place), the MLA dual norm with group-128 q codes and
 * bf16 kv (eps 1e-6 on both sides), the QK norm + NeoX RoPE with the cache
 * write and k written back (eps 1e-6), the residual-add norm with zero padding
 * (bf16, eps 1e-5), and the MLA RoPE with the [kv_c | k_pe] cache write.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rra.h"

static const char* g_dir;

static void fail(const char* what, const char* detail) {
  fprintf(stderr, "rra_c_client: %s: %s\n", what, detail);
  exit(1);
}

static void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(what, hipGetErrorString(e));
}

static void rra_check(int rc, const char* what) {
  if (rc != RRA_OK) fail(what, rra_status_string(rc));
}

static void path_of(char* buf, size_t n, const char* name) {
  if (snprintf(buf, n, "%s/%s.bin", g_dir, name) >= (int)n) fail(name, "path too long");
}

/* Reads NAME.bin, which must hold exactly `bytes` bytes, into new device memory. */
static void* load(const char* name, size_t bytes) {
  char path[4096];
  path_of(path, sizeof path, name);
  FILE* f = fopen(path, "rb");
  if (!f) fail(path, "cannot open");
  void* host = malloc(bytes ? bytes : 1);
  if (!host) fail(path, "out of host memory");
  const size_t got = fread(host, 1, bytes, f);
  const int extra = fgetc(f);
  fclose(f);
  if (got != bytes || extra != EOF) fail(path, "size differs from the shapes");
  void* dev = NULL;
  hip_check(hipMalloc(&dev, bytes ? bytes : 1), "hipMalloc");
  hip_check(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
  free(host);
  return dev;
}

static void* alloc_dev(size_t bytes) {
  void* dev = NULL;
  hip_check(hipMalloc(&dev, bytes ? bytes : 1), "hipMalloc");
  return dev;
}

/* Writes `bytes` bytes of device memory to NAME.bin. */
static void save(const char* name, const void* dev, size_t bytes) {
  char path[4096];
  path_of(path, sizeof path, name);
  void* host = malloc(bytes ? bytes : 1);
  if (!host) fail(path, "out of host memory");
  hip_check(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
  FILE* f = fopen(path, "wb");
  if (!f) fail(path, "cannot create");
  if (fwrite(host, 1, bytes, f) != bytes) fail(path, "short write");
  if (fclose(f) != 0) fail(path, "close failed");
  free(host);
}

static void expect_status(int rc, int want, const char* what) {
  if (rc != want) {
    fprintf(stderr, "rra_c_client: %s returned %d (%s), expected %d (%s)\n", what, rc,
            rra_status_string(rc), want, rra_status_string(want));
    exit(1);
  }
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  g_dir = argv[1];
  if (rra_abi_version() != RRA_ABI_VERSION) fail("rra_abi_version", "library and header differ");

  char path[4096];
  path_of(path, sizeof path, "shapes");
  path[strlen(path) - 4] = '\0';
  strcat(path, ".txt");
  FILE* f = fopen(path, "r");
  if (!f) fail(path, "cannot open");
  long long sz[36];
  int n = 0;
  while (n < 36 && fscanf(f, "%lld", &sz[n]) == 1) ++n;
  fclose(f);
  if (n != 36) fail(path, "expected 36 integers");
  const long long Tn = sz[0], Hn = sz[1], Ts = sz[2], Is = sz[3];
  const long long Tr = sz[4], Hq = sz[5], Hkv = sz[6], D = sz[7], nb = sz[8], bs = sz[9];
  const long long max_pos = sz[10], theta = sz[11], Tm = sz[12], Hqm = sz[13], Hkvm = sz[14];
  const long long Tq = sz[15], Hqq = sz[16], Hkq = sz[17], Dq = sz[18], nbq = sz[19];
  const long long bsq = sz[20], mpq = sz[21], thq = sz[22];
  const long long Tp = sz[23], Hp = sz[24], Hpad = sz[25];
  const long long Tmr = sz[26], Hmr = sz[27], nope = sz[28], rdim = sz[29], lora = sz[30];
  const long long nbm = sz[31], bsm = sz[32], mpm = sz[33], thm = sz[34], neoxm = sz[35];

  hipStream_t stream;
  hip_check(hipStreamCreate(&stream), "hipStreamCreate");
  void* st = (void*)stream;
  const size_t u16 = sizeof(uint16_t), f32 = sizeof(float), i64 = sizeof(int64_t);

  /* Residual add + RMSNorm + per-token FP8 (section "RMSNorm + Quantization"). */
  const size_t nn = (size_t)(Tn * Hn);
  uint16_t* x = load("norm_x", nn * u16);
  uint16_t* res = load("norm_res", nn * u16);
  uint16_t* w = load("norm_w", (size_t)Hn * u16);
  uint8_t* codes = alloc_dev(nn);
  float* scales = alloc_dev((size_t)Tn * f32);
  rra_check(fused_add_rmsnorm_quant(x, Hn, res, Hn, w, 1e-5f, RRA_Q_PER_TOKEN, 0, NULL, codes,
                                    Hn, scales, Tn, Hn, st),
            "fused_add_rmsnorm_quant");

  /* SiLU-and-Mul + group-128 FP8 (section "SiLU+Mul + Quantization"). */
  uint16_t* sin_ = load("silu_in", (size_t)(Ts * 2 * Is) * u16);
  uint8_t* scodes = alloc_dev((size_t)(Ts * Is));
  float* sscales = alloc_dev((size_t)(Ts * (Is / 128)) * f32);
  rra_check(silu_mul_quant(sin_, 2 * Is, RRA_Q_PER_GROUP, 128, NULL, scodes, Is, sscales, Ts, Is,
                           st),
            "silu_mul_quant");

  /* RoPE + paged KV write (section "RoPE + KV-Cache Update"), q in place. */
  const size_t qn = (size_t)(Tr * Hq * D), kn = (size_t)(Tr * Hkv * D);
  const size_t cn = (size_t)(nb * bs * Hkv * D);
  uint16_t* q = load("rope_q", qn * u16);
  uint16_t* k = load("rope_k", kn * u16);
  uint16_t* v = load("rope_v", kn * u16);
  int64_t* pos = load("rope_pos", (size_t)Tr * i64);
  int64_t* slot = load("rope_slot", (size_t)Tr * i64);
  uint16_t* kc = load("rope_kc", cn * u16);
  uint16_t* vc = load("rope_vc", cn * u16);
  float* cos_sin = alloc_dev((size_t)(max_pos * D) * f32);
  rra_check(rope_cos_sin_cache(cos_sin, max_pos, (int)D, (double)theta, st),
            "rope_cos_sin_cache");
  rra_check(rope_kv_write(pos, q, Hq * D, q, Hq * D, k, Hkv * D, v, Hkv * D, cos_sin, max_pos,
                          slot, kc, vc, Tr, (int)Hq, (int)Hkv, (int)D, (int)D, (int)bs, nb, 1,
                          RRA_BF16, st),
            "rope_kv_write");

  /* MLA dual RMSNorm, q to group-128 FP8 (section "MLA Dual RMSNorm"). */
  uint16_t* mq = load("mla_q", (size_t)(Tm * Hqm) * u16);
  uint16_t* mkv = load("mla_kv", (size_t)(Tm * Hkvm) * u16);
  uint16_t* mqw = load("mla_qw", (size_t)Hqm * u16);
  uint16_t* mkvw = load("mla_kvw", (size_t)Hkvm * u16);
  uint8_t* mqo = alloc_dev((size_t)(Tm * Hqm));
  float* mqs = alloc_dev((size_t)(Tm * (Hqm / 128)) * f32);
  uint16_t* mkvo = alloc_dev((size_t)(Tm * Hkvm) * u16);
  rra_check(dual_rmsnorm_quant(mq, Hqm, mqw, 1e-6f, mkv, Hkvm, mkvw, 1e-6f, RRA_Q_PER_GROUP, 128,
                               mqo, Hqm, mqs, mkvo, Hkvm, Tm, Hqm, Hkvm, st),
            "dual_rmsnorm_quant");

  /* QK norm + RoPE + cache write, k written back (section "QK Norm + RoPE"). */
  const size_t qkw = (size_t)((Hqq + 2 * Hkq) * Dq), qkc = (size_t)(nbq * bsq * Hkq * Dq);
  uint16_t* qkv = load("qk_qkv", (size_t)Tq * qkw * u16);
  uint16_t* qkqw = load("qk_qw", (size_t)Dq * u16);
  uint16_t* qkkw = load("qk_kw", (size_t)Dq * u16);
  int64_t* qkpos = load("qk_pos", (size_t)Tq * i64);
  int64_t* qkslot = load("qk_slot", (size_t)Tq * i64);
  uint16_t* qkkc = load("qk_kc", qkc * u16);
  uint16_t* qkvc = load("qk_vc", qkc * u16);
  float* qkcs = alloc_dev((size_t)(mpq * Dq) * f32);
  rra_check(rope_cos_sin_cache(qkcs, mpq, (int)Dq, (double)thq, st), "rope_cos_sin_cache (qk)");
  rra_check(qk_norm_rope_kv_write(qkpos, qkv, (int64_t)qkw, qkqw, qkkw, 1e-6f, qkcs, mpq, qkslot,
                                  qkkc, qkvc, 1, Tq, (int)Hqq, (int)Hkq, (int)Dq, (int)Dq,
                                  (int)bsq, nbq, 1, st),
            "qk_norm_rope_kv_write");

  /* Residual add + RMSNorm + zero padding (section "RMSNorm + Padding"). */
  uint16_t* px = load("pad_x", (size_t)(Tp * Hp) * u16);
  uint16_t* pres = load("pad_res", (size_t)(Tp * Hp) * u16);
  uint16_t* pw = load("pad_w", (size_t)Hp * u16);
  uint16_t* pout = alloc_dev((size_t)(Tp * Hpad) * u16);
  rra_check(fused_add_rmsnorm_pad(px, Hp, pres, Hp, pw, 1e-5f, pout, Hpad, Tp, Hp, Hpad,
                                  RRA_BF16, st),
            "fused_add_rmsnorm_pad");

  /* MLA q_pe / k_pe RoPE + [kv_c | k_pe] cache write, q_pe in place in q. */
  const size_t mrw = (size_t)(Hmr * (nope + rdim)), mrc = (size_t)(nbm * bsm * (lora + rdim));
  uint16_t* mrq = load("mr_q", (size_t)Tmr * mrw * u16);
  uint16_t* mrk = load("mr_kpe", (size_t)(Tmr * rdim) * u16);
  uint16_t* mrkv = load("mr_kvc", (size_t)(Tmr * lora) * u16);
  int64_t* mrpos = load("mr_pos", (size_t)Tmr * i64);
  int64_t* mrslot = load("mr_slot", (size_t)Tmr * i64);
  uint16_t* mrcache = load("mr_cache", mrc * u16);
  float* mrcs = alloc_dev((size_t)(mpm * rdim) * f32);
  rra_check(rope_cos_sin_cache(mrcs, mpm, (int)rdim, (double)thm, st), "rope_cos_sin_cache (mla)");
  rra_check(mla_rope_kv_write(mrpos, mrq + nope, (int64_t)mrw, nope + rdim, mrk, rdim, mrkv, lora,
                              mrcs, mpm, mrslot, mrcache, Tmr, (int)Hmr, (int)lora, (int)rdim,
                              (int)bsm, nbm, (int)neoxm, st),
            "mla_rope_kv_write");

  hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");

  /* Argument errors are caught on the host and launch nothing. */
  expect_status(fused_add_rmsnorm_quant(NULL, Hn, res, Hn, w, 1e-5f, RRA_Q_PER_TOKEN, 0, NULL,
                                        codes, Hn, scales, Tn, Hn, st),
                RRA_ERR_NULL, "fused_add_rmsnorm_quant without x");
  expect_status(fused_add_rmsnorm_quant(x, Hn, res, Hn, w, 1e-5f, RRA_Q_PER_GROUP, 96, NULL,
                                        codes, Hn, scales, Tn, Hn, st),
                RRA_ERR_UNSUPPORTED, "fused_add_rmsnorm_quant with group 96");
  expect_status(silu_mul_quant(sin_, 2 * Is, RRA_Q_PER_GROUP, 128, NULL, scodes, Is, sscales, -1,
                               Is, st),
                RRA_ERR_SHAPE, "silu_mul_quant with T = -1");
  expect_status(rope_kv_write(pos, q, Hq * D, q, Hq * D, k, Hkv * D, v, Hkv * D, cos_sin, max_pos,
                              slot, kc, vc, Tr, (int)Hq, (int)Hkv, (int)D, (int)D, (int)bs, nb, 1,
                              7, st),
                RRA_ERR_UNSUPPORTED, "rope_kv_write with dtype 7");
  expect_status(dual_rmsnorm_quant(mq + 1, Hqm, mqw, 1e-6f, mkv, Hkvm, mkvw, 1e-6f,
                                   RRA_Q_PER_GROUP, 128, mqo, Hqm, mqs, mkvo, Hkvm, Tm, Hqm, Hkvm,
                                   st),
                RRA_ERR_ALIGN, "dual_rmsnorm_quant with a misaligned q");
  expect_status(fused_add_rmsnorm_quant(NULL, Hn, NULL, Hn, w, 1e-5f, RRA_Q_PER_TOKEN, 0, NULL,
                                        NULL, Hn, NULL, 0, Hn, st),
                RRA_OK, "fused_add_rmsnorm_quant with T = 0");

  save("out_norm_codes", codes, nn);
  save("out_norm_scales", scales, (size_t)Tn * f32);
  save("out_norm_res", res, nn * u16);
  save("out_silu_codes", scodes, (size_t)(Ts * Is));
  save("out_silu_scales", sscales, (size_t)(Ts * (Is / 128)) * f32);
  save("out_rope_cos_sin", cos_sin, (size_t)(max_pos * D) * f32);
  save("out_rope_q", q, qn * u16);
  save("out_rope_kc", kc, cn * u16);
  save("out_rope_vc", vc, cn * u16);
  save("out_mla_q", mqo, (size_t)(Tm * Hqm));
  save("out_mla_qs", mqs, (size_t)(Tm * (Hqm / 128)) * f32);
  save("out_mla_kv", mkvo, (size_t)(Tm * Hkvm) * u16);
  save("out_qk_qkv", qkv, (size_t)Tq * qkw * u16);
  save("out_qk_kc", qkkc, qkc * u16);
  save("out_qk_vc", qkvc, qkc * u16);
  save("out_pad", pout, (size_t)(Tp * Hpad) * u16);
  save("out_pad_res", pres, (size_t)(Tp * Hp) * u16);
  save("out_mr_q", mrq, (size_t)Tmr * mrw * u16);
  save("out_mr_cache", mrcache, mrc * u16);

  void* bufs[] = {x, res, w, codes, scales, sin_, scodes, sscales, q, k, v, pos, slot, kc, vc,
                  cos_sin, mq, mkv, mqw, mkvw, mqo, mqs, mkvo, qkv, qkqw, qkkw, qkpos, qkslot,
                  qkkc, qkvc, qkcs, px, pres, pw, pout, mrq, mrk, mrkv, mrpos, mrslot, mrcache,
                  mrcs};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) hip_check(hipFree(bufs[i]), "hipFree");
  hip_check(hipStreamDestroy(stream), "hipStreamDestroy");
  printf("rra_c_client: seven entry points and six status checks done\n");
  return 0;
}
