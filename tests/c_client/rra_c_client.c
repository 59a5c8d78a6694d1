/*
 * rra_c_client.c - a plain C11 caller of the rra.h C ABI, with no Python and no
 * torch.  It runs the four step entry points (fused_add_rmsnorm_quant,
 * silu_mul_quant, rope_kv_write, dual_rmsnorm_quant) and rope_cos_sin_cache on
 * inputs read from raw files, and writes their outputs back as raw files.  A
 * GPU test runs it beside the Python binding on the same inputs and requires
 * byte-identical outputs.  Test infrastructure: nothing in the library uses it.
 *
 * Usage: rra_c_client DIR
 *   DIR/shapes.txt holds, whitespace-separated:
 *     T_norm H_norm  T_silu I_silu  T_rope Hq Hkv D num_blocks block_size
 *     max_pos theta  T_mla Hq_mla Hkv_mla
 *   Inputs (little-endian, row-major, contiguous): norm_x, norm_res, norm_w,
 *   silu_in, rope_q, rope_k, rope_v, rope_pos, rope_slot, rope_kc, rope_vc,
 *   mla_q, mla_kv, mla_qw, mla_kvw (each NAME.bin).
 *   Outputs: out_norm_codes, out_norm_scales, out_norm_res, out_silu_codes,
 *   out_silu_scales, out_rope_cos_sin, out_rope_q, out_rope_kc, out_rope_vc,
 *   out_mla_q, out_mla_qs, out_mla_kv (each NAME.bin).
 * It also checks that a few invalid calls return the documented statuses
 * without launching.  Exit status 0 on success; on any failure it prints the
 * call and its status string and exits 1.
 *
 * Workloads (the fused patterns of the vLLM page "Fusion torch.compile
 * passes", one call each): the residual-add norm with per-token scales (eps
 * 1e-5), SiLU-and-Mul with group-128 scales, GPT-NeoX RoPE with the paged KV
 * write (q rotated in place), and the MLA dual norm with group-128 q codes and
 * bf16 kv (eps 1e-6 on both sides).
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
  long long Tn, Hn, Ts, Is, Tr, Hq, Hkv, D, nb, bs, max_pos, theta, Tm, Hqm, Hkvm;
  const int n = fscanf(f, "%lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld",
                       &Tn, &Hn, &Ts, &Is, &Tr, &Hq, &Hkv, &D, &nb, &bs, &max_pos, &theta, &Tm,
                       &Hqm, &Hkvm);
  fclose(f);
  if (n != 15) fail(path, "expected 15 integers");

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

  void* bufs[] = {x, res, w, codes, scales, sin_, scodes, sscales, q, k, v, pos, slot, kc, vc,
                  cos_sin, mq, mkv, mqw, mkvw, mqo, mqs, mkvo};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) hip_check(hipFree(bufs[i]), "hipFree");
  hip_check(hipStreamDestroy(stream), "hipStreamDestroy");
  printf("rra_c_client: four entry points and six status checks done\n");
  return 0;
}
