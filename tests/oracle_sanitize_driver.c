/*
 * Drives every oracle entry point on small inputs in exactly sized heap
 * buffers, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitize.py): an out-of-bounds access or undefined
 * operation anywhere in the oracle aborts the run.  Covers every quant mode,
 * both RoPE pairings, bf16 and fp16 elements, strided rows, padding slots,
 * partial rotary width, and the contract errors (duplicate or out-of-range
 * slots, positions past the table).  Values come from a fixed LCG.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rra_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* [-1, 1) */
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_state >> 11) / 4503599627370496.0 - 1.0;
}

static uint16_t* bf16_array(int64_t n, double scale) {
  uint16_t* a = malloc((size_t)n * sizeof *a);
  for (int64_t i = 0; i < n; ++i) a[i] = orc_bf16_encode(scale * uniform());
  return a;
}

static uint16_t* f16_array(int64_t n, double scale) {
  uint16_t* a = malloc((size_t)n * sizeof *a);
  for (int64_t i = 0; i < n; ++i) a[i] = orc_f16_encode(scale * uniform());
  return a;
}

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if ((got == 0) != (want == 0)) {
    fprintf(stderr, "%s: status %d, expected %s\n", what, got, want ? "an error" : "success");
    ++failures;
  }
}

static void norm_cases(void) {
  const int64_t T = 5, H = 256, S = H + 24; /* strided rows */
  for (int mode = 1; mode <= 3; ++mode) {
    for (int g = 64; g <= 128; g += 64) {
      uint16_t* x = bf16_array(T * S, 2.0);
      uint16_t* r = bf16_array(T * S, 2.0);
      uint16_t* w = bf16_array(H, 1.0);
      uint8_t* out = malloc((size_t)(T * S));
      float* sc = malloc((size_t)(T * (H / 64)) * sizeof *sc);
      const int gs = mode == 3 ? g : 0;
      expect(orc_fused_add_rmsnorm_quant(x, S, r, S, w, 1e-5f, mode, gs, 0.05f, out, S, sc, T, H),
             0, "fused_add_rmsnorm_quant");
      expect(orc_fused_add_rmsnorm_quant(x, S, NULL, 0, w, 1e-5f, mode, gs, 0.05f, out, S, sc, T,
                                         H),
             0, "rmsnorm_quant without residual");
      expect(orc_unfused_add_rmsnorm_quant(x, S, r, S, w, 1e-5f, mode, gs, 0.05f, out, S, sc, T,
                                           H),
             0, "unfused_add_rmsnorm_quant");
      expect(orc_fused_add_rmsnorm_quant(x, S, r, S, w, 1e-5f, 3, 96, 0.05f, out, S, sc, T, H), 1,
             "group size 96");
      free(x), free(r), free(w), free(out), free(sc);
    }
  }
  for (int dt = 0; dt <= 1; ++dt) { /* padding op, bf16 and fp16 */
    const int64_t Hp = H + 40;
    uint16_t* x = dt ? f16_array(T * H, 2.0) : bf16_array(T * H, 2.0);
    uint16_t* r = dt ? f16_array(T * H, 2.0) : bf16_array(T * H, 2.0);
    uint16_t* w = dt ? f16_array(H, 1.0) : bf16_array(H, 1.0);
    uint16_t* out = malloc((size_t)(T * Hp) * sizeof *out);
    expect(orc_fused_add_rmsnorm_pad(x, H, r, H, w, 1e-5f, out, Hp, T, H, Hp, dt), 0,
           "fused_add_rmsnorm_pad");
    free(x), free(r), free(w), free(out);
  }
}

static void silu_cases(void) {
  const int64_t T = 3, I = 384;
  uint16_t* in = bf16_array(T * 2 * I, 4.0);
  uint8_t* out = malloc((size_t)(T * I));
  float* sc = malloc((size_t)(T * (I / 64)) * sizeof *sc);
  expect(orc_silu_mul_quant(in, 2 * I, 3, 128, 0.f, out, I, sc, T, I), 0, "silu group 128");
  expect(orc_silu_mul_quant(in, 2 * I, 3, 64, 0.f, out, I, sc, T, I), 0, "silu group 64");
  expect(orc_silu_mul_quant(in, 2 * I, 1, 0, 0.05f, out, I, sc, T, I), 0, "silu static");
  expect(orc_unfused_silu_mul_quant(in, 2 * I, 3, 128, 0.f, out, I, sc, T, I), 0,
         "unfused silu");
  free(in), free(out), free(sc);
}

static void dual_cases(void) {
  const int64_t T = 4, Hq = 384, Hkv = 128;
  for (int mode = 0; mode <= 3; mode += 1) {
    if (mode == 1) continue; /* static is not offered for the q latent */
    uint16_t* q = bf16_array(T * Hq, 2.0);
    uint16_t* kv = bf16_array(T * Hkv, 2.0);
    uint16_t* qw = bf16_array(Hq, 1.0);
    uint16_t* kvw = bf16_array(Hkv, 1.0);
    void* qo = malloc((size_t)(T * Hq) * 2);
    float* qs = malloc((size_t)(T * (Hq / 64)) * sizeof *qs);
    uint16_t* kvo = malloc((size_t)(T * Hkv) * sizeof *kvo);
    const int g = mode == 3 ? 128 : 0;
    expect(orc_dual_rmsnorm_quant(q, Hq, qw, 1e-6f, kv, Hkv, kvw, 1e-6f, mode, g, qo, Hq, qs, kvo,
                                  Hkv, T, Hq, Hkv),
           0, "dual_rmsnorm_quant");
    expect(orc_unfused_dual_rmsnorm_quant(q, Hq, qw, 1e-6f, kv, Hkv, kvw, 1e-6f, mode, g, qo, Hq,
                                          qs, kvo, Hkv, T, Hq, Hkv),
           0, "unfused dual");
    free(q), free(kv), free(qw), free(kvw), free(qo), free(qs), free(kvo);
  }
}

static void rope_cases(void) {
  const int64_t T = 6, max_pos = 32, nb = 4;
  const int Hq = 3, Hkv = 2, bs = 4;
  for (int D = 64; D <= 128; D += 64) {
    for (int neox = 0; neox <= 1; ++neox) {
      for (int dt = 0; dt <= 1; ++dt) {
        const int rot = neox ? D : D / 2; /* partial rotary for GPT-J */
        uint16_t* q = dt ? f16_array(T * Hq * D, 1.0) : bf16_array(T * Hq * D, 1.0);
        uint16_t* k = dt ? f16_array(T * Hkv * D, 1.0) : bf16_array(T * Hkv * D, 1.0);
        uint16_t* v = dt ? f16_array(T * Hkv * D, 1.0) : bf16_array(T * Hkv * D, 1.0);
        uint16_t* qo = malloc((size_t)(T * Hq * D) * sizeof *qo);
        uint16_t* ko = malloc((size_t)(T * Hkv * D) * sizeof *ko);
        const int64_t cache_n = nb * bs * Hkv * D;
        uint16_t* kc = calloc((size_t)cache_n, sizeof *kc);
        uint16_t* vc = calloc((size_t)cache_n, sizeof *vc);
        int64_t pos[6] = {0, 5, 31, 7, 2, 9};
        int64_t slots[6] = {3, -1, 15, 0, 8, -1};
        expect(orc_rope_kv_write(pos, q, Hq * D, qo, Hq * D, k, Hkv * D, v, Hkv * D, 1e4, max_pos,
                                 slots, kc, vc, T, Hq, Hkv, D, rot, bs, nb, neox, dt),
               0, "rope_kv_write");
        expect(orc_unfused_rope_kv_write(pos, q, Hq * D, qo, Hq * D, k, Hkv * D, ko, v, Hkv * D,
                                         1e4, max_pos, slots, kc, vc, T, Hq, Hkv, D, rot, bs, nb,
                                         neox, dt),
               0, "unfused rope_kv_write");
        int64_t dup[6] = {3, 4, 3, 0, 8, -1};
        expect(orc_rope_kv_write(pos, q, Hq * D, qo, Hq * D, k, Hkv * D, v, Hkv * D, 1e4, max_pos,
                                 dup, kc, vc, T, Hq, Hkv, D, rot, bs, nb, neox, dt),
               1, "duplicate slots");
        int64_t far[6] = {3, 4, 16, 0, 8, -1}; /* slot 16 = nb * bs */
        expect(orc_rope_kv_write(pos, q, Hq * D, qo, Hq * D, k, Hkv * D, v, Hkv * D, 1e4, max_pos,
                                 far, kc, vc, T, Hq, Hkv, D, rot, bs, nb, neox, dt),
               1, "slot past the cache");
        int64_t late[6] = {0, 5, 32, 7, 2, 9}; /* position max_pos */
        expect(orc_rope_kv_write(late, q, Hq * D, qo, Hq * D, k, Hkv * D, v, Hkv * D, 1e4,
                                 max_pos, slots, kc, vc, T, Hq, Hkv, D, rot, bs, nb, neox, dt),
               1, "position past the table");
        free(q), free(k), free(v), free(qo), free(ko), free(kc), free(vc);
      }
    }
  }
}

static void qk_cases(void) {
  const int64_t T = 5, max_pos = 16, nb = 3;
  const int Hq = 2, Hkv = 1, D = 128, bs = 2;
  for (int neox = 0; neox <= 1; ++neox) {
    for (int cached = 0; cached <= 1; ++cached) {
      const int64_t row = (Hq + 2 * Hkv) * D;
      uint16_t* qkv = bf16_array(T * row, 1.0);
      uint16_t* qw = bf16_array(D, 1.0);
      uint16_t* kw = bf16_array(D, 1.0);
      uint16_t* kc = calloc((size_t)(nb * bs * Hkv * D), sizeof *kc);
      uint16_t* vc = calloc((size_t)(nb * bs * Hkv * D), sizeof *vc);
      int64_t pos[5] = {0, 15, 3, 8, 1};
      int64_t slots[5] = {5, 0, -1, 2, 3};
      expect(orc_qk_norm_rope_kv_write(pos, qkv, row, qw, kw, 1e-6f, 1e6, max_pos,
                                       cached ? slots : NULL, kc, vc, 1, T, Hq, Hkv, D, D, bs, nb,
                                       neox),
             0, "qk_norm_rope_kv_write");
      expect(orc_unfused_qk_norm_rope_kv_write(pos, qkv, row, qw, kw, 1e-6f, 1e6, max_pos,
                                               cached ? slots : NULL, kc, vc, 1, T, Hq, Hkv, D, D,
                                               bs, nb, neox),
             0, "unfused qk_norm_rope_kv_write");
      free(qkv), free(qw), free(kw), free(kc), free(vc);
    }
  }
}

static void mla_cases(void) {
  const int64_t T = 4, max_pos = 8, nb = 2;
  const int Hq = 3, nope = 32, rope = 64, lora = 96, bs = 4;
  for (int neox = 0; neox <= 1; ++neox) {
    const int64_t qs = Hq * (nope + rope);
    uint16_t* q = bf16_array(T * qs, 1.0);
    uint16_t* kpe = bf16_array(T * rope, 1.0);
    uint16_t* kvc = bf16_array(T * lora, 1.0);
    uint16_t* cache = calloc((size_t)(nb * bs * (lora + rope)), sizeof *cache);
    int64_t pos[4] = {0, 7, 3, 1};
    int64_t slots[4] = {7, -1, 0, 4};
    expect(orc_mla_rope_kv_write(pos, q + nope, qs, nope + rope, kpe, rope, kvc, lora, 1e4,
                                 max_pos, slots, cache, T, Hq, lora, rope, bs, nb, neox),
           0, "mla_rope_kv_write");
    free(q), free(kpe), free(kvc), free(cache);
  }
}

static void codec_cases(void) {
  float in[6] = {0.f, -0.f, 448.f, 1e-9f, -3.5f, 500.f};
  uint8_t codes[6];
  uint16_t bits[6];
  double back[6];
  orc_e4m3fn_encode_f32_array(in, codes, 6);
  orc_bf16_encode_f32_array(in, bits, 6);
  orc_e4m3fn_decode_array(codes, back, 6);
  if (orc_e4m3fn_cross_check(0x3F000000u, 0x3F010000u) != 0) {
    fprintf(stderr, "e4m3fn encoders disagree\n");
    ++failures;
  }
}

int main(void) {
  codec_cases();
  norm_cases();
  silu_cases();
  dual_cases();
  rope_cases();
  qk_cases();
  mla_cases();
  if (failures) return 1;
  puts("oracle sanitizer run: clean");
  return 0;
}
