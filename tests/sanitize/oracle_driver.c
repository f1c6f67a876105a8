/* Drives every oracle function on small inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py; CPU only).
 * The inputs are bytes from a fixed linear congruential sequence: every bit
 * pattern of the quant fields is a valid code, and the fp16 scale fields are
 * overwritten with small finite values. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_half(uint16_t h);
float orc_logit(const void* x, int x_dtype, int64_t x_off, const float* w, int d);
void orc_router_logits(const void* x, int x_dtype, int T, int d, const float* W, int E, float* z);
void orc_topk(const float* z, int T, int E, int k, int32_t* idx);
float orc_sigmoid32(float z);
void orc_bias_keys(const float* z, int T, int E, const float* b, float* key);
void orc_route_weights(const float* z, const int32_t* idx, int T, int E, int k, float* wt);
void orc_bucket(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                int32_t* pos);
int orc_dequant(int fmt, const uint8_t* blocks, int64_t n_blocks, const uint8_t* grid, double* out);
int orc_dequant_rows(int fmt, const uint8_t* rows, int64_t n_rows, int K, const uint8_t* grid, const uint8_t* cb,
                     double* out);
double orc_e4m3(int b);
int orc_ffn(int E, int d, int f, int k, int fmt_gu, int fmt_dn, const uint8_t* w_gate, const uint8_t* w_up,
            const uint8_t* w_down, const uint8_t* grid, const uint8_t* cb, int has_shared, int fmt_sh, const uint8_t* s_gate,
            const uint8_t* s_up, const uint8_t* s_down, const float* down_gain, const void* x, int x_dtype, int T,
            const int32_t* tokens, int n_tok, const int32_t* idx, const float* wt, float* y);
int orc_ffn_grouped(int E, int d, int f, int k, int fmt_gu, int fmt_dn, const uint8_t* w_gate, const uint8_t* w_up,
                    const uint8_t* w_down, const uint8_t* grid, const uint8_t* cb, int has_shared, int fmt_sh,
                    const uint8_t* s_gate,
                    const uint8_t* s_up, const uint8_t* s_down, const float* down_gain, const void* x, int x_dtype,
                    int T, const int32_t* tokens, int n_tok, const int32_t* idx, const float* wt, float* y);

static uint32_t lcg = 12345u;
static uint32_t next(void) { return lcg = lcg * 1664525u + 1013904223u; }
static float unif(void) { return (float)(next() >> 8) / 16777216.0f - 0.5f; }

static int bw(int fmt) { return fmt == 3 || fmt == 5 ? 32 : 256; }
static int bb(int fmt) { return fmt == 1 ? 66 : fmt == 2 ? 84 : fmt == 4 ? 144 : fmt == 5 ? 17 : 34; }

/* random blocks with scale fields set to 2^-10 (fp16 0x1400; E8M0 0x75) */
static uint8_t* blocks(int fmt, int n) {
  uint8_t* b = (uint8_t*)malloc((size_t)n * bb(fmt));
  for (int i = 0; i < n * bb(fmt); i++) b[i] = (uint8_t)(next() >> 24);
  for (int i = 0; i < n; i++) {
    uint8_t* p = b + (size_t)i * bb(fmt);
    if (fmt == 5) { p[0] = 0x75; continue; }
    p[0] = 0x00; p[1] = 0x14;
    if (fmt == 2 || fmt == 4) { p[2] = 0x00; p[3] = 0x14; }
  }
  return b;
}

/* bytes of one row of K weights (VQ rows: gain, 12-bit stream, 13-bit plane) */
static int row_bytes(int fmt, int K) {
  if (fmt == 6 || fmt == 7) return 2 + 3 * K / 16 + (fmt == 7 ? K / 64 : 0);
  return K / bw(fmt) * bb(fmt);
}

/* a random matrix of `rows` rows of K weights */
static uint8_t* matrix(int fmt, int rows, int K) {
  if (fmt != 6 && fmt != 7) return blocks(fmt, rows * K / bw(fmt));
  int rb = row_bytes(fmt, K);
  uint8_t* b = (uint8_t*)malloc((size_t)rows * rb);
  for (int i = 0; i < rows * rb; i++) b[i] = (uint8_t)(next() >> 24);
  for (int r = 0; r < rows; r++) { b[(size_t)r * rb] = 0x00; b[(size_t)r * rb + 1] = 0x14; }
  return b;
}

int main(void) {
  enum { E = 6, k = 2, d = 256, f = 256, T = 5 };
  double acc = 0.0;
  for (int h = 0; h < 65536; h++) {
    double v = orc_half((uint16_t)h);
    if (isfinite(v)) acc += v * 1e-9;
  }
  uint8_t grid[256 * 8];
  for (int i = 0; i < 256 * 8; i++) grid[i] = (uint8_t)(2 * (next() % 4) + 1);
  float x[T * d], W[E * d], z[T * E], key[T * E], wt[T * k], bias[E], y[T * d], y2[T * d], gain[E * d];
  uint16_t xb[T * d];
  for (int i = 0; i < T * d; i++) { x[i] = unif() * 4; xb[i] = (uint16_t)(next() >> 16) & 0x3fff; }
  for (int i = 0; i < E * d; i++) { W[i] = unif() * 0.1f; gain[i] = 1.0f + unif(); }
  for (int e = 0; e < E; e++) bias[e] = unif() * 0.1f;
  acc += orc_logit(xb, 1, 0, W, d);
  orc_router_logits(x, 0, T, d, W, E, z);
  int32_t idx[T * k];
  orc_bias_keys(z, T, E, bias, key);
  orc_topk(key, T, E, k, idx);
  orc_topk(z, T, E, k, idx);
  orc_route_weights(z, idx, T, E, k, wt);
  for (int i = -100; i <= 100; i++) acc += orc_sigmoid32((float)i);
  int32_t counts[E], offsets[E + 1], perm[T * k], pos[T * k];
  orc_bucket(idx, T, k, E, counts, offsets, perm, pos);
  /* codebook of 8192 E4M3 codewords, bit 3 cleared: even exponent fields, never 15, all finite */
  static uint8_t cb[8192 * 8];
  for (int i = 0; i < 8192 * 8; i++) cb[i] = (uint8_t)(next() >> 24) & 0xf7;
  for (int c = 0; c < 256; c++) acc += isnan(orc_e4m3(c)) ? 0.0 : orc_e4m3(c) * 1e-9;
  for (int fmt = 1; fmt <= 5; fmt++) {
    uint8_t* b = blocks(fmt, 3);
    double w[3 * 256];
    if (orc_dequant(fmt, b, 3, grid, w) != 0) return 2;
    for (int i = 0; i < 3 * bw(fmt); i++) acc += w[i];
    free(b);
  }
  for (int fmt = 6; fmt <= 7; fmt++) {
    uint8_t* b = matrix(fmt, 3, 256);
    double w[3 * 256];
    if (orc_dequant_rows(fmt, b, 3, 256, NULL, cb, w) != 0) return 9;
    if (orc_dequant_rows(fmt, b, 3, 256, NULL, NULL, w) != -1) return 10;
    for (int i = 0; i < 3 * 256; i++) acc += w[i];
    free(b);
  }
  const int fmts[5][3] = {{1, 2, 3}, {4, 4, 3}, {3, 1, 2}, {5, 5, 3}, {7, 6, 3}};
  for (int c = 0; c < 5; c++) {
    const int fgu = fmts[c][0], fdn = fmts[c][1], fsh = fmts[c][2];
    uint8_t* g = matrix(fgu, E * f, d);
    uint8_t* u = matrix(fgu, E * f, d);
    uint8_t* dn = matrix(fdn, E * d, f);
    uint8_t* sg = matrix(fsh, f, d);
    uint8_t* su = matrix(fsh, f, d);
    uint8_t* sd = matrix(fsh, d, f);
    int32_t tok[3] = {4, 0, 4};
    if (orc_ffn(E, d, f, k, fgu, fdn, g, u, dn, grid, cb, 1, fsh, sg, su, sd, c ? gain : NULL, x, 0, T, NULL, 0, idx,
                wt, y) != 0) return 3;
    if (orc_ffn_grouped(E, d, f, k, fgu, fdn, g, u, dn, grid, cb, 1, fsh, sg, su, sd, c ? gain : NULL, x, 0, T, NULL, 0,
                        idx, wt, y2) != 0) return 4;
    if (memcmp(y, y2, sizeof y) != 0) return 5;
    if (orc_ffn_grouped(E, d, f, k, fgu, fdn, g, u, dn, grid, cb, 0, 0, NULL, NULL, NULL, NULL, xb, 1, T, tok, 3, idx,
                        wt, y2) != 0) return 6;
    int32_t bad[T * k];
    memcpy(bad, idx, sizeof bad);
    bad[3] = E;
    if (orc_ffn_grouped(E, d, f, k, fgu, fdn, g, u, dn, grid, cb, 0, 0, NULL, NULL, NULL, NULL, x, 0, T, NULL, 0, bad,
                        wt, y2) != -1) return 7;
    if (orc_ffn(E, d, f, k, fgu, fdn, g, u, dn, grid, cb, 0, 0, NULL, NULL, NULL, NULL, x, 0, T, NULL, 0, bad, wt,
                y2) != -1) return 8;
    for (int i = 0; i < T * d; i++) acc += y[i];
    free(g); free(u); free(dn); free(sg); free(su); free(sd);
  }
  printf("OK %g\n", acc);
  return 0;
}
