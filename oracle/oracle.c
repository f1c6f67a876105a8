/*
 * oracle.c -- plain, slow, obviously correct CPU oracle of the routed-expert
 * MoE layer.  TEST INFRASTRUCTURE ONLY: the product path never loads it;
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may call it.  It shares no code, header or table with the GPU library; it
 * restates the definitions from the pages and from the byte layouts in its
 * own words.
 *
 * What is computed, step by step:
 *   router logits  fp32, in the fixed order given at orc_logit()
 *   selection      exact top-k on the logits, ties to the lower index (with
 *                  a router bias: on the keys sigmoid32(z) + b, orc_bias_keys)
 *   mixing weights sigmoid of the chosen logits, normalised to sum one (fp64)
 *   bucketing      stable counting sort of the flat routes by expert
 *   dequantisation every weight exactly, in fp64 (block formats; VQ rows
 *                  with a per-layer E4M3 codebook)
 *   expert FFN     h = silu(G x) * (U x), ye = D h, all in fp64
 *   combine        y = sum_j wt_j * (g_e * ye_j) + shared(x), fp64, rounded
 *                  to fp32 (g_e the optional per-channel down gains, else 1)
 *
 * Sources: the layer's sum y = sum_k rw_k * ye_k + ysh with ye taken before
 * the routing weight is the per-layer MoE sum on "YoungAi -- DeepSeek V4.1
 * Flash on one DGX Spark", section 4.2, with the sidecar's per-channel down
 * gains and selection-only router bias optional (same section).  384
 * experts with 6 chosen per token: same page, section 2.2.  The format mix
 * (IQ2_XXS-like gate/up, Q2_K-like down, Q8 shared expert, unquantized
 * router): "Running DeepSeek V4 Flash on an RTX 5080 with 16GB VRAM Under
 * Linux/WSL2 via DS4", model section, and the txtmix teardown "ds4 拆解",
 * section 3.  The 8-dimensional VQ routed format (one 12- or 13-bit index
 * per 8 weights, one fp16 gain per row, E4M3 codewords shared by a layer):
 * YoungAi page, section 4.1.  The pages name no score function, activation, summation order
 * or byte layout; the readings used here are: sigmoid scores, selection on
 * the raw logit, SwiGLU experts with silu(g) = g / (1 + exp(-g)), the fixed
 * router order below, and the byte layouts restated at each decoder.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math:
 * the router order relies on IEEE fmaf and plain additions).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_IQ2 1
#define ORC_Q2K 2
#define ORC_Q8 3
#define ORC_Q4K 4
#define ORC_MX4 5
#define ORC_VQ12 6
#define ORC_VQ13 7

/* ---------------------------------------------------------------------- */
/* scalar decoding of stored numbers                                      */
/* ---------------------------------------------------------------------- */

/* IEEE binary16 -> double, exactly (normal, subnormal, inf, nan). */
double orc_half(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25);
  return sign ? -v : v;
}

/* bf16 bits -> fp32, exactly (the bits are the upper half of an fp32). */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t rd32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static float x_at(const void* x, int x_dtype, int64_t i) {
  if (x_dtype == ORC_BF16) return bf16_to_f32(((const uint16_t*)x)[i]);
  return ((const float*)x)[i];
}

/* ---------------------------------------------------------------------- */
/* router                                                                  */
/* ---------------------------------------------------------------------- */

/*
 * One router logit in fp32.  The pages give no summation order; exact
 * indices on both sides need one.  Order used: 64 partial sums start at
 * +0; element i goes to partial (i / 4) mod 64, each partial consuming its
 * elements in increasing i with one fused multiply-add each; the partials
 * are then folded pairwise, halving the count each step: p[l] += p[l + s]
 * for s = 32, 16, 8, 4, 2, 1; the logit is p[0].
 */
float orc_logit(const void* x, int x_dtype, int64_t x_off, const float* w, int d) {
  float p[64];
  for (int l = 0; l < 64; l++) p[l] = 0.0f;
  for (int i = 0; i < d; i++) {
    int l = (i / 4) % 64;
    p[l] = fmaf(x_at(x, x_dtype, x_off + i), w[i], p[l]);
  }
  for (int s = 32; s >= 1; s /= 2)
    for (int l = 0; l < s; l++) p[l] = p[l] + p[l + s];
  return p[0];
}

/* z[t][e] for all tokens and experts; W is [E][d] fp32, expert-major. */
void orc_router_logits(const void* x, int x_dtype, int T, int d, const float* W, int E, float* z) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) z[(int64_t)t * E + e] = orc_logit(x, x_dtype, (int64_t)t * d, W + (int64_t)e * d, d);
}

/*
 * Exact top-k: repeatedly take the best expert not taken yet.  "Best" is
 * the larger logit; among equal logits (IEEE equality, so -0 equals +0)
 * the lower index wins because the scan keeps the first maximum it meets.
 * Selecting on the logit rather than on sigmoid(logit) gives the same
 * order in exact arithmetic (sigmoid is strictly increasing).
 */
void orc_topk(const float* z, int T, int E, int k, int32_t* idx) {
  for (int t = 0; t < T; t++) {
    const float* zt = z + (int64_t)t * E;
    char* taken = (char*)calloc((size_t)E, 1);
    for (int r = 0; r < k; r++) {
      int best = -1;
      for (int e = 0; e < E; e++)
        if (!taken[e] && (best < 0 || zt[e] > zt[best])) best = e;
      taken[best] = 1;
      idx[(int64_t)t * k + r] = best;
    }
    free(taken);
  }
}

/*
 * Selection keys with a router bias (the sidecar's selection-only bias,
 * YoungAi page, section 4.2: the bias moves which experts are chosen and
 * leaves the mixing weights alone): key_e = sigmoid32(z_e) + b_e in fp32,
 * then the same top-k as above on the keys.  sigmoid32 is a fixed sequence
 * of IEEE fp32 operations (the pages give none; any implementation that
 * performs exactly these operations reproduces every bit):
 *   z clamped to [-80, 80]; t = -z
 *   n = rint(t * log2(e)) by adding and subtracting 1.5 * 2^23
 *   r = (t - n * ln2_hi) - n * ln2_lo        (ln2_hi has 16 significant bits,
 *                                            so n * ln2_hi is exact)
 *   p = ((((((r/720 + 1/120) r + 1/24) r + 1/6) r + 1/2) r + 1) r + 1)
 *       (Taylor coefficients of e^r, Horner, each step a product then a sum)
 *   e = p * 2^n                               (exact: 2^n built from bits)
 *   sigmoid32 = 1 / (1 + e)                   (correctly rounded division)
 * The constants are the fp32 values of the hex literals below.
 */
float orc_sigmoid32(float z) {
  const float log2e = 0x1.715476p+0f, ln2_hi = 0x1.62e400p-1f, ln2_lo = 0x1.7f7d1cp-20f;
  const float c720 = 0x1.6c16c2p-10f, c120 = 0x1.111112p-7f, c24 = 0x1.555556p-5f, c6 = 0x1.555556p-3f;
  const float shifter = 0x1.8p+23f;
  float zc = z < -80.0f ? -80.0f : (z > 80.0f ? 80.0f : z);
  float t = -zc;
  float kf = t * log2e;
  float n = (kf + shifter) - shifter;
  float r = (t - n * ln2_hi) - n * ln2_lo;
  float p = c720;
  p = p * r + c120;
  p = p * r + c24;
  p = p * r + c6;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  union {
    uint32_t u;
    float f;
  } two_n;
  two_n.u = (uint32_t)((int)n + 127) << 23;
  float e = p * two_n.f;
  return 1.0f / (1.0f + e);
}

void orc_bias_keys(const float* z, int T, int E, const float* b, float* key) {
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) key[(int64_t)t * E + e] = orc_sigmoid32(z[(int64_t)t * E + e]) + b[e];
}

/*
 * Mixing weights: s_j = 1 / (1 + exp(-z_j)) for the k selected experts, in
 * double precision; w_j = s_j / (s_0 + ... + s_{k-1}) with the sum taken in
 * rank order; stored as fp32.  No extra routed scaling factor.  Selection
 * keys and mixing weights are separate quantities (YoungAi page, section
 * 4.2: a selection bias leaves the mixing weights untouched); with no bias
 * both come from the same logit.
 */
void orc_route_weights(const float* z, const int32_t* idx, int T, int E, int k, float* wt) {
  for (int t = 0; t < T; t++) {
    double s[64], sum = 0.0;
    for (int j = 0; j < k; j++) {
      double zj = (double)z[(int64_t)t * E + idx[(int64_t)t * k + j]];
      s[j] = 1.0 / (1.0 + exp(-zj));
    }
    for (int j = 0; j < k; j++) sum += s[j];
    for (int j = 0; j < k; j++) wt[(int64_t)t * k + j] = (float)(s[j] / sum);
  }
}

/*
 * Bucketing: a stable counting sort of the flat routes r = t*k + j by their
 * expert idx[r].  counts, exclusive offsets (offsets[E] = n), perm = routes
 * ordered by (expert, r), pos = inverse of perm.  Grouping a chunk's tokens
 * by expert is what lets one pass over an expert's weights serve all of
 * its rows (YoungAi page, section 4.4, the verify-batch expert kernel).
 */
void orc_bucket(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                int32_t* pos) {
  int64_t n = (int64_t)T * k;
  for (int e = 0; e < E; e++) counts[e] = 0;
  for (int64_t r = 0; r < n; r++) counts[idx[r]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int e = 0; e < E; e++) next[e] = offsets[e];
  for (int64_t r = 0; r < n; r++) {
    int32_t p = next[idx[r]]++;
    perm[p] = (int32_t)r;
    pos[r] = p;
  }
  free(next);
}

/* ---------------------------------------------------------------------- */
/* dequantisation (every value exact in fp64)                              */
/* ---------------------------------------------------------------------- */

/*
 * IQ2XXS_L block, 256 weights in 66 bytes: fp16 d; then for sub-block
 * j = 0..7 two little-endian words A_j, B_j.  A_j byte i is the grid row of
 * 8-weight group 4j+i; B_j bits 7i..7i+6 are that group's 7 stored signs
 * and bits 28..31 the sub-block scale s.  The 8th sign of a group is the
 * parity of its 7 stored signs.  w = d * (2s+1) * grid[row][p] * sign.
 */
static void deq_iq2(const uint8_t* b, const uint8_t* grid, double* w) {
  double d = orc_half(rd16(b));
  for (int j = 0; j < 8; j++) {
    uint32_t A = rd32(b + 2 + 8 * j), B = rd32(b + 6 + 8 * j);
    int s = (int)(B >> 28);
    for (int i = 0; i < 4; i++) {
      int row = (int)((A >> (8 * i)) & 255u);
      int sg = (int)((B >> (7 * i)) & 127u);
      int parity = __builtin_popcount((unsigned)sg) & 1;
      for (int p = 0; p < 8; p++) {
        int neg = p < 7 ? (sg >> p) & 1 : parity;
        double v = d * (double)(2 * s + 1) * (double)grid[row * 8 + p];
        w[32 * j + 8 * i + p] = neg ? -v : v;
      }
    }
  }
}

/*
 * Q2K_L block, 256 weights in 84 bytes: fp16 d, fp16 dmin, 16 bytes of
 * (scale low nibble, min high nibble) per 16-weight sub-block, 64 bytes of
 * 2-bit quants (weight i in bits 2(i%4) of byte i/4).
 * w_i = d * sc_j * q_i - dmin * m_j, j = i / 16.
 */
static void deq_q2k(const uint8_t* b, double* w) {
  double d = orc_half(rd16(b)), dmin = orc_half(rd16(b + 2));
  for (int i = 0; i < 256; i++) {
    int j = i / 16;
    int sc = b[4 + j] & 15, m = b[4 + j] >> 4;
    int q = (b[20 + i / 4] >> (2 * (i % 4))) & 3;
    w[i] = d * (double)sc * (double)q - dmin * (double)m;
  }
}

/*
 * Q4K_L block (the 4-bit routed variant: the "ds4f-q4" models of "Running
 * DeepSeek V4 Flash on an RTX 5080 ...", model section, whose routed Q4_K
 * layout has the grouped kernels named in its CUDA section), 256 weights in
 * 144 bytes: fp16 d, fp16 dmin; 8 bytes, one per 32-weight sub-block j,
 * holding the low 4 bits of the 6-bit scale sc_j (low nibble) and of the
 * 6-bit min m_j (high nibble); 4 bytes, byte p holding the top two bits of
 * sc_2p, m_2p, sc_2p+1, m_2p+1 (bit pairs 0-1, 2-3, 4-5, 6-7); 128 bytes of
 * 4-bit quants (weight i in bits 4(i%2) of byte i/2).
 * w_i = d * sc_j * q_i - dmin * m_j, j = i / 32.
 */
static void deq_q4k(const uint8_t* b, double* w) {
  double d = orc_half(rd16(b)), dmin = orc_half(rd16(b + 2));
  for (int j = 0; j < 8; j++) {
    int top = b[12 + j / 2] >> (4 * (j % 2));
    int sc = (b[4 + j] & 15) | ((top & 3) << 4);
    int m = (b[4 + j] >> 4) | (((top >> 2) & 3) << 4);
    for (int t = 0; t < 32; t++) {
      int i = 32 * j + t;
      int q = (b[16 + i / 2] >> (4 * (i % 2))) & 15;
      w[i] = d * (double)sc * (double)q - dmin * (double)m;
    }
  }
}

/*
 * MXFP4_L block (the native MXFP4 routed experts of "Running DeepSeek V4
 * Flash on an RTX 5080 ...", model section: FP4 values with one shared
 * scale per 32 weights, 4.25 bits per weight as the YoungAi page, section
 * 4.1, counts them), 32 weights in 17 bytes: byte 0 is an E8M0 scale, the
 * power of two 2^(s - 127); bytes 1..16 hold E2M1 codes, weight 2i in the
 * low nibble of byte 1 + i and weight 2i + 1 in the high nibble.
 * An E2M1 code has a sign bit (bit 3), a 2-bit exponent E (bits 2..1) and a
 * 1-bit mantissa M (bit 0): |value| = M / 2 when E = 0 (subnormal), else
 * (1 + M / 2) * 2^(E - 1).  w = 2^(s - 127) * value.  (s = 255, the E8M0
 * not-a-number, is not a valid block.)
 */
static double e2m1(int c) {
  int E = (c >> 1) & 3, M = c & 1;
  double mag = E == 0 ? 0.5 * M : (1.0 + 0.5 * M) * ldexp(1.0, E - 1);
  return (c & 8) ? -mag : mag;
}

static void deq_mx4(const uint8_t* b, double* w) {
  double scale = ldexp(1.0, (int)b[0] - 127);
  for (int i = 0; i < 32; i++) {
    int c = (b[1 + i / 2] >> (4 * (i % 2))) & 15;
    w[i] = scale * e2m1(c);
  }
}

/*
 * E4M3 byte (the FP8 codewords of the YoungAi page, section 4.1): sign bit
 * 7, 4-bit exponent E (bits 6..3, bias 7), 3-bit mantissa M; |value| =
 * M / 8 * 2^-6 for E = 0, else (1 + M / 8) * 2^(E - 7); E = 15 with M = 7 is
 * not a number (not a valid codeword); there are no infinities.
 */
double orc_e4m3(int b) {
  int E = (b >> 3) & 15, M = b & 7;
  if (E == 15 && M == 7) return NAN;
  double mag = E == 0 ? ldexp((double)M, -9) : ldexp((double)(8 + M), E - 10);
  return (b & 128) ? -mag : mag;
}

/*
 * VQ rows (the 8-dimensional vector quantization of the YoungAi page,
 * section 4.1: every 8 consecutive weights of a routed-expert row are one
 * 12-bit or 13-bit index into a per-layer codebook, times one fp16 gain per
 * row).  A row of K weights is:
 *   bytes 0-1                fp16 gain g,
 *   next 3K/16 bytes         the 12-bit index stream: index j occupies bits
 *                            12j .. 12j + 11 of the stream, least
 *                            significant bit first (bit b of the stream is
 *                            bit b % 8 of byte b / 8),
 *   next K/64 bytes (VQ13)   the bit plane: bit j (bit j % 8 of byte j / 8)
 *                            is bit 12 of index j (the "12 + 1" layout).
 *   w[8j + i] = g * codebook[index_j][i], codewords as E4M3 bytes [n][8].
 */
static int64_t vq_row_bytes(int fmt, int K) { return 2 + 3 * (int64_t)K / 16 + (fmt == ORC_VQ13 ? K / 64 : 0); }

static void deq_vq_row(int fmt, const uint8_t* row, int K, const uint8_t* cb, double* w) {
  double g = orc_half(rd16(row));
  const uint8_t* stream = row + 2;
  const uint8_t* plane = stream + 3 * K / 16;
  for (int j = 0; j < K / 8; j++) {
    int idx = 0;
    for (int b = 0; b < 12; b++) {
      int64_t bit = 12 * (int64_t)j + b;
      idx |= ((stream[bit / 8] >> (bit % 8)) & 1) << b;
    }
    if (fmt == ORC_VQ13) idx |= ((plane[j / 8] >> (j % 8)) & 1) << 12;
    for (int i = 0; i < 8; i++) w[8 * j + i] = g * orc_e4m3(cb[8 * idx + i]);
  }
}

/* Q8_0_L block, 32 weights in 34 bytes: fp16 d then int8 q[32]; w = d q. */
static void deq_q8(const uint8_t* b, double* w) {
  double d = orc_half(rd16(b));
  for (int i = 0; i < 32; i++) w[i] = d * (double)(int8_t)b[2 + i];
}

static int block_weights(int fmt) { return fmt == ORC_Q8 || fmt == ORC_MX4 ? 32 : 256; }
static int block_bytes(int fmt) {
  return fmt == ORC_IQ2 ? 66 : fmt == ORC_Q2K ? 84 : fmt == ORC_Q4K ? 144 : fmt == ORC_MX4 ? 17 : 34;
}

/* Bytes of one row of K weights in `fmt`. */
static int64_t row_bytes_of(int fmt, int K) {
  if (fmt == ORC_VQ12 || fmt == ORC_VQ13) return vq_row_bytes(fmt, K);
  return (int64_t)(K / block_weights(fmt)) * block_bytes(fmt);
}

/* Decode n_blocks consecutive blocks of `fmt` into fp64. Returns 0 on success. */
int orc_dequant(int fmt, const uint8_t* blocks, int64_t n_blocks, const uint8_t* grid, double* out) {
  if (fmt != ORC_IQ2 && fmt != ORC_Q2K && fmt != ORC_Q8 && fmt != ORC_Q4K && fmt != ORC_MX4) return -1;
  int bw = block_weights(fmt), bb = block_bytes(fmt);
  for (int64_t i = 0; i < n_blocks; i++) {
    const uint8_t* b = blocks + i * bb;
    double* w = out + i * bw;
    if (fmt == ORC_IQ2)
      deq_iq2(b, grid, w);
    else if (fmt == ORC_Q2K)
      deq_q2k(b, w);
    else if (fmt == ORC_Q4K)
      deq_q4k(b, w);
    else if (fmt == ORC_MX4)
      deq_mx4(b, w);
    else
      deq_q8(b, w);
  }
  return 0;
}

/*
 * Decode n_rows consecutive rows of K weights of any format (the block
 * formats row by row, VQ rows with the codebook cb).  Returns 0 on success.
 */
int orc_dequant_rows(int fmt, const uint8_t* rows, int64_t n_rows, int K, const uint8_t* grid, const uint8_t* cb,
                     double* out) {
  int64_t rb = row_bytes_of(fmt, K);
  for (int64_t r = 0; r < n_rows; r++) {
    if (fmt == ORC_VQ12 || fmt == ORC_VQ13) {
      if (!cb) return -1;
      deq_vq_row(fmt, rows + r * rb, K, cb, out + r * K);
    } else if (orc_dequant(fmt, rows + r * rb, K / block_weights(fmt), grid, out + r * K) != 0) {
      return -1;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* expert FFN                                                              */
/* ---------------------------------------------------------------------- */

/*
 * out[n] = sum_i W[n][i] * v[i] over the `rows` rows of one matrix of
 * `fmt` (row n of expert matrix starts at n * row_bytes), fp64 throughout,
 * each dot product summed in increasing i.
 */
static void matvec(int fmt, const uint8_t* mat, int rows, int K, const uint8_t* grid, const uint8_t* cb,
                   const double* v, double* out) {
  int64_t row_bytes = row_bytes_of(fmt, K);
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < rows; n++) {
      orc_dequant_rows(fmt, mat + (int64_t)n * row_bytes, 1, K, grid, cb, w);
      double acc = 0.0;
      for (int i = 0; i < K; i++) acc += w[i] * v[i];
      out[n] = acc;
    }
    free(w);
  }
}

/* silu(g) = g * sigmoid(g) = g / (1 + exp(-g)). */
static double silu(double g) { return g / (1.0 + exp(-g)); }

/*
 * One SwiGLU expert on one token: out = D (silu(G x) * (U x)).
 * G, U: [f][d]; D: [d][f].
 */
/* Whether fmt names a format this file decodes (VQ rows need a codebook). */
static int fmt_usable(int fmt, const uint8_t* cb) {
  if (fmt == ORC_VQ12 || fmt == ORC_VQ13) return cb != NULL;
  return fmt == ORC_IQ2 || fmt == ORC_Q2K || fmt == ORC_Q8 || fmt == ORC_Q4K || fmt == ORC_MX4;
}

static void expert(int fmt_gu, const uint8_t* G, const uint8_t* U, int fmt_dn, const uint8_t* D, int d, int f,
                   const uint8_t* grid, const uint8_t* cb, const double* x, double* out, double* g, double* u) {
  matvec(fmt_gu, G, f, d, grid, cb, x, g);
  matvec(fmt_gu, U, f, d, grid, cb, x, u);
  for (int n = 0; n < f; n++) g[n] = silu(g[n]) * u[n];
  matvec(fmt_dn, D, d, f, grid, cb, g, out);
}

static int64_t mat_bytes(int fmt, int rows, int K) { return (int64_t)rows * row_bytes_of(fmt, K); }

/*
 * Expert FFN of a layer for the tokens listed in `tokens` (n_tok of them;
 * NULL means tokens 0..T-1) with caller-given routes idx/wt [T][k]:
 *   acc = sum_j wt[t][j] * (g_e * D_e(silu(G_e x_t) * (U_e x_t)))  (j in rank order)
 *       + D_s(silu(G_s x_t) * (U_s x_t))                            (if has_shared)
 * where g_e is expert e's per-output-channel down gain (down_gain [E][d],
 * the sidecar's gains of the YoungAi page, section 4.2) or one when
 * down_gain is NULL.
 *   y[row] = fp32(acc)  (round to nearest even), row = position in `tokens`.
 * The routing weight multiplies each expert's down-projection output, as in
 * the per-layer sum of the YoungAi page, section 4.2.
 */
int orc_ffn(int E, int d, int f, int k, int fmt_gu, int fmt_dn, const uint8_t* w_gate, const uint8_t* w_up,
            const uint8_t* w_down, const uint8_t* grid, const uint8_t* cb, int has_shared, int fmt_sh,
            const uint8_t* s_gate,
            const uint8_t* s_up, const uint8_t* s_down, const float* down_gain, const void* x, int x_dtype, int T,
            const int32_t* tokens, int n_tok, const int32_t* idx, const float* wt, float* y) {
  if (!fmt_usable(fmt_gu, cb) || !fmt_usable(fmt_dn, cb) || (has_shared && !fmt_usable(fmt_sh, cb))) return -1;
  int64_t gu_bytes = mat_bytes(fmt_gu, f, d), dn_bytes = mat_bytes(fmt_dn, d, f);
  double* xv = (double*)malloc(sizeof(double) * (size_t)d);
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double* ye = (double*)malloc(sizeof(double) * (size_t)d);
  double* g = (double*)malloc(sizeof(double) * (size_t)f);
  double* u = (double*)malloc(sizeof(double) * (size_t)f);
  int count = tokens ? n_tok : T, status = 0;
  for (int r = 0; r < count && status == 0; r++) {
    int t = tokens ? tokens[r] : r;
    if (t < 0 || t >= T) {
      status = -1;
      break;
    }
    for (int i = 0; i < d; i++) xv[i] = (double)x_at(x, x_dtype, (int64_t)t * d + i);
    for (int i = 0; i < d; i++) acc[i] = 0.0;
    for (int j = 0; j < k; j++) {
      int e = idx[(int64_t)t * k + j];
      if (e < 0 || e >= E) {
        status = -1;
        break;
      }
      expert(fmt_gu, w_gate + e * gu_bytes, w_up + e * gu_bytes, fmt_dn, w_down + e * dn_bytes, d, f, grid, cb, xv,
             ye, g, u);
      double w = (double)wt[(int64_t)t * k + j];
      if (down_gain)
        for (int i = 0; i < d; i++) acc[i] += w * ((double)down_gain[(int64_t)e * d + i] * ye[i]);
      else
        for (int i = 0; i < d; i++) acc[i] += w * ye[i];
    }
    if (status != 0) break;
    if (has_shared) {
      expert(fmt_sh, s_gate, s_up, fmt_sh, s_down, d, f, grid, cb, xv, ye, g, u);
      for (int i = 0; i < d; i++) acc[i] += ye[i];
    }
    for (int i = 0; i < d; i++) y[(int64_t)r * d + i] = (float)acc[i];
  }
  free(xv);
  free(acc);
  free(ye);
  free(g);
  free(u);
  return status;
}

/*
 * The same function as orc_ffn, with the loops over tokens and experts
 * interchanged: every expert that a listed token routes to is dequantised
 * once, then each of its (token, rank) pairs is evaluated with exactly the
 * operations orc_ffn performs for it (fp64 dot products in increasing input
 * order, the SwiGLU, the down projection), and the results are combined per
 * token in rank order, then the shared expert, as orc_ffn does.  Every output
 * is therefore bitwise the same as orc_ffn's; only the number of
 * dequantisations changes (once per expert instead of once per token and
 * route), which makes hundreds of tokens of a full-size layer affordable.
 */
static void matvec_deq(const double* W, int rows, int K, const double* v, double* out) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < rows; n++) {
    const double* w = W + (int64_t)n * K;
    double acc = 0.0;
    for (int i = 0; i < K; i++) acc += w[i] * v[i];
    out[n] = acc;
  }
}

static double* deq_matrix(int fmt, const uint8_t* mat, int rows, int K, const uint8_t* grid, const uint8_t* cb) {
  int64_t row_bytes = row_bytes_of(fmt, K);
  double* W = (double*)malloc(sizeof(double) * (size_t)rows * (size_t)K);
  if (!W) return NULL;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < rows; n++) orc_dequant_rows(fmt, mat + (int64_t)n * row_bytes, 1, K, grid, cb, W + (int64_t)n * K);
  return W;
}

/* out = D (silu(G x) * (U x)) with dequantised G, U [f][d] and D [d][f]. */
static void expert_deq(const double* G, const double* U, const double* D, int d, int f, const double* x,
                       double* out, double* g, double* u) {
  matvec_deq(G, f, d, x, g);
  matvec_deq(U, f, d, x, u);
  for (int n = 0; n < f; n++) g[n] = silu(g[n]) * u[n];
  matvec_deq(D, d, f, g, out);
}

int orc_ffn_grouped(int E, int d, int f, int k, int fmt_gu, int fmt_dn, const uint8_t* w_gate, const uint8_t* w_up,
                    const uint8_t* w_down, const uint8_t* grid, const uint8_t* cb, int has_shared, int fmt_sh,
                    const uint8_t* s_gate,
                    const uint8_t* s_up, const uint8_t* s_down, const float* down_gain, const void* x, int x_dtype,
                    int T, const int32_t* tokens, int n_tok, const int32_t* idx, const float* wt, float* y) {
  if (!fmt_usable(fmt_gu, cb) || !fmt_usable(fmt_dn, cb) || (has_shared && !fmt_usable(fmt_sh, cb))) return -1;
  int64_t gu_bytes = mat_bytes(fmt_gu, f, d), dn_bytes = mat_bytes(fmt_dn, d, f);
  int count = tokens ? n_tok : T;
  for (int r = 0; r < count; r++) {
    int t = tokens ? tokens[r] : r;
    if (t < 0 || t >= T) return -1;
    for (int j = 0; j < k; j++) {
      int e = idx[(int64_t)t * k + j];
      if (e < 0 || e >= E) return -1;
    }
  }
  double* ye = (double*)calloc((size_t)count * k * d, sizeof(double));    /* [r][j][d] */
  double* ysh = (double*)calloc((size_t)count * d, sizeof(double));       /* [r][d] */
  double* xv = (double*)malloc(sizeof(double) * (size_t)d);
  double* g = (double*)malloc(sizeof(double) * (size_t)f);
  double* u = (double*)malloc(sizeof(double) * (size_t)f);
  if (!ye || !ysh || !xv || !g || !u) {
    free(ye); free(ysh); free(xv); free(g); free(u);
    return -2;
  }
  int status = 0;
  for (int e = 0; e < E && status == 0; e++) {
    int used = 0;
    for (int r = 0; r < count && !used; r++) {
      int t = tokens ? tokens[r] : r;
      for (int j = 0; j < k; j++) used |= idx[(int64_t)t * k + j] == e;
    }
    if (!used) continue;
    double* G = deq_matrix(fmt_gu, w_gate + e * gu_bytes, f, d, grid, cb);
    double* U = deq_matrix(fmt_gu, w_up + e * gu_bytes, f, d, grid, cb);
    double* D = deq_matrix(fmt_dn, w_down + e * dn_bytes, d, f, grid, cb);
    if (!G || !U || !D) status = -2;
    for (int r = 0; r < count && status == 0; r++) {
      int t = tokens ? tokens[r] : r;
      for (int j = 0; j < k; j++) {
        if (idx[(int64_t)t * k + j] != e) continue;
        for (int i = 0; i < d; i++) xv[i] = (double)x_at(x, x_dtype, (int64_t)t * d + i);
        expert_deq(G, U, D, d, f, xv, ye + ((int64_t)r * k + j) * d, g, u);
      }
    }
    free(G); free(U); free(D);
  }
  if (status == 0 && has_shared) {
    double* G = deq_matrix(fmt_sh, s_gate, f, d, grid, cb);
    double* U = deq_matrix(fmt_sh, s_up, f, d, grid, cb);
    double* D = deq_matrix(fmt_sh, s_down, d, f, grid, cb);
    if (!G || !U || !D) status = -2;
    for (int r = 0; r < count && status == 0; r++) {
      int t = tokens ? tokens[r] : r;
      for (int i = 0; i < d; i++) xv[i] = (double)x_at(x, x_dtype, (int64_t)t * d + i);
      expert_deq(G, U, D, d, f, xv, ysh + (int64_t)r * d, g, u);
    }
    free(G); free(U); free(D);
  }
  if (status == 0) {
    for (int r = 0; r < count; r++) {
      int t = tokens ? tokens[r] : r;
      for (int i = 0; i < d; i++) {
        double acc = 0.0;
        for (int j = 0; j < k; j++) {
          int e = idx[(int64_t)t * k + j];
          double w = (double)wt[(int64_t)t * k + j], v = ye[((int64_t)r * k + j) * d + i];
          if (down_gain)
            acc += w * ((double)down_gain[(int64_t)e * d + i] * v);
          else
            acc += w * v;
        }
        if (has_shared) acc += ysh[(int64_t)r * d + i];
        y[(int64_t)r * d + i] = (float)acc;
      }
    }
  }
  free(ye); free(ysh); free(xv); free(g); free(u);
  return status;
}

/* Routing of the listed tokens: logits, exact top-k and mixing weights. */
void orc_route(const void* x, int x_dtype, int T, int d, const float* W, int E, int k, float* z, int32_t* idx,
               float* wt) {
  orc_router_logits(x, x_dtype, T, d, W, E, z);
  orc_topk(z, T, E, k, idx);
  orc_route_weights(z, idx, T, E, k, wt);
}

/* Threads for the parallel regions that follow (n >= 1); bench uses it for
 * a single-thread rate beside the all-cores one. */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Number of OpenMP threads a parallel region would use (reported by bench). */
int orc_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
