/*
 * moe.h -- C ABI of libqmoe: a routed-expert MoE feed-forward layer with
 * 2-bit block-quantized experts, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (sources are the pages this library follows):
 *
 *   - A router scores every expert of a layer and keeps the best top_k of
 *     them per token (DeepSeek V4.1 Flash layers have 384 experts and pick 6:
 *     "YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 2.2).  The
 *     router itself is not quantized ("Running DeepSeek V4 Flash on an RTX
 *     5080 with 16GB VRAM Under Linux/WSL2 via DS4", model section: only the
 *     routed experts are quantized; shared experts, projections and routing
 *     stay at higher precision).
 *   - Routed experts store gate/up in an IQ2_XXS-like codebook format and
 *     down in a Q2_K-like format (same model section; the Flash Q2 file name
 *     in the txtmix teardown "ds4 拆解", section 3, also names a Q8 shared
 *     expert, hence the Q8_0-like shared-expert format below).
 *   - Each expert is a SwiGLU FFN: h = silu(G x) * (U x), ye = D h.
 *   - The per-layer output is the weighted sum of the chosen experts' down
 *     projections plus the always-on shared expert:
 *         y_t = sum_j wt[t][j] * (g_e * ye_e(x_t)) + ysh(x_t),  e = idx[t][j]
 *     (YoungAi page, section 4.2, the engine's per-layer MoE sum), where ye
 *     is taken before the routing weight is applied and g_e is expert e's
 *     optional per-output-channel down gain (the sidecar's gains; one when
 *     moe_layer.down_gain is NULL), applied element-wise.
 *
 * Router definition used by every entry point (the pages name no score
 * function, summation order or tie rule; these are this library's readings):
 *   z[t][e]   = fp32 dot(x_t, W_r[e]) in the FIXED ORDER defined below;
 *   selection = the top_k experts by z (descending), equal z resolved to the
 *               smaller expert index, IEEE comparison (-0 == +0);
 *               idx[t][0..k-1] lists them best first ("rank order");
 *   weights   = s_j = sigmoid(z_j) over the selected experts, computed in
 *               double precision; wt[t][j] = s_j / (s_0 + ... + s_{k-1})
 *               (the sum taken in rank order), stored as fp32.
 *   Fixed fp32 order of z: with d = d_model and 64 partial sums p[0..63]
 *   starting at +0.0f, element i of the dot product belongs to partial
 *   p[(i / 4) % 64]; each partial takes its elements in increasing i, one
 *   fused multiply-add (fmaf, single rounding) each; then for s = 32, 16,
 *   8, 4, 2, 1 in that order, p[l] = p[l] + p[l + s] for every l < s; z is
 *   p[0].  bf16 activations are widened to fp32 exactly before use.
 *   Ranking on z rather than on sigmoid(z) gives the same order in exact
 *   arithmetic and keeps the selection independent of any exp routine.
 *   With a router bias b (moe_layer.router_bias / the bias argument of
 *   moe_route_topk, the sidecar's selection-only bias of the YoungAi page,
 *   section 4.2) the selection ranks key[t][e] = sigmoid32(z[t][e]) + b[e]
 *   (one fp32 addition) instead of z, with the same tie rule; the weights
 *   are unchanged (still from z).  sigmoid32 is this fixed sequence of
 *   IEEE fp32 operations, each rounded on its own:
 *     zc = z clamped to [-80, 80]; t = -zc; kf = t * 0x1.715476p+0;
 *     n = (kf + 0x1.8p+23) - 0x1.8p+23;
 *     r = (t - n * 0x1.62e400p-1) - n * 0x1.7f7d1cp-20;
 *     p = 0x1.6c16c2p-10; then p = p * r + c for c = 0x1.111112p-7,
 *       0x1.555556p-5, 0x1.555556p-3, 0.5, 1, 1 in turn;
 *     e = p * 2^n (2^n exact from its bits); sigmoid32 = 1 / (1 + e).
 *
 * -------------------------------------------------------------------------
 * Weight formats (canonical layout; all fields little-endian; the pages give
 * only the format families, so the byte layouts are this library's own).
 * A "row" is one output channel of a matrix; blocks run along the input
 * dimension K.  A matrix tensor holds n_experts matrices back to back:
 *   [expert][row][K / weights_per_block] blocks.
 * gate/up matrices have d_ff rows and K = d_model; down has d_model rows and
 * K = d_ff.
 *
 * MOE_FMT_IQ2XXS_L -- 256 weights in 66 bytes (2.0625 bits per weight):
 *   bytes 0-1   d, IEEE binary16 (fp16)
 *   for sub-block j = 0..7 (weights 32j .. 32j+31), at byte 2 + 8j:
 *     u32 A_j : byte i (i = 0..3) is the grid row of group g = 4j + i
 *     u32 B_j : bits 7i .. 7i+6 are the 7 stored sign bits of group 4j + i,
 *               bits 28..31 are the 4-bit sub-block scale s_j
 *   group g covers weights 8g .. 8g+7; for element p of the group
 *     mag   = grid[row][p], a value in {1, 3, 5, 7}
 *     neg_p = bit p of the stored sign bits for p < 7; for p = 7 it is the
 *             parity (popcount & 1) of the 7 stored bits, so every group has
 *             an even number of negative weights
 *     w     = d * (2 s_j + 1) * mag * (neg_p ? -1 : +1)
 *   The grid is a caller-supplied uint8 table [256][8] (moe_layer.iq2_grid).
 *
 * MOE_FMT_Q2K_L -- 256 weights in 84 bytes (2.625 bits per weight):
 *   bytes 0-1 d (fp16), bytes 2-3 dmin (fp16),
 *   bytes 4..19  one byte per 16-weight sub-block j: low nibble sc_j,
 *                high nibble m_j,
 *   bytes 20..83 2-bit quants: q_i = (byte[20 + i/4] >> (2 (i % 4))) & 3,
 *   w_i = d * sc_j * q_i - dmin * m_j  with j = i / 16.
 *
 * MOE_FMT_Q4K_L -- 256 weights in 144 bytes (4.5 bits per weight), the
 *   4-bit routed-expert variant (the "ds4f-q4" models of "Running DeepSeek
 *   V4 Flash on an RTX 5080 ...", model section, whose routed Q4_K layout
 *   has the grouped kernels of that page's CUDA section); routed gate/up and
 *   down only, not the shared expert:
 *   bytes 0-1 d (fp16), bytes 2-3 dmin (fp16),
 *   bytes 4..11  one byte per 32-weight sub-block j: low nibble = the low 4
 *                bits of the 6-bit scale sc_j, high nibble = the low 4 bits
 *                of the 6-bit min m_j,
 *   bytes 12..15 byte p (p = 0..3) holds the top two bits of sc_2p (bits
 *                0-1), m_2p (2-3), sc_2p+1 (4-5) and m_2p+1 (6-7),
 *   bytes 16..143 4-bit quants: q_i = (byte[16 + i/2] >> (4 (i % 2))) & 15,
 *   w_i = d * sc_j * q_i - dmin * m_j  with j = i / 32.
 *
 * MOE_FMT_Q8_0_L -- 32 weights in 34 bytes (8.5 bits per weight):
 *   bytes 0-1 d (fp16), bytes 2..33 int8 q[32];  w_i = d * q_i.
 *
 * MOE_FMT_MXFP4_L -- 32 weights in 17 bytes (4.25 bits per weight), the
 *   native MXFP4 routed experts ("Running DeepSeek V4 Flash on an RTX 5080
 *   ...", model section: FP4 values with one shared scale per 32 weights);
 *   routed gate/up and down only, not the shared expert:
 *   byte 0       E8M0 scale exponent s (0..254): scale = 2^(s - 127),
 *   bytes 1..16  E2M1 codes: code_i = (byte[1 + i/2] >> (4 (i % 2))) & 15;
 *                bit 3 is the sign, bits 2..1 the exponent E, bit 0 the
 *                mantissa M: |value| = M/2 for E = 0, else (1 + M/2) 2^(E-1)
 *                (0, 0.5, 1, 1.5, 2, 3, 4, 6),
 *   w_i = 2^(s - 127) * value(code_i).
 *
 * MOE_FMT_VQ12_L / MOE_FMT_VQ13_L -- rows of 8-dimensional vector-quantized
 *   weights, the routed-expert base format of "YoungAi -- DeepSeek V4.1 Flash
 *   on one DGX Spark", section 4.1: every 8 consecutive weights of a row are
 *   one 12-bit (1.5 bits per weight) or 13-bit (1.625) index into the
 *   layer's codebook, times one fp16 gain per row; routed gate/up and down
 *   only.  There are no blocks: a tensor is [expert][row] rows of
 *   2 + 3K/16 (+ K/64 for 13 bits) bytes, K a multiple of 64:
 *   bytes 0-1          gain g (fp16),
 *   next 3K/16 bytes   the low 12 bits of every index as one little-endian
 *                      bit stream: index j occupies stream bits 12j ..
 *                      12j + 11, bit b of the stream being bit b % 8 of
 *                      stream byte b / 8,
 *   next K/64 bytes    (13 bits only) the bit plane: bit j % 8 of plane byte
 *                      j / 8 is bit 12 of index j (the page's "12 + 1"
 *                      layout, which keeps the 12-bit stream's geometry);
 *   w[8j + i] = g * C[idx_j][i]  (i = 0..7).
 *   The codebook C (moe_layer.vq_codebook) is uint8 [n][8]: codeword c is 8
 *   E4M3 bytes (sign bit 7, exponent bits 6..3 with bias 7, mantissa bits
 *   2..0; exponent 0 is subnormal, M/8 * 2^-6; the largest finite value is
 *   448; 0x7f and 0xff are not numbers and must not occur), n = 4096 or 8192
 *   (moe_layer.vq_codes), at least 2^bits for every VQ matrix of the layer.
 *   One codebook serves all experts and the three matrices of a layer (same
 *   page and section), so a layer's routed gate/up and down are either both
 *   VQ formats (of either width) or neither.
 *
 * Device layout (MOE_LAYOUT_DEVICE).  The compute entry points read weights
 * only in this layout, produced from the canonical one by moe_repack (the
 * map is a bijection on bytes and the total size is unchanged).  Every
 * scale field is hoisted into its own plane so that each quant stream is
 * 16-byte aligned and can be read with 128-bit loads.  For a tensor of
 * R = n_experts * rows rows and nb blocks per row:
 *   IQ2XXS_L : plane D  fp16 d[R][nb]                 (2 R nb bytes), then
 *              plane P  payload[R][nb][64]: the 64 bytes after d, unchanged
 *   Q2K_L    : plane DM {fp16 d, fp16 dmin}[R][nb]    (4 R nb bytes), then
 *              plane S  scale bytes[R][nb][16], then
 *              plane Q  quant bytes[R][nb][64]
 *   Q4K_L    : plane DM {fp16 d, fp16 dmin}[R][nb]    (4 R nb bytes), then
 *              plane S  scale bytes[R][nb][12], then
 *              plane Q  quant bytes[R][nb][128]
 *   Q8_0_L   : plane D  fp16 d[R][nb]                 (2 R nb bytes), then
 *              plane Q  int8 q[R][nb][32]
 *   MXFP4_L  : plane S  E8M0 s[R][nb]                 (R nb bytes), then
 *              plane Q  codes[R][nb][16]
 *   VQ12_L   : plane G  fp16 gain[R]                   (2 R bytes), then
 *              plane I  index stream[R][3K/16]
 *   VQ13_L   : planes G and I as for VQ12_L, then
 *              plane B  bit plane[R][K/64]
 *   (nb counts 256-weight superblocks for IQ2XXS_L/Q2K_L/Q4K_L and 32-weight
 *   blocks for Q8_0_L and MXFP4_L.)  Plane offsets follow from R and nb alone.
 * -------------------------------------------------------------------------
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer unless its comment says [host].
 *     moe_layer descriptors are [host] structs read only during the call.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     for a call's data and retains no pointer after a call returns; what it
 *     keeps until the process ends is the fixed scratch array of
 *     moe_layer_forward_noalloc and the GEMM library's handle and plans of
 *     the dense shared expert (moe_expert_ffn_prefill), made on first use.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     MOE_OK means "validated and enqueued on stream", not "finished".  A
 *     kernel fault surfaces at the caller's next synchronisation.
 *   - Arguments are validated before anything is enqueued: a call that
 *     returns an error has launched nothing.  moe_last_error() then gives a
 *     message (thread-local, valid until the next call on that thread).
 *   - T = 0 is a valid no-op for every entry point that takes T.
 *   - Identical inputs give bitwise identical outputs (no floating-point
 *     atomics anywhere; every reduction has a fixed order).  One exception:
 *     a prefill call with a Q8 shared expert recorded under stream capture
 *     before its chunk size's GEMM plans exist runs that expert on the
 *     grouped kernels (other rounding, the same accuracy).
 *   - Size limits: 1 <= n_experts <= 1024; 1 <= top_k <= min(n_experts, 16);
 *     d_model and d_ff are powers of two in [256, 8192]; 0 <= T <= 65536.
 *     Pointers must be 16-byte aligned (torch allocations are 256-byte).
 *   - Numeric preconditions (not checked): activations and router weights
 *     are finite; expert inputs to the down projection (the SwiGLU outputs)
 *     stay inside the fp16 range; caller-supplied idx entries lie in
 *     [0, n_experts) and are distinct within a token.
 *   - Outputs y are fp32 [T][d_model]; idx int32 [T][top_k]; wt fp32
 *     [T][top_k].  Activations x are fp32 or bf16 [T][d_model].
 */
#ifndef QMOE_MOE_H
#define QMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null/misaligned pointer, bad size, bad T/k */
#define MOE_ERR_UNSUPPORTED (-2) /* unknown format, layout, dtype or ABI version */
#define MOE_ERR_WORKSPACE (-3)   /* workspace smaller than moe_workspace_bytes() */
#define MOE_ERR_HIP (-4)         /* the HIP runtime reported an error */

/* Activation dtypes. */
#define MOE_F32 0
#define MOE_BF16 1

/* Weight formats (see the layout notes above). */
#define MOE_FMT_NONE 0
#define MOE_FMT_IQ2XXS_L 1
#define MOE_FMT_Q2K_L 2
#define MOE_FMT_Q8_0_L 3
#define MOE_FMT_Q4K_L 4    /* routed experts only */
#define MOE_FMT_MXFP4_L 5  /* routed experts only */
#define MOE_FMT_VQ12_L 6   /* routed experts only; needs moe_layer.vq_codebook */
#define MOE_FMT_VQ13_L 7   /* routed experts only; needs a codebook of 8192 codewords */

/* Weight layouts. */
#define MOE_LAYOUT_CANONICAL 0
#define MOE_LAYOUT_DEVICE 1

/* Workspace queries. */
#define MOE_OP_ROUTE 0   /* moe_route_topk */
#define MOE_OP_DECODE 1  /* moe_expert_ffn_decode */
#define MOE_OP_PREFILL 2 /* moe_expert_ffn_prefill */
#define MOE_OP_LAYER 3   /* moe_layer_forward, either path */

/* Path choice for moe_layer_forward. */
#define MOE_PATH_AUTO 0    /* decode path for T <= MOE_AUTO_DECODE_MAX_T, else prefill */
#define MOE_PATH_DECODE 1  /* streaming GEMV path (T <= MOE_DECODE_MAX_T only) */
#define MOE_PATH_PREFILL 2 /* bucketing + grouped MFMA GEMM path */
#define MOE_DECODE_MAX_T 8
/* Where MOE_PATH_AUTO switches to prefill: the largest T at which the decode
 * path (in consecutive calls of at most MOE_DECODE_MAX_T tokens) measured
 * faster than one prefill call on the 384-expert, top-6, d=4096, f=2048
 * layer (bench.py, crossover with the caller's routes: 24 tokens 318
 * against 389 us, 32 tokens 424 against 414 us).  Under MOE_PATH_AUTO,
 * moe_layer_forward runs such T in chunks of MOE_DECODE_MAX_T tokens; the
 * workspace covers one chunk. */
#define MOE_AUTO_DECODE_MAX_T 24

/* moe_repack directions. */
#define MOE_REPACK_TO_DEVICE 0
#define MOE_REPACK_TO_CANONICAL 1

/*
 * One MoE layer.  [host] struct; the weight pointers are device pointers to
 * tensors in `layout`.  Compute entry points require MOE_LAYOUT_DEVICE.
 * Routed gate/up and down may each be any of the formats above; the shared
 * expert (if present) uses fmt_shared (IQ2XXS_L, Q2K_L or Q8_0_L) for its
 * three matrices and has d_ff rows in gate/up like the routed experts.
 * iq2_grid is required whenever any matrix is IQ2XXS_L; vq_codebook and
 * vq_codes whenever a routed matrix is VQ12_L or VQ13_L (otherwise they are
 * not read).
 */
typedef struct moe_layer {
  uint32_t abi_version;       /* must equal MOE_ABI_VERSION */
  int32_t n_experts;          /* E */
  int32_t d_model;            /* d: width of x and y */
  int32_t d_ff;               /* f: expert hidden width */
  int32_t top_k;              /* k */
  int32_t fmt_gate_up;        /* format of w_gate and w_up */
  int32_t fmt_down;           /* format of w_down */
  int32_t layout;             /* layout of all weight tensors below */
  const void* w_gate;         /* [E][f rows][d] */
  const void* w_up;           /* [E][f rows][d] */
  const void* w_down;         /* [E][d rows][f] */
  const uint8_t* iq2_grid;    /* uint8 [256][8], values in {1,3,5,7} */
  const float* w_router;      /* fp32 [E][d], expert-major */
  int32_t has_shared;         /* 0 or 1 */
  int32_t fmt_shared;         /* format of the shared expert's matrices */
  const void* s_gate;         /* [f rows][d] */
  const void* s_up;           /* [f rows][d] */
  const void* s_down;         /* [d rows][f] */
  const float* router_bias;   /* nullable fp32 [E]: selection-only router bias */
  const float* down_gain;     /* nullable fp32 [E][d], 16-byte aligned: down gains */
  const uint8_t* vq_codebook; /* E4M3 codewords [vq_codes][8], 16-byte aligned (VQ formats) */
  int32_t vq_codes;           /* 4096 or 8192 (VQ formats) */
} moe_layer;

/* ABI version compiled into the library (== MOE_ABI_VERSION of its header). */
int moe_abi_version(void);

/* [host] Message for the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* [host] Static name of a status code. */
const char* moe_status_string(int status);

/*
 * Bytes of one weight tensor of `fmt` holding n_experts matrices of `rows`
 * rows by K inputs (identical for both layouts).  *bytes is [host].
 */
int moe_matrix_bytes(int32_t fmt, int32_t n_experts, int32_t rows, int32_t K,
                     size_t* bytes);

/*
 * Workspace needed by an entry point (op = MOE_OP_*) for T tokens.  Only
 * n_experts, d_model, d_ff, top_k and has_shared of L are read (for
 * MOE_OP_ROUTE only n_experts and d_model).  *bytes is [host].  The
 * workspace is caller-owned device memory with no required contents; its
 * contents after a call are unspecified.  Calls that overlap in time (on
 * different streams) need separate workspaces.
 */
int moe_workspace_bytes(const moe_layer* L, int32_t T, int32_t op,
                        size_t* bytes);

/*
 * Repack one weight tensor between the canonical and the device layout
 * (direction = MOE_REPACK_TO_DEVICE or MOE_REPACK_TO_CANONICAL).  src and
 * dst are distinct device buffers of moe_matrix_bytes() bytes.  Device-only
 * copies of the weights with aligned quant streams follow the practice of
 * re-aligning expert payloads at load time described on the YoungAi page,
 * section 4.4 (decode, VQ expert kernel).
 */
int moe_repack(int32_t fmt, int32_t n_experts, int32_t rows, int32_t K,
               const void* src, void* dst, int32_t direction, void* stream);

/*
 * Prepare a whole layer for the compute entry points: every weight tensor of
 * `canonical` (layout MOE_LAYOUT_CANONICAL, all other fields as for the
 * compute calls) is converted to the device layout, as moe_repack does, into
 * the buffers the caller put in device_out->w_gate, w_up, w_down (and
 * s_gate, s_up, s_down if the layer has a shared expert), each
 * moe_matrix_bytes() of its tensor, 16-byte aligned, overlapping no source
 * and no other destination.  Then *device_out [host] becomes *canonical with
 * those six pointers and layout = MOE_LAYOUT_DEVICE: the grid, router, bias,
 * gain and codebook arrays have a single layout and are shared, not copied.
 * Everything is validated before the first launch; on an error *device_out
 * is left unchanged.  Device copies with aligned quant streams follow the
 * load-time payload re-alignment of the YoungAi page, section 4.4 (decode,
 * VQ expert kernel); one call per layer keeps the layout internals behind
 * the narrow interface of the ds4 timeline's public header.
 */
int moe_prepare_weights(const moe_layer* canonical, moe_layer* device_out,
                        void* stream);

/*
 * Router and exact top-k (definition at the top of this header).
 *   w_router fp32 [E][d]; bias nullable fp32 [E] (selection on the biased
 *   keys when given); x [T][d] in x_dtype; idx int32 [T][k] (rank order);
 *   wt fp32 [T][k].  Workspace: moe_workspace_bytes(MOE_OP_ROUTE).
 */
int moe_route_topk(const float* w_router, const float* bias, int32_t E,
                   int32_t d, const void* x, int32_t x_dtype, int32_t T,
                   int32_t k, int32_t* idx, float* wt, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * Token-to-expert bucketing of the T*k routes (flat route r = t*k + j with
 * key idx[r]): a stable counting sort.
 *   counts[e]  = number of routes with key e                  int32 [E]
 *   offsets[e] = counts[0] + ... + counts[e-1]; offsets[E] = T*k  [E+1]
 *   perm       = the routes r sorted by (key, r)               int32 [T*k]
 *   pos[r]     = position of route r inside perm               int32 [T*k]
 * idx entries must lie in [0, E).  The result is unique, so it is compared
 * bit for bit.  Grouping the routes of one expert lets one pass over that
 * expert's weights serve all of its tokens (the YoungAi page, section 4.4,
 * describes reading each chosen expert's bits once for a batch of rows).
 */
int moe_bucket(const int32_t* idx, int32_t T, int32_t k, int32_t E,
               int32_t* counts, int32_t* offsets, int32_t* perm,
               int32_t* pos, void* stream);

/*
 * Expert FFN for given routes on the streaming-GEMV (decode) path:
 *   y_t = sum_j wt[t][j] * D_e(silu(G_e x_t) * (U_e x_t)) + shared(x_t),
 *   e = idx[t][j].  Requires T <= MOE_DECODE_MAX_T.
 * Decode reads every selected weight once per token and is bound by HBM
 * bytes (YoungAi page, section 4.4: decoding is memory-bound).
 */
int moe_expert_ffn_decode(const moe_layer* L, const void* x, int32_t x_dtype,
                          int32_t T, const int32_t* idx, const float* wt,
                          float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * The same function on the prefill path: bucketing, then grouped GEMMs that
 * dequantize expert tiles into exact small integers for bf16/fp16 MFMA
 * (the YoungAi page, section 4.4, runs prefill experts on 16-bit matrix
 * units with exact products), then a fixed-order combine.
 *   bucket_out (nullable) receives counts | offsets | perm, int32
 *   [E + (E + 1) + T*k], exactly as moe_bucket defines them.
 * A Q8 shared expert runs as dense fp16 GEMMs (hipBLASLt) on fp16 copies of
 * its weights that each call writes into the workspace (its size counts
 * them: 2 * 3 * d * f bytes more), as the RTX 5080 page's table of launcher
 * variables lists an optional Q8-to-F16 weight conversion.  The first call
 * of a token count (rounded up to a multiple of 64) on a device makes that
 * size's GEMM plans, which may allocate; under stream capture a call whose
 * plans do not exist yet runs the shared expert on the grouped kernels
 * instead (the same function, other rounding), so capture after one eager
 * call of the same size to record the dense path.
 */
int moe_expert_ffn_prefill(const moe_layer* L, const void* x, int32_t x_dtype,
                           int32_t T, const int32_t* idx, const float* wt,
                           float* y, int32_t* bucket_out, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Whole layer: router + top-k + expert FFN (+ shared expert) -> y.
 *   path = MOE_PATH_AUTO | MOE_PATH_DECODE | MOE_PATH_PREFILL.
 *   idx_out / wt_out are nullable [T][k] outputs of the routing step.
 */
int moe_layer_forward(const moe_layer* L, const void* x, int32_t x_dtype,
                      int32_t T, float* y, int32_t* idx_out, float* wt_out,
                      int32_t path, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same computation with the
 * same kernels as moe_layer_forward (bitwise the same outputs), except that
 * a Q8 shared expert on the prefill path runs on the grouped kernels rather
 * than as dense GEMMs (other rounding, the same accuracy); the workspace is
 * a fixed array of MOE_NOALLOC_SCRATCH_BYTES that the library holds in each
 * device's memory from its load until the process ends.  Nothing is
 * allocated by the call (the first call on a device looks up that device's
 * array).  That covers every decode call (T <= 8 at any supported shape)
 * and short prefill chunks; a call that would need more (the workspace of
 * moe_layer_forward on its path, less the dense shared expert's buffers)
 * returns MOE_ERR_WORKSPACE and enqueues nothing.  Every call on one device shares
 * that device's array, and the array keeps the last call's contents (no
 * call needs it cleared): calls that overlap in time on one device (several
 * streams or host threads) race, and must be ordered by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_layer_forward_noalloc(const moe_layer* L, const void* x, int32_t x_dtype,
                              int32_t T, float* y, int32_t* idx_out,
                              float* wt_out, int32_t path, void* stream);

/*
 * Per-kernel timing with HIP events recorded on the stream each kernel is
 * launched on.  Eager use only: do not enable it while a stream is being
 * captured into a graph.  moe_profile_collect synchronises the recorded
 * events and returns, per kernel name, the number of launches and their
 * summed duration in milliseconds.  names is [host] char[max][48].
 */
int moe_profile_enable(int32_t on);
int moe_profile_reset(void);
int moe_profile_collect(int32_t max_kernels, char* names, int64_t* launches,
                        double* total_ms, int32_t* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_MOE_H */
