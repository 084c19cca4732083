/*
 * qgemv.h -- C ABI of the MI355X (gfx950) quantized-weight GEMV library.
 *
 * y = W.x where W stays packed in device memory and is decoded in registers
 * while it streams.  Every pointer argument is a DEVICE pointer owned by the
 * caller; the library keeps no reference to any of them after the call
 * returns and allocates no device memory.  Work is enqueued asynchronously on
 * `stream` (a hipStream_t; NULL means the default stream); a return value of
 * QGEMV_OK means the work was validated and launched, not that it finished.
 *
 * All arguments are validated on the host before any pointer is used; a
 * refused call returns a nonzero qgemv_status, launches nothing and touches
 * no memory.  qgemv_strerror() names the condition.  There is no silent
 * fallback to another implementation.
 *
 * Activations x are f32 [S][I] row-major (S vectors of length I), outputs y
 * are f32 [S][O] row-major and are overwritten.  S ranges over 1..8.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QGEMV_OK = 0,
    QGEMV_E_NULL = 1,      /* a required pointer is NULL                      */
    QGEMV_E_DIMS = 2,      /* S, I, O, E, T or K out of range                 */
    QGEMV_E_GS = 3,        /* group size is not an even number >= 2           */
    QGEMV_E_ALIGN = 4,     /* an f32 / int32 pointer is not 4-byte aligned    */
    QGEMV_E_K256 = 5,      /* I is not a multiple of 256 (MQ4-v2, FWHT-256)   */
    QGEMV_E_IDS = 6,       /* expert strides too small for one expert         */
    QGEMV_E_WORKSPACE = 7, /* workspace NULL or smaller than required         */
    QGEMV_E_HIP = 8        /* the HIP runtime reported an error at launch     */
} qgemv_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *qgemv_strerror(int status);

/* Library version, e.g. "0.1.0" (static string). */
const char *qgemv_version(void);

/* Largest S (vectors per call) the GEMV entry points accept. */
#define QGEMV_MAX_S 8

/*
 * Grouped int4 ("fmt=4"): colibri PR #457 "metal: grouped-int4 (fmt=4) GEMV
 * support", sections 1 and 3.
 *   w       u8  [O][(I+1)/2]  two unsigned nibbles per byte; column 2k is the
 *                             low nibble of byte k, column 2k+1 the high one;
 *                             for odd I the last high nibble is ignored
 *   scales  f32 [O][ceil(I/gs)]  weight (o,i) = (nibble - 8) * scales[o][i/gs]
 *   x       f32 [S][I],  y f32 [S][O]
 *   gs      even, 2 .. 2^24; any I >= 1 (a last partial group is allowed)
 * Rows whose bytes are 16-byte aligned (I % 32 == 0, w and x 16-byte
 * aligned) with gs % 32 == 0 take the streaming kernel (S > 4 runs in groups
 * of up to 4 vectors, each group streaming the weights once).  It stages x
 * per 32 columns as a 22-bit shared-exponent fixed point and forms exact
 * integer nibble x digit sums, accumulated in f32; activations holding an
 * infinity or NaN, or whose estimated error in that form would exceed
 * 3e-6 relative on y (a large value next to much smaller ones), are
 * multiplied per element in f32 instead.  Every other valid shape takes a
 * slower general kernel with the same result definition.
 */
int qgemv_i4g(const void *w, const float *scales, const float *x, float *y,
              int S, int I, int O, int gs, void *stream);

/*
 * Grouped int4 for many tokens at once (prompt prefill): the same product as
 * qgemv_i4g, Y[S][O] = X[S][I] . W^T, for any S >= 1, on the matrix cores
 * (f32 MFMA: weights decoded to f32 as (q - 8) * s, products and sums in
 * f32).  colibri PR #457 "metal: grouped-int4 (fmt=4) GEMV support",
 * sections 1 and 3 (format); the pages route many-token products to a
 * separate matrix-unit GEMM path from a token-count threshold.
 *   w, scales, gs  as qgemv_i4g;  x f32 [S][I], y f32 [S][O] (overwritten)
 * Fast path: I % 32 == 0, gs % 32 == 0, w 4-byte and x 16-byte aligned;
 * other shapes run the GEMV eight tokens per launch.
 */
int qgemv_i4g_prefill(const void *w, const float *scales, const float *x, float *y, int S,
                      int I, int O, int gs, void *stream);

/*
 * fp8-e4m3 with 128x128 block scales ("fmt=7"): colibri PR #528 "fmt=7:
 * fp8-e4m3-b128 passthrough weight format", section "Design".
 *   w          u8  [O][I]    OCP E4M3-FN codes (bias 7, subnormals, +-0;
 *                            0x7F / 0xFF are NaN and poison their row)
 *   scale_inv  f32 [ceil(O/128)][ceil(I/128)] row-major block order;
 *              weight (o,i) = e4m3(w[o][i]) * scale_inv[o/128][i/128]
 *              (a multiply, whatever the name says)
 *   x          f32 [S][I],  y f32 [S][O]
 * Rows with I % 16 == 0 and 16-byte aligned w and x take the streaming
 * kernel (vectors that do not fit its LDS staging together are staged in
 * column phases inside the launch); other shapes a general kernel.
 */
int qgemv_fp8b128(const void *w, const float *scale_inv, const float *x,
                  float *y, int S, int I, int O, void *stream);

/*
 * fp8-e4m3 with UE8M0 block scales: the same weight geometry as
 * qgemv_fp8b128 with one scale byte per 128x128 block holding a power-of-two
 * exponent (colibri PR #528, section "Design": dtype F8_E8M0, one byte per
 * block).  The page names the dtype without its decode; the reading taken is
 * the dtype's definition: scale = 2^(e - 127), e = 255 is NaN.
 *   scale_e8m0  u8 [ceil(O/128)][ceil(I/128)] row-major block order;
 *               weight (o,i) = e4m3(w[o][i]) * 2^(scale_e8m0[o/128][i/128] - 127)
 *   w, x, y     as qgemv_fp8b128
 */
int qgemv_fp8b128_ue8m0(const void *w, const uint8_t *scale_e8m0, const float *x, float *y,
                        int S, int I, int O, void *stream);

/*
 * MQ4-v2: hipfire "MQ4 V2" page, sections 2 and 4.
 *   w      u8 [O][I/256][136]; per 256-weight group, little-endian:
 *          bytes 0..3  dword: fp16 scale (low 16 bits), fp16 zero (high 16)
 *                      of weights 0..127,
 *          bytes 4..7  the same pair for weights 128..255,
 *          bytes 8..135  128 payload bytes, weight j = nibble j (byte j/2,
 *                      low nibble for even j);  weight = q * scale + zero
 *   x_rot  f32 [S][I] activations already rotated into the weights' space
 *          (qgemv_fwht256),  y f32 [S][O];  I % 256 == 0
 */
int qgemv_mq4v2(const void *w, const float *x_rot, float *y, int S, int I,
                int O, void *stream);

/*
 * MQ4 v1 (qt=13) and MQ4C pad (qt=45): hipfire "MQ4 V2", sections 1b and 1e.
 * The same 136-byte groups and payload as qgemv_mq4v2 (128 nibble bytes at
 * [8..136), weight j = nibble j, low nibble first; w = q * scale + zero),
 * with one header for all 256 weights of a group:
 *   v1    f32 scale at byte 0, f32 zero at byte 4
 *   MQ4C  fp16 scale (low half) and fp16 zero (high half) of the dword at
 *         byte 0; bytes 4..7 are the zero pad and are not read
 * x_rot, y, S, I, O and refusals as qgemv_mq4v2.
 */
int qgemv_mq4v1(const void *w, const float *x_rot, float *y, int S, int I, int O,
                void *stream);
int qgemv_mq4c(const void *w, const float *x_rot, float *y, int S, int I, int O,
               void *stream);

/*
 * MQ4-v2 encoder: hipfire "MQ4 V2", section 3.  W f32 [O][I] holds weights
 * already in the rotated space (I % 256 == 0, 16-byte aligned); w_out
 * receives O * (I/256) * 136 bytes (8-byte aligned) in the qgemv_mq4v2
 * layout.  Per 128-weight half: lo, hi = min, max; step = (hi - lo) / 15 in
 * f32; the stored scale and zero are the fp16 (nearest even) roundings of
 * step and lo; each code is q = clamp(rint((w - z) / s), 0, 15) against the
 * stored, f16-rounded s and z (so decoding reproduces the encoder's own
 * reconstruction).  A stored scale of 0 (a constant half, or a step below
 * fp16's range) gives q = 0; an extreme of -0 counts as +0.  W must be
 * finite.
 */
int qgemv_mq4v2_encode(const float *W, void *w_out, int I, int O, void *stream);

/*
 * MQ4-v2 GEMV on unrotated activations: the FWHT-256 pre-rotation below
 * (hipfire "MQ4 V2", section 1) fused into the GEMV (sections 2 and 4),
 *     y = W . x_rot,  x_rot = (1/16) H256 (signs (.) x) per 256-column block,
 * with x_rot bit-identical to qgemv_fwht256's output and y as qgemv_mq4v2
 * computes it from that x_rot, in one launch.
 *   w      as qgemv_mq4v2, 8-byte aligned;  x f32 [S][I], 16-byte aligned;
 *   signs  int8 [I] (each +1 or -1), 8-byte aligned;  y f32 [S][O];
 *   I % 256 == 0.
 * Refusals: QGEMV_E_ALIGN for other alignments, QGEMV_E_DIMS when one
 * vector's staged activations exceed the LDS (I above 40000); rotate with
 * qgemv_fwht256 and call qgemv_mq4v2 for those.
 * Speed: every workgroup rotates all S vectors itself, so the fused call
 * pays off for few vectors only.  At 8192 x 8192: S = 1 9.5 us against 10.9
 * us for the two calls, S = 2 13.2 against 14.0, S = 3 equal, S = 4 29.9
 * against 22.7 (there the two calls are faster).
 */
int qgemv_mq4v2_rot(const void *w, const float *x, const int8_t *signs, float *y, int S,
                    int I, int O, void *stream);

/*
 * FWHT-256 pre-rotation of activations for MQ4 weights (hipfire "MQ4 V2",
 * section 1: the weights are FWHT-256 rotated with per-element signs).
 * Per 256-element block b of each vector:
 *     x_rot[b] = (1/16) * H256 * (signs[b] (.) x[b])
 * with H256 the Sylvester Hadamard matrix H[i][j] = (-1)^popcount(i&j).
 *   x f32 [S][I], signs int8 [I] (each +1 or -1), x_rot f32 [S][I];
 *   I % 256 == 0; x and x_rot must be 16-byte aligned and may be the same
 *   buffer (in-place rotation).
 */
int qgemv_fwht256(const float *x, const int8_t *signs, float *x_rot, int S,
                  int I, void *stream);

/*
 * Router top-k that feeds qgemv_moe_topk: regolith audit "phase 0 + phase 2
 * m5 air validation", section 2.1 (columns at or past the expert count are
 * masked out of the softmax; the logits row stride may exceed it) and
 * section 2.2 (the gates are the picked experts' probabilities renormalised
 * over the picked set).
 *   logits  f32 [T][ld], experts 0..E-1 of each row valid (ld >= E); finite
 *   ids     int32 [T][K]: the K most probable experts, most probable first;
 *           equal probabilities rank by the lower expert index
 *   gates   f32 [T][K]: g_k = exp(l_k - m) / sum over picks j of exp(l_j - m)
 *   1 <= E <= 1024, 1 <= K <= min(E, 64)
 */
int qgemv_router_topk(const float *logits, int T, int E, int ld, int K, int32_t *ids,
                      float *gates, void *stream);

/*
 * Routed experts over grouped-int4 matrices: regolith audit "phase 0 +
 * phase 2 m5 air validation", section 2.2 (the gates are the selection
 * probabilities renormalised over the selected experts) and colibri PR #457,
 * section 4 (routed experts are grouped-int4 matrices).
 *   y[t][o] = sum_k gates[t][k] * (W_{ids[t][k]} . x[t])[o]
 * summed over k in ascending order (deterministic; no atomics).
 *   w        expert e's packed weights (layout as qgemv_i4g, [O x I]) start
 *            at byte e*w_stride;  scales  expert e's f32 scales start at
 *            element e*s_stride;  E experts
 *   ids      int32 [T][K] device array; an id outside [0, E) makes row t of
 *            y NaN (it is never dereferenced) and sets a flag in the
 *            workspace (qgemv_moe_topk_error)
 *   gates    f32 [T][K],  x f32 [T][I],  y f32 [T][O] (overwritten)
 *   T in 1..8, K in 1..64, gs even 2 .. 2^24
 *   workspace  device scratch of at least qgemv_moe_topk_workspace(T, K, O)
 *              bytes, 4-byte aligned: the per-token error flags; its
 *              contents are overwritten.
 * Each distinct expert of the call is streamed once: every token that
 * selected it is multiplied from the same weight registers (an id repeated
 * within a token is counted per slot).  When T * K > 64, or the tokens'
 * staged activations exceed the LDS (about seven of 7168 columns), the
 * tokens run in groups and an expert shared across groups is read once per
 * group.  The routing never leaves the device.
 */
size_t qgemv_moe_topk_workspace(int T, int K, int O);
int qgemv_moe_topk(const void *w, const float *scales, long long w_stride,
                   long long s_stride, int E, const int32_t *ids,
                   const float *gates, int T, int K, const float *x, float *y,
                   int I, int O, int gs, void *workspace, size_t ws_bytes,
                   void *stream);
/* Copies the error flag of the last qgemv_moe_topk that used `workspace`
 * into *flag (host int; 0 = all ids in range), synchronising `stream`. */
int qgemv_moe_topk_error(const void *workspace, int *flag, void *stream);

/*
 * qgemv_moe_topk for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid it): the same
 * arguments without the workspace, the same kernels and the same y.  The
 * per-token error flags go to a fixed 256-byte device array of the library
 * (one per GPU, held until the process ends) and are not readable through
 * the ABI; an out-of-range id still makes its token's row of y NaN.  No
 * host or device memory is allocated.  Calls that overlap on one GPU share
 * that array and race on the flags (y is unaffected).  Refusals as
 * qgemv_moe_topk; QGEMV_E_WORKSPACE if the flags would not fit the array
 * (never for T <= 8).
 */
int qgemv_moe_topk_noalloc(const void *w, const float *scales, long long w_stride,
                           long long s_stride, int E, const int32_t *ids, const float *gates,
                           int T, int K, const float *x, float *y, int I, int O, int gs,
                           void *stream);

/*
 * Decode-only entry points: write the decoded f32 weights W[O][I], each the
 * format's definition rounded once to f32 -- grouped int4 (q - 8) * s
 * (colibri PR #457, section 3), fp8 e4m3 * block scale (colibri PR #528,
 * section "Design"), MQ4 q * scale + zero (hipfire "MQ4 V2", sections 1b,
 * 1e and 4) -- with the device's nibble / fp8 / fp16 converters.  They are
 * the bit-exact decode check of those converters and layouts.  The 4-bit
 * GEMVs do not form these values: they multiply q - 8 (packed nibbles XOR 8)
 * with fixed-point activation digits; their decode is checked through
 * one-hot activations instead.  Arguments as the GEMV of the same format.
 */
int qgemv_dequant_i4g(const void *w, const float *scales, float *W, int I,
                      int O, int gs, void *stream);
int qgemv_dequant_fp8b128(const void *w, const float *scale_inv, float *W,
                          int I, int O, void *stream);
int qgemv_dequant_fp8b128_ue8m0(const void *w, const uint8_t *scale_e8m0, float *W, int I,
                                int O, void *stream);
int qgemv_dequant_mq4v2(const void *w, float *W, int I, int O, void *stream);
int qgemv_dequant_mq4v1(const void *w, float *W, int I, int O, void *stream);
int qgemv_dequant_mq4c(const void *w, float *W, int I, int O, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
