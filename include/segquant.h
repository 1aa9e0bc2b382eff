/*
 * segquant.h -- C ABI of libsegquant: the DualScale x SegLinear W8A8 linear
 * layer on AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization
 *        Framework for Diffusion Models", paper notes (papernotes.org,
 *        CVPR 2026): "SegLinear" (output- and input-segmented patterns and
 *        their equations), "DualScale" (split, scales, reconstruction,
 *        hardware-native execution), framework table (AMax calibrator).
 *   [P2] "SegQuant", project page (hliangzhao.me/works/segquant.html):
 *        section 2 (SegLinear equations), section 3 (polarity-aware
 *        quantisation Q_dual, s+ and s-, reconstruction, one batched launch
 *        with a fused epilogue).
 *
 * What the layer computes (Y = X W, X in R^{M x K}, W in R^{K x N}):
 *   split      X+ = max(X,0), X- = min(X,0)                     [P1 DualScale]
 *   scales     s+ = max(X)/127, s- = |min(X)|/128, per K-segment  [P2 s.3]
 *   quantise   q+ = clamp(rne(fp32(x+ * inv+)), 0, 127)
 *              q- = clamp(rne(fp32(x- * inv-)), -128, 0)          [P2 s.3 Q_dual]
 *   products   A+_i = q+_i W_q,i and A-_i = q-_i W_q,i (int32, exact) over
 *              the K-range of segment i, both halves against one W tile
 *   epilogue   y = sum_i w_scale[i][n] (s+_i A+_i + s-_i A-_i), fp32,
 *              stored bf16 (round to nearest even)      [P1/P2 reconstruction]
 * Output-segmented layers [P1 SegLinear pattern one] differ only in their
 * weight-scale groups, which w_scale expresses per column; input-segmented
 * layers [P1 SegLinear pattern two] carry one (s+, s-) pair and one weight
 * scale group per K-segment.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory and keeps no pointer after the
 *     call returns.  The only scratch memory is the optional, caller-owned
 *     workspace of segquant_gemm_w8a8_seg (its size from
 *     segquant_gemm_workspace_bytes).
 *   - Segment lists are HOST arrays (offset[n], width[n]), read only during
 *     the call: offsets start at 0, are contiguous, widths are positive and
 *     sum to the segmented dimension.  Every K-segment boundary except the
 *     end of K is a multiple of 64 (one MFMA K-step); n <= SEGQ_MAX_KSEG.
 *   - Activation scale table: DEVICE fp32 [4][n_kseg], rows
 *     s_pos, s_neg, inv_pos, inv_neg (segquant_calibrate_amax writes it).
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major with a
 *     leading dimension (elements) >= the row length.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; no call synchronises the host.
 *   - Every call returns SEGQ_OK or a negative status.  All argument checks
 *     run before any HIP call, so an invalid call enqueues nothing and
 *     changes no buffer.  segquant_last_error() gives the thread's detail
 *     text for its last failing call.  Nothing is thrown, printed or aborted.
 *   - The library is thread-safe; its only state is that thread-local text.
 *   - Inputs must not hold NaN.  +-Inf saturates to the end of its half's
 *     code range when that half's inverse scale is nonzero; an infinite
 *     value in a half whose scale is zero is outside the contract.
 */
#ifndef SEGQUANT_H
#define SEGQUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SEGQ_OK 0
#define SEGQ_ERR_NULL (-1)        /* a required pointer is NULL */
#define SEGQ_ERR_SHAPE (-2)       /* a size or leading dimension is invalid */
#define SEGQ_ERR_SEGMENTS (-3)    /* a segment list is malformed */
#define SEGQ_ERR_ALIGN (-4)       /* a size, boundary or pointer is misaligned */
#define SEGQ_ERR_UNSUPPORTED (-5) /* valid but beyond this library's limits */
#define SEGQ_ERR_HIP (-6)         /* a HIP launch or runtime call failed */

/* Limits. */
#define SEGQ_MAX_KSEG 128
/* Widest K-segment whose int32 products cannot overflow:
 * floor((2^31 - 1) / (128 * 127)). */
#define SEGQ_MAX_KSEG_WIDTH 132104

/* Layouts of a quantised activation. */
#define SEGQ_Q_SIGNED 0 /* one int8 plane [M][ld_q] holding q+ + q- (the
                           halves have disjoint support, so this is lossless:
                           q+ = max(Q,0), q- = min(Q,0)) */
#define SEGQ_Q_PLANES 1 /* two int8 planes [2][M][ld_q]: q+ then q- */

/* Flags for segquant_gemm_w8a8_seg. */
#define SEGQ_GEMM_AUTO 0u        /* pick the kernel from the shape */
#define SEGQ_GEMM_FORCE_TILE 1u  /* the MFMA tile kernel, any M */
#define SEGQ_GEMM_FORCE_SMALLM 2u /* the weight-streaming kernel (M <= 16) */
#define SEGQ_GEMM_FUSED_QUANT 4u  /* quantise bf16 input inside the GEMM kernel
                                     even when a workspace is given */
#define SEGQ_GEMM_SINGLE_SCALE 8u /* single-scale W8A8: see segquant_gemm_w8a8_seg */
#define SEGQ_GEMM_W4 16u          /* w_packed holds 4-bit weights (segquant_quantize_weight_w4) */

/* Kernel choices reported by segquant_gemm_kernel_for. */
#define SEGQ_KERNEL_TILE 1
#define SEGQ_KERNEL_SMALLM 2

/*
 * segquant_calibrate_amax -- AMax calibration of the static activation
 * scales [P1 framework table, AMax; P1 DualScale scale equation; P2 s.3].
 * For each K-segment i, over X[:, segment i]:
 *   mx = max(0, max x), mn = min(0, min x)
 *   s_pos = mx/127, s_neg = |mn|/128, inv_pos = 127/mx, inv_neg = 128/|mn|
 * each quotient formed in fp64 and rounded once to fp32; an inverse whose
 * range is zero is 0 (that half then quantises to all zeros).
 *   x_bf16      device bf16 [M][ld_x]
 *   act_scales  device fp32 [4][n_kseg] (output; also used as the reduction
 *               buffer while the call runs)
 * Three short launches on `stream`.  M may be 0 (all scales become 0).
 */
int segquant_calibrate_amax(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                            int32_t n_kseg, const int32_t *kseg_offset,
                            const int32_t *kseg_width, float *act_scales, void *stream);

/*
 * segquant_calibrate_amax_single -- the single-scale baseline's calibration
 * [P2 deployment-cost table, INT8 baseline row; P1 limitations section:
 * DualScale doubles the products, so it may be enabled only for layers whose
 * activations are polarity-asymmetric].  Per K-segment i, one symmetric
 * range a = max(max x, -min x) over X[:, segment i]:
 *   s = a/127, inv = 127/a (fp64 quotients rounded once to fp32; 0 when a = 0)
 * written into BOTH halves of the table (s_pos = s_neg = s, inv_pos =
 * inv_neg = inv).  With such a table the DualScale quantiser yields the
 * plain symmetric codes clamp(rne(fp32(x * inv)), -127, 127), and the layer
 * equals textbook per-segment W8A8; SEGQ_GEMM_SINGLE_SCALE then computes it
 * with one product instead of two.  Arguments and launches as
 * segquant_calibrate_amax.
 */
int segquant_calibrate_amax_single(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                                   int32_t n_kseg, const int32_t *kseg_offset,
                                   const int32_t *kseg_width, float *act_scales, void *stream);

/*
 * segquant_quantize_dualscale -- polarity split and dual-scale quantisation
 * [P1 DualScale split and quantisation scheme; P2 s.3 Q_dual] of a bf16
 * activation, HBM to HBM, for the pre-quantised GEMM path.
 *   x_bf16      device bf16 [M][ld_x]
 *   act_scales  device fp32 [4][n_kseg] (reads the inv rows)
 *   q_out       device int8: SEGQ_Q_SIGNED -> [M][ld_q];
 *               SEGQ_Q_PLANES -> [2][M][ld_q] (q+ plane, then q- plane)
 * One launch.  M may be 0.
 */
int segquant_quantize_dualscale(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                                int32_t n_kseg, const int32_t *kseg_offset,
                                const int32_t *kseg_width, const float *act_scales,
                                int8_t *q_out, int64_t ld_q, int32_t q_layout, void *stream);

/* Activations for segquant_activate_quantize. */
#define SEGQ_ACT_SILU 1 /* z / (1 + exp(-z)) */
#define SEGQ_ACT_GELU 2 /* z/2 * (1 + erf(z / sqrt(2))), the exact form */

/*
 * segquant_activate_quantize -- the producer fused with the quantisation:
 * the SiLU or GELU whose outputs carry the polarity asymmetry DualScale is
 * for [P1 DualScale motivation; P2 section 3], applied to a bf16
 * pre-activation and quantised in the same pass, so the activated bf16 X
 * never round-trips through HBM.  Per element:
 *   x = bf16_rne(act(z))   with act evaluated in fp32 (library expf;
 *                          GELU as z/2 erfc(-z/sqrt 2), which is accurate
 *                          for negative z)
 *   codes of x exactly as segquant_quantize_dualscale
 *   z_bf16      device bf16 [M][ld_z]
 *   act_kind    SEGQ_ACT_SILU or SEGQ_ACT_GELU
 *   act_scales  device fp32 [4][n_kseg], calibrated on x (may be NULL when
 *               q_out is NULL)
 *   q_out       optional device int8, layout and ld_q as for
 *               segquant_quantize_dualscale
 *   x_out       optional device bf16 [M][ld_xo]: x itself (for the offline
 *               calibration, or for another consumer of the bf16 values)
 * At least one of q_out and x_out.  One launch; M may be 0.
 */
int segquant_activate_quantize(const uint16_t *z_bf16, int64_t M, int64_t K, int64_t ld_z,
                               int32_t act_kind, int32_t n_kseg, const int32_t *kseg_offset,
                               const int32_t *kseg_width, const float *act_scales,
                               int8_t *q_out, int64_t ld_q, int32_t q_layout, uint16_t *x_out,
                               int64_t ld_xo, void *stream);

/*
 * segquant_weight_packed_bytes -- size of the packed int8 weight for a
 * K x N layer: K*N bytes when K % 64 == 0 and N % 16 == 0, else 0.
 * The packed layout is tiles of 64 (k) x 16 (n) bytes, 1 KiB each, stored
 * n-tile major: tile (nt, kt) at byte (nt * (K/64) + kt) * 1024; inside a
 * tile, byte (g*16 + j)*16 + b holds W_q[kt*64 + g*16 + b][nt*16 + j]
 * (g in 0..3, j in 0..15, b in 0..15): the operand order of the int8
 * 16x16x64 matrix-core instruction, one 16-byte row per lane.
 */
size_t segquant_weight_packed_bytes(int64_t K, int64_t N);

/*
 * segquant_quantize_weight -- symmetric int8 weight quantisation per group
 * [P1 SegLinear, both patterns: each segment quantised on its own; P2 s.2],
 * packed for the kernels.  The group of (k, n) is (K-segment of k) x
 * (N-segment of n), or (K-segment of k) x {n} when per_column != 0 (then
 * the N-segment list is ignored and may be NULL).  Per group:
 *   a = max |w|, s_w = a/127 and inv_w = 127/a (fp64 quotients rounded
 *   once to fp32; inv_w = 0 when a = 0),
 *   w_q = clamp(rne(fp32(w * inv_w)), -127, 127)
 *   w          device fp32 [K][ld_w] (Y = X W)
 *   w_packed   device int8, segquant_weight_packed_bytes(K, N) bytes
 *   w_scale    device fp32 [n_kseg][N]: the s_w of the group holding
 *              (K-segment i, column n) -- the epilogue's per-column scale
 * Requires K % 64 == 0, N % 16 == 0.  Offline; four short launches.
 */
int segquant_quantize_weight(const float *w, int64_t K, int64_t N, int64_t ld_w,
                             int32_t n_kseg, const int32_t *kseg_offset,
                             const int32_t *kseg_width, int32_t n_nseg,
                             const int32_t *nseg_offset, const int32_t *nseg_width,
                             int32_t per_column, int8_t *w_packed, float *w_scale,
                             void *stream);

/*
 * segquant_quantize_weight_w4 -- the 4-bit weights of W4A8, the pages'
 * second precision [P2 deployment-cost table, SegQuant-4 row; P1
 * experiments, W4A8], with the same groups as segquant_quantize_weight:
 *   s_w = a/7, inv_w = 7/a, w_q = clamp(rne(fp32(w * inv_w)), -7, 7)
 * Packed in 512-byte tiles that mirror the int8 ones (tile (nt, kt) at byte
 * (nt * K/64 + kt) * 512; lane l = g*16 + j of a tile owns bytes l*8 .. l*8+7
 * holding W_q[kt*64 + g*16 + b][nt*16 + j], b = 0..15, as codes + 8 in
 * nibbles: byte i (i = 0..3) of the first dword holds b = i in its low and
 * b = i + 4 in its high nibble, byte i of the second dword b = 8 + i and
 * b = 12 + i).  segquant_weight_packed_bytes_w4(K, N) = K*N/2 bytes.
 * Arguments, w_scale and launches as segquant_quantize_weight.
 */
int segquant_quantize_weight_w4(const float *w, int64_t K, int64_t N, int64_t ld_w,
                                int32_t n_kseg, const int32_t *kseg_offset,
                                const int32_t *kseg_width, int32_t n_nseg,
                                const int32_t *nseg_offset, const int32_t *nseg_width,
                                int32_t per_column, int8_t *w_packed, float *w_scale,
                                void *stream);

size_t segquant_weight_packed_bytes_w4(int64_t K, int64_t N);

/* segquant_unpack_weight_w4 -- 4-bit packed weights -> int8 codes
 * [K][ld_w] row-major (values in [-7, 7]).  For inspection and tests. */
int segquant_unpack_weight_w4(const int8_t *w_packed, int64_t K, int64_t N, int8_t *w_kn,
                              int64_t ld_w, void *stream);

/*
 * segquant_unpack_weight -- inverse of the packing: w_packed -> device int8
 * W_q [K][ld_w] row-major.  For inspection and tests.  One launch.
 */
int segquant_unpack_weight(const int8_t *w_packed, int64_t K, int64_t N, int8_t *w_kn,
                           int64_t ld_w, void *stream);

/*
 * segquant_gemm_w8a8_seg -- the DualScale x SegLinear W8A8 linear layer in
 * ONE launch [P1 DualScale hardware-native execution; P2 s.3: both polarity
 * products in one batched launch, combined in a fused epilogue]:
 *   y[m][n] = bf16( sum_i w_scale[i][n] * (s_pos[i]*A+_i[m][n]
 *                                          + s_neg[i]*A-_i[m][n]) )
 * with A+-_i the exact int32 products of the quantised halves over K-segment
 * i against W_q (both halves read one W tile).  The activation is either
 *   x_bf16 != NULL: bf16 [M][ld_x], quantised inside the kernel with the inv
 *                   rows of act_scales (xq must be NULL), or
 *   xq != NULL:     the output of segquant_quantize_dualscale with the same
 *                   act_scales, layout q_layout, leading dimension ld_q.
 *   w_packed   from segquant_quantize_weight (K x N)
 *   w_scale    device fp32 [n_kseg][N]
 *   act_scales device fp32 [4][n_kseg]
 *   y_bf16     device bf16 [M][ld_y] (output)
 *   acc_debug  optional device int32 [2][n_kseg][M][N]: when not NULL the
 *              kernel also stores every per-segment accumulator A+_i
 *              (plane 0) and A-_i (plane 1); NULL in production.
 *   workspace  optional device scratch of workspace_bytes bytes, 16-byte
 *              aligned, owned by the caller.  With bf16 input and at least
 *              segquant_gemm_workspace_bytes() bytes, the call may quantise
 *              X into it first (the segquant_quantize_dualscale kernel,
 *              signed codes, ld_q = K) and run the GEMM from the codes: two
 *              launches, the same results.  Its contents are undefined
 *              afterwards; calls that share one workspace must be ordered
 *              (same stream).  NULL, or fewer bytes than asked for: one
 *              fused launch.
 *   flags      SEGQ_GEMM_AUTO, or force one kernel for testing
 *              (SEGQ_GEMM_FUSED_QUANT: never use the workspace), or'ed with
 *              SEGQ_GEMM_SINGLE_SCALE: single-scale W8A8.  Only the + half
 *              of act_scales is read: each element is quantised with inv_pos
 *              of its segment (code in [-128, 127]) and
 *                y[m][n] = bf16( sum_i w_scale[i][n] * s_pos[i] * A_i[m][n] )
 *              with A_i the exact int32 product of the signed codes: one
 *              product per element instead of two.  With a table from
 *              segquant_calibrate_amax_single this is the DualScale formula
 *              of that table.  acc_debug then receives A_i in plane 0 and
 *              plane 1 is not written.  Takes bf16 or SEGQ_Q_SIGNED input
 *              (SEGQ_Q_PLANES: SEGQ_ERR_UNSUPPORTED).
 *              SEGQ_GEMM_W4: w_packed is from segquant_quantize_weight_w4
 *              (W4A8; same formula with the 4-bit codes).  The small-M
 *              streaming kernel reads the 4-bit tiles directly (half the
 *              weight bytes); every other shape first widens them to int8
 *              tiles in the workspace, which must then hold K*N bytes (plus
 *              the quantise-first bytes; segquant_gemm_workspace_bytes with
 *              the same flags gives the total), else SEGQ_ERR_UNSUPPORTED.
 * Requires K % 64 == 0, N % 16 == 0, every K-segment width <=
 * SEGQ_MAX_KSEG_WIDTH (each segment's int32 sums stay below 2^31; K itself
 * has no further bound), 16-byte aligned tensor pointers, ld_x and ld_q
 * multiples of 8 and 16 elements, ld_y a multiple of 2.  M may be 0 (no
 * launch).  SEGQ_GEMM_FORCE_SMALLM requires M <= 16.
 */
int segquant_gemm_w8a8_seg(int64_t M, int64_t N, int64_t K,
                           const uint16_t *x_bf16, int64_t ld_x,
                           const int8_t *xq, int64_t ld_q, int32_t q_layout,
                           const int8_t *w_packed, const float *w_scale,
                           int32_t n_kseg, const int32_t *kseg_offset,
                           const int32_t *kseg_width, const float *act_scales,
                           uint16_t *y_bf16, int64_t ld_y, int32_t *acc_debug,
                           void *workspace, size_t workspace_bytes,
                           uint32_t flags, void *stream);

/*
 * segquant_gemm_w8a8_seg_noalloc -- segquant_gemm_w8a8_seg without a
 * workspace and without any device allocation, for callers that cannot
 * allocate: code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, validation, results and errors are those of
 * segquant_gemm_w8a8_seg (same kernels, bit-identical outputs), less the
 * workspace.
 *
 * What the ordinary call would use a workspace for (the quantise-first int8
 * codes, M*K bytes; the int8 widening of 4-bit weights, K*N bytes) comes from
 * a device array of SEGQ_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends (its address is looked up on
 * the first call on each device).  Quantise-first codes that would not fit
 * are replaced by the fused launch (same codes and products); a required
 * widening that does not fit is refused with SEGQ_ERR_UNSUPPORTED before any
 * HIP call.  All calls on one GPU share its array: calls that overlap on one
 * GPU race, so order them (one stream).  The call makes no hipMalloc or
 * hipFree and calls no allocating library routine.
 */
#define SEGQ_NOALLOC_SCRATCH_BYTES (64u << 20)
int segquant_gemm_w8a8_seg_noalloc(int64_t M, int64_t N, int64_t K,
                                   const uint16_t *x_bf16, int64_t ld_x,
                                   const int8_t *xq, int64_t ld_q, int32_t q_layout,
                                   const int8_t *w_packed, const float *w_scale,
                                   int32_t n_kseg, const int32_t *kseg_offset,
                                   const int32_t *kseg_width, const float *act_scales,
                                   uint16_t *y_bf16, int64_t ld_y, int32_t *acc_debug,
                                   uint32_t flags, void *stream);

/*
 * segquant_gemm_workspace_bytes -- the workspace with which
 * segquant_gemm_w8a8_seg, given bf16 input of this shape and these
 * K-segments, quantises first (M * K bytes), or 0 when it quantises inside
 * the GEMM kernel anyway.  The large-M kernel re-quantises each activation
 * tile once per output column tile; from six column tiles on, one separate
 * quantisation pass costs less.  On invalid arguments returns 0 and sets
 * segquant_last_error().
 */
size_t segquant_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t n_kseg,
                                     const int32_t *kseg_offset, const int32_t *kseg_width,
                                     uint32_t flags);

/*
 * segquant_gemm_halves -- which halves a layer needs, from its static scales
 * ([P1] "SegQuant" notes, DualScale section, and its limitations: the
 * negative half exists for polarity-asymmetric activations; with no negative
 * values its term of the reconstruction vanishes).  Host-only: no GPU work.
 *   act_scales_host  HOST fp32 [4][n_kseg], a copy of the table written by
 *                    segquant_calibrate_amax (the scales are static, so the
 *                    copy is taken once, after calibration)
 * Returns SEGQ_GEMM_SINGLE_SCALE when s_neg and inv_neg are 0 in every
 * K-segment (the calibration data held no negative value), else 0.  Or'ed
 * into the flags of segquant_gemm_w8a8_seg with this same table, the layer
 * then runs one product per element instead of two and, for an input with
 * no negative elements, gives exactly the DualScale result (the + half's
 * codes and products are the same; the - half's are all zero).  A negative
 * element, which DualScale with s_neg = 0 quantises to 0, is instead
 * quantised with the + half's scale.  On a NULL table or n_kseg outside
 * [1, SEGQ_MAX_KSEG] returns SEGQ_ERR_NULL or SEGQ_ERR_SEGMENTS and sets
 * segquant_last_error().
 */
int segquant_gemm_halves(const float *act_scales_host, int32_t n_kseg);

/* Which kernel family segquant_gemm_w8a8_seg runs for this shape under
 * `flags` (SEGQ_KERNEL_*), or a negative status when the shape is invalid.
 * SEGQ_KERNEL_TILE is the large-M family: the tile kernel, or, for several
 * K-segments on int8 codes (the quantise-first path included) and for any
 * call whose K exceeds the tile kernel's running int32 sums
 * (K * 128 * 127 >= 2^31), the kernel that stages both operands in LDS and
 * folds each segment's own sums; which of the two depends on the segment
 * list and the activation format, not on the shape alone. */
int segquant_gemm_kernel_for(int64_t M, int64_t N, int64_t K, uint32_t flags);

/* Text for a status code (static storage). */
const char *segquant_status_string(int status);

/* Detail of this thread's last failing call ("" if none); valid until the
 * thread's next call into the library. */
const char *segquant_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int segquant_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGQUANT_H */
