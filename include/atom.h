/*
 * atom.h -- C ABI of the MI355X (gfx950) W4A4 mixed-precision quantized linear layer.
 *
 * The layer (Atom: "Low-bit Quantization for Efficient and Accurate LLM Serving"):
 *   - a fixed set of 128 outlier input channels is moved to the tail of every row and kept
 *     as one INT8 group (quantization record, Fields "Bits", "Activation scheme", "notes":
 *     a 128-channel high-precision group);
 *   - the dense bulk is quantized to INT4 with an independent scale per contiguous group of
 *     128 elements (record, Field "Weight group size" and "notes"; summary page, method
 *     paragraph: per-group scales);
 *   - the product runs on integer operators (index page, Abstract; record, "notes"): one
 *     exact integer dot product per 128-channel group, scaled in fp32 and summed.
 *
 * Conventions for every call below
 *   - Every tensor pointer is a DEVICE pointer into memory the caller owns.  The library
 *     never allocates, frees or synchronizes; work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and the call returns.  Inputs are only read, outputs are
 *     fully overwritten.
 *   - Dense row-major layouts.  Pointers must be 16-byte aligned (ATOM_E_ALIGN otherwise).
 *   - Shapes: K is a multiple of 128 with 256 <= K <= ATOM_MAX_K; rows (M, N) >= 1 and
 *     <= ATOM_MAX_ROWS.  G = K/128 groups: groups 0..G-2 are INT4, group G-1 is the INT8
 *     outlier group.  RB = atom_row_bytes(K) = (K-128)/2 + 128 bytes per packed row.
 *   - Packed row format: the first (K-128)/2 bytes hold the K-128 reordered INT4 codes in
 *     [-7, 7], four bits per code, in units of 16 consecutive codes c0..c15 stored as two
 *     32-bit little-endian words w0, w1.  Code c_i is the 6-bit field
 *     f_i = |c_i| + 32 * (c_i < 0) (the fp6 e2m3 encoding of c_i / 8, a subnormal) at bits
 *     6i .. 6i+5 of a 96-bit string T0 + T1 * 2^32 + T2 * 2^64, and
 *     w0 = T0 | (T2 & 0x18618618), w1 = T1 | (T2 & 0x86186186): the masks are the exponent
 *     bits (3 and 4 of each field) of T0 and T1, which are always zero, and T2's other bits
 *     are zero too.  (Decoding back to fp6 MFMA operands: T0 = w0 & ~0x18618618,
 *     T1 = w1 & ~0x86186186, T2 = (w0 & 0x18618618) | (w1 & 0x86186186).)  The last 128
 *     bytes hold the INT8 outlier codes in [-127, 127], two's complement.  Scales are fp16,
 *     group-major [G, rows].
 *   - Argument checks run on the host before any HIP call and return the status without
 *     enqueuing anything.  A failed launch returns ATOM_E_HIP.  Faults inside a kernel
 *     surface at the caller's next synchronization.  Calls that share no output buffer may
 *     run concurrently on different streams.
 */
#ifndef ATOM_H_
#define ATOM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATOM_GROUP 128        /* elements per quantization group (record, "Weight group size") */
#define ATOM_OUTLIERS 128     /* high-precision outlier channels (record, "notes") */
#define ATOM_MAX_K 65536      /* largest K: the row quantize stages a whole fp16 row (128 KiB) in LDS */
#define ATOM_MAX_ROWS (1 << 24)
#define ATOM_MAX_TILES (1 << 26) /* GEMM: ceil(M/128) * ceil(N/128) output tiles at most */

enum {
  ATOM_OK = 0,
  ATOM_E_NULL = 1,     /* a required pointer is NULL */
  ATOM_E_SHAPE = 2,    /* K not a multiple of 128, K < 256 or > ATOM_MAX_K, rows out of range,
                          GEMM with more than ATOM_MAX_TILES output tiles */
  ATOM_E_ALIGN = 3,    /* a pointer is not 16-byte aligned */
  ATOM_E_OVERLAP = 4,  /* an output range overlaps an input or another output range */
  ATOM_E_HIP = 5,      /* the HIP runtime reported an error when enqueuing */
  ATOM_E_SCRATCH = 6   /* atom_gemm_noalloc: the shape needs more scratch than ATOM_STATIC_SCRATCH_BYTES */
};

/* Bytes of one packed row, (K-128)/2 + 128: the K-128 bulk channels at four bits each and
 * the 128 outlier channels at eight (record, Fields "Bits": w4a4 with the outlier channels at
 * higher precision, and "notes": one 128-channel high-precision group); or -ATOM_E_SHAPE for
 * an invalid K.  Pure host function, no HIP call. */
int64_t atom_row_bytes(int32_t K);

/* Number of 128-channel groups, K/128, each with its own scale (record, Field "Weight group
 * size" and "notes": every contiguous run of 128 elements is quantized independently); groups
 * 0..G-2 are INT4, group G-1 is the INT8 outlier group.  -ATOM_E_SHAPE for an invalid K.  Pure
 * host function, no HIP call. */
int32_t atom_num_groups(int32_t K);

/* Static description of a status code; never NULL. */
const char *atom_strerror(int status);

/*
 * Outlier statistic (offline).  stat[c] = sum over m < M of X[m,c]^2 for every input
 * channel c of fp16 calibration activations X [M, K], returned as the exact sum rounded
 * once to fp64 (round to nearest even), so the value does not depend on summation order.
 * The pages leave the selection statistic open (record, "Activation scheme": a small set of
 * outlier channels kept at higher precision); this is the statistic the layer uses.
 *   X    : const fp16 [M, K]
 *   stat : double [K]                       (output)
 */
int atom_channel_stat(const void *X, int32_t M, int32_t K, double *stat, void *stream);

/*
 * Outlier selection and reorder (offline).  The 128 channels with the largest stat are the
 * outliers (ties go to the lower channel index).  perm lists the non-outlier channels in
 * ascending order followed by the outlier channels in ascending order: reordered channel j
 * takes original channel perm[j], so the outliers form the tail group G-1 (record, "notes":
 * one 128-channel high-precision group).  stat must hold no NaN.
 *   stat : const double [K]
 *   perm : int32 [K]                        (output)
 */
int atom_select_outliers(const double *stat, int32_t K, int32_t *perm, void *stream);

/*
 * Offline weight pack (summary page, method paragraph: weights grouped into small blocks
 * with per-group scales).  Row n of W is reordered through perm and quantized group by
 * group exactly as atom_quantize_act does for a token row.
 *   W    : const fp16 [N, K]      perm : const int32 [K], a permutation of 0..K-1
 *   Wq   : uint8 [N, RB]          sw   : fp16 [G, N]          (outputs)
 * Entries of perm outside 0..K-1 are clamped into range (garbage out, no fault).
 */
int atom_pack_weights(const void *W, const int32_t *perm, int32_t N, int32_t K,
                      void *Wq, void *sw, void *stream);

/*
 * Runtime activation quantize (record, "Activation scheme": dense bulk 4-bit, outlier
 * channels at higher precision; summary page: a dedicated outlier path).  For every token
 * row m and group g of the reordered row x = X[m, perm]:
 *   a = max |x| over the group;  qmax = 7 (g < G-1) or 127 (g = G-1);
 *   s = fp16_rne(fp32(a / qmax));  code = clamp(rint_even(fp32(x / s)), -qmax, qmax),
 *   code = 0 where s == 0.
 *   X    : const fp16 [M, K]      perm : const int32 [K]
 *   Xq   : uint8 [M, RB]          sx   : fp16 [G, M]           (outputs)
 * Elements must be finite: a group holding an inf or NaN gets unspecified codes and scale
 * (no fault).  The same holds for W in atom_pack_weights.
 */
int atom_quantize_act(const void *X, const int32_t *perm, int32_t M, int32_t K,
                      void *Xq, void *sx, void *stream);

/*
 * W4A4 GEMM (index page, Abstract: low-bit integer operators; record, "notes": integer
 * path).  Y[m,n] = fp16_rne( sum_g acc_g[m,n] * sx[g,m] * sw[g,n] ) where
 * acc_g[m,n] = sum over the 128 channels of group g of code_x * code_w is an exact integer;
 * the scale products and the sum over groups are fp32.
 *   Xq : const uint8 [M, RB]   sx : const fp16 [G, M]
 *   Wq : const uint8 [N, RB]   sw : const fp16 [G, N]
 *   Y  : fp16 [M, N]                                           (output)
 */
int atom_gemm(const void *Xq, const void *sx, const void *Wq, const void *sw,
              int32_t M, int32_t N, int32_t K, void *Y, void *stream);

/*
 * Scratch for atom_gemm_ws: bytes of fp32 workspace that let atom_gemm_ws divide each tile's
 * groups among several workgroups (split-K) when the M x N tiles alone would leave most of
 * the GPU idle; 0 when no split is used for this shape; -ATOM_E_SHAPE for invalid shapes.
 */
int64_t atom_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);

/*
 * atom_gemm with caller-provided scratch (the library allocates nothing).  With workspace
 * != NULL and workspace_bytes >= atom_gemm_workspace_bytes(M, N, K) > 0, each split
 * accumulates its groups in fp32 and a second kernel adds the splits in a fixed order and
 * rounds once to fp16 (the sum over groups is then associated differently: results agree
 * with atom_gemm to fp32 rounding, not bit for bit).  Otherwise it is exactly atom_gemm.
 * The workspace must be 16-byte aligned and must not overlap any argument; its contents on
 * entry do not matter and are overwritten.
 */
int atom_gemm_ws(const void *Xq, const void *sx, const void *Wq, const void *sw,
                 int32_t M, int32_t N, int32_t K, void *Y, void *workspace,
                 int64_t workspace_bytes, void *stream);

/*
 * atom_gemm for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same kernels and the same result as
 * atom_gemm_ws with enough workspace, bit for bit, but the split-K scratch is a static buffer
 * inside the library, ATOM_STATIC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends.  No allocation of any kind happens in the call.  The buffer of the
 * current device is used (the stream must belong to it).  Every call on one GPU shares that
 * buffer, so calls that overlap on one GPU (different streams without synchronization) race and
 * give wrong results.  ATOM_E_SCRATCH if the shape's split needs more than the buffer (no valid
 * shape does: the largest needs 19.7 MiB); other errors as for atom_gemm.
 */
#define ATOM_STATIC_SCRATCH_BYTES (24 << 20)
int atom_gemm_noalloc(const void *Xq, const void *sx, const void *Wq, const void *sw, int32_t M, int32_t N, int32_t K,
                      void *Y, void *stream);

/*
 * Per-group integer accumulators (verification aid): acc[g, m, n] = acc_g[m,n] as defined
 * for atom_gemm, computed by the main loop of the kernel atom_gemm runs for this shape (the
 * few-rows kernel for M <= 16, the tiled kernel otherwise; where atom_gemm splits the groups
 * of a 64 x 64 tile between two K parts, the same tiles without the split).  acc is int32
 * [G, M, N] (output, G*M*N*4 bytes).
 */
int atom_gemm_group_acc(const void *Xq, const void *Wq, int32_t M, int32_t N, int32_t K,
                        int32_t *acc, void *stream);

/*
 * The layer's runtime forward in one call (a next step beside the path: the activation quantize
 * fused with the GEMM, summary page, method paragraph: activations take their own quantize and
 * outlier path on the way into the integer GEMM).  Computes exactly what atom_quantize_act
 * (X, perm -> Xq, sx) followed by atom_gemm (-> Y) compute, with the same outputs.
 *   X  : const fp16 [M, K]     perm : const int32 [K]
 *   Wq : const uint8 [N, RB]   sw   : const fp16 [G, N]      (from atom_pack_weights)
 *   Xq : uint8 [M, RB]         sx   : fp16 [G, M]            (outputs, as atom_quantize_act's)
 *   Y  : fp16 [M, N]                                          (output)
 *   workspace : atom_linear_workspace_bytes(M, N, K) bytes of device memory that must be zero
 *               before its first use; every call leaves its control words zero again.
 * When the GEMM runs whole 128 x 128 output tiles and K <= 12288, both steps run in ONE
 * persistent launch: every workgroup first quantizes its share of the activation rows and
 * counts them as ready, then runs its share of the output tiles, each after its rows are ready.
 * No workgroup waits before its own rows are done, so the waits end when every workgroup is
 * resident: the launch takes the resident count for an otherwise idle GPU.  The wait is bounded
 * all the same: if one gives up (another kernel holding compute units meanwhile could cause
 * that), int32 word 9 of the workspace becomes nonzero (read it after the stream completes; it
 * stays set until the caller clears it) and the outputs of that call are not valid.  int32 word
 * 10 sets the wait (0: default bound; > 0: that many polls; < 0: give up at once, which exercises
 * the failure path).  Other shapes run the two kernels one after the other (the split-K scratch,
 * if any, lies after the control words).  Calls sharing one workspace must not overlap (same
 * stream, or synchronized).
 */
int64_t atom_linear_workspace_bytes(int32_t M, int32_t N, int32_t K);
int atom_linear(const void *X, const int32_t *perm, const void *Wq, const void *sw, int32_t M, int32_t N, int32_t K,
                void *Xq, void *sx, void *Y, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * W4A8 variant (a next step beside the W4A4 path; the pages point to INT8 activations only as
 * the precision another method's kernels target).  Activations get INT8 codes in every group
 * (the rule of atom_quantize_act with qmax = 127 for every group); weights keep the W4 rule of
 * atom_pack_weights but a layout the int8 matrix cores unpack cheaply.  The product and the
 * output are defined as for atom_gemm.
 *
 * atom_quantize_act_a8: X const fp16 [M, K], perm const int32 [K] -> Xq uint8 [M, K] (one
 *   two's-complement byte per code, reordered order), sx fp16 [G, M].
 * atom_pack_weights_w4a8: W const fp16 [N, K], perm -> Wq uint8 [N, RB], sw fp16 [G, N].  Codes
 *   and scales equal atom_pack_weights'; the first (K-128)/2 bytes hold the INT4 codes in blocks
 *   of 8 consecutive codes c_0..c_7 as 4 bytes, byte j = (c_j + 8) | (c_{j+4} + 8) << 4
 *   (offset binary); the last 128 bytes hold the INT8 outlier codes, two's complement.
 * atom_gemm_w4a8: Xq [M, K] from atom_quantize_act_a8, Wq [N, RB] from atom_pack_weights_w4a8,
 *   scales as above -> Y fp16 [M, N] = fp16_rne(sum_g acc_g * sx[g,m] * sw[g,n]), fp32 scaling.
 * atom_gemm_w4a8_group_acc: acc int32 [G, M, N] of the same operands (verification aid).
 * atom_gemm_w4a8_workspace_bytes / atom_gemm_w4a8_ws: split-K scratch and the call that uses it,
 *   with the semantics of atom_gemm_workspace_bytes / atom_gemm_ws (any M, including M <= 16).
 * Shapes, alignment, overlap and error rules as for the W4A4 calls.
 */
int atom_quantize_act_a8(const void *X, const int32_t *perm, int32_t M, int32_t K, void *Xq, void *sx,
                         void *stream);
int atom_pack_weights_w4a8(const void *W, const int32_t *perm, int32_t N, int32_t K, void *Wq, void *sw,
                           void *stream);
int atom_gemm_w4a8(const void *Xq, const void *sx, const void *Wq, const void *sw, int32_t M, int32_t N,
                   int32_t K, void *Y, void *stream);
int atom_gemm_w4a8_group_acc(const void *Xq, const void *Wq, int32_t M, int32_t N, int32_t K, int32_t *acc,
                             void *stream);
int64_t atom_gemm_w4a8_workspace_bytes(int32_t M, int32_t N, int32_t K);
int atom_gemm_w4a8_ws(const void *Xq, const void *sx, const void *Wq, const void *sw, int32_t M, int32_t N,
                      int32_t K, void *Y, void *workspace, int64_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATOM_H_ */
