/*
 * swiglu.h -- C ABI of the MI355X (gfx950) fused SwiGLU GEMM library.
 *
 *   Y = SiLU(A . W1) (.) (A . W2),   SiLU(x) = x / (1 + exp(-x))
 *
 * The gated MLP of "Tile-Level Activation Overlap for Efficient LLM
 * Inference" (arXiv 2607.02521; paper text, section 1 Introduction: Gate =
 * A x W1, Up = A x W2, Y = SiLU(Gate) (.) Up).  The fused entry point never
 * writes Gate or Up to device memory: they live in MFMA accumulators
 * (registers) from the contraction to the bf16 store of Y.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every matrix is bf16, passed as its 16-bit patterns (uint16_t), dense
 *    and contiguous: A [M][K], W1 and W2 [K][N], Y / gate_ws / up_ws [M][N]
 *    row-major; the packed weight W_fused (K x 2N) column-major, i.e. a
 *    row-major [2N][K] array whose row c is column c of W_fused.  Exceptions
 *    are stated by the calls they concern: the FP8 calls take one-byte E4M3
 *    codes (uint8_t), swiglu_fused_gemm_strided takes row-strided A and Y.
 *  - Every matrix pointer is a DEVICE pointer, allocated and owned by the
 *    caller.  The library allocates, frees and retains nothing: no pointer is
 *    kept past the call.
 *  - `stream` is a hipStream_t passed as void*; NULL selects the default
 *    stream.  Calls only enqueue work and return; results are valid after the
 *    stream is synchronised.  Errors raised by a kernel while it runs surface
 *    at the caller's synchronisation, as in HIP.
 *  - Arguments are validated before any HIP call: an invalid call launches
 *    nothing and returns a negative swiglu_status.  Preconditions:
 *      M >= 0, N >= 0, K >= 8;  K % 8 == 0 and N % 8 == 0 (each row is a
 *      whole number of 16-byte chunks);  M <= 2^31 - 1, K <= 2^21,
 *      N <= 2^22;
 *      every pointer 16-byte aligned;  outputs do not overlap inputs or
 *      each other.
 *    M == 0 or N == 0 is an empty problem: SWIGLU_OK, nothing launched.
 *  - Outputs are computed with fp32 accumulation of bf16 (or FP8) products
 *    and one round-to-nearest-even to bf16 at the end; the accumulation order
 *    is not specified (results of different variants need not be bitwise
 *    equal).
 *  - Every compute call takes the weights in one form only, the packed
 *    W_fused that swiglu_pack_weights (or swiglu_pack_weights_nk) writes once
 *    per weight set: variant I, variant S, the unfused ablation and the MLP
 *    block read it, and none of them takes W1 and W2 as two separate
 *    [K][N] arrays.  Variant S and the ablation read its even (Gate) and odd
 *    (Up) rows as two row-strided panels, which are exactly the bytes of W1
 *    and W2 in K-contiguous order.  The reason is the operand layout: both
 *    MFMA operands take 8 consecutive k per lane, so K-contiguous weights
 *    give plain 16-byte LDS fragment reads, where [K][N] weights would need
 *    the transposing 8-byte reads at about half the LDS rate.  Accepting
 *    [K][N] W1, W2 in the compute calls would mean a second mainloop or a
 *    transpose inside every call, so the transpose is the pack's job.
 *  - Calls are re-entrant; the only global state is a per-device cache of
 *    the device's architecture and compute-unit count, the static scratch
 *    array of swiglu_fused_gemm_noalloc, and a static array of arrival
 *    counters for the split reduced in the kernel (device memory the library
 *    holds; no call allocates).  The counters start at zero and every call
 *    that completes leaves them at zero; each such call takes the next of 64
 *    counter blocks of its device in turn, so at most 64 of them may run at
 *    once on one device (different streams).
 *  - The code object targets gfx950 only: on another device every launching
 *    call returns SWIGLU_ERR_UNSUPPORTED.
 */
#ifndef SWIGLU_H
#define SWIGLU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swiglu_status {
    SWIGLU_OK = 0,
    SWIGLU_ERR_NULL = -1,        /* a pointer the call needs is NULL            */
    SWIGLU_ERR_SHAPE = -2,       /* a size violates the preconditions above     */
    SWIGLU_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned            */
    SWIGLU_ERR_UNSUPPORTED = -4, /* unknown variant, or the device is not gfx950 */
    SWIGLU_ERR_HIP = -5,         /* a HIP call or kernel launch failed          */
    SWIGLU_ERR_ALIAS = -6        /* an output overlaps an input or another output */
} swiglu_status;

typedef enum swiglu_variant {
    SWIGLU_AUTO = 0,      /* pick by M (swiglu_select_variant)                  */
    SWIGLU_VARIANT_S = 1, /* sequential: Gate loop, SiLU, Up loop, multiply      */
    SWIGLU_VARIANT_I = 2  /* interleaved: one GEMM over W_fused, paired epilogue */
} swiglu_variant;

/*
 * Interleave W1 and W2 column by column into W_fused (the fused weight of the
 * pages' Kernel-2; gist.science technical summary, Method, Kernel-2: even
 * columns belong to Gate, odd columns to Up):
 *
 *     W_fused[k][2n] = W1[k][n],   W_fused[k][2n+1] = W2[k][n]   (0-based)
 *
 * W_fused is stored column-major: the output is the row-major [2N][K] array
 * P with P[2n][k] = W1[k][n] and P[2n+1][k] = W2[k][n], so both operands of
 * every contraction are K-contiguous (the layout the MFMA loaders read).
 * W1, W2: [K][N] device, read only.  W_fused: 2N*K elements, device, written.
 * A pure copy of 16-bit patterns (bit-exact).  Done once per weight set, off
 * the timed path.  K >= 0 here (K == 0 or N == 0 is an empty problem); the
 * other preconditions above apply (K % 8 == 0 and N % 8 == 0: both are row
 * lengths here).
 */
int swiglu_pack_weights(const uint16_t *W1, const uint16_t *W2,
                        uint16_t *W_fused, int64_t K, int64_t N, void *stream);

/*
 * The fused SwiGLU GEMM, Y = bf16( SiLU(A.W1) * (A.W2) ), from the packed
 * weight (swiglu_pack_weights).  Gate and Up never leave registers.
 *
 * variant SWIGLU_VARIANT_I (the pages' Kernel-2; gist.science technical
 *   summary, Method, Kernel-2): one GEMM over all 2N columns of W_fused; its
 *   epilogue pairs accumulator columns 2n (Gate) and 2n+1 (Up) and stores
 *   SiLU(D[m][2n]) * D[m][2n+1].
 * variant SWIGLU_VARIANT_S (the pages' Kernel-1; paper abstract and
 *   gist.science technical summary, Method, Kernel-1): per output tile, the
 *   Gate contraction (even columns), then SiLU on the register-resident Gate
 *   accumulator while the first Up tiles' loads (issued across the Gate->Up
 *   boundary) are in flight, then the Up contraction (odd columns) and a
 *   multiply-and-store epilogue.
 * variant SWIGLU_AUTO: whichever swiglu_select_variant(M, N, K) names.
 *
 * A: [M][K], W_fused: packed [2N][K], Y: [M][N]; device pointers.
 *
 * workspace / workspace_bytes: optional caller-owned device scratch
 * (256-byte aligned, not shared by calls that may run concurrently; no
 * initialisation needed, contents meaningless after the call).  When the
 * output tiles leave the last round of workgroups partly idle, variant I runs
 * that round's tiles whichever way a cost model of the device predicts
 * fastest: whole; as quarter-size tiles in the same kernel (no workspace
 * needed); or, given at least swiglu_workspace_size() bytes of workspace,
 * split along K, the pieces leaving fp32 partial tiles in the workspace that
 * a second kernel on the same stream sums, in a fixed order, before the
 * epilogue.  At M <= 128 with long K (at least 3 pieces of at least 16 K
 * steps of 64, at most 4 pieces) variant I instead splits every tile along K
 * and sums the partials in the same kernel: the last piece of each tile to
 * finish (counted with a library-owned arrival counter, see the global state
 * below) reads the others' partials from the workspace.  Every schedule gives
 * bitwise reproducible results for a given (M, N, K, workspace size, device).
 * NULL or too small: no split.  Variant S does not use it.
 */
int swiglu_fused_gemm(const uint16_t *A, const uint16_t *W_fused, uint16_t *Y,
                      int64_t M, int64_t N, int64_t K, int variant,
                      void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * swiglu_fused_gemm on row-strided views of A and Y, for activations and
 * outputs that are slices of wider tensors (rows of A are lda elements apart,
 * rows of Y ldy elements apart; the packed weight stays contiguous).  Same
 * computation, variants, workspace and preconditions as swiglu_fused_gemm,
 * plus: K <= lda <= 2^21 with lda % 8 == 0 (16-byte aligned rows), and
 * N <= ldy <= 2^22.  Only the M x K elements of A and the M x N elements of Y
 * are accessed; Y's elements between rows are left untouched.  Overlap is
 * judged on the spans [A, A + (M-1)*lda + K) and [Y, Y + (M-1)*ldy + N), so
 * views that interleave rows of one allocation are rejected as overlapping.
 * swiglu_fused_gemm(A, W, Y, M, N, K, ...) is this call with lda = K, ldy = N.
 */
int swiglu_fused_gemm_strided(const uint16_t *A, int64_t lda, const uint16_t *W_fused,
                              uint16_t *Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                              int variant, void *workspace, uint64_t workspace_bytes,
                              void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not allocate, harnesses that forbid it.
 * swiglu_fused_gemm without a workspace argument: the split-tail scratch
 * (fp32 partial tiles) lives in a static device array inside the library,
 * 64 MiB (one fp32 256 x 256 tile per compute unit of a 256-CU device), that
 * each device the library is loaded on holds from the first call on that
 * device until the process ends.  The call allocates nothing (no hipMalloc,
 * no library routine that allocates).  Same computation, variants, schedule
 * choice and preconditions as swiglu_fused_gemm with a workspace of that
 * size (the outputs are bitwise those of swiglu_fused_gemm given a workspace
 * of at least swiglu_workspace_size() bytes).  Every call on a device shares
 * that device's array: calls that may overlap on one device (different
 * streams without ordering between them) race and must not be issued; calls
 * on one stream are ordered and safe.  The scratch needs no initialisation
 * (each partial is written before it is read) and its contents are
 * meaningless after a call.  A device whose compute-unit count needs more
 * scratch than the array holds gets SWIGLU_ERR_UNSUPPORTED, nothing launched.
 */
int swiglu_fused_gemm_noalloc(const uint16_t *A, const uint16_t *W_fused, uint16_t *Y,
                              int64_t M, int64_t N, int64_t K, int variant, void *stream);

/*
 * Bytes of `workspace` that let a call split the tail round along K: variant
 * SWIGLU_VARIANT_I or SWIGLU_AUTO for swiglu_fused_gemm, -1 for
 * swiglu_unfused_ablation, swiglu_down_proj and swiglu_gated_mlp (0 when
 * nothing uses it, e.g. variant S, or for an empty problem; the FP8 call uses
 * variant I's size).  Queries the current device's compute-unit count (a HIP
 * call).  One fp32 256 x 256 tile per compute unit, whatever the shape:
 * 64 MiB on MI355X.
 */
int swiglu_workspace_size(int64_t M, int64_t N, int64_t K, int variant,
                          uint64_t *bytes);

/*
 * The unfused pipeline, kept as an ablation so the saved memory traffic can be
 * measured (paper text, section 1: the unfused form materialises two full
 * intermediate tensors, Gate and Up, between the GEMM and activation stages).
 * Three stream-ordered launches built from the same mainloop, and the same
 * packed weight, as the fused kernels:
 *     gate_ws = bf16(A.W1);  up_ws = bf16(A.W2);
 *     Y = bf16( SiLU(gate_ws) * up_ws )   (fp32 arithmetic, one rounding)
 * gate_ws, up_ws: caller-owned [M][N] device workspaces, written (their
 * contents are part of the result and may be inspected).  workspace /
 * workspace_bytes: as for swiglu_fused_gemm (the two GEMMs use the same
 * scheduler as variant I; size from swiglu_workspace_size(..., -1, ...)).
 */
int swiglu_unfused_ablation(const uint16_t *A, const uint16_t *W_fused,
                            uint16_t *gate_ws, uint16_t *up_ws, uint16_t *Y,
                            int64_t M, int64_t N, int64_t K, void *workspace,
                            uint64_t workspace_bytes, void *stream);

/*
 * Packer for weights in a linear layer's layout (one row per output feature,
 * as a framework's gate and up projection layers store them): W1t and W2t
 * are [N][K] row-major, W1t[n][k] = W1[k][n] and W2t[n][k] = W2[k][n].
 * Writes the same packed W_fused as swiglu_pack_weights [gist.science
 * technical summary, Method, Kernel-2]: row 2n of the [2N][K] array is row n
 * of W1t, row 2n+1 is row n of W2t (a row interleave, bit-exact).
 * W1t, W2t: device, read only; W_fused: 2N*K elements, device, written.
 * K % 8 == 0 (the row length of all three arrays; N is unrestricted),
 * K <= 2^21, N <= 2^22, pointers 16-byte aligned, no overlap between the
 * output and the inputs.  K == 0 or N == 0 is an empty problem.
 */
int swiglu_pack_weights_nk(const uint16_t *W1t, const uint16_t *W2t,
                           uint16_t *W_fused, int64_t K, int64_t N,
                           void *stream);

/*
 * The down projection that closes the gated MLP block, Out = bf16(H . W3)
 * with H [M][N] (the SwiGLU output) and W3 in R^{N x D} (D is the model
 * width, K of the gated GEMM).  The paper measures the SwiGLU stage as a
 * share of the whole MLP block's time (paper text, section 1 Introduction,
 * Figure 1); the block's last GEMM is this one.
 *
 * H: [M][N] row-major device; W3t: W3 stored K-contiguous, i.e. the
 * row-major [D][N] array with W3t[d][n] = W3[n][d] (a linear layer's weight
 * layout); Out: [M][D] row-major device, written.  fp32 accumulation, one
 * round-to-nearest-even.  Preconditions: M >= 0, D >= 0, N >= 8; N % 8 == 0
 * and D % 8 == 0; N <= 2^21, D <= 2^22; pointers 16-byte aligned; Out
 * overlaps no input.  M == 0 or D == 0: SWIGLU_OK, nothing launched.
 * workspace / workspace_bytes: as for swiglu_fused_gemm (the same scheduler;
 * size from swiglu_workspace_size(M, N, D, -1, ...)): with few output tiles
 * (e.g. a narrow model width at small M) it lets the call split the tiles
 * along N so that every compute unit works.
 */
int swiglu_down_proj(const uint16_t *H, const uint16_t *W3t, uint16_t *Out,
                     int64_t M, int64_t N, int64_t D, void *workspace,
                     uint64_t workspace_bytes, void *stream);

/*
 * The gated MLP block (paper text, section 1 Introduction: Gate = A x W1,
 * Up = A x W2, Y = SiLU(Gate) (.) Up; Figure 1: the MLP block the SwiGLU
 * stage is a share of), with its down projection back to the model width K:
 *     H = swiglu_fused_gemm(A, W_fused, variant)      (bf16, [M][N])
 *     Out = bf16(H . W3)                               ([M][K])
 * Two stream-ordered launches (the fused SwiGLU GEMM, then the down
 * projection); Gate and Up never reach device memory, H does (the down
 * projection reduces over all N columns of a row, which span many tiles).
 * A [M][K], W_fused packed [2N][K], W3t [K][N] (W3 in R^{N x K} stored
 * K-contiguous), H [M][N] (caller-owned, written: the block's intermediate),
 * Out [M][K]; all device.  Preconditions: those of swiglu_fused_gemm and of
 * swiglu_down_proj with D = K; H and Out overlap no input and not each other.
 * M == 0: SWIGLU_OK, nothing launched.  workspace: as for swiglu_fused_gemm,
 * shared by the two launches (stream order).
 */
int swiglu_gated_mlp(const uint16_t *A, const uint16_t *W_fused,
                     const uint16_t *W3t, uint16_t *H, uint16_t *Out,
                     int64_t M, int64_t N, int64_t K, int variant,
                     void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * FP8 inputs.  The pages' motivation is that quantisation (FP8, INT4) makes
 * the GEMMs cheaper, so the materialisation the fusion removes costs
 * relatively more (paper text, section 1 Introduction).  Format: OCP FP8 E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; largest finite 448), one byte per value.  Scaling: one
 * power of two per tensor, A = 2^a_exp * A8 and W_fused = 2^w_exp * W8.
 *
 * swiglu_fp8_scale_exp: the smallest exponent e with amax * 2^-e <= 448
 * (host only; 0 for amax <= 0, NaN or beyond the float range).
 *
 * swiglu_quantize_fp8: Q[i] = E4M3(X[i] * 2^-scale_exp) for bf16 X, round to
 * nearest even, finite values beyond 448 and infinities saturated to +-448,
 * NaN -> 0x7F (bit-exact).  X: count bf16 values, Q: count bytes, device;
 * count % 16 == 0, -126 <= scale_exp <= 126, pointers 16-byte aligned, Q does
 * not overlap X.  Quantising the packed weight (swiglu_pack_weights output,
 * count = 2N*K) gives W_fused8; quantising A gives A8.
 *
 * swiglu_fused_gemm_fp8: the fused SwiGLU GEMM on FP8 operands,
 *     Y = bf16( SiLU(2^(a_exp+w_exp) A8.W1_8) * (2^(a_exp+w_exp) A8.W2_8) )
 * with A8 [M][K] and W_fused8 packed [2N][K] (the layout of
 * swiglu_pack_weights, one byte per value); fp32 accumulation of exact FP8
 * products, the scales applied to Gate and Up in fp32 before the activation,
 * one rounding to bf16.  `variant`: SWIGLU_VARIANT_I, SWIGLU_VARIANT_S or
 * SWIGLU_AUTO (swiglu_select_variant), as for swiglu_fused_gemm.
 * Preconditions: those of swiglu_fused_gemm, and K % 16 == 0 (16-byte rows);
 * a_exp, w_exp and a_exp + w_exp in [-126, 126].  workspace: as for
 * swiglu_fused_gemm (variant I's size; variant S does not use it).
 */
int swiglu_fp8_scale_exp(double amax);
int swiglu_quantize_fp8(const uint16_t *X, uint8_t *Q, int64_t count,
                        int scale_exp, void *stream);
int swiglu_fused_gemm_fp8(const uint8_t *A8, const uint8_t *W_fused8,
                          uint16_t *Y, int64_t M, int64_t N, int64_t K,
                          int a_exp, int w_exp, int variant, void *workspace,
                          uint64_t workspace_bytes, void *stream);

/*
 * What a call would launch, as text (host only; queries the current device's
 * compute-unit count): for swiglu_fused_gemm with `variant` (AUTO, S, I) or
 * for swiglu_unfused_ablation (-1), for the down projection of
 * swiglu_gated_mlp over (M, N, K) (-2: an M x K output reducing over N),
 * for swiglu_fused_gemm_fp8 (-3),
 * given a workspace of `workspace_bytes`
 * (0: none), the kernel names with their tile shapes and schedule, e.g.
 * "gemm_tiles_kernel<128x128x64,PairMulEpilogue> (2240 tiles; 512 workgroups)"
 * (the GEMM kernels are persistent: each workgroup loops over its share of
 * the tiles).  Writes at most buf_bytes bytes including the terminating NUL
 * (truncating).  Same shape validation as the calls it describes;
 * SWIGLU_ERR_NULL without buf.
 */
int swiglu_describe_launch(int64_t M, int64_t N, int64_t K, int variant,
                           uint64_t workspace_bytes, char *buf, uint64_t buf_bytes);

/*
 * The ablation's activation stage on its own: Y[i] = bf16(SiLU(gate[i]) *
 * up[i]) for i < count, fp32 arithmetic, one rounding.  count % 8 == 0,
 * count >= 0; pointers 16-byte aligned, device.
 */
int swiglu_silu_mul(const uint16_t *gate, const uint16_t *up, uint16_t *Y,
                    int64_t count, void *stream);

/*
 * The variant SWIGLU_AUTO runs for this shape: SWIGLU_VARIANT_I when
 * M <= swiglu_m_switch(), else SWIGLU_VARIANT_S.  The pages aim the
 * interleaved kernel at small batches and the sequential one at large batches
 * (gist.science technical summary, Method, Kernel-1 and Kernel-2); on MI355X
 * the interleaved kernel measured faster at every M (128 to 16384) of the five
 * benchmark K x N shapes, so the built-in threshold is 2^31 - 1 (always I).
 * Host only, no HIP call.  Returns SWIGLU_ERR_SHAPE for M < 0.
 */
int swiglu_select_variant(int64_t M, int64_t N, int64_t K);

/* The M threshold used by swiglu_select_variant: 2^31 - 1 unless the
 * environment variable SWIGLU_M_SWITCH parses as an integer (e.g. 2048 for the
 * pages' small/large-batch split), which then overrides it. */
int64_t swiglu_m_switch(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *swiglu_status_string(int status);

/* Detail of the last failure on the calling thread (static storage; empty
 * string when the last call succeeded). */
const char *swiglu_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_H */
