/*
 * CPU oracle for the gated-MLP SwiGLU GEMM  Y = SiLU(A.W1) (.) (A.W2).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library; the two meet only through the seeded input generator.
 *
 * Sources.  All citations are to the pages on "Tile-Level Activation Overlap
 * for Efficient LLM Inference" (arXiv 2607.02521):
 *   [paper s1]      the paper's own text, section 1 "Introduction"
 *                   (docshare.wps.com copy of the PDF text);
 *   [abstract]      the paper's abstract (same copy, and the arXiv abstract
 *                   on mlsanity.com);
 *   [gist: X]       the gist.science technical summary, section X
 *                   (an AI-written explainer, lowest authority).
 *
 * What is computed.  The method changes where Gate and Up live (registers,
 * not HBM); the result it reaches is the plain definition of the gated MLP
 * [paper s1: Gate = A x W1, Up = A x W2, Y = SiLU(Gate) (.) Up;
 *  gist: Problem statement].  So the oracle is that definition written out:
 *
 *   1. widen every bf16 input to double (exact);
 *   2. Gate[m,n] = sum_k A[m,k] W1[k,n] and Up[m,n] = sum_k A[m,k] W2[k,n],
 *      accumulated in double with k ascending (each product of two bf16
 *      values is exact in double);
 *   3. s = Gate / (1 + exp(-Gate))   (SiLU = Swish with beta = 1; the pages
 *      name SiLU/Swish without a formula, this is the standard one);
 *   4. y = s * Up in double;
 *   5. Y[m,n] = bf16(y), one rounding, round-to-nearest-even.
 *
 * The interleaved form [gist: Method, Kernel-2] packs W_fused in R^{K x 2N}
 * with even columns from W1 (Gate) and odd columns from W2 (Up), runs one
 * GEMM D = A . W_fused and pairs (D[m,2n], D[m,2n+1]) into
 * SiLU(D[m,2n]) * D[m,2n+1].  It is provided separately so that the
 * invariant "interleaved == separate, bit for bit" can be tested.
 *
 * Weights in the layout of a linear layer ([N][K]: one row per output
 * feature, i.e. W1 and W2 transposed) pack into the same W_fused; the
 * packer for them is written out separately and pinned against slicing.
 *
 * The gated MLP block whose execution time the SwiGLU share is measured
 * against [paper s1, Figure 1: SwiGLU activation and materialisation as a
 * fraction of total MLP time] ends with the down projection back to the
 * model width: Out = Y . W3 with W3 in R^{N x K}.  The pages name the MLP
 * block but print no formula for it; the plain reading is that Y, a bf16
 * tensor like every activation here, is the input of one more GEMM:
 *   Out[m,d] = bf16( sum_n Y_bf16[m,n] W3[n,d] ), double, n ascending.
 *
 * The materialised form rounds Gate and Up to bf16 before the activation,
 * as the unfused eager pipeline does [paper s1: two full intermediate tensors
 * are materialised in HBM between the GEMM and activation stages]; it pins
 * the unfused ablation only.
 *
 * Layout: every matrix is row-major and contiguous; bf16 values travel as
 * their 16-bit patterns (uint16_t).
 *
 * Parity pins (in tests/test_oracle_pins.py): bf16 rounding against bit
 * patterns and against torch's independent float->bf16 cast; SiLU closed
 * forms and the identity SiLU(x) - SiLU(-x) = x; hand-computed 2x3x2 cases;
 * dot products against numpy float64 matmul; the interleave invariant; the
 * pack against numpy slicing; the linear-layer packer against slicing of the
 * transposes; the down projection against numpy float64 matmul, the
 * identity weight and a hand case whose result changes sign if Y is not
 * rounded to bf16 first; the FP8 decoder against torch's float8_e4m3fn for
 * all 256 codes, the FP8 rounding against torch's cast and a brute-force
 * nearest search, and the FP8 GEMM against the bf16 oracle on inputs exact
 * in both formats (with and without scales).  Planted-mistake builds (PLANT_* macros below,
 * compiled only by the tests) show that each plausible slip fails a pin.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- planted mistakes: compiled in only by the mutation tests ---------- */
#ifdef PLANT_SILU_SIGN          /* x / (1 + e^{+x})  instead of e^{-x}     */
#define SILU_EXP_ARG(x) (x)
#else
#define SILU_EXP_ARG(x) (-(x))
#endif

/* ------------------------------------------------------------------------ */
/* bf16 <-> double                                                          */
/* ------------------------------------------------------------------------ */

/* Widening is exact: a bf16 pattern is the top half of an IEEE binary32. */
double swo_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16, ties to even, directly (no detour
 * through binary32, which could round twice).
 *
 * bf16 keeps 8 significant bits and binary32's exponent range.  For |x| in
 * [2^e, 2^(e+1)) the spacing of bf16 values is 2^(e-7); below the smallest
 * normal (2^-126) the spacing stays at the subnormal quantum 2^-133.  The
 * nearest multiple of the spacing is found with nearbyint() under the
 * default rounding mode (nearest, ties to even); scaling by a power of two
 * is exact in double.  Results above the largest finite bf16 become +-inf,
 * as IEEE rounding to nearest prescribes (a tie at the top rounds to the
 * even neighbour 2^128, i.e. overflows).
 */
uint16_t swo_double_to_bf16(double x)
{
    if (isnan(x)) {
        return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    }
    if (x == 0.0 || isinf(x)) {
        float f = (float)x;              /* exact: 0, -0, +-inf */
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    int ex;
    (void)frexp(x, &ex);                 /* |x| = f 2^ex, f in [0.5, 1) */
    int qexp = ex - 8;                   /* spacing 2^((ex-1) - 7)      */
    if (qexp < -133) qexp = -133;
    double q = ldexp(1.0, qexp);
#ifdef PLANT_ROUND_TOWARD_ZERO      /* truncates instead of rounding      */
    double r = trunc(x / q) * q;
#else
    double r = nearbyint(x / q) * q;     /* exact scaling, RNE on the integer */
#endif
    const double bf16_max = ldexp(255.0, 120);  /* (2 - 2^-7) 2^127 */
    if (fabs(r) > bf16_max) {
        return (uint16_t)(signbit(x) ? 0xFF80u : 0x7F80u);
    }
    float f = (float)r;                  /* exact: r is a bf16 value    */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^{-x}).  For very negative x,
 * e^{-x} overflows to +inf and the quotient is -0: no NaN for finite x. */
double swo_silu(double x)
{
    return x / (1.0 + exp(SILU_EXP_ARG(x)));
}

/* ------------------------------------------------------------------------ */
/* the contraction                                                          */
/* ------------------------------------------------------------------------ */

/*
 * One output row of D = A . B over a window of ncols columns of a row-major
 * bf16 B whose rows are ldb elements apart (B points at the window's first
 * column): d[c] = sum_{k=0}^{K-1} A[m,k] B[k,c], double, k ascending.  The
 * loop runs c innermost so that B is read along its rows; the order of the
 * terms of each sum is still k = 0, 1, ..., K-1.
 */
static void row_times_window(const uint16_t *a_row, const uint16_t *B,
                             int64_t K, int64_t ncols, int64_t ldb, double *d)
{
    for (int64_t c = 0; c < ncols; ++c) d[c] = 0.0;
#ifdef PLANT_SKIP_LAST_K            /* drops the k = K-1 term              */
    K = K - 1;
#endif
    for (int64_t k = 0; k < K; ++k) {
        const double a = swo_bf16_to_double(a_row[k]);
        const uint16_t *b = B + k * ldb;
        for (int64_t c = 0; c < ncols; ++c) {
            d[c] += a * swo_bf16_to_double(b[c]);
        }
    }
}

static void row_times_matrix(const uint16_t *a_row, const uint16_t *B,
                             int64_t K, int64_t ncols, double *d)
{
    row_times_window(a_row, B, K, ncols, ncols, d);
}

/* D[M, ncols] = A[M,K] . B[K,ncols] in double (exposed for the pins). */
void swo_matmul(const uint16_t *A, const uint16_t *B, int64_t M, int64_t K,
                int64_t ncols, double *D)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        row_times_matrix(A + m * K, B, K, ncols, D + m * ncols);
    }
}

/* Steps 3-5 for one element. */
static void gate_up_to_y(double g, double u, double *y64, uint16_t *ybf)
{
#ifdef PLANT_SWAP_GATE_UP           /* activates Up instead of Gate       */
    double t = g; g = u; u = t;
#endif
    double y = swo_silu(g) * u;
    if (y64) *y64 = y;
    if (ybf) *ybf = swo_double_to_bf16(y);
}

/*
 * Separate formulation over a list of rows: for each listed row m, every
 * column n of Y.  rows == NULL means rows 0..nrows-1.  Outputs are indexed by
 * position in the list: y64[i*N + n], ybf[i*N + n] (either may be NULL).
 */
void swo_swiglu_rows(const uint16_t *A, const uint16_t *W1, const uint16_t *W2,
                     int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                     double *y64, uint16_t *ybf)
{
    #pragma omp parallel
    {
        double *g = (double *)malloc((size_t)N * sizeof(double));
        double *u = (double *)malloc((size_t)N * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t m = rows ? rows[i] : i;
            row_times_matrix(A + m * K, W1, K, N, g);
#ifdef PLANT_TRANSPOSED_UP          /* reads W2 as if it were [N,K]        */
            for (int64_t n = 0; n < N; ++n) {
                double s = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    s += swo_bf16_to_double(A[m * K + k]) *
                         swo_bf16_to_double(W2[n * K + k]);
                u[n] = s;
            }
#else
            row_times_matrix(A + m * K, W2, K, N, u);
#endif
            for (int64_t n = 0; n < N; ++n) {
                gate_up_to_y(g[n], u[n], y64 ? y64 + i * N + n : NULL,
                             ybf ? ybf + i * N + n : NULL);
            }
        }
        free(g);
        free(u);
    }
}

/*
 * Separate formulation over a column window: for each listed row m, the
 * outputs n in [c0, c1) (the same sums as swo_swiglu_rows, fewer columns).
 * Outputs are indexed by position: y64[i*(c1-c0) + j], ybf[...] hold
 * Y[rows[i], c0 + j] (either may be NULL).
 */
void swo_swiglu_block(const uint16_t *A, const uint16_t *W1, const uint16_t *W2,
                      int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                      int64_t c0, int64_t c1, double *y64, uint16_t *ybf)
{
    const int64_t w = c1 - c0;
#ifdef PLANT_BLOCK_OFFSET           /* the window starts one column late   */
    const int64_t first = c0 + 1 < N ? c0 + 1 : c0;
#else
    const int64_t first = c0;
#endif
    #pragma omp parallel
    {
        double *g = (double *)malloc((size_t)w * sizeof(double));
        double *u = (double *)malloc((size_t)w * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t m = rows[i];
            row_times_window(A + m * K, W1 + first, K, w, N, g);
            row_times_window(A + m * K, W2 + first, K, w, N, u);
            for (int64_t j = 0; j < w; ++j) {
                gate_up_to_y(g[j], u[j], y64 ? y64 + i * w + j : NULL,
                             ybf ? ybf + i * w + j : NULL);
            }
        }
        free(g);
        free(u);
    }
}

/* Separate formulation, all M rows. */
void swo_swiglu_separate(const uint16_t *A, const uint16_t *W1,
                         const uint16_t *W2, int64_t M, int64_t N, int64_t K,
                         double *y64, uint16_t *ybf)
{
    swo_swiglu_rows(A, W1, W2, N, K, NULL, M, y64, ybf);
}

/*
 * Interleaved formulation [gist: Method, Kernel-2]: one contraction against
 * W_fused [K, 2N], then pair adjacent columns: column 2n is Gate n, column
 * 2n+1 is Up n (0-based).
 */
void swo_swiglu_interleaved(const uint16_t *A, const uint16_t *Wf, int64_t M,
                            int64_t N, int64_t K, double *y64, uint16_t *ybf)
{
    #pragma omp parallel
    {
        double *d = (double *)malloc((size_t)(2 * N) * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            row_times_matrix(A + m * K, Wf, K, 2 * N, d);
            for (int64_t n = 0; n < N; ++n) {
                gate_up_to_y(d[2 * n], d[2 * n + 1],
                             y64 ? y64 + m * N + n : NULL,
                             ybf ? ybf + m * N + n : NULL);
            }
        }
        free(d);
    }
}

/*
 * Single outputs, one by one: out[i] for (rows[i], cols[i]).  Used to check
 * full-size GPU results on a sample.
 */
void swo_swiglu_points(const uint16_t *A, const uint16_t *W1, const uint16_t *W2,
                       int64_t N, int64_t K, const int64_t *rows,
                       const int64_t *cols, int64_t count, double *y64,
                       uint16_t *ybf)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = rows[i], n = cols[i];
        double g = 0.0, u = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = swo_bf16_to_double(A[m * K + k]);
            g += a * swo_bf16_to_double(W1[k * N + n]);
            u += a * swo_bf16_to_double(W2[k * N + n]);
        }
        gate_up_to_y(g, u, y64 ? y64 + i : NULL, ybf ? ybf + i : NULL);
    }
}

/* W_fused[k, 2n] = W1[k, n],  W_fused[k, 2n+1] = W2[k, n]  [gist: Kernel-2]. */
void swo_pack(const uint16_t *W1, const uint16_t *W2, uint16_t *Wf,
              int64_t K, int64_t N)
{
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t n = 0; n < N; ++n) {
#ifdef PLANT_PACK_UP_EVEN           /* puts Up in the even columns        */
            Wf[k * 2 * N + 2 * n] = W2[k * N + n];
            Wf[k * 2 * N + 2 * n + 1] = W1[k * N + n];
#else
            Wf[k * 2 * N + 2 * n] = W1[k * N + n];
            Wf[k * 2 * N + 2 * n + 1] = W2[k * N + n];
#endif
        }
    }
}

/*
 * Materialised (unfused) pipeline: Gate and Up are rounded to bf16 before
 * the activation, as an eager two-GEMM + activation pipeline stores them
 * [paper s1].  gate/up outputs are the bf16 intermediates; y is
 * bf16(SiLU(gate_bf16) * up_bf16) with one final rounding.  Any output may
 * be NULL.
 */
void swo_swiglu_materialised(const uint16_t *A, const uint16_t *W1,
                             const uint16_t *W2, int64_t M, int64_t N,
                             int64_t K, uint16_t *gate, uint16_t *up,
                             uint16_t *ybf)
{
    #pragma omp parallel
    {
        double *g = (double *)malloc((size_t)N * sizeof(double));
        double *u = (double *)malloc((size_t)N * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            row_times_matrix(A + m * K, W1, K, N, g);
            row_times_matrix(A + m * K, W2, K, N, u);
            for (int64_t n = 0; n < N; ++n) {
                const uint16_t gb = swo_double_to_bf16(g[n]);
                const uint16_t ub = swo_double_to_bf16(u[n]);
                if (gate) gate[m * N + n] = gb;
                if (up) up[m * N + n] = ub;
                if (ybf) {
                    const double y = swo_silu(swo_bf16_to_double(gb)) *
                                     swo_bf16_to_double(ub);
                    ybf[m * N + n] = swo_double_to_bf16(y);
                }
            }
        }
        free(g);
        free(u);
    }
}

/* Element-wise activation stage alone: y[i] = bf16(SiLU(g[i]) * u[i]). */
void swo_silu_mul(const uint16_t *g, const uint16_t *u, int64_t count,
                  uint16_t *ybf)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const double y = swo_silu(swo_bf16_to_double(g[i])) *
                         swo_bf16_to_double(u[i]);
        ybf[i] = swo_double_to_bf16(y);
    }
}

/*
 * Packer for weights in a linear layer's layout: W1t and W2t are [N][K]
 * (row n holds column n of W1, resp. W2).  The output is the same W_fused
 * [K, 2N] as swo_pack:  W_fused[k, 2n] = W1t[n, k],  W_fused[k, 2n+1] =
 * W2t[n, k]  [gist: Kernel-2].
 */
void swo_pack_nk(const uint16_t *W1t, const uint16_t *W2t, uint16_t *Wf,
                 int64_t K, int64_t N)
{
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t n = 0; n < N; ++n) {
#ifdef PLANT_PACK_NK_UNTRANSPOSED   /* reads [N][K] as if it were [K][N]  */
            Wf[k * 2 * N + 2 * n] = W1t[k * N + n];
            Wf[k * 2 * N + 2 * n + 1] = W2t[k * N + n];
#else
            Wf[k * 2 * N + 2 * n] = W1t[n * K + k];
            Wf[k * 2 * N + 2 * n + 1] = W2t[n * K + k];
#endif
        }
    }
}

/*
 * Down projection of the MLP block: Out[m, d] = bf16( sum_n H[m, n] W3[n, d] )
 * for H [M][N] and W3 [N][D] (D is the model width, K of the gated GEMM),
 * double, n ascending, one rounding.  out64 (unrounded) may be NULL.
 */
void swo_down_proj(const uint16_t *H, const uint16_t *W3, int64_t M, int64_t N,
                   int64_t D, double *out64, uint16_t *outbf)
{
    #pragma omp parallel
    {
        double *o = (double *)malloc((size_t)D * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            row_times_matrix(H + m * N, W3, N, D, o);
            for (int64_t d = 0; d < D; ++d) {
                if (out64) out64[m * D + d] = o[d];
                outbf[m * D + d] = swo_double_to_bf16(o[d]);
            }
        }
        free(o);
    }
}

/*
 * The gated MLP block [paper s1]: H = bf16(SiLU(A.W1) * (A.W2)) as in
 * swo_swiglu_separate, then Out = bf16(H . W3) with W3 [N][K] (the output
 * has the model width K of the input).  hbf (the bf16 H, [M][N]) is
 * written; the down projection reads H as rounded.
 */
void swo_gated_mlp(const uint16_t *A, const uint16_t *W1, const uint16_t *W2,
                   const uint16_t *W3, int64_t M, int64_t N, int64_t K,
                   uint16_t *hbf, uint16_t *outbf)
{
#ifdef PLANT_MLP_UNROUNDED_H        /* feeds the unrounded product onward   */
    double *h64 = (double *)malloc((size_t)(M * N) * sizeof(double));
    swo_swiglu_separate(A, W1, W2, M, N, K, h64, hbf);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t d = 0; d < K; ++d) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                s += h64[m * N + n] * swo_bf16_to_double(W3[n * K + d]);
            outbf[m * K + d] = swo_double_to_bf16(s);
        }
    }
    free(h64);
#else
    swo_swiglu_separate(A, W1, W2, M, N, K, NULL, hbf);
    swo_down_proj(hbf, W3, M, N, K, NULL, outbf);
#endif
}

/* ------------------------------------------------------------------------ */
/* FP8 inputs (the pages' motivation: quantisation to FP8 makes the GEMMs    */
/* cheaper, so materialisation costs relatively more [paper s1]).            */
/*                                                                           */
/* Format: OCP FP8 E4M3 -- 1 sign bit, 4 exponent bits with bias 7, 3        */
/* mantissa bits, subnormals at exponent 0 (m/8 * 2^-6), no infinities,      */
/* S.1111.111 is NaN, largest finite value 448.  Scaling: one power of two   */
/* per tensor, A ~= 2^a_exp * A8 and W_fused ~= 2^w_exp * W8, so Gate =      */
/* 2^(a_exp+w_exp) * (A8 . W1_8) and likewise Up.                             */
/* ------------------------------------------------------------------------ */

#ifdef PLANT_FP8_BIAS8              /* the exponent bias of the FNUZ variant */
#define FP8_BIAS 8
#else
#define FP8_BIAS 7
#endif

double swo_fp8_to_double(uint8_t q)
{
    const int e = (q >> 3) & 15, m = q & 7;
    double v;
    if (e == 15 && m == 7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)m, 1 - FP8_BIAS - 3);        /* (m/8) 2^(1-bias)     */
    } else {
        v = ldexp(8.0 + m, e - FP8_BIAS - 3);          /* (1 + m/8) 2^(e-bias) */
    }
    return (q & 0x80) ? -v : v;
}

/*
 * Round a double to the nearest E4M3 value, ties to even; finite values
 * beyond the largest (448), and infinities, saturate to +-448; NaN -> 0x7F.
 * For |x| in [2^e, 2^(e+1)) with e >= -6 the spacing is 2^(e-3); below 2^-6
 * it stays at the subnormal quantum 2^-9.
 */
uint8_t swo_double_to_fp8(double x)
{
    if (isnan(x)) return 0x7F;
    const uint8_t s = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (isinf(a) || a > 448.0) return (uint8_t)(s | 0x7E);
    if (a == 0.0) return s;
    int ex;
    (void)frexp(a, &ex);                      /* a in [2^(ex-1), 2^ex)      */
    int e = ex - 1;
    if (e < -6) e = -6;
    const double q = ldexp(1.0, e - 3);
    double r = nearbyint(a / q) * q;          /* exact scaling, RNE         */
    if (r > 448.0) r = 448.0;                 /* 480 is not a finite value  */
    if (r == 0.0) return s;
    int er;
    (void)frexp(r, &er);
    er -= 1;                                  /* r in [2^er, 2^(er+1))      */
    if (er < -6) return (uint8_t)(s | (uint8_t)(r / ldexp(1.0, -9)));
    const int m = (int)(r / ldexp(1.0, er - 3)) - 8;
    return (uint8_t)(s | (uint8_t)(((er + 7) << 3) | m));
}

/* q[i] = fp8(x[i] * 2^-scale_exp) for bf16 x (the scaling is exact). */
void swo_quantize_fp8(const uint16_t *x, int64_t count, int scale_exp,
                      uint8_t *q)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        q[i] = swo_double_to_fp8(ldexp(swo_bf16_to_double(x[i]), -scale_exp));
    }
}

/*
 * The fused SwiGLU GEMM on FP8 inputs, for a list of rows (rows == NULL:
 * rows 0..nrows-1): A8 [M][K]; WfT8 is W_fused stored by columns, [2N][K]
 * (row 2n = Gate column n, row 2n+1 = Up column n [gist: Kernel-2]).
 *   g = 2^(a_exp+w_exp) sum_k A8[m,k] WfT8[2n,k],  u likewise with 2n+1
 * (each product of two FP8 values is exact in double; k ascending), then
 * y = SiLU(g) u and one rounding to bf16.  Outputs by list position.
 */
void swo_swiglu_fp8_rows(const uint8_t *A8, const uint8_t *WfT8, int64_t N,
                         int64_t K, const int64_t *rows, int64_t nrows,
                         int a_exp, int w_exp, double *y64, uint16_t *ybf)
{
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = swo_fp8_to_double((uint8_t)c);
    #pragma omp parallel
    {
        double *a = (double *)malloc((size_t)K * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t m = rows ? rows[i] : i;
            for (int64_t k = 0; k < K; ++k) a[k] = table[A8[m * K + k]];
            for (int64_t n = 0; n < N; ++n) {
                const uint8_t *wg = WfT8 + (2 * n) * K;
                const uint8_t *wu = WfT8 + (2 * n + 1) * K;
                double g = 0.0, u = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    g += a[k] * table[wg[k]];
                    u += a[k] * table[wu[k]];
                }
                g = ldexp(g, a_exp + w_exp);
#ifndef PLANT_FP8_SCALE_ONCE        /* leaves Up unscaled                  */
                u = ldexp(u, a_exp + w_exp);
#endif
                gate_up_to_y(g, u, y64 ? y64 + i * N + n : NULL,
                             ybf ? ybf + i * N + n : NULL);
            }
        }
        free(a);
    }
}

/* Threads the OpenMP runtime will use for a parallel region. */
#ifdef _OPENMP
int swo_num_threads(void) { return omp_get_max_threads(); }
#else
int swo_num_threads(void) { return 1; }
#endif
