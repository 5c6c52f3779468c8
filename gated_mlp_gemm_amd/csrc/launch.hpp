// Host-side launchers of the kernels in kernels.hip.  Arguments are assumed
// validated by the C ABI layer (api.cpp); each launcher enqueues on `stream`
// and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swiglu {

// Caller-owned scratch for the split-tail schedule (may be empty: base == nullptr).
struct GemmWorkspace {
    void *base;
    uint64_t bytes;
    int cus;          // compute units of the device
    int tile;         // variant I / ablation GEMM tile: 0 = by the cost model, 256 or 128 = forced
    int tail;         // partly idle last round: 0 = by the cost model, else a TailChoice
    unsigned *counters;   // arrival counters for a split reduced in the kernel (zero between calls)
    int max_counters;     // counters available at `counters`
};
// How the tiles of a partly idle last round run (GemmWorkspace::tail).
enum TailChoice { kTailAuto = 0, kTailWhole = 1, kTailPieces = 2, kTailQuarters = 3, kTailFixup = 4 };
// Scratch that lets the single-accumulator GEMMs split the tiles of a partial
// last round along K (the same for every shape: one fp32 256 x 256 tile slot
// per compute unit).
uint64_t partials_bytes(int cus);
uint64_t workspace_bytes_for(int cus);

// Text naming the kernels (tile shape, schedule) a GEMM over an M x cols
// output would launch (snprintf semantics).
// fused_i: the variant-I GEMM (its M <= 128 tile choice differs from the
// ablation's and the down projection's).
int describe_gemm(int M, int cols, int K, const GemmWorkspace &ws, const char *epi, char *buf,
                  size_t n, bool fused_i = false);
int describe_fused_sequential(int M, int N, int K, const GemmWorkspace &ws, char *buf, size_t n);

hipError_t launch_pack(const uint16_t *W1, const uint16_t *W2, uint16_t *Wf, int64_t K,
                       int64_t N, hipStream_t stream);
// Linear-layer-layout weights W1t, W2t [N][K] -> packed [2N][K] (row interleave).
hipError_t launch_pack_nk(const uint16_t *W1t, const uint16_t *W2t, uint16_t *Wf, int64_t K,
                          int64_t N, hipStream_t stream);
hipError_t launch_silu_mul(const uint16_t *g, const uint16_t *u, uint16_t *y, int64_t count,
                           hipStream_t stream);
// lda / ldy: elements from one row of A / Y to the next (K / N when contiguous).
hipError_t launch_fused_interleaved(const uint16_t *A, int lda, const uint16_t *Wf, uint16_t *Y,
                                    int ldy, int M, int N, int K, const GemmWorkspace &ws,
                                    hipStream_t stream);
// ws: only its compute-unit count (the persistent kernel's grid) and tail
// choice are used
hipError_t launch_fused_sequential(const uint16_t *A, int lda, const uint16_t *Wf, uint16_t *Y,
                                   int ldy, int M, int N, int K, const GemmWorkspace &ws,
                                   hipStream_t stream);
// phase 0: C = A . W1 (Gate columns of W_fused), phase 1: C = A . W2 (Up columns)
hipError_t launch_gemm_store(const uint16_t *A, const uint16_t *Wf, int phase, uint16_t *C,
                             int M, int N, int K, const GemmWorkspace &ws, hipStream_t stream);
// Out [M][D] = bf16(H [M][N] . W3), W3 given K-contiguous as W3t [D][N].
hipError_t launch_down_proj(const uint16_t *H, const uint16_t *W3t, uint16_t *Out, int M, int N,
                            int D, const GemmWorkspace &ws, hipStream_t stream);
// FP8 (E4M3) path: q = fp8(x * 2^-scale_exp); variant I on FP8 operands with
// the epilogue scaling Gate and Up by `scale` (= 2^(a_exp + w_exp)).
hipError_t launch_quantize_fp8(const uint16_t *x, uint8_t *q, int64_t count, int scale_exp,
                               hipStream_t stream);
hipError_t launch_fused_interleaved_fp8(const uint8_t *A8, const uint8_t *Wf8, uint16_t *Y,
                                        int M, int N, int K, float scale,
                                        const GemmWorkspace &ws, hipStream_t stream);
hipError_t launch_fused_sequential_fp8(const uint8_t *A8, const uint8_t *Wf8, uint16_t *Y, int M,
                                       int N, int K, float scale, hipStream_t stream);
int describe_gemm_fp8(int M, int cols, int K, const GemmWorkspace &ws, char *buf, size_t n);
// Largest workgroup count any launcher uses for an M x cols output tile grid.
int64_t max_tiles(int64_t M, int64_t cols);

}  // namespace swiglu
