// HIP kernels of the fused SwiGLU GEMM library (gfx950 only).
//
// Citations are to the pages on "Tile-Level Activation Overlap for Efficient
// LLM Inference" (arXiv 2607.02521): [paper s1] = the paper's own text,
// section 1 Introduction; [abstract] = its abstract; [gist: X] = the
// gist.science technical summary, section X.
#include "launch.hpp"

#include "device.hpp"
#include "gemm_core.hpp"
#include "split_tail.hpp"

#include <cmath>
#include <cstdio>

namespace swiglu {

// ---------------------------------------------------------------------------
// Weight packer [gist: Method, Kernel-2]: W_fused[k][2n] = W1[k][n],
// W_fused[k][2n+1] = W2[k][n], stored column-major: column c of W_fused is
// the K-contiguous row c of the [2N][K] array the MFMA loaders read.  One
// workgroup transposes a 64(k) x 64(n) block of W1 and of W2 through LDS
// (coalesced 16-byte loads of rows of W, coalesced 16-byte stores of rows of
// the packed array).  A pure 16-bit permutation.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ W1,
                                                   const uint16_t *__restrict__ W2,
                                                   uint16_t *__restrict__ Wf, int K, int N) {
    constexpr int T = 64, PITCH = T + 8;   // row pitch 144 B keeps 16-byte alignment
    __shared__ __attribute__((aligned(16))) uint16_t tile[2][T][PITCH];
    const int k0 = blockIdx.y * T;
    const int n0 = blockIdx.x * T;
    const int tid = threadIdx.x;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint16_t *W = w == 0 ? W1 : W2;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + i * 256;           // chunk of the 64 x 64 block
            const int row = c >> 3, cc = c & 7;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (k0 + row < K && n0 + cc * 8 < N)
                v = gload16(W + (int64_t)(k0 + row) * N + n0 + cc * 8);
            *reinterpret_cast<u32x4 *>(&tile[w][row][cc * 8]) = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * 256;               // chunk of the 128 output rows x 64 k
        const int orow = c >> 3, kc = c & 7;
        const int j = orow >> 1, w = orow & 1;     // even rows: Gate (W1), odd rows: Up (W2)
        if (n0 + j >= N || k0 + kc * 8 >= K) continue;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = static_cast<uint32_t>(tile[w][kc * 8 + 2 * e][j]) |
                   (static_cast<uint32_t>(tile[w][kc * 8 + 2 * e + 1][j]) << 16);
        gstore16(Wf + (int64_t)(2 * (n0 + j) + w) * K + k0 + kc * 8, v);
    }
}

// ---------------------------------------------------------------------------
// Weight packer for weights in a linear layer's layout, W1t and W2t [N][K]
// (row n holds column n of W1, resp. W2): the packed [2N][K] array takes row
// n of W1t as its row 2n and row n of W2t as its row 2n+1 [gist: Method,
// Kernel-2], so the pack is a row interleave: every thread copies one 16-byte
// chunk, coalesced on both sides (grid-stride).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_nk_kernel(const uint16_t *__restrict__ W1t,
                                                      const uint16_t *__restrict__ W2t,
                                                      uint16_t *__restrict__ Wf,
                                                      int64_t chunks_per_row, int64_t nchunks) {
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t orow = c / chunks_per_row, kc = c - orow * chunks_per_row;
        const uint16_t *src = (orow & 1) ? W2t : W1t;
        const u32x4 v = gload16(src + ((orow >> 1) * chunks_per_row + kc) * 8);
        gstore16(Wf + c * 8, v);
    }
}

// ---------------------------------------------------------------------------
// Ablation activation stage: Y = bf16(SiLU(gate) * up), fp32 arithmetic,
// one rounding.  HBM-bound: 8 elements (three 16-byte accesses) per thread
// per iteration, grid-stride.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
    return __builtin_bit_cast(float, v & 0xFFFF0000u);
}

__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t *__restrict__ g,
                                                       const uint16_t *__restrict__ u,
                                                       uint16_t *__restrict__ y,
                                                       int64_t nchunks) {
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const u32x4 gv = gload16(g + c * 8);
        const u32x4 uv = gload16(u + c * 8);
        u32x4 out;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            out[d] = pack_bf16x2(silu(bf16_lo(gv[d])) * bf16_lo(uv[d]),
                                 silu(bf16_hi(gv[d])) * bf16_hi(uv[d]));
        }
        gstore16(y + c * 8, out);
    }
}

// ---------------------------------------------------------------------------
// FP8 quantizer: q = E4M3(x * 2^-scale_exp) for bf16 x, round to nearest even,
// finite values beyond 448 (and infinities) saturated to +-448, NaN -> 0x7F.
// The scaling is exact in fp32 (a power of two); values below 2^-6 round on
// the subnormal grid of spacing 2^-9.  16 values (32 bytes in, 16 out) per
// thread per iteration, grid-stride.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fp8_e4m3_rne_sat(float v) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(v);
    if (a != a) return 0x7Fu;                                   // NaN
    if (a >= 464.0f) return sign | 0x7Eu;                       // rounds past 448: saturate
    if (a < 0.015625f) {                                        // below 2^-6: multiples of 2^-9
        const uint32_t m = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));   // 0..8, exact
        return sign | m;                                        // m = 8 is 2^-6 (code 0x08)
    }
    // normal: keep 3 of the 23 fraction bits, round to nearest even on the rest
    const uint32_t ab = bits & 0x7FFFFFFFu;
    const uint32_t r = ab + 0x7FFFFu + ((ab >> 20) & 1u);
    const uint32_t e = (r >> 23) - 127u + 7u;                   // 1..15 (a < 464)
    const uint32_t code = (e << 3) | ((r >> 20) & 7u);
    return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t *__restrict__ x,
                                                           uint8_t *__restrict__ q,
                                                           float inv_scale, int64_t nchunks) {
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const u32x4 lo = gload16(x + c * 16);
        const u32x4 hi = gload16(x + c * 16 + 8);
        u32x4 out;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u32x4 &src = d < 2 ? lo : hi;
            const uint32_t w0 = src[(d & 1) * 2], w1 = src[(d & 1) * 2 + 1];
            out[d] = fp8_e4m3_rne_sat(bf16_lo(w0) * inv_scale) |
                     (fp8_e4m3_rne_sat(bf16_hi(w0) * inv_scale) << 8) |
                     (fp8_e4m3_rne_sat(bf16_lo(w1) * inv_scale) << 16) |
                     (fp8_e4m3_rne_sat(bf16_hi(w1) * inv_scale) << 24);
        }
        *reinterpret_cast<u32x4 *>(q + c * 16) = out;
    }
}

// Output stores of the epilogues go through a buffer resource that spans the
// tile's valid rows of a row-major [M][ld] bf16 matrix.  A store whose offset
// lies past those rows, or that carries kOutOfRange (the column is past the
// end), is dropped by the hardware, so an epilogue needs neither a branch nor
// a 64-bit address per element: one 32-bit lane offset per column group plus
// a per-row term that is the same for all lanes.  With ld <= 2^22 and at most
// 256 rows every offset stays below 2^32 (kOutOfRange + row term included).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(uint16_t *base, int m0, int rows,
                                                           int ld) {
    return make_rsrc(base + static_cast<int64_t>(m0) * ld,
                     static_cast<uint32_t>(rows) * static_cast<uint32_t>(ld) * 2u);
}
// `off` is the lane's byte offset and `soff` a uniform one (a row term):
// both count in the range check, so a row past the resource is dropped too,
// and the uniform part costs no vector instruction.
__device__ __forceinline__ void store_b16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff,
                                          uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, static_cast<int>(off), static_cast<int>(soff), 0);
}
// Variant I's output Y is written once and never read back by the kernel.
// With the 32x32 MFMA layout (FP8 operands; bf16 at M <= 128) its stores
// carry the non-temporal hint (nt), so they do not displace the A and weight
// panels that tiles still running read from L2 and the Infinity Cache:
// measured against plain stores, FP8 7.6-10.7 % faster at M=2048 K=1536
// N=8960 and M=512 K=3584 N=18944.  With the 16x16 layout a store covers
// 32-byte pieces of four rows, and under the hint partly written lines left
// L2 early: 2.1-2.4x Y's bytes written (plain stores: 1.0x), and plain stores
// are faster on all four bf16 workloads above M = 128 (1.2-4.2 %, same box).
// Variant S keeps plain stores, and so do the ablation's Gate and Up, which
// the next kernel reads back.
template <bool kNt>
__device__ __forceinline__ void store_y_b16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff,
                                            uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, static_cast<int>(off), static_cast<int>(soff),
                                          kNt ? 2 /* nt */ : 0);
}
// The high 16 bits of v, with the same range check and hint
// (buffer_store_short_d16_hi, which the store builtin does not produce: it
// would shift first).
template <bool kNt>
__device__ __forceinline__ void store_y_b16_hi(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               uint32_t soff, uint32_t v) {
    if constexpr (kNt)
        asm volatile("buffer_store_short_d16_hi %0, %1, %2, %3 offen nt" ::"v"(v), "v"(off),
                     "s"(r), "s"(soff)
                     : "memory");
    else
        asm volatile("buffer_store_short_d16_hi %0, %1, %2, %3 offen" ::"v"(v), "v"(off), "s"(r),
                     "s"(soff)
                     : "memory");
}
// The same without the hint (variant S).
__device__ __forceinline__ void store_b16_hi(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff,
                                             uint32_t v) {
    store_y_b16_hi<false>(r, off, soff, v);
}

// Lane byte offsets of the two 16-column groups of a 32x32 accumulator block
// in a row-major bf16 matrix with ld elements a row (col_r(r) / 16 selects
// one): the lane's row `lrow` (relative to the store resource's first row),
// columns c0 and c0 + 16 (relative to `col_base`); a column at or past
// `cols_valid` gets kOutOfRange.  MI = 32 blocks use only the first.
__device__ __forceinline__ void lane_offsets(uint32_t (&voff)[2], uint32_t lrow, int c0,
                                             int cols_valid, int col_base, int ld) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = c0 + 16 * h;
        voff[h] = c < cols_valid ? (lrow * static_cast<uint32_t>(ld) +
                                    static_cast<uint32_t>(col_base + c)) * 2u
                                 : kOutOfRange;
    }
}

// ---------------------------------------------------------------------------
// Variant I [gist: Method, Kernel-2]: one GEMM D = A . W_fused over tiles of
// the [M, 2N] grid; the epilogue pairs each Gate accumulator column D[m,2n]
// with its Up partner D[m,2n+1] and stores SiLU(D[m,2n]) * D[m,2n+1].
//
// Epilogues work in units of accumulator blocks: unit<S>(a0, a1, u, ...)
// finishes unit u (u < TM * TN / unit_blocks<S>()) of a wave from its
// unit_blocks<S>() 32x32 blocks a0 (and a1), given in order.
//
// Paired layout (wave tiles an even number of 32x32 blocks wide): the weight
// panel is loaded de-interleaved (KMajor::pairs), so block 2p of a wave holds
// the Gate columns and block 2p+1 the Up columns of the same 32 outputs, each
// output column in one lane: every lane finishes its own 16 outputs of the
// unit with no lane exchange, and one conversion packs two of them.
// Interleaved layout (one block wide, the 128x64 tiles): in the 32x32 MFMA
// accumulator layout every lane holds one column, so a Gate column 2n sits in
// an even lane and its Up partner 2n+1 in the next lane, at the same register
// indices; the even lane finishes registers 0..7 (it receives the partner's
// Up values), the odd lane registers 8..15 (it receives Gate values), one DPP
// lane swap per output.
// ---------------------------------------------------------------------------
// kScaled: the accumulators hold D / scale (FP8 operands with power-of-two
// tensor scales), so Gate and Up are scale * D before the activation.
template <bool kScaled>
struct PairMulEpilogueT {
    uint16_t *Y;
    int M, N;
    int ldy;       // elements from one row of Y to the next (>= N)
    float scale;   // used only when kScaled

    __device__ __forceinline__ float scaled(float x) const {
        if constexpr (kScaled) return x * scale;
        else return x;
    }

    template <class S>
    static constexpr bool paired() { return S::TN % 2 == 0; }
    template <class S>
    static constexpr int unit_blocks() { return paired<S>() ? 2 : 1; }

    // kFromAcc: the blocks are MFMA accumulators (AGPRs), read out in order
    // (read_acc); else ordinary values (the split reduction's sums).
    template <class S, bool kFromAcc = true>
    __device__ __forceinline__ void unit(const typename S::Acc &a0, const typename S::Acc &a1,
                                         int u, int m0, int n0, int tid) const {
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int wm = wave / S::WN, wn = wave % S::WN;
        const int rows_valid = min(S::BM, M - m0);
        const int y0 = n0 / 2;                 // first Y column of the tile
        const int ycols_valid = min(S::BN / 2, N - y0);
        const __amdgpu_buffer_rsrc_t r = out_rsrc(Y, m0, rows_valid, ldy);
        uint32_t voff[2];
        if constexpr (paired<S>()) {
            constexpr int kPairBlocks = S::TN / 2;
            const int tm = u / kPairBlocks, tp = u % kPairBlocks;
            const typename S::Acc &g = a0, &up = a1;
            const uint32_t lrow = static_cast<uint32_t>(wm * S::kWaveM + tm * 32 + S::row_l(lane));
            lane_offsets(voff, lrow, wn * (S::kWaveN / 2) + tp * 32 + S::col_l(lane), ycols_valid,
                         y0, ldy);
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                // registers i, i+1: rows row_r(i) and row_r(i) + 1, one column
                const float g0 = scaled(acc_value<kFromAcc>(g.get(i)));
                const float g1 = scaled(acc_value<kFromAcc>(g.get(i + 1)));
                const float u0 = scaled(acc_value<kFromAcc>(up.get(i)));
                const float u1 = scaled(acc_value<kFromAcc>(up.get(i + 1)));
                const uint32_t v = pack_bf16x2(silu(g0) * u0, silu(g1) * u1);
                const uint32_t roff =
                    static_cast<uint32_t>(S::row_r(i)) * static_cast<uint32_t>(ldy) * 2u;
                store_y_b16<S::MI == 32>(r, voff[S::col_r(i) / 16], roff, static_cast<uint16_t>(v));
                store_y_b16_hi<S::MI == 32>(r, voff[S::col_r(i) / 16],
                                            roff + static_cast<uint32_t>(ldy) * 2u, v);
            }
        } else {
            const int tm = u / S::TN, tn = u % S::TN;
            const bool odd = lane & 1;
            // even lanes finish accumulator registers 0..7, odd lanes 8..15,
            // which sit 16 rows further down (row_r(8 + p) = 16 + row_r(p))
            const uint32_t lrow = static_cast<uint32_t>(wm * S::kWaveM + S::row_l(lane) + (odd ? 16 : 0));
            // the Y column of the pair (Gate column, Up column) the lane is in
            const int c0 = wn * S::kWaveN + tn * 32 + (S::col_l(lane) & ~1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ycol = (c0 + 16 * h) >> 1;
                voff[h] = ycol < ycols_valid
                              ? (lrow * static_cast<uint32_t>(ldy) + static_cast<uint32_t>(y0 + ycol)) * 2u
                              : kOutOfRange;
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const float lo = a0.get(p), hi = a0.get(8 + p);
                const float recv = swap_adjacent_lanes(by_lane_parity(hi, lo));
                const float gate = scaled(by_lane_parity(lo, recv));
                const float upv = scaled(by_lane_parity(recv, hi));
                const uint32_t roff = static_cast<uint32_t>(tm * 32 + S::row_r(p)) *
                                      static_cast<uint32_t>(ldy) * 2u;
                store_y_b16<S::MI == 32>(r, voff[S::col_r(p) / 16], roff, to_bf16(silu(gate) * upv));
            }
        }
    }

    template <class S>
    __device__ __forceinline__ void apply(const typename S::Acc (&acc)[S::TM][S::TN], int m0,
                                          int n0, int tid) const {
        constexpr int kUnits = S::TM * S::TN / unit_blocks<S>();
        __builtin_amdgcn_sched_barrier(0);   // nothing of the epilogue moves into the mainloop
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            if constexpr (paired<S>()) {
                const int tm = u / (S::TN / 2), tp = u % (S::TN / 2);
                unit<S>(acc[tm][2 * tp], acc[tm][2 * tp + 1], u, m0, n0, tid);
            } else {
                unit<S>(acc[u / S::TN][u % S::TN], acc[u / S::TN][u % S::TN], u, m0, n0, tid);
            }
            __builtin_amdgcn_sched_barrier(0);   // one unit's temporaries live at a time
        }
    }

    // Accumulator block of unit u's k-th block (index tm * TN + tn).
    template <class S>
    __device__ __forceinline__ static int unit_block(int u, int k) {
        if constexpr (paired<S>())
            return (u / (S::TN / 2)) * S::TN + 2 * (u % (S::TN / 2)) + k;
        else
            return u;
    }
};

using PairMulEpilogue = PairMulEpilogueT<false>;
using PairMulEpilogueFp8 = PairMulEpilogueT<true>;

// Ablation GEMM epilogue: C = bf16(acc), so that Gate and Up are materialised
// as an eager pipeline does [paper s1].
struct StoreEpilogue {
    uint16_t *C;
    int M, N;

    template <class S, bool kFromAcc = true>
    __device__ __forceinline__ void block(const typename S::Acc &a, int tm, int tn, int m0,
                                          int n0, int tid) const {
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int wm = wave / S::WN, wn = wave % S::WN;
        const int rows_valid = min(S::BM, M - m0);
        const int cols_valid = min(S::BN, N - n0);
        const __amdgpu_buffer_rsrc_t r = out_rsrc(C, m0, rows_valid, N);
        const uint32_t lrow = static_cast<uint32_t>(wm * S::kWaveM + S::row_l(lane));
        uint32_t voff[2];
        lane_offsets(voff, lrow, wn * S::kWaveN + tn * 32 + S::col_l(lane), cols_valid, n0, N);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t roff =
                static_cast<uint32_t>(tm * 32 + S::row_r(i)) * static_cast<uint32_t>(N) * 2u;
            store_b16(r, voff[S::col_r(i) / 16], roff, to_bf16(acc_value<kFromAcc>(a.get(i))));
        }
    }

    template <class S>
    __device__ __forceinline__ void apply(const typename S::Acc (&acc)[S::TM][S::TN], int m0,
                                          int n0, int tid) const {
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < S::TN; ++tn) {
                block<S>(acc[tm][tn], tm, tn, m0, n0, tid);
                __builtin_amdgcn_sched_barrier(0);   // one block's temporaries live at a time
            }
    }

    template <class S>
    static constexpr bool paired() { return false; }
    template <class S>
    static constexpr int unit_blocks() { return 1; }
    template <class S, bool kFromAcc = true>
    __device__ __forceinline__ void unit(const typename S::Acc &a0, const typename S::Acc &, int u,
                                         int m0, int n0, int tid) const {
        block<S, kFromAcc>(a0, u / S::TN, u % S::TN, m0, n0, tid);
    }
    template <class S>
    __device__ __forceinline__ static int unit_block(int u, int) { return u; }
};

// K steps [kb, ke) of the S tile at (m0, n0) of D = A . B^T, into acc.
// The K steps [0, len) of one tile into `acc`.  With 16x16 MFMAs the first
// step's MFMAs start the accumulators (C = 0): no vector instructions zero its
// 256 registers first.  32x32 MFMAs accumulate onto zeros (zero_acc_mi32
// before the prologue's wait, while the loads are in flight).
template <class S>
__device__ __forceinline__ void zero_acc_mi32(typename S::Acc (&acc)[S::TM][S::TN]) {
    if constexpr (S::MI != 16) zero_acc<S>(acc);
}
template <class S, class Issue>
__device__ __forceinline__ void run_tile(Pipeline<S> &pl, const Issue &issue, int len,
                                         typename S::Acc (&acc)[S::TM][S::TN]) {
    if constexpr (S::MI == 16) pl.run_init(issue, 0, len, len, acc);
    else pl.run(issue, 0, len, len, acc);
}

template <class S, bool kEven = false>
__device__ __forceinline__ void tile_mainloop(SWIGLU_LDS char *lds, const KMajor &A,
                                              const KMajor &B, int M, int K, int m0, int n0,
                                              int kb, int ke, int nk,
                                              typename S::Acc (&acc)[S::TM][S::TN]) {
    Pipeline<S> pl;
    pl.init(lds);
    TileLoader<S> ld;
    ld.init(A, m0, B, n0, K);
    const int len = ke - kb;
    // steps past the range load nothing (K step nk is past the end of K)
    auto issue = [&](int s, int part, SWIGLU_LDS char *dst, int j) {
        ld.template issue<kEven>(s < len ? kb + s : nk, part, dst, j);
    };
    zero_acc_mi32<S>(acc);
    pl.prologue(issue);
    run_tile<S>(pl, issue, len, acc);
    pl.drain(acc);
}

// The quarter-size tile of a 4-wave shape S, used for a tail round: half the
// rows and columns, with as many stages (up to 4) as S's LDS holds, so that a
// lone workgroup on a CU still keeps several K steps of loads in flight.
template <class S>
constexpr bool kQuarterable =
    S::kOccupancy == 1 && S::kWaves == 4 && S::BM % 128 == 0 && S::BN % 128 == 0;

template <class S>
struct QuarterOf {
    static constexpr int kStage = (S::BM / 2 + S::BN / 2) * S::kRowBytes;
    static constexpr int kStages = S::kLdsBytes / kStage < 4 ? S::kLdsBytes / kStage : 4;
    using type = TileShape<S::BM / 2, S::BN / 2, S::BK, 2, 2, kStages, S::EB, kStages, S::MI>;
};

enum TailMode { kTailNone = 0, kTailSplit = 1, kTailQuarter = 2, kTailReduceInKernel = 3 };

// One accumulator per tile: D = A . B^T over the tiles of `sch`, then `epi`.
// Persistent: workgroup b runs whole tiles b, b + grid, ... below sch.dp
// (XCD-ordered), one after the other; before the epilogue of each it puts the
// first K steps of its next tile in flight, so their load latency hides behind
// the epilogue and no workgroup launch sits between tiles.  Then it takes its
// share of the tiles [dp, dp + split_tiles) of a partly idle last round:
//  - with kTailSplit: work item j (j = b, b + grid, ...) is piece j % pieces
//    of split tile dp + j / pieces, which stores its partial (split_tail.hpp)
//    for split_reduce_kernel to finish;
//  - with kTailQuarter: work item q is quarter q % 4 (row half q/2 % 2, column
//    half q % 2) of tile dp + q / 4, run whole as a quarter-size tile.
//
// kEven: K is a multiple of BK (the loads' offsets are fixed per tile, see
// PanelLoader::issue); the kernel runs the body compiled for its K.
template <class S, class Epi, int TAIL, bool kEven>
__device__ __forceinline__ void gemm_tiles_body(char *smem, const KMajor &Ak, const KMajor &B,
                                                int M, int K, const Epi &epi,
                                                const Schedule &sch) {
    SWIGLU_LDS char *lds = (SWIGLU_LDS char *)smem;
    const int b = blockIdx.x;
    const int grid = sch.grid;

    if (b < sch.dp) {
        Pipeline<S> pl;
        pl.init(lds);
        TileLoader<S> ld;
        int j = b, tm, tn;
        tile_coords(xcd_order(j, sch.dp), sch.tiles_m, sch.tiles_n, sch.group_m, tm, tn);
        ld.init(Ak, tm * S::BM, B, tn * S::BN, K);
        const int nk = sch.nk;
        // steps past the end load nothing (K step nk is past the end of K)
        auto issue = [&](int s, int part, SWIGLU_LDS char *dst, int j) {
            ld.template issue<kEven>(s < nk ? s : nk, part, dst, j);
        };
        pl.prologue_issue(issue);
        for (; j < sch.dp; j += grid) {
            typename S::Acc acc[S::TM][S::TN];
            zero_acc_mi32<S>(acc);
            pl.prologue_wait();
            run_tile<S>(pl, issue, nk, acc);
            pl.drain(acc);
            const int m0 = tm * S::BM, n0 = tn * S::BN;
            if (j + grid < sch.dp) {
                tile_coords(xcd_order(j + grid, sch.dp), sch.tiles_m, sch.tiles_n, sch.group_m, tm,
                            tn);
                ld.init(Ak, tm * S::BM, B, tn * S::BN, K);
                pl.prologue_issue(issue);
            }
            epi.template apply<S>(acc, m0, n0, threadIdx.x);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if constexpr (TAIL == kTailQuarter) {
        using Q = typename QuarterOf<S>::type;
        static_assert(Q::kLdsBytes <= S::kLdsBytes, "quarter ring fits the tile's LDS");
        const int nq = 4 * sch.split_tiles;
        for (int i = b; i < nq; i += grid) {
            const int q = xcd_order(i, nq);
            int tm, tn;
            tile_coords(sch.dp + q / 4, sch.tiles_m, sch.tiles_n, sch.group_m, tm, tn);
            const int m0 = tm * S::BM + ((q >> 1) & 1) * Q::BM;
            const int n0 = tn * S::BN + (q & 1) * Q::BN;
            if (m0 >= M || n0 >= B.rows) continue;   // quarter wholly past the output's edge
            typename Q::Acc acc[Q::TM][Q::TN];
            tile_mainloop<Q, kEven>(lds, Ak, B, M, K, m0, n0, 0, sch.nk, sch.nk, acc);
            epi.template apply<Q>(acc, m0, n0, threadIdx.x);
        }
    } else if constexpr (TAIL == kTailReduceInKernel) {
        // every tile split, reduced by its last piece (split_tail.hpp); the
        // arrival count is broadcast through LDS word 0 (the ring is idle
        // between work items)
        unsigned *arrival = reinterpret_cast<unsigned *>(smem);
        const int np = sch.split_tiles * sch.pieces;
        for (int j = b; j < np; j += grid) {
            const int i = j / sch.pieces;
            const int piece = j % sch.pieces;
            const int kb = piece * sch.nk / sch.pieces;
            const int ke = (piece + 1) * sch.nk / sch.pieces;
            int tm, tn;
            tile_coords(sch.dp + i, sch.tiles_m, sch.tiles_n, sch.group_m, tm, tn);
            typename S::Acc acc[S::TM][S::TN];
            tile_mainloop<S, kEven>(lds, Ak, B, M, K, tm * S::BM, tn * S::BN, kb, ke, sch.nk, acc);
            const float *slots = sch.partials + static_cast<int64_t>(i) * sch.pieces * S::BM * S::BN;
            store_partial_coherent<S>(sch.partials + static_cast<int64_t>(j) * S::BM * S::BN,
                                      acc, threadIdx.x);
            wait_vmcnt<0>();   // this wave's partial is visible device-wide
            __syncthreads();   // ... and every wave's
            if (threadIdx.x == 0)
                *arrival = __hip_atomic_fetch_add(sch.counters + i, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const unsigned seen = *arrival;
            __syncthreads();   // read by all before the next item's loads reuse LDS
            if (seen + 1 != static_cast<unsigned>(sch.pieces)) continue;
            // the last piece: the counter is free for the next call
            if (threadIdx.x == 0)
                __hip_atomic_store(sch.counters + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            constexpr int kUnitBlocks = Epi::template unit_blocks<S>();
            constexpr int kUnits = S::TM * S::TN / kUnitBlocks;
#pragma unroll
            for (int u = 0; u < kUnits; ++u) {
                typename S::Acc a[kUnitBlocks];
#pragma unroll
                for (int k = 0; k < kUnitBlocks; ++k) {
                    const int blk = Epi::template unit_block<S>(u, k);
                    a[k] = sum_pieces_fixup<S>(slots, sch.pieces, piece, acc, blk / S::TN,
                                               blk % S::TN, threadIdx.x);
                }
                epi.template unit<S, false>(a[0], a[kUnitBlocks - 1], u, tm * S::BM, tn * S::BN,
                                            threadIdx.x);
                __builtin_amdgcn_sched_barrier(0);   // one unit's temporaries live at a time
            }
        }
    } else if constexpr (TAIL == kTailSplit) {
        const int np = sch.split_tiles * sch.pieces;
        for (int j = b; j < np; j += grid) {
            const int t = sch.dp + j / sch.pieces;
            const int piece = j % sch.pieces;
            const int kb = piece * sch.nk / sch.pieces;
            const int ke = (piece + 1) * sch.nk / sch.pieces;
            int tm, tn;
            tile_coords(t, sch.tiles_m, sch.tiles_n, sch.group_m, tm, tn);
            typename S::Acc acc[S::TM][S::TN];
            tile_mainloop<S, kEven>(lds, Ak, B, M, K, tm * S::BM, tn * S::BN, kb, ke, sch.nk, acc);
            store_partial<S>(sch.partials + static_cast<int64_t>(j) * S::BM * S::BN, acc,
                             threadIdx.x);
        }
    }
}
template <class S, class Epi, int TAIL>
__global__ __launch_bounds__(S::kThreads, S::kOccupancy) void gemm_tiles_kernel(
    KMajor Ak, KMajor B, int M, int K, Epi epi, Schedule sch) {
    __shared__ __attribute__((aligned(16))) char smem[S::kLdsBytes];
    if (K % S::BK == 0) gemm_tiles_body<S, Epi, TAIL, true>(smem, Ak, B, M, K, epi, sch);
    else gemm_tiles_body<S, Epi, TAIL, false>(smem, Ak, B, M, K, epi, sch);
}

// The split tiles' epilogue: one single-wave workgroup per (split tile, GEMM
// wave, epilogue unit), so the partials' reads spread over as many CUs as
// possible (against four waves per workgroup: the M=128 down projection,
// 18 pieces, 15.6 -> 14.3 us a call; M=2048 K=1536 N=8960 with a 5-way split
// tail 121.1 -> 119.4 us; same results).  The wave takes the
// registers of the GEMM wave it stands for -- its lane l holds what GEMM
// thread 64 w + l held, summed over the pieces -- so the epilogue's lane
// layout is the GEMM's.
template <class S, class Epi>
__global__ __launch_bounds__(64) void split_reduce_kernel(Epi epi, Schedule sch) {
    constexpr int kUnitBlocks = Epi::template unit_blocks<S>();
    constexpr int kUnits = S::TM * S::TN / kUnitBlocks;
    constexpr int kPerTile = S::kWaves * kUnits;
    const int item = blockIdx.x;
    const int i = item / kPerTile;                 // split tile
    const int w = (item % kPerTile) / kUnits;      // GEMM wave
    const int u = item % kUnits;                   // epilogue unit
    const int x = w * 64 + static_cast<int>(threadIdx.x & 63);
    typename S::Acc a[kUnitBlocks];
#pragma unroll
    for (int k = 0; k < kUnitBlocks; ++k)
        a[k] = sum_pieces<S>(sch, i, Epi::template unit_block<S>(u, k), x);
    int tm, tn;
    tile_coords(sch.dp + i, sch.tiles_m, sch.tiles_n, sch.group_m, tm, tn);
    epi.template unit<S, false>(a[0], a[kUnitBlocks - 1], u, tm * S::BM, tn * S::BN, x);
}

// ---------------------------------------------------------------------------
// Variant S [abstract; gist: Method, Kernel-1]: per output tile, the Gate
// contraction, then SiLU on the register-resident Gate accumulator while the
// loads of the next Up tiles are in flight, then the Up contraction and the
// multiply-and-store epilogue.  The prefetch runs straight across the Gate->Up
// boundary: the last Gate step already stages Up tile 0, and Up tile 1 is
// requested before the SiLU pass starts, so SiLU overlaps those loads (and the
// scheduler may interleave it with the first Up MFMAs, which use other
// registers).
// ---------------------------------------------------------------------------
template <class S>
//
// On FP8 operands (S::EB == 1) the accumulators hold D / scale: Gate and Up
// are scaled by `scale` (= 2^(a_exp + w_exp)) before SiLU and the product.
__global__ __launch_bounds__(S::kThreads, S::kOccupancy) void fused_sequential_kernel(
    const void *__restrict__ A, const void *__restrict__ Wf, uint16_t *__restrict__ Y,
    int M, int N, int K, int lda, int ldy, float scale, int tiles_m, int tiles_n) {
    constexpr bool kScaled = S::EB == 1;
    __shared__ __attribute__((aligned(16))) char smem[S::kLdsBytes];
    SWIGLU_LDS char *lds = (SWIGLU_LDS char *)smem;

    int tm_, tn_;
    tile_coords(tiles_m, tiles_n, 8, tm_, tn_);
    const int m0 = tm_ * S::BM;
    const int n0 = tn_ * S::BN;            // first output (Y) column of the tile
    const int rows_valid = min(S::BM, M - m0);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int nk = (K + S::BK - 1) / S::BK;

    // One step sequence of 2*nk K steps: steps [0, nk) contract against the
    // Gate columns of W_fused (even packed rows), steps [nk, 2nk) against the
    // Up columns (odd packed rows); the loads run ahead across the boundary.
    TileLoader<S> ld;
    ld.init(KMajor{A, M, 1, 0, 0, lda}, m0, KMajor{Wf, N, 2, 0}, n0, K);
    PanelLoader<S, S::BN, S::kDmaB> up;
    up.init(KMajor{Wf, N, 2, 1}, n0, K);
    auto issue = [&](int t, int part, SWIGLU_LDS char *dst, int j) {
        if (t < nk) ld.issue(t, part, dst, j);
        else ld.issue(t - nk, part, dst, j, up);   // t - nk >= nk loads nothing
    };
    Pipeline<S> pl;
    pl.init(lds);
    typename S::Acc g[S::TM][S::TN], u[S::TM][S::TN];
    zero_acc<S>(g);
    zero_acc<S>(u);

    constexpr int kBlocks = S::TM * S::TN;
    constexpr int kSiluSteps = (kBlocks + S::kKSub - 1) / S::kKSub;
    // Gate loop
    pl.prologue(issue);
    pl.run(issue, 0, nk, 2 * nk, g);

    // SiLU window: the first Up K steps run with one 32x32 Gate block activated
    // per k-substep, so the VALU/transcendental work interleaves with the Up
    // MFMAs (independent registers) while the Up tiles stream into LDS.
#pragma unroll
    for (int j = 0; j < kSiluSteps; ++j) {
        if (j < nk) {
            pl.step(issue, nk + j, 2 * nk, u, [&](int ks) {
                const int b = j * S::kKSub + ks;
                if (b < kBlocks) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float x = g[b / S::TN][b % S::TN].get(i);
                        if constexpr (kScaled) x *= scale;
                        g[b / S::TN][b % S::TN].set(i, silu(x));
                    }
                }
            });
        }
    }
    // (only when K is shorter than the window) the blocks not yet activated
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
        if (b >= nk * S::kKSub) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = g[b / S::TN][b % S::TN].get(i);
                if constexpr (kScaled) x *= scale;
                g[b / S::TN][b % S::TN].set(i, silu(x));
            }
        }
    }
    // rest of the Up loop
    pl.run(issue, nk + kSiluSteps, 2 * nk, 2 * nk, u);
    pl.drain();

    // multiply and store (two rows per conversion, through a buffer resource
    // over the tile's valid rows, as variant I's epilogue)
    const int cols_valid = min(S::BN, N - n0);
    const __amdgpu_buffer_rsrc_t r = out_rsrc(Y, m0, rows_valid, ldy);
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm) {
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn) {
            const uint32_t lrow = static_cast<uint32_t>(wm * S::kWaveM + tm * 32 + S::row_l(lane));
            uint32_t voff[2];
            lane_offsets(voff, lrow, wn * S::kWaveN + tn * 32 + S::col_l(lane), cols_valid, n0,
                         ldy);
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                float u0 = u[tm][tn].get(i), u1 = u[tm][tn].get(i + 1);
                if constexpr (kScaled) {
                    u0 *= scale;
                    u1 *= scale;
                }
                const uint32_t v = pack_bf16x2(g[tm][tn].get(i) * u0, g[tm][tn].get(i + 1) * u1);
                const uint32_t roff =
                    static_cast<uint32_t>(S::row_r(i)) * static_cast<uint32_t>(ldy) * 2u;
                store_b16(r, voff[S::col_r(i) / 16], roff, static_cast<uint16_t>(v));
                store_b16_hi(r, voff[S::col_r(i) / 16], roff + static_cast<uint32_t>(ldy) * 2u, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Variant S, persistent [abstract; gist: Method, Kernel-1]: the same
// sequence per output tile (Gate contraction, SiLU on the register-resident
// Gate accumulator while the first Up steps run, Up contraction, multiply and
// store), on tiles as large as variant I's in registers -- BM x BN outputs
// with BM x BN Gate and BM x BN Up accumulators -- and with variant I's
// persistent loop: workgroup b runs tiles b, b + grid, ... (XCD-ordered), and
// puts the first K steps of its next tile in flight before the epilogue of
// the current one.  bf16 operands; 16x16 MFMAs.
// ---------------------------------------------------------------------------
// SiLU on a Gate accumulator block of 16x16 quads, each quad written back to
// its AGPRs (the empty tie keeps the compiler from moving the activated block
// into VGPRs, which the Up loop's fragments need).
// After the last assembly MFMA into `acc`: wait until its results are
// written, and redefine the accumulators after that wait, so that no copy
// the compiler makes of them (it does not know the MFMAs' latency) can read
// them earlier.
template <class S>
__device__ __forceinline__ void settle_acc(typename S::Acc (&acc)[S::TM][S::TN]) {
    wait_mfma_results();
#pragma unroll
    for (int a = 0; a < S::TM; ++a)
#pragma unroll
        for (int c = 0; c < S::TN; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) asm volatile("" : "+a"(acc[a][c].v[q]));
}

// The S epilogue of one tile: Y = g * Up with g = SiLU(Gate), two rows per conversion,
// through a buffer resource over the tile's valid rows.
template <class S>
__device__ __forceinline__ void seq_epilogue(const typename S::Acc (&g)[S::TM][S::TN],
                                             const typename S::Acc (&u)[S::TM][S::TN],
                                             uint16_t *Y, int M, int N, int ldy, int m0, int n0) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int rows_valid = min(S::BM, M - m0);
    const int cols_valid = min(S::BN, N - n0);
    const __amdgpu_buffer_rsrc_t r = out_rsrc(Y, m0, rows_valid, ldy);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < S::TM; ++a) {
#pragma unroll
        for (int c = 0; c < S::TN; ++c) {
            const uint32_t lrow = static_cast<uint32_t>(wm * S::kWaveM + a * 32 + S::row_l(lane));
            uint32_t voff[2];
            lane_offsets(voff, lrow, wn * S::kWaveN + c * 32 + S::col_l(lane), cols_valid, n0,
                         ldy);
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float u0 = read_acc(u[a][c].get(i)), u1 = read_acc(u[a][c].get(i + 1));
                const float g0 = read_acc(g[a][c].get(i)), g1 = read_acc(g[a][c].get(i + 1));
                const uint32_t v = pack_bf16x2(g0 * u0, g1 * u1);   // g: SiLU(Gate) already
                const uint32_t roff =
                    static_cast<uint32_t>(S::row_r(i)) * static_cast<uint32_t>(ldy) * 2u;
                store_b16(r, voff[S::col_r(i) / 16], roff, static_cast<uint16_t>(v));
                store_b16_hi(r, voff[S::col_r(i) / 16], roff + static_cast<uint32_t>(ldy) * 2u, v);
            }
            __builtin_amdgcn_sched_barrier(0);   // one block's temporaries live at a time
        }
    }
}

// The loaders of an S tile: the A rows and the Gate panel (even packed rows),
// and the Up panel (odd packed rows), of the tile at (m0, n0).
template <class S, bool kEven = false>
struct SeqLoaders {
    TileLoader<S> ld;
    PanelLoader<S, S::BN, S::kDmaB> up;
    int nk;

    __device__ __forceinline__ void init(const void *A, const void *Wf, int M, int N, int K,
                                         int lda, int m0, int n0) {
        nk = (K + S::BK - 1) / S::BK;
        ld.init(KMajor{A, M, 1, 0, 0, lda}, m0, KMajor{Wf, N, 2, 0, 0, 0}, n0, K);
        up.init(KMajor{Wf, N, 2, 1, 0, 0}, n0, K);
    }
    // Step t of the tile's sequence of 2 nk K steps: Gate steps [0, nk), Up
    // steps [nk, 2 nk); steps past the end load nothing.  (A uniform select of
    // the panel, not a branch: these loads are issued one by one among the
    // MFMAs.)
    __device__ __forceinline__ void operator()(int t, int part, SWIGLU_LDS char *dst,
                                               int j) const {
        const bool gate = t < nk;
        ld.template issue<kEven>(gate ? t : t - nk, part, dst, j, gate ? ld.b : up);
    }
};

// SiLU on every Gate accumulator, in place: read out through volatile
// assembly (so after the wait for the Gate MFMAs), written back and pinned to
// the accumulator registers.
template <class S>
__device__ __forceinline__ void silu_acc(typename S::Acc (&g)[S::TM][S::TN]) {
#pragma unroll
    for (int a = 0; a < S::TM; ++a)
#pragma unroll
        for (int c = 0; c < S::TN; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 x = g[a][c].v[q];
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = silu(read_acc(x[e]));
                g[a][c].v[q] = y;
                asm volatile("" : "+a"(g[a][c].v[q]));
            }
}

// The two contractions of an S tile, each started by its first K step's
// MFMAs (C = 0), with SiLU applied to the Gate accumulators in between --
// while the first Up K steps' loads, issued during the last Gate steps, are
// in flight, and before any Up MFMA runs: the compiler, which does not know
// the assembly MFMAs' latency, must have no reason to copy accumulators next
// to MFMAs still writing them.
template <class S, bool kEven>
__device__ __forceinline__ void seq_contractions(Pipeline<S> &pl, const SeqLoaders<S, kEven> &issue,
                                                 typename S::Acc (&g)[S::TM][S::TN],
                                                 typename S::Acc (&u)[S::TM][S::TN]) {
    const int nk = issue.nk;
    pl.run_init(issue, 0, nk, 2 * nk, g);
    settle_acc<S>(g);
    silu_acc<S>(g);
    pl.run_init(issue, nk, 2 * nk, 2 * nk, u);
    pl.drain(u);
}

// Variant S, persistent, on 16x16 MFMAs: workgroup b runs whole tiles b,
// b + grid, ... below dp (XCD-ordered) and puts the first K steps of its next
// tile in flight before each epilogue; then its share of the 4 * quarter_tiles
// quarter-size tiles of the last round's tiles [dp, dp + quarter_tiles)
// (quarter q: row half q/2 % 2, column half q % 2 of tile dp + q / 4), each run
// on its own with a deeper ring.
template <class S, bool kEven>
__device__ __forceinline__ void fused_sequential_persistent_body(
    char *smem, const void *__restrict__ A, const void *__restrict__ Wf, uint16_t *__restrict__ Y,
    int M, int N, int K, int lda, int ldy, int tiles_m, int tiles_n, int dp, int quarter_tiles) {
    SWIGLU_LDS char *lds = (SWIGLU_LDS char *)smem;
    const int grid = gridDim.x;
    const int b = blockIdx.x;

    if (b < dp) {
        SeqLoaders<S, kEven> issue;
        int j = b, tm, tn;
        tile_coords(xcd_order(j, dp), tiles_m, tiles_n, 8, tm, tn);
        issue.init(A, Wf, M, N, K, lda, tm * S::BM, tn * S::BN);
        Pipeline<S> pl;
        pl.init(lds);
        pl.prologue_issue(issue);
        for (; j < dp; j += grid) {
            typename S::Acc g[S::TM][S::TN], u[S::TM][S::TN];
            pl.prologue_wait();
            seq_contractions<S>(pl, issue, g, u);
            const int m0 = tm * S::BM, n0 = tn * S::BN;
            if (j + grid < dp) {
                tile_coords(xcd_order(j + grid, dp), tiles_m, tiles_n, 8, tm, tn);
                issue.init(A, Wf, M, N, K, lda, tm * S::BM, tn * S::BN);
                pl.prologue_issue(issue);
            }
            seq_epilogue<S>(g, u, Y, M, N, ldy, m0, n0);
        }
    }

    using Q = typename QuarterOf<S>::type;
    static_assert(Q::kLdsBytes <= S::kLdsBytes, "quarter ring fits the tile's LDS");
    const int nq = 4 * quarter_tiles;
    for (int i = b; i < nq; i += grid) {
        const int q = xcd_order(i, nq);
        int tm, tn;
        tile_coords(dp + q / 4, tiles_m, tiles_n, 8, tm, tn);
        const int m0 = tm * S::BM + ((q >> 1) & 1) * Q::BM;
        const int n0 = tn * S::BN + (q & 1) * Q::BN;
        if (m0 >= M || n0 >= N) continue;   // quarter wholly past the output's edge
        SeqLoaders<Q, kEven> issue;
        issue.init(A, Wf, M, N, K, lda, m0, n0);
        Pipeline<Q> pl;
        pl.init(lds);
        typename Q::Acc g[Q::TM][Q::TN], u[Q::TM][Q::TN];
        pl.prologue(issue);
        seq_contractions<Q>(pl, issue, g, u);
        seq_epilogue<Q>(g, u, Y, M, N, ldy, m0, n0);
    }
}
template <class S>
__global__ __launch_bounds__(S::kThreads, 1) void fused_sequential_persistent_kernel(
    const void *__restrict__ A, const void *__restrict__ Wf, uint16_t *__restrict__ Y, int M,
    int N, int K, int lda, int ldy, int tiles_m, int tiles_n, int dp, int quarter_tiles) {
    static_assert(S::MI == 16 && S::EB == 2, "16x16 MFMAs on bf16 operands");
    __shared__ __attribute__((aligned(16))) char smem[S::kLdsBytes];
    if (K % S::BK == 0)
        fused_sequential_persistent_body<S, true>(smem, A, Wf, Y, M, N, K, lda, ldy, tiles_m,
                                                  tiles_n, dp, quarter_tiles);
    else
        fused_sequential_persistent_body<S, false>(smem, A, Wf, Y, M, N, K, lda, ldy, tiles_m,
                                                   tiles_n, dp, quarter_tiles);
}

// ---------------------------------------------------------------------------
// Tile shapes and launchers
// ---------------------------------------------------------------------------
// I and the ablation GEMMs: 4 waves, one per SIMD, each with a 128x128 block
// (256 accumulator registers, in AGPRs), BK = 64 and a two-stage ring (128 KiB
// of LDS); measured 10-16 % faster than an 8-wave ping-pong 256x256x32 shape
// on M=2048..8192 outputs.  16x16x32 MFMAs: under the power-limited clock of
// sustained MFMA load they deliver about 12 % more than 32x32x16 ones (an
// MFMA-only loop on random operands, all CUs: 1978 against 1760 TFLOP/s),
// and this kernel runs 4-5 % faster with them at M=4096 K=8192 N=29568 and
// M=8192 K=5120 N=13824 (equal at M <= 2048).  A third stage for the weight
// panel (B ring 3 deep, all 160 KiB of LDS): +0.8 % at M=4096 K=8192
// N=29568, +1.1 % at M=8192 K=5120 N=13824, +2.6 % at M=2048 K=1536 N=8960
// with the interleaved 16x16 schedule (a third A stage instead: 9 % slower).
using ShapeWide = TileShape<256, 256, 64, 2, 2, 2, 2, 3, 16>;
// The alternative for I and the ablation GEMMs: 128x128x64 tiles, 4 waves of
// 64x64, two stages (64 KiB), so two workgroups share a CU and one's prologue
// and epilogue overlap the other's mainloop; four times the tiles also fill
// the last round better.  Chosen per call by quad_tiles_faster().  16x16x32
// MFMAs, as the 256x256 shape.
using ShapeQuad = TileShape<128, 128, 64, 2, 2, 2, 2, 2, 16>;
// M <= 128 split along K and reduced in the kernel: five-stage rings (160 KiB),
// so a piece of up to five K steps has all its loads in flight at once
using ShapeSplitK = TileShape<128, 128, 64, 2, 2, 5, 2, 5, 16>;
// S: 128x128 output tiles, 4 waves each holding 64x64 Gate and Up
// accumulators, two stages (64 KiB), two workgroups per CU; measured against
// 256x128x64 (one per CU, 3 stages): 34 % faster at M=2048 K=1536 N=8960, 7 %
// at M=8192 K=5120 N=13824, equal at M=4096 K=8192 N=29568.  32x32x16
// MFMAs: with two workgroups per CU each wave has 256 registers, which the
// 16x16 form's doubled fragment registers next to the Gate and Up
// accumulators exceed.
using ShapeSeq = TileShape<128, 128, 64, 2, 2, 2>;
// S above M = 128, persistent: 256 x 128 output tiles (Gate and Up each 128 x
// 64 per wave: 256 accumulator registers, as variant I's 256x256 tile),
// 16x16 MFMAs, rings of 3 A and 3 B stages (144 KiB).
using ShapeSeqP = TileShape<256, 128, 64, 2, 2, 3, 2, 3, 16>;
// M <= 128 (all paths): 128x64 tiles, which put twice the workgroups of a
// 128x128 tile on the weight stream, with BK = 64 and four stages (96 KiB) to
// keep HBM loads in flight; measured with weights streamed from HBM against
// 128x64x32 x 4 stages: 21 % faster at M=128 K=896 N=4864, 24-29 % on K =
// 5120..8192 (up to 4.2 TB/s of weights).  32x32x16 MFMAs: the 16x16x32
// form measured 2 % slower here (M = 128, bound by the weight stream).
using ShapeSmall = TileShape<128, 64, 64, 2, 2, 4>;
// Variant I on FP8 operands: the same three shapes with K steps of 128 FP8
// values, so every tile row of a stage is 128 bytes and the LDS rings, load
// counts and swizzles are those of the bf16 shapes.
using ShapeWide8 = TileShape<256, 256, 128, 2, 2, 2, 1>;
using ShapeQuad8 = TileShape<128, 128, 128, 2, 2, 2, 1>;
using ShapeSmall8 = TileShape<128, 64, 128, 2, 2, 4, 1>;
using ShapeSeq8 = TileShape<128, 128, 128, 2, 2, 2, 1>;

static inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

template <class S, class Kern, class... Args>
static hipError_t launch_tiles(Kern kernel, int M, int cols, hipStream_t stream, Args... args) {
    const int tiles_m = cdiv(M, S::BM);
    const int tiles_n = cdiv(cols, S::BN);
    hipLaunchKernelGGL(kernel, dim3(tiles_m * tiles_n), dim3(S::kThreads), 0, stream, args...,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_pack(const uint16_t *W1, const uint16_t *W2, uint16_t *Wf, int64_t K,
                       int64_t N, hipStream_t stream) {
    const dim3 grid(cdiv(N, 64), cdiv(K, 64));
    hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, stream, W1, W2, Wf, (int)K, (int)N);
    return hipGetLastError();
}

hipError_t launch_pack_nk(const uint16_t *W1t, const uint16_t *W2t, uint16_t *Wf, int64_t K,
                          int64_t N, hipStream_t stream) {
    const int64_t per_row = K / 8, chunks = 2 * N * per_row;
    const int64_t blocks = (chunks + 255) / 256;
    const int grid = static_cast<int>(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(pack_nk_kernel, dim3(grid), dim3(256), 0, stream, W1t, W2t, Wf, per_row,
                       chunks);
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(const uint16_t *x, uint8_t *q, int64_t count, int scale_exp,
                               hipStream_t stream) {
    const int64_t chunks = count / 16;
    const int64_t blocks = (chunks + 255) / 256;
    const int grid = static_cast<int>(blocks < 65536 ? blocks : 65536);
    const float inv_scale = std::ldexp(1.0f, -scale_exp);
    hipLaunchKernelGGL(quantize_fp8_kernel, dim3(grid), dim3(256), 0, stream, x, q, inv_scale,
                       chunks);
    return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t *g, const uint16_t *u, uint16_t *y, int64_t count,
                           hipStream_t stream) {
    const int64_t chunks = count / 8;
    const int64_t blocks = (chunks + 255) / 256;
    const int grid = static_cast<int>(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(silu_mul_kernel, dim3(grid), dim3(256), 0, stream, g, u, y, chunks);
    return hipGetLastError();
}

// Schedule cost model (MI355X, microseconds).  A round of workgroups costs
// kRoundUs plus nk K steps of its tile shape; a split tail also pays the
// reduction (kReduceUs plus its partials, written once and read once, at
// kPartialBytesPerUs).  Fitted to 375 timings of variant I with inputs
// streamed from HBM: the five K x N shapes of the benchmark workloads, M from
// 256 to 16384, each forced through every tile shape and tail schedule
// (RMS error 7 %); on those points the schedule it picks is on average within
// 0.5 % of the measured-fastest (at most 4.1 %).
constexpr double kRoundUs = 3.7;
constexpr double kReduceUs = 3.4;
constexpr double kPartialBytesPerUs = 6.4e6;

// One K step of a round of S tiles: 1.69 for 256x256x64 (one per CU), 1.03
// for 128x128x64 (two per CU, so twice the tiles per round); other shapes
// scaled from the first by tile volume and workgroups per CU.
// (Per K step of 128-byte tile rows: an FP8 step of 128 k takes the MFMA
// cycles and the load bytes of a bf16 step of 64 k.)
template <class S>
constexpr double step_us() {
    constexpr int kRow = S::kRowBytes;
    if (S::BM == 256 && S::BN == 256 && kRow == 128 && S::kOccupancy == 1) return 1.69;
    if (S::BM == 128 && S::BN == 128 && kRow == 128 && S::kOccupancy == 2) return 1.03;
    return 1.69 * (static_cast<double>(S::BM) * S::BN * kRow) / (256.0 * 256.0 * 128.0) *
           S::kOccupancy;
}

// One K step of a round of quarter-size tiles (QuarterOf<S>) in the S kernel:
// 0.59 for the 128x128 quarters of 256x256x64.
template <class S>
constexpr double quarter_step_us() {
    return 0.59 * (static_cast<double>(S::BM) * S::BN * S::kRowBytes) / (256.0 * 256.0 * 128.0);
}

// Work schedule for a single-accumulator GEMM over an M x cols output (see
// split_tail.hpp): all tiles whole unless the last round is partly idle.  Then
// its L tiles run whichever way the cost model predicts fastest:
//  - whole: one more round;
//  - as 4L quarter-size tiles (kQuarterable shapes: one workgroup per CU,
//    whose LDS gives a quarter tile a deeper ring): ceil(4L / G) rounds of
//    quarter steps;
//  - split into s = min(G / L, nk) >= 2 pieces (with a workspace): a round of
//    ceil(nk / s) steps plus the reduction.
// ws.tail forces one of them where it applies.  `us`, if given, receives the
// predicted time of the whole schedule.
template <class S>
static Schedule make_schedule(int M, int cols, int K, const GemmWorkspace &ws,
                              double *us = nullptr) {
    Schedule sch{};
    sch.tiles_m = cdiv(M, S::BM);
    sch.tiles_n = cdiv(cols, S::BN);
    sch.nk = cdiv(K, S::BK);
    sch.group_m = 8;
    const int64_t T = static_cast<int64_t>(sch.tiles_m) * sch.tiles_n;
    sch.dp = static_cast<int>(T);
    const int G = ws.cus * S::kOccupancy;           // workgroup slots
    const double round = kRoundUs + sch.nk * step_us<S>();
    if (us) *us = G > 0 ? cdiv(T, G) * round : 0.0;
    if (G <= 0 || ws.tail == kTailWhole) return sch;
    const int64_t L = T % G;
    if (L == 0) return sch;
    const bool forced = ws.tail != kTailAuto;
    double best = round;                            // tail tiles whole
    if (kQuarterable<S> && (!forced || ws.tail == kTailQuarters)) {
        const double t = cdiv(4 * L, G) * (kRoundUs + sch.nk * quarter_step_us<S>());
        if (forced || t < best) {
            best = t;
            sch.dp = static_cast<int>(T - L);
            sch.split_tiles = static_cast<int>(L);
            sch.quartered = 1;
        }
    }
    const bool has_ws = ws.base != nullptr && ws.bytes >= workspace_bytes_for(ws.cus);
    if (has_ws && (!forced || ws.tail == kTailPieces)) {
        const int pieces =
            static_cast<int>(min(static_cast<int64_t>(G) / L, static_cast<int64_t>(sch.nk)));
        const double partials = static_cast<double>(L) * pieces * S::BM * S::BN * 4.0 * 2.0;
        const double t = kRoundUs + cdiv(sch.nk, pieces) * step_us<S>() + kReduceUs +
                         partials / kPartialBytesPerUs;
        if (pieces >= 2 && (forced || t < best)) {
            best = t;
            sch.dp = static_cast<int>(T - L);
            sch.split_tiles = static_cast<int>(L);
            sch.quartered = 0;
            sch.pieces = pieces;
            sch.partials = reinterpret_cast<float *>(ws.base);
        }
    }
    if (us) *us = (T / G) * round + best;
    return sch;
}

// Workgroups of a persistent launch of `sch`: one per slot, or fewer when
// there is less work (unknown slot count: one per whole tile).
template <class S>
static int launch_grid(const Schedule &sch, int cus) {
    const int64_t tail = sch.quartered ? 4LL * sch.split_tiles
                                       : static_cast<int64_t>(sch.split_tiles) * sch.pieces;
    const int64_t work = sch.dp > tail ? sch.dp : tail;
    const int64_t G = static_cast<int64_t>(cus) * S::kOccupancy;
    return static_cast<int>(G > 0 && G < work ? G : work);
}

template <class S, class Epi>
static hipError_t launch_gemm(KMajor A, KMajor B, int M, int cols, int K, Epi epi,
                              const GemmWorkspace &ws, hipStream_t stream) {
    Schedule sch = make_schedule<S>(M, cols, K, ws);
    sch.grid = launch_grid<S>(sch, ws.cus);
    B.pairs = Epi::template paired<S>() ? 1 : 0;   // de-interleaved weight panels
    if (sch.grid <= 0) return hipSuccess;
    if (sch.quartered) {
        if constexpr (kQuarterable<S>) {
            hipLaunchKernelGGL((gemm_tiles_kernel<S, Epi, kTailQuarter>), dim3(sch.grid),
                               dim3(S::kThreads), 0, stream, A, B, M, K, epi, sch);
            return hipGetLastError();
        }
        return hipErrorInvalidConfiguration;   // make_schedule quarters no other shape
    }
    if (sch.pieces == 0) {
        hipLaunchKernelGGL((gemm_tiles_kernel<S, Epi, kTailNone>), dim3(sch.grid),
                           dim3(S::kThreads), 0, stream, A, B, M, K, epi, sch);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemm_tiles_kernel<S, Epi, kTailSplit>), dim3(sch.grid), dim3(S::kThreads),
                       0, stream, A, B, M, K, epi, sch);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // S::kWaves * (epilogue units per wave) single-wave workgroups per split tile
    constexpr int kWavesPerTile = S::kWaves * S::TM * S::TN / Epi::template unit_blocks<S>();
    const int rgrid = sch.split_tiles * kWavesPerTile;
    hipLaunchKernelGGL((split_reduce_kernel<S, Epi>), dim3(rgrid), dim3(64), 0, stream, epi, sch);
    return hipGetLastError();
}

// Tile choice for an M x cols single-accumulator GEMM above M = 128: the
// 128x128 two-per-CU tiles when the cost model predicts their schedule
// faster than the 256x256 tiles' (each with its own best tail).
template <class Wide = ShapeWide, class Quad = ShapeQuad>
static bool quad_tiles_faster(int M, int cols, int K, const GemmWorkspace &ws) {
    if (ws.tile == 256) return false;
    if (ws.tile == 128) return true;
    if (ws.cus <= 0) return false;
    double wide = 0.0, quad = 0.0;
    make_schedule<Wide>(M, cols, K, ws, &wide);
    make_schedule<Quad>(M, cols, K, ws, &quad);
    return quad < wide;
}

// Variant I at M <= 128 streams the packed weight once, so its time follows
// the rows of W_fused the busiest compute unit has to stream: 64 per round
// of 128x64 tiles (one workgroup per CU), or 128 per resident 128x128 tile
// (two share a CU).  The 128x128 tiles are taken when M > 64 and they put no
// more rows on any CU (fewer workgroups, one round).  Measured at M = 128:
// 6-10 % faster on (K, N) = (1536, 8960), (5120, 13824), (8192, 29568), where
// the 128x64 tiles need a second (or fourth) round; the rule keeps 128x64 on
// (896, 4864) and (3584, 18944), where 128x128 tiles ran 64 % and 5 % slower;
// at M <= 64 the 128x64 tiles were as fast or faster on all five shapes.
// The FP8 path applies the same rule (there the 128x128 tiles also gain 10-19 %
// on the first and last of those three shapes; on (3584, 18944) they would be
// 10 % faster but the rule keeps 128x64).
// SWIGLU_I_TILE=128 / 256 forces the 128x128 / 128x64 tiles here.
static bool small_m_quad_tiles(int M, int cols, const GemmWorkspace &ws) {
    if (ws.tile == 128) return true;
    if (ws.tile == 256 || M <= 64 || ws.cus <= 0) return false;
    const int64_t small = cdiv(cols, ShapeSmall::BN), quad = cdiv(cols, ShapeQuad::BN);
    const int64_t rows_small = 64 * ((small + ws.cus - 1) / ws.cus);
    const int64_t rows_quad = 128 * ((quad + ws.cus - 1) / ws.cus);
    return rows_quad <= rows_small;
}

// M <= 128 (one tile row): every tile split into s = min(G / T, nk) pieces
// along K and reduced in the kernel, when 3 <= s <= kMaxFixupPieces and each
// piece has at least 16 K steps, or when SWIGLU_TAIL=fixup forces it (s
// capped); needs the workspace for the partials and a counter block.
// Otherwise a schedule with pieces == 0.  Each piece writes a 64 KiB fp32
// partial and the last reads s - 1 of them, so short pieces lose: against the
// 128x64 tiles run whole (same box, M=128): K=8192 N=4864 44.2 against
// 56.3 us, K=3584 N=4864 24.7 against 29.1, but K=896 N=4864 (3 pieces of 4-5
// steps) 16.0 against 10.4, and M=64 K=8192 N=6144 (2 pieces, no more
// workgroups than 128x64 tiles) 51.7 against 49.1.  More pieces are left to
// the split tail's reduction kernel, which spreads the sums over the chip.
template <class S>
static Schedule make_fixup_schedule(int M, int cols, int K, const GemmWorkspace &ws) {
    Schedule none{};
    if (M > S::BM || ws.cus <= 0 || ws.base == nullptr || ws.counters == nullptr) return none;
    if (ws.tail != kTailAuto && ws.tail != kTailFixup) return none;
    Schedule sch{};
    sch.tiles_m = 1;
    sch.tiles_n = cdiv(cols, S::BN);
    sch.nk = cdiv(K, S::BK);
    sch.group_m = 8;
    const int T = sch.tiles_n;
    int s = ws.cus / T < sch.nk ? ws.cus / T : sch.nk;
    if (ws.tail == kTailAuto && (s < 3 || s > kMaxFixupPieces || sch.nk < 16 * s)) return none;
    if (s > kMaxFixupPieces) s = kMaxFixupPieces;
    if (s < 2 || T > ws.max_counters) return none;
    if (static_cast<uint64_t>(T) * s * S::BM * S::BN * sizeof(float) > ws.bytes) return none;
    sch.dp = 0;
    sch.split_tiles = T;
    sch.pieces = s;
    sch.partials = reinterpret_cast<float *>(ws.base);
    sch.counters = ws.counters;
    sch.grid = T * s;
    return sch;
}

template <class S, class Epi>
static hipError_t launch_reduce_in_kernel(KMajor A, KMajor B, int M, int K, Epi epi,
                                          const Schedule &sch, hipStream_t stream) {
    B.pairs = Epi::template paired<S>() ? 1 : 0;   // de-interleaved weight panels
    hipLaunchKernelGGL((gemm_tiles_kernel<S, Epi, kTailReduceInKernel>), dim3(sch.grid),
                       dim3(S::kThreads), 0, stream, A, B, M, K, epi, sch);
    return hipGetLastError();
}

hipError_t launch_fused_interleaved(const uint16_t *A, int lda, const uint16_t *Wf, uint16_t *Y,
                                    int ldy, int M, int N, int K, const GemmWorkspace &ws,
                                    hipStream_t stream) {
    const KMajor Ak{A, M, 1, 0, 0, lda};
    const KMajor B{Wf, 2 * N, 1, 0};
    const PairMulEpilogue epi{Y, M, N, ldy, 1.0f};
    if (M <= 128) {
        const Schedule fx = make_fixup_schedule<ShapeSplitK>(M, 2 * N, K, ws);
        if (fx.pieces) return launch_reduce_in_kernel<ShapeSplitK>(Ak, B, M, K, epi, fx, stream);
        if (small_m_quad_tiles(M, 2 * N, ws))
            return launch_gemm<ShapeQuad>(Ak, B, M, 2 * N, K, epi, ws, stream);
        return launch_gemm<ShapeSmall>(Ak, B, M, 2 * N, K, epi, ws, stream);
    }
    if (quad_tiles_faster(M, 2 * N, K, ws))
        return launch_gemm<ShapeQuad>(Ak, B, M, 2 * N, K, epi, ws, stream);
    return launch_gemm<ShapeWide>(Ak, B, M, 2 * N, K, epi, ws, stream);
}

// The kernels launch_fused_interleaved / launch_fused_sequential /
// launch_gemm_store (one of the ablation's two GEMMs) would run, as text.
template <class S>
static int describe(const char *kernel, const char *epi, const Schedule &sch, int cus,
                    char *buf, size_t n) {
    const int wgs = launch_grid<S>(sch, cus);
    if (sch.pieces)
        return std::snprintf(buf, n,
                             "%s<%dx%dx%d,%s> (%d whole tiles + %d tiles split %d ways along K;"
                             " %d workgroups) + split_reduce_kernel",
                             kernel, S::BM, S::BN, S::BK, epi, sch.dp, sch.split_tiles,
                             sch.pieces, wgs);
    if (sch.quartered)
        return std::snprintf(buf, n,
                             "%s<%dx%dx%d,%s> (%d tiles + %d tiles run as %d %dx%d tiles;"
                             " %d workgroups)",
                             kernel, S::BM, S::BN, S::BK, epi, sch.dp, sch.split_tiles,
                             4 * sch.split_tiles, S::BM / 2, S::BN / 2, wgs);
    return std::snprintf(buf, n, "%s<%dx%dx%d,%s> (%d tiles; %d workgroups)", kernel, S::BM,
                         S::BN, S::BK, epi, sch.dp, wgs);
}

int describe_gemm(int M, int cols, int K, const GemmWorkspace &ws, const char *epi, char *buf,
                  size_t n, bool fused_i) {
    if (M <= 128 && fused_i) {
        using P = ShapeSplitK;
        const Schedule fx = make_fixup_schedule<P>(M, cols, K, ws);
        if (fx.pieces)
            return std::snprintf(buf, n,
                                 "gemm_tiles_kernel<%dx%dx%d,%s> (%d tiles split %d ways along K,"
                                 " reduced in the kernel; %d workgroups)",
                                 P::BM, P::BN, P::BK, epi, fx.split_tiles, fx.pieces, fx.grid);
    }
    if (M <= 128 && fused_i && small_m_quad_tiles(M, cols, ws))
        return describe<ShapeQuad>("gemm_tiles_kernel", epi,
                                   make_schedule<ShapeQuad>(M, cols, K, ws), ws.cus, buf, n);
    if (M <= 128)
        return describe<ShapeSmall>("gemm_tiles_kernel", epi,
                                    make_schedule<ShapeSmall>(M, cols, K, ws), ws.cus, buf, n);
    if (quad_tiles_faster(M, cols, K, ws))
        return describe<ShapeQuad>("gemm_tiles_kernel", epi,
                                   make_schedule<ShapeQuad>(M, cols, K, ws), ws.cus, buf, n);
    return describe<ShapeWide>("gemm_tiles_kernel", epi, make_schedule<ShapeWide>(M, cols, K, ws),
                               ws.cus, buf, n);
}

// Work schedule of the persistent S kernel: whole 256x128 tiles, unless the
// last round is partly idle; then its L tiles run whichever way is predicted
// faster (ws.tail forces one): whole (one more round), or as 4L quarter-size
// tiles (ceil(4L / G) rounds of quarter steps).
struct SeqSchedule {
    int tiles_m, tiles_n;
    int dp;              // tiles [0, dp) run whole
    int quarter_tiles;   // tiles [dp, dp + quarter_tiles) run as four quarters each
    int grid;
};
// One K step of a round of whole tiles, and of a round of quarter tiles
// (measured: rounds of 256x128 and 128x64 tiles at M=4096 K=8192 N=29568 and
// M=2048 K=1536 N=8960; a quarter step takes 0.65 of a whole one for a
// quarter of its work).  Over 13 shapes from M=256 to 8192 the choice is
// the faster one, or within 2 % of it.
constexpr double kSeqStepUs = 0.9;
constexpr double kSeqQuarterStepUs = 0.6;

static SeqSchedule make_seq_schedule(int M, int N, int K, const GemmWorkspace &ws) {
    using P = ShapeSeqP;
    SeqSchedule s{};
    s.tiles_m = cdiv(M, P::BM);
    s.tiles_n = cdiv(N, P::BN);
    const int64_t T = static_cast<int64_t>(s.tiles_m) * s.tiles_n;
    s.dp = static_cast<int>(T);
    const int G = ws.cus;
    const int64_t L = G > 0 ? T % G : 0;
    if (L > 0 && ws.tail != kTailWhole) {
        const int nk = cdiv(K, P::BK);
        const double whole = kRoundUs + 2 * nk * kSeqStepUs;
        const double quarters = cdiv(4 * L, G) * (kRoundUs + 2 * nk * kSeqQuarterStepUs);
        if (ws.tail == kTailQuarters || quarters < whole) {
            s.dp = static_cast<int>(T - L);
            s.quarter_tiles = static_cast<int>(L);
        }
    }
    const int64_t work = s.dp > 4LL * s.quarter_tiles ? s.dp : 4LL * s.quarter_tiles;
    s.grid = static_cast<int>(G > 0 && G < work ? G : work);
    return s;
}

int describe_fused_sequential(int M, int N, int K, const GemmWorkspace &ws, char *buf, size_t n) {
    if (M <= 128)
        return std::snprintf(buf, n, "fused_sequential_kernel<%dx%dx%d> (%lld tiles)",
                             ShapeSmall::BM, ShapeSmall::BN, ShapeSmall::BK,
                             static_cast<long long>(cdiv(M, ShapeSmall::BM)) * cdiv(N, ShapeSmall::BN));
    using P = ShapeSeqP;
    const SeqSchedule s = make_seq_schedule(M, N, K, ws);
    if (s.quarter_tiles)
        return std::snprintf(buf, n,
                             "fused_sequential_persistent_kernel<%dx%dx%d> (%d tiles + %d tiles "
                             "run as %d %dx%d tiles; %d workgroups)",
                             P::BM, P::BN, P::BK, s.dp, s.quarter_tiles, 4 * s.quarter_tiles,
                             P::BM / 2, P::BN / 2, s.grid);
    return std::snprintf(buf, n,
                         "fused_sequential_persistent_kernel<%dx%dx%d> (%d tiles; %d workgroups)",
                         P::BM, P::BN, P::BK, s.dp, s.grid);
}

// Variant I on FP8 operands: the same GEMM over W_fused with K steps of 128
// FP8 values (128-byte tile rows, as bf16's 64), the f8f6f4 MFMA, and the
// paired epilogue scaling Gate and Up by 2^(a_exp + w_exp) before SiLU.
hipError_t launch_fused_interleaved_fp8(const uint8_t *A8, const uint8_t *Wf8, uint16_t *Y,
                                        int M, int N, int K, float scale,
                                        const GemmWorkspace &ws, hipStream_t stream) {
    const KMajor Ak{A8, M, 1, 0};
    const KMajor B{Wf8, 2 * N, 1, 0};
    const PairMulEpilogueFp8 epi{Y, M, N, N, scale};
    if (M <= 128) {
        if (small_m_quad_tiles(M, 2 * N, ws))
            return launch_gemm<ShapeQuad8>(Ak, B, M, 2 * N, K, epi, ws, stream);
        return launch_gemm<ShapeSmall8>(Ak, B, M, 2 * N, K, epi, ws, stream);
    }
    if (quad_tiles_faster<ShapeWide8, ShapeQuad8>(M, 2 * N, K, ws))
        return launch_gemm<ShapeQuad8>(Ak, B, M, 2 * N, K, epi, ws, stream);
    return launch_gemm<ShapeWide8>(Ak, B, M, 2 * N, K, epi, ws, stream);
}

int describe_gemm_fp8(int M, int cols, int K, const GemmWorkspace &ws, char *buf, size_t n) {
    const char *epi = "PairMulEpilogueFp8";
    if (M <= 128 && small_m_quad_tiles(M, cols, ws))
        return describe<ShapeQuad8>("gemm_tiles_kernel", epi,
                                    make_schedule<ShapeQuad8>(M, cols, K, ws), ws.cus, buf, n);
    if (M <= 128)
        return describe<ShapeSmall8>("gemm_tiles_kernel", epi,
                                     make_schedule<ShapeSmall8>(M, cols, K, ws), ws.cus, buf, n);
    if (quad_tiles_faster<ShapeWide8, ShapeQuad8>(M, cols, K, ws))
        return describe<ShapeQuad8>("gemm_tiles_kernel", epi,
                                    make_schedule<ShapeQuad8>(M, cols, K, ws), ws.cus, buf, n);
    return describe<ShapeWide8>("gemm_tiles_kernel", epi,
                                make_schedule<ShapeWide8>(M, cols, K, ws), ws.cus, buf, n);
}

hipError_t launch_fused_sequential(const uint16_t *A, int lda, const uint16_t *Wf, uint16_t *Y,
                                   int ldy, int M, int N, int K, const GemmWorkspace &ws,
                                   hipStream_t stream) {
    const void *a = A, *w = Wf;
    if (M <= 128)
        return launch_tiles<ShapeSmall>(fused_sequential_kernel<ShapeSmall>, M, N, stream, a, w,
                                        Y, M, N, K, lda, ldy, 1.0f);
    using P = ShapeSeqP;
    const SeqSchedule s = make_seq_schedule(M, N, K, ws);
    if (s.grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(fused_sequential_persistent_kernel<P>, dim3(s.grid), dim3(P::kThreads), 0,
                       stream, a, w, Y, M, N, K, lda, ldy, s.tiles_m, s.tiles_n, s.dp,
                       s.quarter_tiles);
    return hipGetLastError();
}

// Variant S on FP8 operands: the same kernel with K steps of 128 FP8 values.
hipError_t launch_fused_sequential_fp8(const uint8_t *A8, const uint8_t *Wf8, uint16_t *Y, int M,
                                       int N, int K, float scale, hipStream_t stream) {
    const void *a = A8, *w = Wf8;
    if (M <= 128)
        return launch_tiles<ShapeSmall8>(fused_sequential_kernel<ShapeSmall8>, M, N, stream, a, w,
                                         Y, M, N, K, K, N, scale);
    return launch_tiles<ShapeSeq8>(fused_sequential_kernel<ShapeSeq8>, M, N, stream, a, w, Y, M,
                                   N, K, K, N, scale);
}

// C [M][cols] = bf16(A . B^T) for a K-contiguous operand B of `cols` logical
// rows: the ablation's GEMMs and the down projection.
static hipError_t launch_store_gemm(const uint16_t *A, const KMajor &B, uint16_t *C, int M,
                                    int cols, int K, const GemmWorkspace &ws,
                                    hipStream_t stream) {
    const KMajor Ak{A, M, 1, 0};
    const StoreEpilogue epi{C, M, cols};
    if (M <= 128) return launch_gemm<ShapeSmall>(Ak, B, M, cols, K, epi, ws, stream);
    if (quad_tiles_faster(M, cols, K, ws))
        return launch_gemm<ShapeQuad>(Ak, B, M, cols, K, epi, ws, stream);
    return launch_gemm<ShapeWide>(Ak, B, M, cols, K, epi, ws, stream);
}

hipError_t launch_gemm_store(const uint16_t *A, const uint16_t *Wf, int phase, uint16_t *C,
                             int M, int N, int K, const GemmWorkspace &ws, hipStream_t stream) {
    return launch_store_gemm(A, KMajor{Wf, N, 2, phase}, C, M, N, K, ws, stream);
}

hipError_t launch_down_proj(const uint16_t *H, const uint16_t *W3t, uint16_t *Out, int M, int N,
                            int D, const GemmWorkspace &ws, hipStream_t stream) {
    return launch_store_gemm(H, KMajor{W3t, D, 1, 0}, Out, M, D, N, ws, stream);
}

// One 256x256 fp32 slot per CU: a split schedule has at most one piece per
// workgroup slot, and a CU holds one 256x256 workgroup or two of the smaller
// shapes (whose slots are a quarter the size or less).
uint64_t partials_bytes(int cus) {
    return static_cast<uint64_t>(cus) * ShapeWide::BM * ShapeWide::BN * sizeof(float);
}

uint64_t workspace_bytes_for(int cus) { return partials_bytes(cus); }

int64_t max_tiles(int64_t M, int64_t cols) {
    // the most workgroups any launcher above creates for an M x cols output
    const int64_t small = ((M + 127) / 128) * ((cols + 63) / 64);
    const int64_t wide = ((M + 255) / 256) * ((cols + 127) / 128);
    // 256x256 tiles with the tail quartered: at most four workgroups a tile
    const int64_t quartered = 4 * ((M + 255) / 256) * ((cols + 255) / 256);
    const int64_t most = small > wide ? small : wide;
    return most > quartered ? most : quartered;
}

}  // namespace swiglu
