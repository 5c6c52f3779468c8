// Device side of the tiled GEMM kernels: output stores, the variant-I and
// store epilogues, the persistent tile kernel with its tail schedules, its
// split-tail reduction, the variant-S kernels, and the tile shapes.
//
// Citations are to the pages on "Tile-Level Activation Overlap for Efficient
// LLM Inference" (arXiv 2607.02521): [paper s1] = the paper's own text,
// section 1 Introduction; [abstract] = its abstract; [gist: X] = the
// gist.science technical summary, section X.
//
// The kernel templates are instantiated only in kernel_instances.hip, once per
// object (see the Launch structs at the end); the dispatch code in kernels.hip
// includes this header for the shapes and epilogue types and calls the
// Launch structs' run().
#pragma once

#include "device.hpp"
#include "gemm_core.hpp"
#include "split_tail.hpp"

namespace swiglu {

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

// The K steps [0, len) of one tile into `acc`.  With 16x16 MFMAs the first
// step's MFMAs start the accumulators (C = 0): no vector instructions zero its
// 256 registers first.  32x32 MFMAs accumulate onto zeros (zero_acc_mi32
// before the prologue's wait, while the loads are in flight).
template <class S>
__device__ __forceinline__ void zero_acc_mi32(typename S::Acc (&acc)[S::TM][S::TN]) {
    if constexpr (S::MI != 16) zero_acc<S>(acc);
}
// kUnroll: the ring walked in unrolled periods (the loads' offsets are fixed
// per tile when K is a multiple of BK, so only that body takes it).
template <class S, bool kUnroll = false, class Issue>
__device__ __forceinline__ void run_tile(Pipeline<S> &pl, const Issue &issue, int len,
                                         typename S::Acc (&acc)[S::TM][S::TN]) {
    if constexpr (S::MI == 16) pl.template run_init0<kUnroll>(issue, len, len, acc);
    else pl.run(issue, 0, len, len, acc);
}

// K steps [kb, ke) of the S tile at (m0, n0) of D = A . B^T, into acc.
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
    run_tile<S, kEven>(pl, issue, len, acc);
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
// the epilogue and no workgroup launch sits between tiles.  It also takes its
// share of the tiles [dp, dp + split_tiles) of the partly idle last round:
// quartered tiles before its whole tiles, so that the workgroups with such a
// share run their whole tiles out of step with the others and the epilogues
// of a round, which all store their tile at once when every workgroup starts
// together, are spread out (M=2048 K=1536 N=8960: 101.9 -> 96.2 us a call,
// M=512 K=3584 N=18944: 125.6 -> 119-123); split pieces after them (before
// them measured 2.5 % slower on M=4096 K=8192 N=29568, 0.6 % on M=8192
// K=5120 N=13824):
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

    auto whole_tiles = [&] {
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
                run_tile<S, kEven>(pl, issue, nk, acc);
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
    };

    if constexpr (TAIL == kTailQuarter) {
        // the quarter-size tiles first: the workgroups that have one then
        // finish their whole tiles a quarter tile later than the others, so
        // the epilogues of a round do not all store at the same moment
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
        whole_tiles();
    } else {
        whole_tiles();
    }
    if constexpr (TAIL == kTailReduceInKernel) {
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
    pl.template run_init0<kEven>(issue, nk, 2 * nk, g);
    settle_acc<S>(g);
    silu_acc<S>(g);
    pl.template run_init<kEven>(issue, nk, 2 * nk, 2 * nk, u);
    pl.drain(u);
}

// Variant S, persistent, on 16x16 MFMAs: workgroup b runs whole tiles b,
// b + grid, ... below dp (XCD-ordered), putting the first K steps of its next
// tile in flight before each epilogue, and its share of the 4 * quarter_tiles
// quarter-size tiles of the last round's tiles [dp, dp + quarter_tiles)
// (quarter q: row half q/2 % 2, column half q % 2 of tile dp + q / 4), each on
// its own with a deeper ring, before or after them (below).
template <class S, bool kEven>
__device__ __forceinline__ void fused_sequential_persistent_body(
    char *smem, const void *__restrict__ A, const void *__restrict__ Wf, uint16_t *__restrict__ Y,
    int M, int N, int K, int lda, int ldy, int tiles_m, int tiles_n, int dp, int quarter_tiles) {
    SWIGLU_LDS char *lds = (SWIGLU_LDS char *)smem;
    const int grid = gridDim.x;
    const int b = blockIdx.x;

    // The quarter-size tiles of the last round before the whole tiles when a
    // tile is at most 64 K steps long (as in gemm_tiles_body: those
    // workgroups then run their whole tiles out of step with the rest and the
    // epilogues of a round spread out; M=2048 K=1536 N=8960 119.1 -> 115.9
    // us), after them on longer tiles (at K=8192 N=29568 quarters first
    // measured 8.5 % slower at M=256 and 11 % at M=2048).
    using Q = typename QuarterOf<S>::type;
    static_assert(Q::kLdsBytes <= S::kLdsBytes, "quarter ring fits the tile's LDS");
    const int nq = 4 * quarter_tiles;
    const bool quarters_first = (K + S::BK - 1) / S::BK <= 64;
    // tile rows walked together, as the GEMM kernels' schedule chooses them
    const int group_m = tiles_m <= 8 && (K + S::BK - 1) / S::BK <= 32 ? 4 : 8;
#pragma nounroll
    for (int pass = 0; pass < 2; ++pass) {
        if ((pass == 0) == quarters_first) {
            for (int i = b; i < nq; i += grid) {
                const int q = xcd_order(i, nq);
                int tm, tn;
                tile_coords(dp + q / 4, tiles_m, tiles_n, group_m, tm, tn);
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
        } else if (b < dp) {
            SeqLoaders<S, kEven> issue;
            int j = b, tm, tn;
            tile_coords(xcd_order(j, dp), tiles_m, tiles_n, group_m, tm, tn);
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
                    tile_coords(xcd_order(j + grid, dp), tiles_m, tiles_n, group_m, tm, tn);
                    issue.init(A, Wf, M, N, K, lda, tm * S::BM, tn * S::BN);
                    pl.prologue_issue(issue);
                }
                seq_epilogue<S>(g, u, Y, M, N, ldy, m0, n0);
            }
        }
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
// 5120..8192 (up to 4.2 TB/s of weights); five or six stages (120 / 144 KiB,
// still one workgroup per CU) ran 0-14 % slower for variants I and S and the
// ablation at M = 32 and 128 on all five K x N workload shapes.  32x32x16
// MFMAs: the 16x16x32 form measured 2 % slower here (M = 128, bound by the
// weight stream).
using ShapeSmall = TileShape<128, 64, 64, 2, 2, 4>;
// Variant I on FP8 operands: the same three shapes with K steps of 128 FP8
// values, so every tile row of a stage is 128 bytes and the LDS rings, load
// counts and swizzles are those of the bf16 shapes (the 256x256 one with a
// three-stage weight ring, as bf16's: 0-1.3 % faster than two stages).
using ShapeWide8 = TileShape<256, 256, 128, 2, 2, 2, 1, 3>;
using ShapeQuad8 = TileShape<128, 128, 128, 2, 2, 2, 1>;
using ShapeSmall8 = TileShape<128, 64, 128, 2, 2, 4, 1>;
using ShapeSeq8 = TileShape<128, 128, 128, 2, 2, 2, 1>;

// ---------------------------------------------------------------------------
// Launches of the kernel templates above.  Each run() enqueues one launch on
// `stream` and returns its status.  They are defined and explicitly
// instantiated in kernel_instances.hip, which is compiled once per entry of
// its instance list: the K loops unrolled over a whole ring period make each
// tile-kernel instance a large function to compile, and separate objects
// let the build compile them in parallel.
// ---------------------------------------------------------------------------
// gemm_tiles_kernel<S, Epi, TAIL> on `grid` workgroups over the tiles of `sch`
template <class S, class Epi, int TAIL>
struct TilesLaunch {
    static hipError_t run(int grid, const KMajor &A, const KMajor &B, int M, int K,
                          const Epi &epi, const Schedule &sch, hipStream_t stream);
};
// split_reduce_kernel<S, Epi> on `grid` single-wave workgroups
template <class S, class Epi>
struct ReduceLaunch {
    static hipError_t run(int grid, const Epi &epi, const Schedule &sch, hipStream_t stream);
};
// fused_sequential_kernel<S>, one workgroup per S tile of the M x N output
template <class S>
struct SequentialLaunch {
    static hipError_t run(const void *A, const void *Wf, uint16_t *Y, int M, int N, int K,
                          int lda, int ldy, float scale, hipStream_t stream);
};
// fused_sequential_persistent_kernel<S> on `grid` workgroups
template <class S>
struct PersistentSequentialLaunch {
    static hipError_t run(int grid, const void *A, const void *Wf, uint16_t *Y, int M, int N,
                          int K, int lda, int ldy, int tiles_m, int tiles_n, int dp,
                          int quarter_tiles, hipStream_t stream);
};

}  // namespace swiglu
