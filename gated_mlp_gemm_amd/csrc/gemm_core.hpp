// The bf16 MFMA mainloop shared by every GEMM-shaped kernel of the library:
// the interleaved fused kernel, the sequential fused kernel and the unfused
// ablation's plain-store GEMM all run this code, so that their timings differ
// only by what the method changes (where Gate and Up live).
//
// One workgroup computes a BM x BN tile of D = A . B^T where both operands are
// K-contiguous row panels ("NT" form):
//   A: rows of the activations [M][K];
//   B: rows of the packed weight W_fused^T [2N][K] (column c of W_fused is row
//      c here), optionally every second row (the Gate or the Up columns).
// K is consumed in steps of BK.
//
// Pipeline.  K steps stream through two rings of LDS buffers, STAGES of A
// panels and BSTAGES of B panels, filled by direct-to-LDS buffer loads
// (buffer_load_dwordx4 ... lds: no VGPR staging, no LDS write instructions),
// STAGES-1 (BSTAGES-1) steps ahead of the MFMAs: an operand whose ring is one
// stage deeper is loaded one more step ahead (the LDS left beside a ring of
// two 256x256 stages holds exactly one more panel).  The compiler does not
// track those LDS writes, so completion is awaited by hand (s_waitcnt vmcnt
// with a count of the later loads still allowed in flight, derived from the
// issue order at compile time) before a workgroup barrier; see the pipeline
// driver below.  Every step issues exactly one group of loads per operand
// (groups past the end of K read nothing), which keeps the vmcnt arithmetic
// uniform.
//
// LDS layout: the A ring, STAGES tiles [BM][BK], then the B ring, BSTAGES
// tiles [BN][BK], 16-byte chunks with the
// chunk index XOR-swizzled by the row, so that the 16 lanes one LDS cycle
// serves (256 B) hit 16 different bank groups.  Fragment reads are one
// ds_read_b128 per lane per 32x32x16 MFMA operand (8 consecutive k of one
// row), which on gfx950 streams 256 B per clock, twice the rate of the
// transposing 64-bit reads a [K][N] weight layout would need.  A direct-to-LDS
// load writes 64 consecutive chunks per wave, so the swizzle is applied on the
// global side: the lane that lands on physical chunk p fetches the logical
// chunk that belongs there.
//
// Edges.  Rows past the end of an operand fall outside its buffer range and
// load as zeros; chunks at k >= K are masked explicitly, so the K tail
// contributes nothing.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace swiglu {

// EB is the operand element size in bytes: 2 for bf16, 1 for FP8 E4M3.  MI
// is the MFMA that computes each 32x32 accumulator block:
//   MI = 32: one v_mfma_f32_32x32x16_bf16 per 16 k (bf16: one 16-byte chunk
//            per lane and operand), or one v_mfma_f32_32x32x64_f8f6f4 per 64 k
//            (FP8: two chunks per lane);
//   MI = 16: four v_mfma_f32_16x16x32_bf16 per 32 k, one per 16x16 quarter
//            of the block (bf16 only; one chunk per lane and 16-row half).
// Per flop the 16x16 instruction reads and writes half the accumulator
// registers of the 32x32 one.  A K step of BK elements moves BK * EB bytes
// per tile row either way.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int EB_ = 2,
          int BSTAGES_ = STAGES_, int MI_ = 32>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int STAGES = STAGES_;     // A ring
    static constexpr int BSTAGES = BSTAGES_;   // B ring
    static constexpr int MI = MI_;
    static constexpr int EB = EB_;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int TM = kWaveM / 32;          // 32x32 MFMA blocks per wave (M)
    static constexpr int TN = kWaveN / 32;          // 32x32 MFMA blocks per wave (N)
    static constexpr int kMfmaK = EB == 2 ? (MI == 16 ? 32 : 16) : 64;   // k per MFMA
    static constexpr int kKSub = BK / kMfmaK;       // MFMA k-substeps per K step
    // 16-byte LDS reads per lane, operand and 32-row block in one substep:
    // consecutive chunks of one row (MI = 32), or the two 16-row halves (MI = 16)
    static constexpr int kFragChunks = kMfmaK * EB / 32;
    static constexpr int kMfmaPerBlock = MI == 16 ? 4 : 1;   // per block and substep
    using Acc = typename std::conditional<MI == 16, Acc16, Acc32>::type;
    static constexpr int kElemsPerChunk = 16 / EB;
    static constexpr int kChunksPerRow = BK * EB / 16;   // 16-byte chunks per tile row
    static constexpr int kRowBytes = BK * EB;
    static constexpr int kABytes = BM * kRowBytes;
    static constexpr int kBBytes = BN * kRowBytes;
    static constexpr int kBRing = STAGES * kABytes;   // LDS offset of the B ring
    static constexpr int kLdsBytes = kBRing + BSTAGES * kBBytes;
    // direct-to-LDS loads per wave per K step (each moves 64 x 16 B = 1 KiB)
    static constexpr int kDmaA = kABytes / (kThreads * 16);
    static constexpr int kDmaB = kBBytes / (kThreads * 16);
    static constexpr int kDmaPerStep = kDmaA + kDmaB;
    // workgroups resident per CU that the kernel is built for: two when two
    // fit the 160 KiB of LDS (the kernel then keeps to 256 registers a lane)
    static constexpr int kOccupancy = (2 * kLdsBytes <= 160 * 1024) ? 2 : 1;

    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(EB == 2 || EB == 1, "bf16 or FP8 operands");
    static_assert(MI == 32 || (MI == 16 && EB == 2), "16x16 MFMAs for bf16 operands only");
    static_assert(EB == 2 ? (BK == 32 || BK == 64) : BK == 128,
                  "BK: 32 or 64 bf16 elements, or 128 FP8 elements");
    static_assert(kABytes % (kThreads * 16) == 0 && kDmaA >= 1, "A tile must split evenly");
    static_assert(kBBytes % (kThreads * 16) == 0 && kDmaB >= 1, "B tile must split evenly");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup is 160 KiB");
    static_assert(STAGES >= 2 && STAGES <= 16 && BSTAGES >= 2 && BSTAGES <= 16, "ring depth");
    static_assert(kDmaA * STAGES + kDmaB * BSTAGES < 64, "vmcnt is a 6-bit counter");
    static_assert(kWaves == 4, "4 waves, one per SIMD (the pipeline below)");

    // Row and column, within its 32x32 block, of accumulator register r of
    // lane l: row_l(l) + row_r(r) and col_l(l) + col_r(r) (device.hpp gives
    // the MFMA layouts).
    __device__ __forceinline__ static int row_l(int lane) {
        return MI == 16 ? 4 * (lane >> 4) : 4 * (lane >> 5);
    }
    static constexpr int row_r(int r) { return MI == 16 ? 16 * (r >> 3) + (r & 3) : 8 * (r >> 2) + (r & 3); }
    __device__ __forceinline__ static int col_l(int lane) { return MI == 16 ? (lane & 15) : (lane & 31); }
    static constexpr int col_r(int r) { return MI == 16 ? 16 * ((r >> 2) & 1) : 0; }
};

// Chunk swizzle of a tile row.  The 16 lanes of one LDS cycle read 16
// consecutive rows at the same logical chunk; the XOR spreads them over 16
// distinct 16-byte bank groups of the 256 B bank period (and is periodic in 32
// rows, so 32-row MFMA blocks share it).
template <class S>
__device__ __forceinline__ int swz(int row) {
    if constexpr (S::kChunksPerRow == 4) return ((row >> 1) ^ (row >> 3)) & 3;  // 64 B rows
    else return (row >> 1) & 7;                                                 // 128 B rows
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // dword3 0x00020000: raw (untyped) 32-bit data format, the CDNA setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             static_cast<int>(bytes), 0x00020000);
}

// One 16-byte-per-lane direct-to-LDS load; `lds` is the wave's 1 KiB block.
// IMM, the instruction's immediate offset, is added to the global address
// and to the LDS destination alike: loads into consecutive KiB of LDS can
// share one LDS base (M0) when their global offsets are reduced by IMM.
template <int IMM = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, SWIGLU_LDS char *lds,
                                      uint32_t voff, uint32_t soff) {
    static_assert(IMM >= 0 && IMM < 4096, "12-bit immediate offset");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, reinterpret_cast<SWIGLU_LDS void *>(lds), 16,
                                             static_cast<int>(voff), static_cast<int>(soff), IMM,
                                             0);
}

// An offset no buffer range admits: loads through it return nothing/zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// Workgroup barrier that the compiler may not move memory operations across
// (and that does not imply a full memory fence).
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A K-contiguous operand: logical row r is physical row r*stride + offset of
// a row-major [rows*stride][K] matrix whose rows are ld elements apart (ld = 0:
// K, the rows are contiguous).  (stride 2 selects the Gate (offset 0)
// or Up (offset 1) columns of the interleaved packed weight.)
struct KMajor {
    const void *base;   // elements of the tile shape's size (bf16 or FP8)
    int rows;        // logical rows
    int stride;
    int offset;
    // 1: the operand is the interleaved packed weight read as one matrix and
    // each 64-row group of a panel is loaded de-interleaved: LDS rows
    // 32g' .. 32g'+31 of the group get its even (Gate) rows, the next 32 its
    // odd (Up) rows (pair_row).  Then the Gate and Up columns of one output
    // column meet in the same lane of two adjacent 32x32 accumulator blocks.
    int pairs;
    // Elements from one physical row to the next (a row-strided view); 0: K
    // (contiguous rows).
    int ld;
};

// Panel row whose data lands in LDS row `r` of a de-interleaved panel: within
// each 64-row group, LDS rows 0..31 take the group's rows 0, 2, ..., 62 and
// LDS rows 32..63 its rows 1, 3, ..., 63.
__device__ __forceinline__ int pair_row(int r) {
    return (r & ~63) + 2 * (r & 31) + ((r >> 5) & 1);
}

// The direct-to-LDS loads of one tile panel (NROWS rows) of a KMajor
// operand: NDMA loads per wave per K step.  Load j of a wave fills the 1 KiB
// LDS block j * kWaves + wave: LDS rows r0 + j R (R = 256 / kChunksPerRow,
// r0 = (64 wave + lane) / kChunksPerRow < R), and every load of a lane reads
// the same chunk column, because the swizzle is periodic in R rows.  So a
// lane keeps one byte offset and one K limit for all its loads, and load j
// adds a uniform row distance (dj, in scalar registers) to that offset.
template <class S, int NROWS, int NDMA>
struct PanelLoader {
    static constexpr int R = S::kWaves * 64 / S::kChunksPerRow;   // LDS rows between loads
    static_assert(R % 32 == 0, "the row swizzle and the pair layout repeat every 32 rows");
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff;         // byte offset of this lane's chunk of load 0 at k0 = 0
    int klim;              // K minus the first k of that chunk: step k0 loads iff k0 < klim
    uint32_t row_bytes;    // uniform: bytes from one panel row to the next
    int pairs;             // uniform: a de-interleaved panel (KMajor::pairs)
    int lds_base;          // uniform: LDS byte offset of the wave's block of load 0
    // When K is a multiple of BK (issue<true>): each load's offset, computed
    // once per panel, for a wave-major assignment of the LDS blocks: the
    // loads go in groups of kGroup, and group g of a wave fills kGroup
    // consecutive KiB, blocks (g kWaves + wave) kGroup + i, so that the
    // group's loads share one M0 and differ in the immediate offset i KiB
    // (vo holds the offset less that immediate).  The LDS contents are those
    // of the other assignment: block b holds LDS rows b * 1024 / kRowBytes on.
    static constexpr int kGroup = NDMA < 4 ? NDMA : 4;
    static_assert(NDMA % kGroup == 0, "whole groups of loads");
    uint32_t vo[NDMA];
    int lds_even;          // uniform: LDS byte offset of the wave's group 0
    int klen;

    // Panel = logical rows [r0, r0 + NROWS) of `op`.
    __device__ __forceinline__ void init(const KMajor &op, int r0, int K) {
        const int64_t phys0 = static_cast<int64_t>(r0) * op.stride + op.offset;
        const int64_t phys_end = static_cast<int64_t>(op.rows) * op.stride;  // past the matrix
        const int64_t pitch = op.ld > 0 ? op.ld : K;      // elements per physical row
        const char *panel = static_cast<const char *>(op.base) + phys0 * pitch * S::EB;
        // (past the last row's K elements nothing is read: those chunks are masked)
        int64_t bytes = (phys_end - phys0) * pitch * S::EB;
        if (bytes < 0) bytes = 0;
        if (bytes > 0x7FFFFFF0LL) bytes = 0x7FFFFFF0LL;
        rsrc = make_rsrc(panel, static_cast<uint32_t>(bytes));
        klen = K;
        const int lane = threadIdx.x & 63;
        // uniform per wave: keeps the LDS destinations (M0) in scalar registers
        const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
        const int p = wave * 64 + lane;                   // physical chunk of load 0
        const int row = p / S::kChunksPerRow;             // its LDS row (< R)
        const int c = (p % S::kChunksPerRow) ^ swz<S>(row);
        pairs = op.pairs;
        const int grow = pairs ? pair_row(row) : row;     // panel row it holds
        row_bytes = static_cast<uint32_t>(op.stride) * static_cast<uint32_t>(pitch) * S::EB;
        voff = static_cast<uint32_t>(grow) * row_bytes + c * 16u;
        klim = K - c * S::kElemsPerChunk;
        lds_base = wave * 1024;
        lds_even = wave * kGroup * 1024;
        // (the rows of a block i of a group are at least 8 i: offsets >= i KiB
        // whenever a row has at least 128 bytes, as when K is a multiple of BK)
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
            const int g = j / kGroup, i = j % kGroup;
            const int blk = (g * S::kWaves + wave) * kGroup + i;
            const int r = blk * (1024 / S::kRowBytes) + lane / S::kChunksPerRow;
            const int cj = (lane % S::kChunksPerRow) ^ swz<S>(r);
            const int gr = pairs ? pair_row(r) : r;
            vo[j] = static_cast<uint32_t>(gr) * row_bytes + cj * 16u - static_cast<uint32_t>(i) * 1024u;
        }
    }

    // Uniform bytes from load 0's panel row to load j's: the LDS distance
    // j R rows, or in a de-interleaved panel pair_row(j R) (R is a multiple
    // of 32).
    __device__ __forceinline__ uint32_t dj(int j) const {
        return static_cast<uint32_t>(pairs ? pair_row(j * R) : j * R) * row_bytes;
    }

    // Branch-free, so that the loads can be scheduled among the MFMAs of the
    // same K step: at k >= K (the K tail, or a step past the end) a lane's
    // chunks get an out-of-range offset and load nothing.
    // (No test on the step as a whole: a uniform condition would be turned
    // back into a branch.  k0 <= K + BK keeps kOutOfRange + dj + 2 k0 below
    // 2^32: dj < 2^31 for at most 256 rows of at most 2^21 elements.)
    // Load `only` of the panel, or all NDMA loads when only < 0.
    //  kEven (K a multiple of BK): every chunk of a step below K is inside K,
    //  so the loads take the offsets computed at init with no per-lane
    //  arithmetic (each vector instruction among the MFMAs delays them by
    //  about as much as it takes to issue).  A step at or past K (the ring
    //  running ahead of a tile's last step) loads the last step again, into a
    //  stage no step reads (a uniform clamp: no per-lane masking).
    template <int... J>
    __device__ __forceinline__ void issue_even(uint32_t soff, SWIGLU_LDS char *panel_lds, int only,
                                               std::integer_sequence<int, J...>) const {
        (
            [&] {
                if (only < 0 || only == J)
                    dma16<(J % kGroup) * 1024>(
                        rsrc, panel_lds + lds_even + (J / kGroup) * S::kWaves * kGroup * 1024,
                        vo[J], soff);
            }(),
            ...);
    }
    template <bool kEven = false>
    __device__ __forceinline__ void issue(int k0, SWIGLU_LDS char *panel_lds, int only = -1) const {
        if constexpr (kEven) {
            const uint32_t soff = static_cast<uint32_t>(k0 < klen ? k0 : klen - S::BK) * S::EB;
            issue_even(soff, panel_lds, only, std::make_integer_sequence<int, NDMA>{});
        } else {
            const uint32_t soff = static_cast<uint32_t>(k0) * S::EB;
            const uint32_t v0 = k0 < klim ? voff : kOutOfRange;
#pragma unroll
            for (int j = 0; j < NDMA; ++j)
                if (only < 0 || only == j)
                    dma16(rsrc, panel_lds + lds_base + j * S::kWaves * 1024, v0 + dj(j), soff);
        }
    }
};

// Loader of one output tile: the A panel and the B panel of each K step.
template <class S>
struct TileLoader {
    PanelLoader<S, S::BM, S::kDmaA> a;
    PanelLoader<S, S::BN, S::kDmaB> b;
    int K;

    __device__ __forceinline__ void init(const KMajor &A, int m0, const KMajor &B, int n0,
                                         int K_) {
        K = K_;
        a.init(A, m0, K_);
        b.init(B, n0, K_);
    }

    // Load the A (part 0) or B (part 1, from panel `bp`) panel of K step
    // `kstep` into the ring buffer `dst` (only its load `only`, if >= 0);
    // kstep >= ceil(K/BK) loads nothing.
    template <bool kEven = false>
    __device__ __forceinline__ void issue(int kstep, int part, SWIGLU_LDS char *dst, int only,
                                          const PanelLoader<S, S::BN, S::kDmaB> &bp) const {
        const int k0 = kstep * S::BK;
        if (part == 0) a.template issue<kEven>(k0, dst, only);
        else bp.template issue<kEven>(k0, dst, only);
    }
    template <bool kEven = false>
    __device__ __forceinline__ void issue(int kstep, int part, SWIGLU_LDS char *dst,
                                          int only = -1) const {
        issue<kEven>(kstep, part, dst, only, b);
    }
};

// Fragment registers of one k-substep: raw MFMA operands, kFragChunks
// 16-byte chunks per block.
template <class S>
struct Frags {
    u32x4 a[S::TM][S::kFragChunks];
    u32x4 b[S::TN][S::kFragChunks];
};

// LDS reads issued as inline assembly.  The compiler neither tracks their
// completion nor sees them as LDS accesses; the pipelines wait for them with
// wait_frags().  Keeping the fragment reads out of the compiler's view keeps
// its waitcnt pass from draining the in-flight direct-to-LDS loads (vmcnt(0))
// around LDS reads it cannot prove independent of them.
template <int OFF>
__device__ __forceinline__ u32x4 asm_read_b128(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// Per-lane LDS byte offsets of the fragment reads, relative to a ring buffer,
// one per k-substep and read j for each operand (the swizzle mixes the chunk
// index into the address); 32-row blocks tm / tn are +32 rows (the swizzle
// is periodic in 32 rows).
//  MI = 32: lane l (half h = l / 32) reads the kFragChunks consecutive chunks
//           starting at chunk kFragChunks * (2 KS + h) of row l % 32: for bf16
//           the 8 k of its MFMA operand; for FP8 32 consecutive k;
//  MI = 16: read j is row 16 j + l % 16 (the block's 16-row half j), chunk
//           4 KS + l / 16: the 8 k of the lane's operand of the 16x16 MFMAs
//           of that half.
// The same lane-to-k assignment serves both operands, so whatever order an
// MFMA gives the k within a lane, the products pair A and B at equal k.
template <class S>
struct FragOffsets {
    uint32_t a[S::kKSub][S::kFragChunks];
    uint32_t b[S::kKSub][S::kFragChunks];

    __device__ __forceinline__ void init(int wm, int wn, int lane) {
#pragma unroll
        for (int ks = 0; ks < S::kKSub; ++ks)
#pragma unroll
            for (int j = 0; j < S::kFragChunks; ++j) {
                int ra, rb, c;
                if constexpr (S::MI == 16) {
                    ra = wm * S::kWaveM + 16 * j + (lane & 15);
                    rb = wn * S::kWaveN + 16 * j + (lane & 15);
                    c = ks * 4 + (lane >> 4);
                } else {
                    ra = wm * S::kWaveM + (lane & 31);
                    rb = wn * S::kWaveN + (lane & 31);
                    c = (ks * 2 + (lane >> 5)) * S::kFragChunks + j;
                }
                a[ks][j] = static_cast<uint32_t>(ra * S::kRowBytes + ((c ^ swz<S>(ra)) * 16));
                b[ks][j] = static_cast<uint32_t>(rb * S::kRowBytes + ((c ^ swz<S>(rb)) * 16));
            }
    }
};

template <class S, int I>
__device__ __forceinline__ void read_a_blocks(uint32_t p, Frags<S> &f, int j) {
    if constexpr (I < S::TM) {
        f.a[I][j] = asm_read_b128<I * 32 * S::kRowBytes>(p);
        read_a_blocks<S, I + 1>(p, f, j);
    }
}
template <class S, int I>
__device__ __forceinline__ void read_b_blocks(uint32_t p, Frags<S> &f, int j) {
    if constexpr (I < S::TN) {
        f.b[I][j] = asm_read_b128<I * 32 * S::kRowBytes>(p);
        read_b_blocks<S, I + 1>(p, f, j);
    }
}

// Issue the fragment reads of k-substep KS from the A and B ring buffers at
// LDS addresses `sa` and `sb`.
template <class S, int KS>
__device__ __forceinline__ void read_frags(uint32_t sa, uint32_t sb, const FragOffsets<S> &o,
                                           Frags<S> &f) {
#pragma unroll
    for (int j = 0; j < S::kFragChunks; ++j) {
        read_a_blocks<S, 0>(sa + o.a[KS][j], f, j);
        read_b_blocks<S, 0>(sb + o.b[KS][j], f, j);
    }
}

// Load issue order of the pipeline below, and the vmcnt waits it implies.
// K step t's panels are loaded in group g = t - STAGES (A) and t - BSTAGES
// (B); the prologue issues the groups -max(STAGES, BSTAGES) .. -1, and the
// last substep of step t issues group t.  Inside a group the panel of the
// shallower ring goes first (A when the depths are equal), so that the panel
// needed soonest is never queued behind the one needed later.
template <class S>
struct IssueOrder {
    static constexpr bool kAFirst = S::STAGES <= S::BSTAGES;
    static constexpr int kDeep = S::STAGES > S::BSTAGES ? S::STAGES : S::BSTAGES;

    // Loads issued after both panels of K step `s` when the groups up to
    // `last` have been issued (vmcnt counts completions in issue order, so
    // waiting for at most this many outstanding loads means step s landed).
    static constexpr int loads_after(int s, int last) {
        int total = 0, end_a = 0, end_b = 0;
        for (int g = -kDeep; g <= last; ++g) {
            for (int k = 0; k < 2; ++k) {
                const bool a_part = (k == 0) == kAFirst;
                const int step = g + (a_part ? S::STAGES : S::BSTAGES);
                if (step < 0) continue;
                total += a_part ? S::kDmaA : S::kDmaB;
                if (step == s) (a_part ? end_a : end_b) = total;
            }
        }
        return total - (end_a > end_b ? end_a : end_b);
    }
    // before step 0 (the prologue has issued groups up to -1)
    static constexpr int kWaitPrologue = loads_after(0, -1);
    // before step t+1, in step t (groups up to t-1 issued); the same for every t
    static constexpr int kWaitSteady = loads_after(2 * kDeep + 3, 2 * kDeep + 1);
    static_assert(loads_after(2 * kDeep + 4, 2 * kDeep + 2) == kWaitSteady, "steady state");
    // every wait from the first step on is the steady one
    static constexpr bool steady_from_start() {
        for (int t = 0; t <= 2 * kDeep; ++t)
            if (loads_after(t + 1, t - 1) != kWaitSteady) return false;
        return true;
    }
    static_assert(steady_from_start(), "the first steps wait as the steady state does");
    static_assert(kWaitPrologue < 64 && kWaitSteady < 64, "vmcnt is a 6-bit counter");
};

// Wait until every fragment read issued so far has landed, and make the
// fragment registers of `f` depend on that wait (volatile asm statements keep
// their order, so each empty "+v" statement, which the MFMAs depend on, stays
// after the wait).
template <class S>
__device__ __forceinline__ void wait_frags(Frags<S> &f) {
    asm volatile("s_waitcnt lgkmcnt(0)");
#pragma unroll
    for (int j = 0; j < S::kFragChunks; ++j) {
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) asm volatile("" : "+v"(f.a[tm][j]));
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn) asm volatile("" : "+v"(f.b[tn][j]));
    }
}

// The MFMAs of one k-substep (32x32 MFMAs; the 16x16 ones go through mma16).
template <class S>
__device__ __forceinline__ void mma(const Frags<S> &f, typename S::Acc (&acc)[S::TM][S::TN]) {
    static_assert(S::MI == 32, "16x16 MFMAs: mma16");
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn) {
            if constexpr (S::EB == 2) {
                acc[tm][tn].v = mfma_32x32x16(__builtin_bit_cast(bf16x8, f.a[tm][0]),
                                              __builtin_bit_cast(bf16x8, f.b[tn][0]),
                                              acc[tm][tn].v);
            } else {
                acc[tm][tn].v = mfma_32x32x64_fp8(f.a[tm][0], f.a[tm][1], f.b[tn][0], f.b[tn][1],
                                                  acc[tm][tn].v);
            }
        }
}

// Fragment read R of k-substep KS (R < kFragChunks (TM + TN), in the order of
// read_frags: for each read j, the TM A blocks, then the TN B blocks).
template <class S, int KS, int R>
__device__ __forceinline__ void read_frag_one(uint32_t sa, uint32_t sb, const FragOffsets<S> &o,
                                              Frags<S> &f) {
    constexpr int kPer = S::TM + S::TN;
    constexpr int j = R / kPer, b = R % kPer;
    if constexpr (b < S::TM)
        f.a[b][j] = asm_read_b128<b * 32 * S::kRowBytes>(sa + o.a[KS][j]);
    else
        f.b[b - S::TM][j] = asm_read_b128<(b - S::TM) * 32 * S::kRowBytes>(sb + o.b[KS][j]);
}

// Where a substep's fragment reads find their ring stage.  RuntimeReads: the
// stages' LDS addresses sa / sb, known at run time (a per-lane add per read
// address).  FixedReads: stage offsets OFFA / OFFB from the LDS base known at
// compile time (a ring walked in unrolled groups of its period): each read
// address is a loop-invariant per-lane base plus the 64 KiB-aligned part of
// the offset, and the rest rides in the instruction's immediate offset.
template <class S>
struct RuntimeReads {
    uint32_t sa, sb;
    const FragOffsets<S> *o;
    template <int KS, int R>
    __device__ __forceinline__ void read(Frags<S> &f) const {
        read_frag_one<S, KS, R>(sa, sb, *o, f);
    }
};
template <class S, int OFFA, int OFFB>
struct FixedReads {
    uint32_t lds_addr;
    const FragOffsets<S> *o;
    template <int OFF>
    __device__ __forceinline__ static u32x4 at(uint32_t lane_base) {
        static_assert((OFF & 0xFFFF) + 16 <= 0x10000, "16-bit immediate offset");
        return asm_read_b128<(OFF & 0xFFFF)>(lane_base + static_cast<uint32_t>(OFF & ~0xFFFF));
    }
    template <int KS, int R>
    __device__ __forceinline__ void read(Frags<S> &f) const {
        constexpr int kPer = S::TM + S::TN;
        constexpr int j = R / kPer, b = R % kPer;
        if constexpr (b < S::TM)
            f.a[b][j] = at<OFFA + b * 32 * S::kRowBytes>(lds_addr + o->a[KS][j]);
        else
            f.b[b - S::TM][j] = at<OFFB + (b - S::TM) * 32 * S::kRowBytes>(lds_addr + o->b[KS][j]);
    }
};

// The 16x16 MFMAs of one k-substep, issued one by one (inline assembly, in
// program order) on the fragments `cur`, and between them:
//  - the fragment reads of the next k-substep KSN (from the ring buffers at
//    LDS addresses sa / sb, into `nxt`): read R after MFMA R n / (2 r) of the
//    n, so that all r of them go out in the first half of the substep and
//    have landed when the next substep starts;
//  - if kLoads > 0, `load(d)` after MFMA d n / kLoads (the direct-to-LDS
//    loads of the substep that refills the ring).
// A 16x16x32 MFMA keeps the MFMA pipe busy for only 16 cycles, so a run of
// reads or loads issued back to back would leave it idle; spread out, each
// issues in the shadow of the MFMA before it.  (The compiler's scheduler
// cannot interleave them: it does not see the assembly MFMAs.)  The reads
// write the other fragment buffer, which the previous substep's MFMAs read:
// those were issued before these reads, and a read's data lands long after
// an MFMA has taken its operands.
template <class S, int KSN, bool kReads, int kLoads, int kBegin, int kEnd, bool kInit, int I,
          class Reads, class Load, int... R, int... D>
__device__ __forceinline__ void mma16_at(const Frags<S> &cur, Frags<S> &nxt, const Reads &rd,
                                         typename S::Acc (&acc)[S::TM][S::TN], const Load &load,
                                         std::integer_sequence<int, R...>,
                                         std::integer_sequence<int, D...>) {
    constexpr int kSpan = kEnd - kBegin;
    constexpr int kNReads = sizeof...(R);
    constexpr int tm = I / (4 * S::TN), tn = (I / 4) % S::TN, sm = (I / 2) % 2, sn = I % 2;
    // quad 2 sm + sn of block (tm, tn): rows 16 sm, columns 16 sn
    if constexpr (kInit) mfma_16x16x32_init(acc[tm][tn].v[2 * sm + sn], cur.a[tm][sm], cur.b[tn][sn]);
    else mfma_16x16x32_acc(acc[tm][tn].v[2 * sm + sn], cur.a[tm][sm], cur.b[tn][sn]);
    (
        [&] {
            if constexpr (kReads && kBegin + R * (kSpan / 2) / kNReads == I)
                rd.template read<KSN, R>(nxt);
        }(),
        ...);
    (
        [&] {
            if constexpr (kLoads > 0 && kBegin + D * kSpan / (kLoads > 0 ? kLoads : 1) == I)
                load(D);
        }(),
        ...);
}
// MFMAs [kBegin, kEnd) of the substep, with the reads (if kReads) and loads
// spread over that range; kInit: they start the accumulators (C = 0).
template <class S, int KSN, bool kReads, int kLoads, int kBegin, int kEnd, bool kInit = false,
          int I = kBegin, class Reads, class Load>
__device__ __forceinline__ void mma16(const Frags<S> &cur, Frags<S> &nxt, const Reads &rd,
                                      typename S::Acc (&acc)[S::TM][S::TN], const Load &load) {
    static_assert(S::MI == 16, "16x16 MFMAs");
    if constexpr (I < kEnd) {
        mma16_at<S, KSN, kReads, kLoads, kBegin, kEnd, kInit, I>(
            cur, nxt, rd, acc, load,
            std::make_integer_sequence<int, S::kFragChunks * (S::TM + S::TN)>{},
            std::make_integer_sequence<int, (kLoads > 0 ? kLoads : 1)>{});
        mma16<S, KSN, kReads, kLoads, kBegin, kEnd, kInit, I + 1>(cur, nxt, rd, acc, load);
    }
}

template <class S>
__device__ __forceinline__ void zero_acc(typename S::Acc (&acc)[S::TM][S::TN]) {
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[tm][tn].set_quad(q, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    // (assembly MFMAs read them: the accumulator writes' two wait states)
    if constexpr (S::MI == 16) asm volatile("s_nop 1");
}

// ---------------------------------------------------------------------------
// Plain pipeline (4 waves, one per SIMD).  A "step sequence" is a run of K
// steps numbered 0..total-1; `issue(t, part, dst, j)` loads the A (part 0)
// or B (part 1) panel of sequence step t into the ring buffer `dst` (only its
// load j if j >= 0).  Before step
// t+1 is read, each wave waits until its loads of step t+1 have landed (the
// later loads IssueOrder counts may stay in flight), then the workgroup meets
// at one barrier, which also proves that every wave has finished reading
// step t's buffers; they are refilled with step t+STAGES (A) and
// t+BSTAGES (B) right after it.  The barrier sits before the MFMAs of step
// t's last k-substep, so those MFMAs overlap the first fragment reads of step
// t+1; within a step the reads of substep ks+1 overlap the MFMAs of substep
// ks.
// ---------------------------------------------------------------------------
template <class S>
struct Pipeline {
    SWIGLU_LDS char *lds;
    uint32_t lds_addr;
    FragOffsets<S> off;
    Frags<S> f[2];

    using Order = IssueOrder<S>;
    static constexpr int kMfma16 = S::TM * S::TN * 4;   // 16x16 MFMAs per substep
    // 16x16 MFMAs of the last substep issued before its wait and barrier, so
    // the MFMA pipe works while the workgroup meets: an eighth of the
    // substep's.  Measured with the 256x256 tile's 64: with the ring stages
    // computed at run time, 16 was fastest of 0, 4, 8, 16, 24, 32, 40 (+1 %
    // and +5 % over none at M=4096 K=8192 N=29568 and M=2048 K=1536 N=8960);
    // with the unrolled ring walk (fewer instructions to issue around the
    // barrier) 2, 4 and 8 are within 0.3 % of each other and 0.2-1.5 %
    // faster than 16 on those two workloads, M=8192 K=5120 N=13824 and
    // variant S, 24 and 32 are 0.8-4.6 % slower (more delays the refill loads).
    static constexpr int kEarlyMfma = kMfma16 / 8;
    static_assert(S::MI != 16 || (kEarlyMfma > 0 && kEarlyMfma < kMfma16),
                  "MFMAs on both sides of the barrier");

    __device__ __forceinline__ SWIGLU_LDS char *stage_a(int t) const {
        return lds + (t % S::STAGES) * S::kABytes;
    }
    __device__ __forceinline__ SWIGLU_LDS char *stage_b(int t) const {
        return lds + S::kBRing + (t % S::BSTAGES) * S::kBBytes;
    }
    __device__ __forceinline__ uint32_t addr_a(int t) const {
        return lds_addr + static_cast<uint32_t>((t % S::STAGES) * S::kABytes);
    }
    __device__ __forceinline__ uint32_t addr_b(int t) const {
        return lds_addr + static_cast<uint32_t>(S::kBRing + (t % S::BSTAGES) * S::kBBytes);
    }

    // Group g of the issue order: the A panel of step g + STAGES and the B
    // panel of step g + BSTAGES (each skipped if before step 0), the
    // shallower ring's first.
    template <class Issue>
    __device__ __forceinline__ void issue_group(const Issue &issue, int g) const {
        const int ta = g + S::STAGES, tb = g + S::BSTAGES;
        if constexpr (Order::kAFirst) {
            if (ta >= 0) issue(ta, 0, stage_a(ta), -1);
            if (tb >= 0) issue(tb, 1, stage_b(tb), -1);
        } else {
            if (tb >= 0) issue(tb, 1, stage_b(tb), -1);
            if (ta >= 0) issue(ta, 0, stage_a(ta), -1);
        }
    }
    // Load d (d < kDmaPerStep) of steady-state group g, in the group's issue
    // order.
    // (SA, SB >= 0: group g's stages, known at compile time in an unrolled ring)
    template <int SA = -1, int SB = -1, class Issue>
    __device__ __forceinline__ void issue_one(const Issue &issue, int g, int d) const {
        const int ta = g + S::STAGES, tb = g + S::BSTAGES;
        constexpr int kFirst = Order::kAFirst ? S::kDmaA : S::kDmaB;
        const bool first = d < kFirst;
        const bool a_part = first == Order::kAFirst;
        const int j = first ? d : d - kFirst;
        if constexpr (SA >= 0) {
            if (a_part) issue(ta, 0, lds + SA * S::kABytes, j);
            else issue(tb, 1, lds + S::kBRing + SB * S::kBBytes, j);
        } else {
            if (a_part) issue(ta, 0, stage_a(ta), j);
            else issue(tb, 1, stage_b(tb), j);
        }
    }
    // Ring period: the steps after which both rings are back at stage 0.
    static constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }
    static constexpr int kPeriod = S::STAGES / gcd(S::STAGES, S::BSTAGES) * S::BSTAGES;
    // Fragment reads of step t (stage offsets known when PH >= 0: t % kPeriod == PH).
    template <int PH>
    __device__ __forceinline__ auto reads_of(int t) const {
        if constexpr (PH >= 0)
            return FixedReads<S, (PH % S::STAGES) * S::kABytes,
                              S::kBRing + (PH % S::BSTAGES) * S::kBBytes>{lds_addr, &off};
        else
            return RuntimeReads<S>{addr_a(t), addr_b(t), &off};
    }

    __device__ __forceinline__ void init(SWIGLU_LDS char *lds_) {
        lds = lds_;
        lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_));
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
        off.init(wave / S::WN, wave % S::WN, lane);
    }

    // The prologue in two halves, so that a persistent workgroup can put the
    // loads of its next tile in flight before it runs the current tile's
    // epilogue (the ring must be idle: after drain()).
    template <class Issue>
    __device__ __forceinline__ void prologue_issue(const Issue &issue) {
#pragma unroll
        for (int g = -Order::kDeep; g < 0; ++g) issue_group(issue, g);
    }
    __device__ __forceinline__ void prologue_wait() {
        wait_vmcnt<Order::kWaitPrologue>();
        block_barrier();
        read_frags<S, 0>(addr_a(0), addr_b(0), off, f[0]);
    }
    template <class Issue>
    __device__ __forceinline__ void prologue(const Issue &issue) {
        prologue_issue(issue);
        prologue_wait();
    }

    // kInit: the step starts the accumulators (16x16 MFMAs only: its first
    // substep's MFMAs take C = 0, no zero_acc() before it).
    template <int KS, bool kInit, int PH, class Issue, class Hook>
    __device__ __forceinline__ void substeps(const Issue &issue, int t, int total,
                                             typename S::Acc (&acc)[S::TM][S::TN], const Hook &hook) {
        constexpr int last = S::kKSub - 1;
        __builtin_amdgcn_sched_barrier(0);   // keep the previous substep's MFMAs above this wait
        wait_frags<S>(f[KS & 1]);
        if constexpr (KS < last) {
            if constexpr (S::MI == 16) {
                hook(KS);
                mma16<S, KS + 1, true, 0, 0, kMfma16, kInit && KS == 0>(
                    f[KS & 1], f[(KS + 1) & 1], reads_of<PH>(t), acc, [](int) {});
            } else {
                read_frags<S, KS + 1>(addr_a(t), addr_b(t), off, f[(KS + 1) & 1]);
                hook(KS);
                mma<S>(f[KS & 1], acc);
            }
            substeps<KS + 1, kInit, PH>(issue, t, total, acc, hook);
        } else {
            // Step t+1's loads have landed (own wait, then everyone's via the
            // barrier), and every wave has finished reading stage t.  The
            // first fragment reads of step t+1 go out before this substep's
            // MFMAs (an LDS read lands asynchronously: its destination must
            // not be registers that MFMAs issued just before it still read),
            // and the refill of step t's buffers (group t: steps t+STAGES and
            // t+BSTAGES) after them, in one
            // straight-line block, so the scheduler can place those loads --
            // which write LDS, not registers -- among the MFMAs instead of
            // leaving the MFMA pipe idle while they are issued.  After the
            // last step the loads are masked dummies (the issue lambda maps
            // steps past the end to nothing) and the reads are unused; drain()
            // waits for them.
            if constexpr (S::MI == 16) {
                // the first kEarlyMfma MFMAs of this substep (operands already
                // in registers) go out before the wait and the barrier
                hook(KS);
                mma16<S, 0, false, 0, 0, kEarlyMfma>(f[KS & 1], f[(KS + 1) & 1],
                                                     RuntimeReads<S>{0, 0, &off}, acc, [](int) {});
                wait_vmcnt<Order::kWaitSteady>();
                block_barrier();
                constexpr int kNext = PH >= 0 ? (PH + 1) % kPeriod : -1;
                mma16<S, 0, true, S::kDmaPerStep, kEarlyMfma, kMfma16>(
                    f[KS & 1], f[(KS + 1) & 1], reads_of<kNext>(t + 1), acc, [&](int d) {
                        if constexpr (PH >= 0)
                            issue_one<PH % S::STAGES, PH % S::BSTAGES>(issue, t, d);
                        else
                            issue_one(issue, t, d);
                    });
            } else {
                wait_vmcnt<Order::kWaitSteady>();
                block_barrier();
                read_frags<S, 0>(addr_a(t + 1), addr_b(t + 1), off, f[(KS + 1) & 1]);
                hook(KS);
                mma<S>(f[KS & 1], acc);
                issue_group(issue, t);
                interleave_mfma_and_loads();
            }
        }
    }

    // Scheduling pattern for the last substep: one MFMA, then its share of
    // the step's direct-to-LDS loads, and so on (sched_group_barrier masks:
    // 0x008 MFMA, 0x020 VMEM read).
    __device__ __forceinline__ static void interleave_mfma_and_loads() {
        constexpr int kMfma = S::TM * S::TN * S::kMfmaPerBlock;
        constexpr int kPer = (S::kDmaPerStep + kMfma - 1) / kMfma;
#pragma unroll
        for (int i = 0; i < kMfma; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, kPer, 0);
        }
    }

    // PH >= 0: t % kPeriod == PH, so every ring stage the step touches is a
    // compile-time offset (no stage arithmetic in the step).
    template <bool kInit = false, int PH = -1, class Issue, class Hook>
    __device__ __forceinline__ void step(const Issue &issue, int t, int total,
                                         typename S::Acc (&acc)[S::TM][S::TN], const Hook &hook) {
        static_assert(S::kKSub % 2 == 0, "fragment double buffer alternates per substep");
        static_assert(!kInit || S::MI == 16, "accumulator start by MFMA: 16x16 path");
        static_assert(PH < 0 || S::MI == 16, "fixed stages: 16x16 path");
        substeps<0, kInit, PH>(issue, t, total, acc, hook);
    }
    // Steps t0 .. t0 + kPeriod - 1 with t0 % kPeriod == P0 (I counts them).
    template <int P0, int I, class Issue>
    __device__ __forceinline__ void steps_of_period(const Issue &issue, int t0, int total,
                                                    typename S::Acc (&acc)[S::TM][S::TN]) {
        if constexpr (I < kPeriod) {
            step<false, (P0 + I) % kPeriod>(issue, t0 + I, total, acc, [](int) {});
            steps_of_period<P0, I + 1>(issue, t0, total, acc);
        }
    }

    // Steps [t_begin, t_end).  kUnroll (16x16 MFMAs): whole periods of the
    // ring starting at a multiple of kPeriod run as one unrolled group of
    // steps with compile-time stages; the steps before the first and after
    // the last such group run with the stages computed at run time.  (Those
    // per-step stage computations -- the remainder by 3 of a three-stage ring,
    // the per-stage read addresses -- sat between the MFMAs of the steps.)
    template <bool kUnroll = false, class Issue>
    __device__ __forceinline__ void run(const Issue &issue, int t_begin, int t_end, int total,
                                        typename S::Acc (&acc)[S::TM][S::TN]) {
        int t = t_begin;
        if constexpr (kUnroll && S::MI == 16) {
            for (; t < t_end && t % kPeriod != 0; ++t) step(issue, t, total, acc, [](int) {});
            for (; t + kPeriod <= t_end; t += kPeriod) steps_of_period<0, 0>(issue, t, total, acc);
        }
        for (; t < t_end; ++t) step(issue, t, total, acc, [](int) {});
    }
    // The same, with step t_begin (< t_end) starting the accumulators.
    template <bool kUnroll = false, class Issue>
    __device__ __forceinline__ void run_init(const Issue &issue, int t_begin, int t_end, int total,
                                             typename S::Acc (&acc)[S::TM][S::TN]) {
        step<true>(issue, t_begin, total, acc, [](int) {});
        run<kUnroll>(issue, t_begin + 1, t_end, total, acc);
    }
    // Steps [0, t_end), step 0 starting the accumulators.  kUnroll: the
    // unrolled groups start right after it, at step 1 (phase 1 of the ring
    // period), so that only (t_end - 1) % kPeriod steps run the generic step.
    template <bool kUnroll = false, class Issue>
    __device__ __forceinline__ void run_init0(const Issue &issue, int t_end, int total,
                                              typename S::Acc (&acc)[S::TM][S::TN]) {
        step<true>(issue, 0, total, acc, [](int) {});
        int t = 1;
        if constexpr (kUnroll && S::MI == 16)
            for (; t + kPeriod <= t_end; t += kPeriod) steps_of_period<1, 0>(issue, t, total, acc);
        for (; t < t_end; ++t) step(issue, t, total, acc, [](int) {});
    }

    __device__ __forceinline__ void drain() {
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        block_barrier();
        // the last assembly MFMAs' results are read from here on
        if constexpr (S::MI == 16) wait_mfma_results();
    }
    // drain(), then redefine the accumulators after its wait, so that every
    // later read of them depends on the wait (the compiler does not know the
    // assembly MFMAs' latency and could otherwise move a read above it).
    __device__ __forceinline__ void drain(typename S::Acc (&acc)[S::TM][S::TN]) {
        drain();
        if constexpr (S::MI == 16) {
#pragma unroll
            for (int a = 0; a < S::TM; ++a)
#pragma unroll
                for (int c = 0; c < S::TN; ++c)
#pragma unroll
                    for (int q = 0; q < 4; ++q) asm volatile("" : "+a"(acc[a][c].v[q]));
        }
    }
};

// Tile order.  tile_coords() walks a tile index t over the tile grid in
// groups of `group_m` tile rows (tiles close in t share A rows and B columns);
// xcd_order() renumbers workgroup ids, which the hardware dispatches
// round-robin over the 8 XCDs (id mod 8), so that each XCD receives a
// contiguous run of indices and its L2 sees neighbouring tiles.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m,
                                            int &tm, int &tn) {
    const int width = group_m * tiles_n;
    const int group = t / width;
    const int first_m = group * group_m;
    const int rows_in_group = min(tiles_m - first_m, group_m);
    const int in_group = t % width;
    tm = first_m + in_group % rows_in_group;
    tn = in_group / rows_in_group;
}
__device__ __forceinline__ int xcd_order(int bid, int nb) {
    const int per = nb / 8;
    return (bid < per * 8) ? (bid % 8) * per + bid / 8 : bid;
}
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int group_m, int &tm,
                                            int &tn) {
    tile_coords(xcd_order(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace swiglu
