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
// Pipeline.  K steps stream through a ring of STAGES LDS buffers filled by
// direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds: no VGPR staging,
// no LDS write instructions), STAGES-1 steps ahead of the MFMAs.  The
// compiler does not track those LDS writes, so completion is awaited by hand
// (s_waitcnt vmcnt with a count of the later steps still allowed in flight)
// before a workgroup barrier; see the pipeline driver below.  Every step
// issues exactly one group of loads (groups past the end of K read nothing),
// which keeps the vmcnt arithmetic uniform.
//
// LDS layout: A tile [BM][BK] then B tile [BN][BK], 16-byte chunks with the
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

#include "device.hpp"

namespace swiglu {

// EB is the operand element size in bytes: 2 for bf16 (v_mfma_f32_32x32x16_bf16,
// 16 k per MFMA, one 16-byte chunk per lane and operand), 1 for FP8 E4M3
// (v_mfma_f32_32x32x64_f8f6f4, 64 k per MFMA, two chunks per lane).  A K step
// of BK elements moves BK * EB bytes per tile row either way.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int EB_ = 2>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int STAGES = STAGES_;
    static constexpr int EB = EB_;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int TM = kWaveM / 32;          // 32x32 MFMA blocks per wave (M)
    static constexpr int TN = kWaveN / 32;          // 32x32 MFMA blocks per wave (N)
    static constexpr int kMfmaK = EB == 2 ? 16 : 64;   // k per MFMA
    static constexpr int kKSub = BK / kMfmaK;       // MFMA k-substeps per K step
    static constexpr int kFragChunks = kMfmaK * EB / 32;   // 16-byte chunks per lane and operand
    static constexpr int kElemsPerChunk = 16 / EB;
    static constexpr int kChunksPerRow = BK * EB / 16;   // 16-byte chunks per tile row
    static constexpr int kRowBytes = BK * EB;
    static constexpr int kABytes = BM * kRowBytes;
    static constexpr int kBBytes = BN * kRowBytes;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kLdsBytes = kStageBytes * STAGES;
    // direct-to-LDS loads per wave per K step (each moves 64 x 16 B = 1 KiB)
    static constexpr int kDmaA = kABytes / (kThreads * 16);
    static constexpr int kDmaB = kBBytes / (kThreads * 16);
    static constexpr int kDmaPerStep = kDmaA + kDmaB;
    // workgroups resident per CU that the kernel is built for: two when two
    // fit the 160 KiB of LDS (the kernel then keeps to 256 registers a lane)
    static constexpr int kOccupancy = (2 * kLdsBytes <= 160 * 1024) ? 2 : 1;

    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(EB == 2 || EB == 1, "bf16 or FP8 operands");
    static_assert(EB == 2 ? (BK == 32 || BK == 64) : BK == 128,
                  "BK: 32 or 64 bf16 elements, or 128 FP8 elements");
    static_assert(kABytes % (kThreads * 16) == 0 && kDmaA >= 1, "A tile must split evenly");
    static_assert(kBBytes % (kThreads * 16) == 0 && kDmaB >= 1, "B tile must split evenly");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup is 160 KiB");
    static_assert(STAGES >= 2 && STAGES <= 8, "ring depth");
    static_assert(kDmaPerStep * (STAGES - 1) < 64, "vmcnt is a 6-bit counter");
    static_assert(kWaves == 4, "4 waves, one per SIMD (the pipeline below)");
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
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, SWIGLU_LDS char *lds,
                                      uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, reinterpret_cast<SWIGLU_LDS void *>(lds), 16,
                                             static_cast<int>(voff), static_cast<int>(soff), 0,
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
// operand: NDMA loads per wave per K step.
template <class S, int NROWS, int NDMA>
struct PanelLoader {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff[NDMA];   // byte offset of this lane's chunk at k0 = 0 (from the panel base)
    int kcol[NDMA];        // first k of that chunk
    int lds_off[NDMA];     // LDS byte offset (within the panel) of the wave's 1 KiB block

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
        const int lane = threadIdx.x & 63;
        // uniform per wave: keeps the LDS destinations (M0) in scalar registers
        const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
            const int block = j * S::kWaves + wave;
            const int p = block * 64 + lane;                  // physical chunk in the panel
            const int row = p / S::kChunksPerRow;             // LDS row
            const int c = (p % S::kChunksPerRow) ^ swz<S>(row);
            const int grow = op.pairs ? pair_row(row) : row;  // panel row it holds
            voff[j] = static_cast<uint32_t>(grow * op.stride) * static_cast<uint32_t>(pitch) * S::EB +
                      c * 16u;
            kcol[j] = c * S::kElemsPerChunk;
            lds_off[j] = block * 1024;
        }
    }

    // Branch-free, so that the loads can be scheduled among the MFMAs of the
    // same K step: chunks at k >= K (the K tail, or a step past the end) get
    // an out-of-range offset and load nothing.
    // (No test on the step as a whole: a uniform condition would be turned
    // back into a branch.  k0 <= K + BK keeps kOutOfRange + 2 k0 below 2^32.)
    __device__ __forceinline__ void issue(int k0, int K, SWIGLU_LDS char *panel_lds) const {
        const uint32_t soff = static_cast<uint32_t>(k0) * S::EB;
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
            const uint32_t v = (k0 + kcol[j] < K) ? voff[j] : kOutOfRange;
            dma16(rsrc, panel_lds + lds_off[j], v, soff);
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

    // Load K step `kstep` into `stage` with B panel `bp`; kstep >= ceil(K/BK)
    // loads nothing.
    __device__ __forceinline__ void issue(int kstep, SWIGLU_LDS char *stage,
                                          const PanelLoader<S, S::BN, S::kDmaB> &bp) const {
        const int k0 = kstep * S::BK;
        a.issue(k0, K, stage);
        bp.issue(k0, K, stage + S::kABytes);
    }
    __device__ __forceinline__ void issue(int kstep, SWIGLU_LDS char *stage) const {
        issue(kstep, stage, b);
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

// Per-lane LDS byte offsets of the fragment reads, relative to a stage base,
// one per k-substep and 16-byte chunk for each operand (the swizzle mixes the
// chunk index into the address); 32-row blocks tm / tn are +32 rows (the
// swizzle has period 32).  Lane l (half h = l / 32) takes the kFragChunks
// consecutive chunks starting at chunk kFragChunks * (2 KS + h) of its row:
// for bf16 the 8 k of its MFMA operand; for FP8 32 consecutive k.  The same
// lane-to-k assignment serves both operands, so whatever order the FP8 MFMA
// gives those k within a lane, the products pair A and B at equal k.
template <class S>
struct FragOffsets {
    uint32_t a[S::kKSub][S::kFragChunks];
    uint32_t b[S::kKSub][S::kFragChunks];

    __device__ __forceinline__ void init(int wm, int wn, int lane) {
        const int h = lane >> 5;
        const int ra = wm * S::kWaveM + (lane & 31);
        const int rb = wn * S::kWaveN + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < S::kKSub; ++ks)
#pragma unroll
            for (int j = 0; j < S::kFragChunks; ++j) {
                const int c = (ks * 2 + h) * S::kFragChunks + j;
                a[ks][j] = static_cast<uint32_t>(ra * S::kRowBytes + ((c ^ swz<S>(ra)) * 16));
                b[ks][j] = static_cast<uint32_t>(S::kABytes + rb * S::kRowBytes +
                                                 ((c ^ swz<S>(rb)) * 16));
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

// Issue the fragment reads of k-substep KS from the stage at LDS address `stage`.
template <class S, int KS>
__device__ __forceinline__ void read_frags(uint32_t stage, const FragOffsets<S> &o,
                                           Frags<S> &f) {
#pragma unroll
    for (int j = 0; j < S::kFragChunks; ++j) {
        read_a_blocks<S, 0>(stage + o.a[KS][j], f, j);
        read_b_blocks<S, 0>(stage + o.b[KS][j], f, j);
    }
}

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

template <class S>
__device__ __forceinline__ void mma(const Frags<S> &f, f32x16 (&acc)[S::TM][S::TN]) {
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn) {
            if constexpr (S::EB == 2)
                acc[tm][tn] = mfma_32x32x16(__builtin_bit_cast(bf16x8, f.a[tm][0]),
                                            __builtin_bit_cast(bf16x8, f.b[tn][0]), acc[tm][tn]);
            else
                acc[tm][tn] = mfma_32x32x64_fp8(f.a[tm][0], f.a[tm][1], f.b[tn][0], f.b[tn][1],
                                                acc[tm][tn]);
        }
}

template <class S>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[S::TM][S::TN]) {
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[tm][tn][i] = 0.0f;
}

// ---------------------------------------------------------------------------
// Plain pipeline (4 waves, one per SIMD).  A "step sequence" is a run of K
// steps numbered 0..total-1; `issue(t, stage)` loads sequence step t into an
// LDS stage.  Before step t+1 is read, each wave waits until at most
// STAGES-2 later steps' loads are outstanding, then the workgroup meets at
// one barrier, which also proves that every wave has finished reading step
// t's buffer; that buffer is refilled with step t+STAGES right after it.  The
// barrier sits before the MFMAs of step t's last k-substep, so those MFMAs
// overlap the first fragment reads of step t+1; within a step the reads of
// substep ks+1 overlap the MFMAs of substep ks.
// ---------------------------------------------------------------------------
template <class S>
struct Pipeline {
    SWIGLU_LDS char *lds;
    uint32_t lds_addr;
    FragOffsets<S> off;
    Frags<S> f[2];

    __device__ __forceinline__ SWIGLU_LDS char *stage(int t) const {
        return lds + (t % S::STAGES) * S::kStageBytes;
    }
    __device__ __forceinline__ uint32_t stage_addr(int t) const {
        return lds_addr + static_cast<uint32_t>((t % S::STAGES) * S::kStageBytes);
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
        for (int t = 0; t < S::STAGES; ++t) issue(t, stage(t));
    }
    __device__ __forceinline__ void prologue_wait() {
        wait_vmcnt<S::kDmaPerStep * (S::STAGES - 1)>();
        block_barrier();
        read_frags<S, 0>(stage_addr(0), off, f[0]);
    }
    template <class Issue>
    __device__ __forceinline__ void prologue(const Issue &issue) {
        prologue_issue(issue);
        prologue_wait();
    }

    template <int KS, class Issue, class Hook>
    __device__ __forceinline__ void substeps(const Issue &issue, int t, int total,
                                             f32x16 (&acc)[S::TM][S::TN], const Hook &hook) {
        constexpr int last = S::kKSub - 1;
        __builtin_amdgcn_sched_barrier(0);   // keep the previous substep's MFMAs above this wait
        wait_frags<S>(f[KS & 1]);
        if constexpr (KS < last) {
            read_frags<S, KS + 1>(stage_addr(t), off, f[(KS + 1) & 1]);
            hook(KS);
            mma<S>(f[KS & 1], acc);
            substeps<KS + 1>(issue, t, total, acc, hook);
        } else {
            // Step t+1's loads have landed (own wait, then everyone's via the
            // barrier), and every wave has finished reading stage t.  The
            // first fragment reads of step t+1 go out before this substep's
            // MFMAs (an LDS read lands asynchronously: its destination must
            // not be registers that MFMAs issued just before it still read),
            // and the refill of stage t (step t+STAGES) after them, in one
            // straight-line block, so the scheduler can place those loads --
            // which write LDS, not registers -- among the MFMAs instead of
            // leaving the MFMA pipe idle while they are issued.  After the
            // last step the loads are masked dummies (the issue lambda maps
            // steps past the end to nothing) and the reads are unused; drain()
            // waits for them.
            wait_vmcnt<S::kDmaPerStep * (S::STAGES - 2)>();
            block_barrier();
            read_frags<S, 0>(stage_addr(t + 1), off, f[(KS + 1) & 1]);
            hook(KS);
            mma<S>(f[KS & 1], acc);
            issue(t + S::STAGES, stage(t));
            interleave_mfma_and_loads();
        }
    }

    // Scheduling pattern for the last substep: one MFMA, then its share of
    // the step's direct-to-LDS loads, and so on (sched_group_barrier masks:
    // 0x008 MFMA, 0x020 VMEM read).
    __device__ __forceinline__ static void interleave_mfma_and_loads() {
        constexpr int kMfma = S::TM * S::TN;
        constexpr int kPer = (S::kDmaPerStep + kMfma - 1) / kMfma;
#pragma unroll
        for (int i = 0; i < kMfma; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, kPer, 0);
        }
    }

    template <class Issue, class Hook>
    __device__ __forceinline__ void step(const Issue &issue, int t, int total,
                                         f32x16 (&acc)[S::TM][S::TN], const Hook &hook) {
        static_assert(S::kKSub % 2 == 0, "fragment double buffer alternates per substep");
        substeps<0>(issue, t, total, acc, hook);
    }

    template <class Issue>
    __device__ __forceinline__ void run(const Issue &issue, int t_begin, int t_end, int total,
                                        f32x16 (&acc)[S::TM][S::TN]) {
        for (int t = t_begin; t < t_end; ++t) step(issue, t, total, acc, [](int) {});
    }

    __device__ __forceinline__ void drain() {
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        block_barrier();
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
