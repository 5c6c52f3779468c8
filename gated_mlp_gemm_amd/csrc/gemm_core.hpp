// The bf16 MFMA mainloop shared by every GEMM-shaped kernel of the library:
// the interleaved fused kernel, the sequential fused kernel and the unfused
// ablation's plain-store GEMM all run this code, so that their timings differ
// only by what the method changes (where Gate and Up live).
//
// One workgroup computes a BM x BN tile of D = A . B, where
//   A is row-major [rows][K]   (K contiguous; the activations),
//   B is row-major [K][cols]   (cols contiguous; W1, W2 or W_fused),
// in K steps of BK.
//
// Pipeline.  K steps stream through a ring of STAGES LDS buffers filled by
// direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds: no VGPR staging,
// no LDS write instructions), STAGES-1 steps ahead of the MFMAs.  The
// compiler does not track those LDS writes, so completion is awaited by hand:
// before step t+1 is read, each wave waits until at most (STAGES-2) later
// steps' loads are outstanding (s_waitcnt vmcnt), then the workgroup meets at
// one barrier.  That barrier also proves that every wave has finished reading
// step t's buffer, which is refilled with step t+STAGES right after it.  The
// barrier sits before the MFMAs of step t's last k-substep, so those MFMAs
// overlap the first fragment reads of step t+1.  Every step issues exactly one
// group of loads (groups past the end of K read nothing), which keeps the
// vmcnt arithmetic uniform.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that the fragment reads of a
// wave spread over all banks):
//   A tile: [BM][BK]; physical chunk = chunk ^ swz_a(row);
//           fragment read: one ds_read_b128 per lane (8 consecutive k).
//   B tile: [BK][BN] exactly as in memory (n contiguous);
//           physical chunk = chunk ^ swz_b(k);
//           fragment read: two ds_read_b64_tr_b16 per lane, which transpose
//           4 k-rows x 16 columns across each 16-lane group so that every lane
//           receives 8 consecutive k of one column (the MFMA B layout).
// A direct-to-LDS load writes 64 consecutive 16-byte chunks per wave, so the
// swizzle is applied on the global side: the lane that lands on physical chunk
// p fetches the logical chunk that belongs there.
//
// Edges.  Rows past the end of A and k past the end of B fall outside the
// buffer ranges and load as zeros; the K tail of A is masked explicitly.
// Columns of B past `cols` may load neighbouring data of the same matrix; they
// only feed accumulator columns that are never stored.
#pragma once

#include "device.hpp"

namespace swiglu {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int STAGES = STAGES_;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int TM = kWaveM / 32;          // 32x32 MFMA blocks per wave (M)
    static constexpr int TN = kWaveN / 32;          // 32x32 MFMA blocks per wave (N)
    static constexpr int kKSub = BK / 16;           // MFMA k-substeps per K step
    static constexpr int kAChunksPerRow = BK / 8;
    static constexpr int kBChunksPerRow = BN / 8;
    static constexpr int kABytes = BM * BK * 2;
    static constexpr int kBBytes = BK * BN * 2;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kLdsBytes = kStageBytes * STAGES;
    // direct-to-LDS loads per wave per K step (each moves 64 x 16 B = 1 KiB)
    static constexpr int kDmaA = kABytes / (kThreads * 16);
    static constexpr int kDmaB = kBBytes / (kThreads * 16);
    static constexpr int kDmaPerStep = kDmaA + kDmaB;

    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
    static_assert(kABytes % (kThreads * 16) == 0 && kDmaA >= 1, "A tile must split evenly");
    static_assert(kBBytes % (kThreads * 16) == 0 && kDmaB >= 1, "B tile must split evenly");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup is 160 KiB");
    static_assert(STAGES >= 2 && STAGES <= 8, "ring depth");
    static_assert(kDmaPerStep * (STAGES - 1) < 64, "vmcnt is a 6-bit counter");
    static_assert(BN >= 64, "B swizzle needs at least 8 chunks per row");
};

// Swizzles (see the layout note above).
template <class S>
__device__ __forceinline__ int swz_a(int row) {
    if constexpr (S::kAChunksPerRow == 4) return ((row >> 1) ^ (row >> 3)) & 3;
    else return (row >> 1) & 7;
}
template <class S>
__device__ __forceinline__ int swz_b(int k) {
    return (4 * (k & 3)) & (S::kBChunksPerRow - 1);
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

// Global -> LDS loader of one tile's K steps.  The B operand may change
// between K-step ranges (the sequential variant runs W1 steps then W2 steps).
template <class S>
struct TileLoader {
    __amdgpu_buffer_rsrc_t rsrc_a;
    uint32_t a_voff[S::kDmaA];   // byte offset of this lane's A chunk at k0 = 0
    int a_kcol[S::kDmaA];        // first k of that chunk
    uint32_t b_voff[S::kDmaB];   // byte offset of this lane's B chunk within a K step
    int K;
    int ldb;

    __device__ __forceinline__ void init(const uint16_t *A_tile, int lda, int rows_valid, int K_,
                                         int ldb_) {
        K = K_;
        ldb = ldb_;
        rsrc_a = make_rsrc(A_tile, static_cast<uint32_t>(rows_valid) * lda * 2u);
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int j = 0; j < S::kDmaA; ++j) {
            const int p = (j * S::kWaves + wave) * 64 + lane;   // physical chunk
            const int row = p / S::kAChunksPerRow;
            const int c = (p % S::kAChunksPerRow) ^ swz_a<S>(row);
            a_voff[j] = static_cast<uint32_t>(row) * lda * 2u + c * 16u;
            a_kcol[j] = c * 8;
        }
#pragma unroll
        for (int j = 0; j < S::kDmaB; ++j) {
            const int p = (j * S::kWaves + wave) * 64 + lane;
            const int k = p / S::kBChunksPerRow;
            const int c = (p % S::kBChunksPerRow) ^ swz_b<S>(k);
            b_voff[j] = static_cast<uint32_t>(k) * ldb_ * 2u + c * 16u;
        }
    }

    // Load K step `kstep` (of a K-long contraction against B_tile = B + n0)
    // into `stage`.  kstep >= ceil(K/BK) loads nothing (keeps vmcnt uniform).
    __device__ __forceinline__ void issue(int kstep, const uint16_t *B_tile, int n0,
                                          SWIGLU_LDS char *stage) const {
        const int wave = threadIdx.x >> 6;
        const int k0 = kstep * S::BK;
        const bool live = k0 < K;
        SWIGLU_LDS char *la = stage;
        SWIGLU_LDS char *lb = stage + S::kABytes;
        const uint32_t soff = live ? static_cast<uint32_t>(k0) * 2u : 0u;
        if (live && k0 + S::BK <= K) {
#pragma unroll
            for (int j = 0; j < S::kDmaA; ++j)
                dma16(rsrc_a, la + (j * S::kWaves + wave) * 1024, a_voff[j], soff);
        } else {
            // K tail (or a step past the end): mask the chunks at k >= K
#pragma unroll
            for (int j = 0; j < S::kDmaA; ++j) {
                const uint32_t v = (live && k0 + a_kcol[j] < K) ? a_voff[j] : kOutOfRange;
                dma16(rsrc_a, la + (j * S::kWaves + wave) * 1024, v, soff);
            }
        }
        // B: rebase on row k0 so that offsets stay small; the range ends at the
        // last element of B, so rows k >= K load as zeros.
        int64_t remaining = live ? (static_cast<int64_t>(K - k0) * ldb - n0) * 2 : 0;
        if (remaining > 0x7FFFFFF0LL) remaining = 0x7FFFFFF0LL;
        const uint16_t *b_base = B_tile + (live ? static_cast<int64_t>(k0) * ldb : 0);
        const __amdgpu_buffer_rsrc_t rsrc_b =
            make_rsrc(b_base, static_cast<uint32_t>(remaining));
#pragma unroll
        for (int j = 0; j < S::kDmaB; ++j)
            dma16(rsrc_b, lb + (j * S::kWaves + wave) * 1024, b_voff[j], 0u);
    }
};

// Fragment registers of one k-substep: raw 16-byte MFMA operands.
template <class S>
struct Frags {
    u32x4 a[S::TM];
    u32x4 b[S::TN];
};

// LDS reads issued as inline assembly.  The compiler neither tracks their
// completion nor sees them as LDS accesses; the pipeline waits for them with
// wait_frags() (below).  Keeping every fragment read out of the compiler's
// view is deliberate: its waitcnt pass treats a transposing LDS read as
// possibly aliasing the in-flight direct-to-LDS loads and would otherwise
// drain every outstanding load (vmcnt(0)) before each one.
template <int OFF>
__device__ __forceinline__ u32x4 asm_read_b128(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 asm_read_tr_b64(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// Per-lane LDS byte offsets of the fragment reads, relative to a stage base.
// A: one per k-substep (the swizzle mixes the substep into the address);
//    the 32-row blocks tm are +tm*32 rows (the swizzle has period 32 in rows).
// B: one per 32-column block tn; substep ks is +16*ks rows and the second
//    transposing read +4 rows (the swizzle has period 4 in k).
template <class S>
struct FragOffsets {
    uint32_t a[S::kKSub];
    uint32_t b[S::TN];

    __device__ __forceinline__ void init(int wm, int wn, int lane) {
        const int h = lane >> 5;
        const int s = lane & 15;
        const int q1 = (lane >> 4) & 1;
        const int row = wm * S::kWaveM + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < S::kKSub; ++ks) {
            const int pc = (ks * 2 + h) ^ swz_a<S>(row);
            a[ks] = static_cast<uint32_t>(row * (S::BK * 2) + pc * 16);
        }
        const int krow = 8 * h + (s >> 2);
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn) {
            const int ncol = wn * S::kWaveN + tn * 32 + 16 * q1 + 4 * (s & 3);
            const int pc = (ncol >> 3) ^ swz_b<S>(krow);
            b[tn] = static_cast<uint32_t>(S::kABytes + krow * (S::BN * 2) + pc * 16 +
                                          ((ncol >> 2) & 1) * 8);
        }
    }
};

// Issue the fragment reads of k-substep KS from the stage at LDS byte address
// `stage` (A: TM x ds_read_b128; B: TN x 2 ds_read_b64_tr_b16).
template <class S, int KS>
__device__ __forceinline__ void read_frags(uint32_t stage, const FragOffsets<S> &o,
                                           Frags<S> &f) {
    const uint32_t abase = stage + o.a[KS];
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm) {
        // tm * 32 rows of BK bf16; the immediate must be a constant expression
        switch (tm) {
            case 0: f.a[0] = asm_read_b128<0>(abase); break;
            case 1: f.a[1] = asm_read_b128<1 * 32 * S::BK * 2>(abase); break;
            case 2: f.a[2] = asm_read_b128<2 * 32 * S::BK * 2>(abase); break;
            case 3: f.a[3] = asm_read_b128<3 * 32 * S::BK * 2>(abase); break;
        }
    }
    constexpr int kRow = S::BN * 2;
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn) {
        const uint32_t p = stage + o.b[tn];
        const u32x2 lo = asm_read_tr_b64<KS * 16 * kRow>(p);
        const u32x2 hi = asm_read_tr_b64<KS * 16 * kRow + 4 * kRow>(p);
        f.b[tn] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
}

// Wait until every fragment read issued so far has landed, and make the
// fragment registers of `f` depend on that wait (so no MFMA reading them can
// be scheduled before it).
template <class S>
__device__ __forceinline__ void wait_frags(Frags<S> &f) {
    static_assert(S::TM <= 4 && S::TN <= 4, "wait_frags ties at most 4+4 fragments");
    if constexpr (S::TM == 4 && S::TN == 4)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),
                       "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
    else if constexpr (S::TM == 4 && S::TN == 2)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),
                       "+v"(f.b[1]));
    else if constexpr (S::TM == 2 && S::TN == 4)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]),
                       "+v"(f.b[3]));
    else if constexpr (S::TM == 2 && S::TN == 2)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.b[0]), "+v"(f.b[1]));
    else if constexpr (S::TM == 2 && S::TN == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.b[0]));
    else if constexpr (S::TM == 1 && S::TN == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.a[0]), "+v"(f.b[0]));
    else
        static_assert(S::TM == 0, "unsupported fragment count");
}

template <class S>
__device__ __forceinline__ void mma(const Frags<S> &f, f32x16 (&acc)[S::TM][S::TN]) {
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
            acc[tm][tn] = mfma_32x32x16(__builtin_bit_cast(bf16x8, f.a[tm]),
                                        __builtin_bit_cast(bf16x8, f.b[tn]), acc[tm][tn]);
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

// Pipeline driver.  A "step sequence" is a run of K steps numbered
// 0..total-1; `issue(t, stage)` loads sequence step t into an LDS stage (the
// sequential variant chains two contractions into one sequence).
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

    // Fill the ring with steps 0..STAGES-1, wait for step 0, read its first fragments.
    template <class Issue>
    __device__ __forceinline__ void prologue(const Issue &issue) {
#pragma unroll
        for (int t = 0; t < S::STAGES; ++t) issue(t, stage(t));
        wait_vmcnt<S::kDmaPerStep * (S::STAGES - 1)>();
        block_barrier();
        read_frags<S, 0>(stage_addr(0), off, f[0]);
    }

    // Substeps KS..last of sequence step t (helper of step()).
    template <int KS, class Issue, class Hook>
    __device__ __forceinline__ void substeps(const Issue &issue, int t, int total,
                                             f32x16 (&acc)[S::TM][S::TN], const Hook &hook) {
        constexpr int last = S::kKSub - 1;
        // keep the previous substep's MFMAs above this wait
        __builtin_amdgcn_sched_barrier(0);
        wait_frags<S>(f[KS & 1]);
        if constexpr (KS < last) {
            read_frags<S, KS + 1>(stage_addr(t), off, f[(KS + 1) & 1]);
            hook(KS);
            mma<S>(f[KS & 1], acc);
            substeps<KS + 1>(issue, t, total, acc, hook);
        } else {
            if (t + 1 < total) {
                wait_vmcnt<S::kDmaPerStep * (S::STAGES - 2)>();
                block_barrier();
                issue(t + S::STAGES, stage(t));
                read_frags<S, 0>(stage_addr(t + 1), off, f[(KS + 1) & 1]);
            }
            hook(KS);
            mma<S>(f[KS & 1], acc);
        }
    }

    // One K step (sequence step t) into acc.  `hook(ks)` runs once per
    // k-substep, next to that substep's MFMAs (the sequential variant uses it
    // to activate the Gate accumulator while the Up MFMAs run); `total` is the
    // length of the whole sequence (no barrier/refill after its last step).
    template <class Issue, class Hook>
    __device__ __forceinline__ void step(const Issue &issue, int t, int total,
                                         f32x16 (&acc)[S::TM][S::TN], const Hook &hook) {
        static_assert(S::kKSub % 2 == 0, "fragment double buffer alternates per substep");
        substeps<0>(issue, t, total, acc, hook);
    }

    // Sequence steps [t_begin, t_end) into acc.
    template <class Issue>
    __device__ __forceinline__ void run(const Issue &issue, int t_begin, int t_end, int total,
                                        f32x16 (&acc)[S::TM][S::TN]) {
        for (int t = t_begin; t < t_end; ++t) step(issue, t, total, acc, [](int) {});
    }

    // Drain: no load may still be writing LDS when the caller reuses it.
    __device__ __forceinline__ void drain() {
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        block_barrier();
    }
};

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup id mod 8); re-number them so that each XCD receives a
// contiguous run of tile ids, then walk tiles in groups of `group_m` tile rows
// so that tiles resident together share A rows and B columns in that XCD's L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int group_m, int &tm,
                                            int &tn) {
    const int bid = blockIdx.x;
    const int nb = tiles_m * tiles_n;
    const int per = nb / 8;
    const int t = (bid < per * 8) ? (bid % 8) * per + bid / 8 : bid;
    const int width = group_m * tiles_n;
    const int group = t / width;
    const int first_m = group * group_m;
    const int rows_in_group = min(tiles_m - first_m, group_m);
    const int in_group = t % width;
    tm = first_m + in_group % rows_in_group;
    tn = in_group / rows_in_group;
}

}  // namespace swiglu
