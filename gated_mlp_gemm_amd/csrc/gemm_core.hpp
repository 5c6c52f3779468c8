// The bf16 MFMA mainloop shared by every GEMM-shaped kernel of the library:
// the interleaved fused kernel, the sequential fused kernel and the unfused
// ablation's plain-store GEMM all run exactly this code, so that their
// timings differ only by what the method changes (where Gate and Up live).
//
// One workgroup computes a BM x BN tile of D = A . B, where
//   A is row-major [rows][K]   (K contiguous; the activations),
//   B is row-major [K][cols]   (cols contiguous; W1, W2 or W_fused),
// in K steps of BK.  Each step stages an A tile and a B tile in LDS
// (STAGES-deep ring, loads for step k+1 in flight while step k computes),
// then every wave runs its (BM/WM) x (BN/WN) block of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators held in registers.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that the fragment reads of a
// wave hit distinct banks):
//   A tile: [BM][BK], physical chunk = chunk ^ ((row >> 1) & (BK/8 - 1));
//           fragment read = one ds_read_b128 per lane (8 consecutive k).
//   B tile: [BK][BN] exactly as stored in memory (n contiguous),
//           physical chunk = chunk ^ ((4 * (k & 3)) & (BN/8 - 1));
//           fragment read = two ds_read_b64_tr_b16 per lane, which transpose
//           4 k-rows x 16 columns across each 16-lane group so that every lane
//           receives 8 consecutive k of one column, the MFMA B layout.
// Global loads are buffer loads: rows past the end of A and k past the end of
// B come back as zeros from the hardware range check; the K tail of A is
// masked explicitly.  Columns of B past `cols` may read neighbouring data of
// the same matrix; they only feed accumulator columns that are never stored.
#pragma once

#include "device.hpp"

namespace swiglu {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_ = 2>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int STAGES = STAGES_;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int TM = kWaveM / 32;          // 32x32 MFMA blocks per wave (M)
    static constexpr int TN = kWaveN / 32;          // 32x32 MFMA blocks per wave (N)
    static constexpr int kKSub = BK / 16;           // MFMA k-steps per K tile
    static constexpr int kAChunksPerRow = BK / 8;
    static constexpr int kBChunksPerRow = BN / 8;
    static constexpr int kABytes = BM * BK * 2;
    static constexpr int kBBytes = BK * BN * 2;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int kLdsBytes = kStageBytes * STAGES;
    static constexpr int kAChunks = BM * BK / 8 / kThreads;   // 16-B loads per thread
    static constexpr int kBChunks = BK * BN / 8 / kThreads;

    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 16 == 0 && BK >= 16, "BK must be a multiple of 16");
    static_assert(BM * BK / 8 % kThreads == 0 && kAChunks >= 1, "A tile must split evenly");
    static_assert(BK * BN / 8 % kThreads == 0 && kBChunks >= 1, "B tile must split evenly");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup is 160 KiB");
    static_assert(STAGES >= 2, "need at least double buffering");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // dword3 0x00020000: raw (untyped) 32-bit data format, the CDNA setting
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                 static_cast<int>(soff), 0);
}

// An offset no buffer range admits: loads through it return zero.
constexpr uint32_t kOutOfRange = 0x80000000u;

template <class S>
struct Mainloop {
    // --- per-thread state --------------------------------------------------
    __amdgpu_buffer_rsrc_t rsrc_a;
    uint32_t a_voff[S::kAChunks];   // byte offset of each A chunk at k0 = 0
    int a_kcol[S::kAChunks];        // first k of each A chunk at k0 = 0
    uint32_t b_voff[S::kBChunks];   // byte offset of each B chunk within a K step
    u32x4 ra[S::kAChunks];
    u32x4 rb[S::kBChunks];

    const uint16_t *a_tile;   // A + m0 * lda
    int lda;
    int K;

    __device__ __forceinline__ void init_a(const uint16_t *A_tile, int lda_, int rows_valid,
                                           int K_) {
        a_tile = A_tile;
        lda = lda_;
        K = K_;
        rsrc_a = make_rsrc(A_tile, static_cast<uint32_t>(rows_valid) * lda_ * 2u);
        const int tid = threadIdx.x;
#pragma unroll
        for (int r = 0; r < S::kAChunks; ++r) {
            const int cid = r * S::kThreads + tid;
            const int row = cid / S::kAChunksPerRow;
            const int kc = cid % S::kAChunksPerRow;
            a_voff[r] = static_cast<uint32_t>(row) * lda_ * 2u + kc * 16u;
            a_kcol[r] = kc * 8;
        }
    }

    __device__ __forceinline__ void init_b_offsets(int ldb) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int r = 0; r < S::kBChunks; ++r) {
            const int cid = r * S::kThreads + tid;
            const int krow = cid / S::kBChunksPerRow;
            const int cc = cid % S::kBChunksPerRow;
            b_voff[r] = static_cast<uint32_t>(krow) * ldb * 2u + cc * 16u;
        }
    }

    // Issue the global loads of K step `kt` (A tile and B tile) into registers.
    // B_tile = B + n0 (first column of the tile); ldb = row pitch of B.
    __device__ __forceinline__ void load(int kt, const uint16_t *B_tile, int ldb, int n0,
                                         int cols_total) {
        const int k0 = kt * S::BK;
        if (k0 + S::BK <= K) {
#pragma unroll
            for (int r = 0; r < S::kAChunks; ++r)
                ra[r] = buffer_load16(rsrc_a, a_voff[r], static_cast<uint32_t>(k0) * 2u);
        } else {
#pragma unroll
            for (int r = 0; r < S::kAChunks; ++r) {
                const uint32_t v = (k0 + a_kcol[r] < K) ? a_voff[r] : kOutOfRange;
                ra[r] = buffer_load16(rsrc_a, v, static_cast<uint32_t>(k0) * 2u);
            }
        }
        // B: rebase on row k0 so that offsets stay small; the range ends at the
        // last element of B, which zero-fills k >= K.
        const uint16_t *b_base = B_tile + static_cast<int64_t>(k0) * ldb;
        const int64_t remaining = (static_cast<int64_t>(K - k0) * ldb - n0) * 2;
        const uint32_t b_bytes =
            static_cast<uint32_t>(remaining < 0x7FFFFFF0LL ? remaining : 0x7FFFFFF0LL);
        const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(b_base, b_bytes);
        (void)cols_total;
#pragma unroll
        for (int r = 0; r < S::kBChunks; ++r) rb[r] = buffer_load16(rsrc_b, b_voff[r], 0u);
    }

    // Write the staged registers into one LDS stage (swizzled).
    __device__ __forceinline__ void store(SWIGLU_LDS char *stage) const {
        const int tid = threadIdx.x;
        SWIGLU_LDS char *la = stage;
        SWIGLU_LDS char *lb = stage + S::kABytes;
#pragma unroll
        for (int r = 0; r < S::kAChunks; ++r) {
            const int cid = r * S::kThreads + tid;
            const int row = cid / S::kAChunksPerRow;
            const int kc = cid % S::kAChunksPerRow;
            const int pc = kc ^ ((row >> 1) & (S::kAChunksPerRow - 1));
            lds_write16(la + row * (S::BK * 2) + pc * 16, ra[r]);
        }
#pragma unroll
        for (int r = 0; r < S::kBChunks; ++r) {
            const int cid = r * S::kThreads + tid;
            const int krow = cid / S::kBChunksPerRow;
            const int cc = cid % S::kBChunksPerRow;
            const int pc = cc ^ ((4 * (krow & 3)) & (S::kBChunksPerRow - 1));
            lds_write16(lb + krow * (S::BN * 2) + pc * 16, rb[r]);
        }
    }
};

// One K tile of MFMA work for the calling wave: acc += A_tile . B_tile over
// the wave's (kWaveM x kWaveN) block.
template <class S>
__device__ __forceinline__ void mma_stage(const SWIGLU_LDS char *stage,
                                          f32x16 (&acc)[S::TM][S::TN], int wm, int wn,
                                          int lane) {
    const SWIGLU_LDS char *la = stage;
    const SWIGLU_LDS char *lb = stage + S::kABytes;
    const int s = lane & 15;
    const int h = lane >> 5;
    const int q1 = (lane >> 4) & 1;
#pragma unroll
    for (int ks = 0; ks < S::kKSub; ++ks) {
        bf16x8 af[S::TM];
        bf16x8 bfr[S::TN];
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            const int row = wm * S::kWaveM + tm * 32 + (lane & 31);
            const int chunk = ks * 2 + h;
            const int pc = chunk ^ ((row >> 1) & (S::kAChunksPerRow - 1));
            af[tm] = __builtin_bit_cast(bf16x8, lds_read16(la + row * (S::BK * 2) + pc * 16));
        }
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn) {
            const int krow = ks * 16 + 8 * h + (s >> 2);
            const int ncol = wn * S::kWaveN + tn * 32 + 16 * q1 + 4 * (s & 3);
            const int chunk = ncol >> 3;
            const int half = (ncol >> 2) & 1;
            const int pc = chunk ^ ((4 * (krow & 3)) & (S::kBChunksPerRow - 1));
            const SWIGLU_LDS char *p = lb + krow * (S::BN * 2) + pc * 16 + half * 8;
            // rows krow and krow + 4 share the swizzle (4 * (k & 3) is periodic in 4)
            const u32x2 lo = lds_read_tr8(p);
            const u32x2 hi = lds_read_tr8(p + 4 * (S::BN * 2));
            const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
            bfr[tn] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < S::TN; ++tn)
                acc[tm][tn] = mfma_32x32x16(af[tm], bfr[tn], acc[tm][tn]);
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

// Full contraction over K for one tile, double-buffered through LDS:
// loads of step kt+1 are in flight while step kt's MFMAs run.
template <class S>
__device__ __forceinline__ void gemm_tile(SWIGLU_LDS char *lds, Mainloop<S> &ml,
                                          const uint16_t *B_tile, int ldb, int n0,
                                          int cols_total, int K,
                                          f32x16 (&acc)[S::TM][S::TN]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / S::WN;
    const int wn = wave % S::WN;
    const int nk = (K + S::BK - 1) / S::BK;
    ml.load(0, B_tile, ldb, n0, cols_total);
    ml.store(lds);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) ml.load(kt + 1, B_tile, ldb, n0, cols_total);
        mma_stage<S>(lds + (kt & 1) * S::kStageBytes, acc, wm, wn, lane);
        if (more) ml.store(lds + ((kt + 1) & 1) * S::kStageBytes);
        __syncthreads();
    }
}

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
