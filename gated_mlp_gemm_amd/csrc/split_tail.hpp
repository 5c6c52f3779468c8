// Work schedule for the single-accumulator GEMM kernels: whole tiles for the
// full rounds; the tiles of a partly idle last round whole, quartered (run as
// quarter-size tiles by the same kernel, see gemm_tiles_kernel) or split along
// K as described here, whichever the launcher's cost model prefers.
//
// One tile per workgroup leaves CUs idle in the last round when the tile count
// T is not a multiple of the CU count G: the M=2048, 2N=17920 output has 560
// tiles of 256x256 for 256 CUs, 3 rounds for 2.19 rounds of work.  Here the
// first R*G tiles (R = T / G full rounds) run whole, one per workgroup, and
// each of the L = T mod G remaining tiles is cut into s = min(G / L, nk)
// pieces of about nk / s K steps, one piece per workgroup: the tail round
// takes nk / s steps instead of nk (for 560 tiles: 2 + 1/5 rounds).  Each
// piece is one (tile, K range) work item of the persistent GEMM kernel; a
// workgroup takes its share of the pieces after its whole tiles, with one
// accumulator set live at a time.
//
// A piece stores its fp32 partial accumulator in its own workspace slot and
// ends.  A second, short kernel on the same stream then sums the s slots of
// each split tile in piece order (so results are bitwise reproducible) and
// runs the epilogue; it gives every 32x32 accumulator block of every split
// tile its own wave, so the reduction is spread over the whole chip rather
// than left to one workgroup per tile.  The stream order is the only
// synchronisation: no counters, atomics or fences.
//
// Workspace (caller-owned device memory, no initialisation needed): G slots of
// BM*BN floats, sized for the largest tile shape.
//
// Reduced in the kernel (fixup): when a whole output's tiles are split (M <= 128
// and few tiles: the reduction launch would cost as much as the GEMM), every
// piece stores its partial with device-scope stores (cache policy sc1: written
// through to the level where every XCD sees it), waits for them to complete,
// and one thread of its workgroup adds 1 to the tile's arrival counter with a
// device-scope atomic.  The piece that sees s - 1 arrivals before its own is
// the last: it resets the counter to 0, reads the other pieces' partials with
// device-scope loads and sums all s in piece order (its own from registers, the
// same additions as the reduction kernel's), then runs the epilogue.  No
// workgroup ever waits for another.  The counters are library-owned device
// memory that starts at zero and that every completed call leaves at zero.
#pragma once

#include "gemm_core.hpp"

namespace swiglu {

struct Schedule {
    int tiles_m, tiles_n;   // tile grid
    int nk;                 // K steps per tile
    int dp;                 // tiles [0, dp) run whole: workgroup b < dp runs one of them
    int pieces;             // K pieces per split tile (0: no split tiles)
    int split_tiles;        // tiles [dp, dp + split_tiles) are split (or quartered)
    int group_m;            // tile order: groups of group_m tile rows (tile_coords)
    int quartered;          // 1: the tail tiles run as four quarter-size tiles instead
    int grid;               // workgroups launched (each loops over its share of the work)
    float *partials;        // one BM*BN slot per piece: slot j = piece j % pieces of split tile j / pieces
    unsigned *counters;     // fixup: one arrival counter per split tile (zero between calls)
};

// Cache policy of the fixup's partial stores and loads: device scope (sc1).
constexpr int kDeviceScope = 16;

// A partial tile is stored thread-major: float4 number i of GEMM thread x at
// float4 index i * threads + x, so every access is a coalesced 16-byte one.
// Float4 number i of a thread holds register quad i%4 of its accumulator
// block i/4 (block = tm * TN + tn).
template <class S>
__device__ __forceinline__ void store_partial(float *slot,
                                              const typename S::Acc (&acc)[S::TM][S::TN],
                                              int tid) {
    f32x4 *dst = reinterpret_cast<f32x4 *>(slot);
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = (tm * S::TN + tn) * 4 + j;
                dst[i * S::kThreads + tid] = acc[tm][tn].quad(j);
            }
}

// store_partial's layout with device-scope stores (the fixup).
template <class S>
__device__ __forceinline__ void store_partial_coherent(float *slot,
                                                       const typename S::Acc (&acc)[S::TM][S::TN],
                                                       int tid) {
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(slot, static_cast<uint32_t>(S::BM * S::BN * sizeof(float)));
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = (tm * S::TN + tn) * 4 + j;
                __builtin_amdgcn_raw_buffer_store_b128(
                    acc[tm][tn].quad(j), r, (i * S::kThreads + tid) * 16, 0, kDeviceScope);
            }
}

// At most this many pieces per tile are reduced in the kernel (the last
// piece holds all the others' loads in flight at once).
constexpr int kMaxFixupPieces = 4;

// The fixup's sum for accumulator block (tm, tn) of GEMM thread `tid` of a
// split tile whose pieces' slots start at `slots`: pieces in order, piece
// `own` from `acc` (read out of the accumulators), the others by device-scope
// loads, all issued before the first addition.
template <class S>
__device__ __forceinline__ typename S::Acc sum_pieces_fixup(
    const float *slots, int pieces, int own, const typename S::Acc (&acc)[S::TM][S::TN], int tm,
    int tn, int tid) {
    const int blk = tm * S::TN + tn;
    f32x4 v[kMaxFixupPieces][4];
#pragma unroll
    for (int p = 0; p < kMaxFixupPieces; ++p) {
        if (p < pieces && p != own) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(
                slots + static_cast<int64_t>(p) * S::BM * S::BN,
                static_cast<uint32_t>(S::BM * S::BN * sizeof(float)));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[p][j] = __builtin_amdgcn_raw_buffer_load_b128(
                    r, ((blk * 4 + j) * S::kThreads + tid) * 16, 0, kDeviceScope);
        }
    }
    f32x4 mine[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 q = acc[tm][tn].quad(j);
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[j][e] = read_acc(q[e]);
    }
    f32x4 sum[4];
#pragma unroll
    for (int p = 0; p < kMaxFixupPieces; ++p) {
        if (p < pieces) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 x = p == own ? mine[j] : v[p][j];
                sum[j] = p == 0 ? x : sum[j] + x;
            }
        }
    }
    typename S::Acc a;
#pragma unroll
    for (int j = 0; j < 4; ++j) a.set_quad(j, sum[j]);
    return a;
}

// Accumulator block `blk` of GEMM thread x of split tile i: the sum, in
// piece order, of the pieces' partials.  The loads of up to four pieces are
// issued together before any is added (a plain loop would wait out one memory
// round trip per piece); the additions still run strictly in piece order, so
// the result does not depend on the grouping.
template <class S>
__device__ __forceinline__ typename S::Acc sum_pieces(const Schedule &sch, int i, int blk,
                                                     int x) {
    constexpr int64_t kSlot4 = static_cast<int64_t>(S::BM) * S::BN / 4;   // float4 per slot
    constexpr int kGroup = 4;
    const f32x4 *first = reinterpret_cast<const f32x4 *>(sch.partials) +
                         static_cast<int64_t>(i) * sch.pieces * kSlot4;
    const int64_t idx0 = static_cast<int64_t>(blk * 4) * S::kThreads + x;
    f32x4 sum[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sum[j] = first[idx0 + j * S::kThreads];
    for (int p = 1; p < sch.pieces; p += kGroup) {
        // every load is issued (past the last piece it re-reads the last one,
        // a valid address); only the additions are conditional
        f32x4 v[kGroup][4];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int64_t q = min(p + g, sch.pieces - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[g][j] = first[q * kSlot4 + idx0 + j * S::kThreads];
        }
#pragma unroll
        for (int g = 0; g < kGroup; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (p + g < sch.pieces) sum[j] += v[g][j];
    }
    typename S::Acc a;
#pragma unroll
    for (int j = 0; j < 4; ++j) a.set_quad(j, sum[j]);
    return a;
}

}  // namespace swiglu
