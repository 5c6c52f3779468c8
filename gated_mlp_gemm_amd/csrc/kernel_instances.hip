// The launches of the tiled GEMM kernels (declared in tile_kernels.hpp),
// explicitly instantiated one group per object.
//
// This file is compiled once per group of the list below, with
// -DSWIGLU_INSTANCE=<group>, into objects of their own that the build
// compiles in parallel: a tile-kernel instance whose K loop is unrolled over
// a whole ring period takes minutes to compile, and one object holding all of
// them would take the sum.  The groups come heaviest first, so that a build
// with fewer workers than groups starts the longest compiles first.  A group
// left out of the list leaves its run() undefined, which the link of the
// library reports.
#include "tile_kernels.hpp"

namespace swiglu {

template <class S, class Epi, int TAIL>
hipError_t TilesLaunch<S, Epi, TAIL>::run(int grid, const KMajor &A, const KMajor &B, int M,
                                          int K, const Epi &epi, const Schedule &sch,
                                          hipStream_t stream) {
    hipLaunchKernelGGL((gemm_tiles_kernel<S, Epi, TAIL>), dim3(grid), dim3(S::kThreads), 0,
                       stream, A, B, M, K, epi, sch);
    return hipGetLastError();
}

template <class S, class Epi>
hipError_t ReduceLaunch<S, Epi>::run(int grid, const Epi &epi, const Schedule &sch,
                                     hipStream_t stream) {
    hipLaunchKernelGGL((split_reduce_kernel<S, Epi>), dim3(grid), dim3(64), 0, stream, epi, sch);
    return hipGetLastError();
}

template <class S>
hipError_t SequentialLaunch<S>::run(const void *A, const void *Wf, uint16_t *Y, int M, int N,
                                    int K, int lda, int ldy, float scale, hipStream_t stream) {
    const int tiles_m = (M + S::BM - 1) / S::BM;
    const int tiles_n = (N + S::BN - 1) / S::BN;
    hipLaunchKernelGGL(fused_sequential_kernel<S>, dim3(tiles_m * tiles_n), dim3(S::kThreads), 0,
                       stream, A, Wf, Y, M, N, K, lda, ldy, scale, tiles_m, tiles_n);
    return hipGetLastError();
}

template <class S>
hipError_t PersistentSequentialLaunch<S>::run(int grid, const void *A, const void *Wf,
                                              uint16_t *Y, int M, int N, int K, int lda,
                                              int ldy, int tiles_m, int tiles_n, int dp,
                                              int quarter_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(fused_sequential_persistent_kernel<S>, dim3(grid), dim3(S::kThreads), 0,
                       stream, A, Wf, Y, M, N, K, lda, ldy, tiles_m, tiles_n, dp,
                       quarter_tiles);
    return hipGetLastError();
}

// The instance list: every (shape, epilogue, tail) the launchers in
// kernels.hip reach.
#if !defined(SWIGLU_INSTANCE)
#error "compile once per group: -DSWIGLU_INSTANCE=<group>"
#elif SWIGLU_INSTANCE == 0
template struct TilesLaunch<ShapeWide, PairMulEpilogue, kTailQuarter>;
#elif SWIGLU_INSTANCE == 1
template struct TilesLaunch<ShapeWide, StoreEpilogue, kTailQuarter>;
#elif SWIGLU_INSTANCE == 2
template struct TilesLaunch<ShapeWide, PairMulEpilogue, kTailSplit>;
#elif SWIGLU_INSTANCE == 3
template struct TilesLaunch<ShapeWide, PairMulEpilogue, kTailNone>;
#elif SWIGLU_INSTANCE == 4
template struct TilesLaunch<ShapeWide, StoreEpilogue, kTailSplit>;
#elif SWIGLU_INSTANCE == 5
template struct TilesLaunch<ShapeWide, StoreEpilogue, kTailNone>;
#elif SWIGLU_INSTANCE == 6
template struct PersistentSequentialLaunch<ShapeSeqP>;
#elif SWIGLU_INSTANCE == 7
template struct TilesLaunch<ShapeQuad, PairMulEpilogue, kTailNone>;
#elif SWIGLU_INSTANCE == 8
template struct TilesLaunch<ShapeQuad, PairMulEpilogue, kTailSplit>;
#elif SWIGLU_INSTANCE == 9
template struct TilesLaunch<ShapeQuad, StoreEpilogue, kTailNone>;
#elif SWIGLU_INSTANCE == 10
template struct TilesLaunch<ShapeQuad, StoreEpilogue, kTailSplit>;
#elif SWIGLU_INSTANCE == 11
template struct TilesLaunch<ShapeSplitK, PairMulEpilogue, kTailReduceInKernel>;
#elif SWIGLU_INSTANCE == 12
template struct TilesLaunch<ShapeWide8, PairMulEpilogueFp8, kTailQuarter>;
template struct TilesLaunch<ShapeWide8, PairMulEpilogueFp8, kTailNone>;
template struct TilesLaunch<ShapeWide8, PairMulEpilogueFp8, kTailSplit>;
#elif SWIGLU_INSTANCE == 13
template struct TilesLaunch<ShapeQuad8, PairMulEpilogueFp8, kTailNone>;
template struct TilesLaunch<ShapeQuad8, PairMulEpilogueFp8, kTailSplit>;
template struct TilesLaunch<ShapeSmall8, PairMulEpilogueFp8, kTailNone>;
template struct TilesLaunch<ShapeSmall8, PairMulEpilogueFp8, kTailSplit>;
#elif SWIGLU_INSTANCE == 14
template struct TilesLaunch<ShapeSmall, PairMulEpilogue, kTailNone>;
template struct TilesLaunch<ShapeSmall, PairMulEpilogue, kTailSplit>;
template struct TilesLaunch<ShapeSmall, StoreEpilogue, kTailNone>;
template struct TilesLaunch<ShapeSmall, StoreEpilogue, kTailSplit>;
#elif SWIGLU_INSTANCE == 15
template struct SequentialLaunch<ShapeSmall>;
template struct SequentialLaunch<ShapeSmall8>;
template struct SequentialLaunch<ShapeSeq8>;
template struct ReduceLaunch<ShapeWide, PairMulEpilogue>;
template struct ReduceLaunch<ShapeQuad, PairMulEpilogue>;
template struct ReduceLaunch<ShapeSmall, PairMulEpilogue>;
template struct ReduceLaunch<ShapeWide, StoreEpilogue>;
template struct ReduceLaunch<ShapeQuad, StoreEpilogue>;
template struct ReduceLaunch<ShapeSmall, StoreEpilogue>;
template struct ReduceLaunch<ShapeWide8, PairMulEpilogueFp8>;
template struct ReduceLaunch<ShapeQuad8, PairMulEpilogueFp8>;
template struct ReduceLaunch<ShapeSmall8, PairMulEpilogueFp8>;
#else
#error "SWIGLU_INSTANCE is past the end of the instance list"
#endif

}  // namespace swiglu
