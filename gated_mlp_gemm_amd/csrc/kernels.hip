// HIP kernels of the fused SwiGLU GEMM library (gfx950 only).
//
// Citations are to the pages on "Tile-Level Activation Overlap for Efficient
// LLM Inference" (arXiv 2607.02521): [paper s1] = the paper's own text,
// section 1 Introduction; [abstract] = its abstract; [gist: X] = the
// gist.science technical summary, section X.
#include "launch.hpp"

#include "tile_kernels.hpp"

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

static inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

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
    // Tile rows walked together by the tile order (tile_coords): 8, or 4 when
    // the output has at most 8 tile rows and a tile at most 32 K steps
    // (measured at M=2048 on the five K x N workload shapes: 4 rows 2-3 %
    // faster at K <= 1536, 1.3-1.7 % slower at K >= 5120; 8 rows best on the
    // large-M workloads).
    sch.group_m = sch.tiles_m <= 8 && sch.nk <= 32 ? 4 : 8;
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
        if constexpr (kQuarterable<S>)
            return TilesLaunch<S, Epi, kTailQuarter>::run(sch.grid, A, B, M, K, epi, sch, stream);
        return hipErrorInvalidConfiguration;   // make_schedule quarters no other shape
    }
    if (sch.pieces == 0)
        return TilesLaunch<S, Epi, kTailNone>::run(sch.grid, A, B, M, K, epi, sch, stream);
    const hipError_t e =
        TilesLaunch<S, Epi, kTailSplit>::run(sch.grid, A, B, M, K, epi, sch, stream);
    if (e != hipSuccess) return e;
    // S::kWaves * (epilogue units per wave) single-wave workgroups per split tile
    constexpr int kWavesPerTile = S::kWaves * S::TM * S::TN / Epi::template unit_blocks<S>();
    const int rgrid = sch.split_tiles * kWavesPerTile;
    return ReduceLaunch<S, Epi>::run(rgrid, epi, sch, stream);
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
    return TilesLaunch<S, Epi, kTailReduceInKernel>::run(sch.grid, A, B, M, K, epi, sch, stream);
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
        return SequentialLaunch<ShapeSmall>::run(a, w, Y, M, N, K, lda, ldy, 1.0f, stream);
    using P = ShapeSeqP;
    const SeqSchedule s = make_seq_schedule(M, N, K, ws);
    if (s.grid <= 0) return hipSuccess;
    return PersistentSequentialLaunch<P>::run(s.grid, a, w, Y, M, N, K, lda, ldy, s.tiles_m,
                                              s.tiles_n, s.dp, s.quarter_tiles, stream);
}

// Variant S on FP8 operands: the same kernel with K steps of 128 FP8 values.
hipError_t launch_fused_sequential_fp8(const uint8_t *A8, const uint8_t *Wf8, uint16_t *Y, int M,
                                       int N, int K, float scale, hipStream_t stream) {
    const void *a = A8, *w = Wf8;
    if (M <= 128) return SequentialLaunch<ShapeSmall8>::run(a, w, Y, M, N, K, K, N, scale, stream);
    return SequentialLaunch<ShapeSeq8>::run(a, w, Y, M, N, K, K, N, scale, stream);
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
