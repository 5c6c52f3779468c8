// C ABI of the fused SwiGLU GEMM library: argument validation, the M-based
// dispatcher between the two fused variants, and kernel launches.
//
// Every argument is checked before the first HIP call, so an invalid call
// launches nothing (and can be exercised on a machine without a GPU).
#include "swiglu.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <atomic>
#include <mutex>

#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return SWIGLU_OK;
}

constexpr int64_t kMaxM = 2147483647;     // 2^31 - 1
constexpr int64_t kMaxK = int64_t(1) << 21;
constexpr int64_t kMaxN = int64_t(1) << 22;
// Built-in M threshold of the dispatcher: every M.  On MI355X variant I was
// faster than variant S at 44 of 45 measured (M, K, N) points -- M from 128 to
// 16384 on each of the five K x N shapes of the workloads, by 10-20 % at large
// M -- and within 1-8 % (run to run) at the other (M = 128, K = 1536, N =
// 8960), so AUTO runs I unless SWIGLU_M_SWITCH sets a smaller threshold.
constexpr int64_t kDefaultMSwitch = kMaxM;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

int check_gemm_shape(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0) return fail(SWIGLU_ERR_SHAPE, "negative size M=%lld N=%lld", (long long)M, (long long)N);
    if (K < 8) return fail(SWIGLU_ERR_SHAPE, "K=%lld must be >= 8", (long long)K);
    if (K % 8 != 0 || N % 8 != 0)
        return fail(SWIGLU_ERR_SHAPE, "K=%lld and N=%lld must be multiples of 8", (long long)K, (long long)N);
    if (M > kMaxM || K > kMaxK || N > kMaxN)
        return fail(SWIGLU_ERR_SHAPE, "size beyond limits (M<=2^31-1, K<=2^21, N<=2^22)");
    if (swiglu::max_tiles(M, 2 * N) > 2147483647)
        return fail(SWIGLU_ERR_SHAPE, "tile grid too large");
    return SWIGLU_OK;
}

// The down projection Out [M][D] = H [M][N] . W3 reduces over N: N is its
// K-like dimension (multiple of 8, at most 2^21) and D its column count.
int check_down_shape(int64_t M, int64_t N, int64_t D) {
    if (M < 0 || D < 0) return fail(SWIGLU_ERR_SHAPE, "negative size M=%lld D=%lld", (long long)M, (long long)D);
    if (N < 8) return fail(SWIGLU_ERR_SHAPE, "N=%lld must be >= 8", (long long)N);
    if (N % 8 != 0 || D % 8 != 0)
        return fail(SWIGLU_ERR_SHAPE, "N=%lld and D=%lld must be multiples of 8", (long long)N, (long long)D);
    if (M > kMaxM || N > kMaxK || D > kMaxN)
        return fail(SWIGLU_ERR_SHAPE, "size beyond limits (M<=2^31-1, N<=2^21, D<=2^22)");
    if (swiglu::max_tiles(M, D) > 2147483647) return fail(SWIGLU_ERR_SHAPE, "tile grid too large");
    return SWIGLU_OK;
}

// swiglu_describe_launch's codes for the down projection of the gated MLP
// and for the FP8 fused call.
constexpr int kDescribeDownProj = -2;
constexpr int kDescribeFp8 = -3;

// Per-device cache: state 1 = gfx950, -1 = other architecture, 0 = not yet
// queried; and the device's compute-unit count (sizes the split-tail schedule).
std::mutex g_dev_mutex;
int g_dev_state[256];
int g_dev_cus[256];


int check_device(int *cus = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SWIGLU_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 256) return fail(SWIGLU_ERR_UNSUPPORTED, "device ordinal %d", dev);
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(SWIGLU_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_dev_cus[dev] = prop.multiProcessorCount;
    }
    if (g_dev_state[dev] != 1)
        return fail(SWIGLU_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
    if (cus) *cus = g_dev_cus[dev];
    return SWIGLU_OK;
}

// SWIGLU_I_TILE=256 or 128 forces the tile of variant I and the ablation
// GEMMs above M = 128, and variant I's 128x64 (256) or 128x128 (128) tiles at
// M <= 128 (testing, measurement); anything else: the cost model / rule.
int tile_override() {
    const char *s = std::getenv("SWIGLU_I_TILE");
    if (s == nullptr) return 0;
    if (std::strcmp(s, "256") == 0) return 256;
    if (std::strcmp(s, "128") == 0) return 128;
    return 0;
}

// SWIGLU_TAIL=whole, split or quarter forces how the tiles of a partly idle
// last round run (split only takes effect with a workspace; quarter only for
// the 256x256 tile); fixup forces variant I at M <= 128 to split all its
// tiles along K and reduce them in the kernel (with a workspace; whole keeps
// it from doing so); unset or anything else: the cost model decides.
int tail_override() {
    const char *s = std::getenv("SWIGLU_TAIL");
    if (s == nullptr) return swiglu::kTailAuto;
    if (std::strcmp(s, "whole") == 0) return swiglu::kTailWhole;
    if (std::strcmp(s, "split") == 0) return swiglu::kTailPieces;
    if (std::strcmp(s, "quarter") == 0) return swiglu::kTailQuarters;
    if (std::strcmp(s, "fixup") == 0) return swiglu::kTailFixup;
    return swiglu::kTailAuto;
}

// Arrival counters of the split GEMM tiles that are reduced in the kernel
// (split_tail.hpp): library-owned device memory, zero when the library is
// loaded and left zero by every call that completes.  Each call takes the
// next of kCounterBlocks blocks of its device's array in turn, so up to
// kCounterBlocks such calls may run at once on one device (on different
// streams).  Host code uses the per-device address from hipGetSymbolAddress.
constexpr int kCounterBlocks = 64;
constexpr int kCountersPerBlock = 1024;
static __device__ __align__(256) unsigned split_counters[kCounterBlocks * kCountersPerBlock] = {};
unsigned *g_counters_ptr[256];   // per device, guarded by g_dev_mutex
unsigned g_counter_next[256];    // next block per device, guarded by g_dev_mutex

// The current device's next counter block, or nullptr (then no call reduces
// in the kernel).
unsigned *next_counter_block() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return nullptr;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_counters_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(split_counters)) != hipSuccess) return nullptr;
        g_counters_ptr[dev] = static_cast<unsigned *>(p);
    }
    const unsigned block = g_counter_next[dev]++ % kCounterBlocks;
    return g_counters_ptr[dev] + static_cast<size_t>(block) * kCountersPerBlock;
}

swiglu::GemmWorkspace make_ws(void *workspace, uint64_t bytes, int cus) {
    swiglu::GemmWorkspace ws{};
    ws.base = bytes > 0 ? workspace : nullptr;
    ws.bytes = workspace ? bytes : 0;
    ws.cus = cus;
    ws.tile = tile_override();
    ws.tail = tail_override();
    ws.counters = ws.base ? next_counter_block() : nullptr;
    ws.max_counters = ws.counters ? kCountersPerBlock : 0;
    return ws;
}

// Library-owned scratch of swiglu_fused_gemm_noalloc: the split-tail partials
// of one call (one fp32 256 x 256 slot per compute unit of a 256-CU device).
// A file-scope device array, so the library allocates nothing at call time;
// each device the library runs on holds its own copy until the process ends.
// Host code never uses the array's name as an address: the per-device device
// address comes from hipGetSymbolAddress (scratch_on_device).
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void *g_scratch_ptr[256];   // per device, guarded by g_dev_mutex

// Device address of this device's `scratch`, looked up once per device with
// that device current (the caller's current device).
int scratch_on_device(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SWIGLU_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 256) return fail(SWIGLU_ERR_UNSUPPORTED, "device ordinal %d", dev);
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(SWIGLU_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SWIGLU_OK;
}

int check_workspace(const void *workspace, uint64_t bytes) {
    if (workspace && bytes > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(SWIGLU_ERR_ALIGN, "workspace must be 256-byte aligned");
    return SWIGLU_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(SWIGLU_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char *swiglu_status_string(int status) {
    switch (status) {
        case SWIGLU_OK: return "ok";
        case SWIGLU_ERR_NULL: return "null pointer";
        case SWIGLU_ERR_SHAPE: return "invalid shape";
        case SWIGLU_ERR_ALIGN: return "pointer not 16-byte aligned";
        case SWIGLU_ERR_UNSUPPORTED: return "unsupported variant or device";
        case SWIGLU_ERR_HIP: return "HIP error";
        case SWIGLU_ERR_ALIAS: return "output overlaps another operand";
        default: return "unknown status";
    }
}

const char *swiglu_last_error(void) { return g_last_error; }

int64_t swiglu_m_switch(void) {
    const char *s = std::getenv("SWIGLU_M_SWITCH");
    if (s != nullptr && *s != '\0') {
        char *end = nullptr;
        const long long v = std::strtoll(s, &end, 10);
        if (end != s && *end == '\0') return v;
    }
    return kDefaultMSwitch;
}

int swiglu_select_variant(int64_t M, int64_t N, int64_t K) {
    (void)N;
    (void)K;
    if (M < 0) return fail(SWIGLU_ERR_SHAPE, "negative M");
    return M <= swiglu_m_switch() ? SWIGLU_VARIANT_I : SWIGLU_VARIANT_S;
}

int swiglu_pack_weights(const uint16_t *W1, const uint16_t *W2, uint16_t *W_fused, int64_t K,
                        int64_t N, void *stream) {
    if (K < 0 || N < 0) return fail(SWIGLU_ERR_SHAPE, "negative size");
    // both are row lengths of 16-byte-chunked rows: N of W1/W2, K of the packed array
    if (K % 8 != 0 || N % 8 != 0)
        return fail(SWIGLU_ERR_SHAPE, "K=%lld and N=%lld must be multiples of 8", (long long)K,
                    (long long)N);
    if (K > kMaxK || N > kMaxN) return fail(SWIGLU_ERR_SHAPE, "size beyond limits");
    if (K == 0 || N == 0) return ok();
    if (!W1 || !W2 || !W_fused) return fail(SWIGLU_ERR_NULL, "W1, W2 and W_fused are required");
    if (!aligned16(W1) || !aligned16(W2) || !aligned16(W_fused))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int64_t wbytes = K * N * 2;
    if (overlap(W_fused, 2 * wbytes, W1, wbytes) || overlap(W_fused, 2 * wbytes, W2, wbytes))
        return fail(SWIGLU_ERR_ALIAS, "W_fused overlaps W1 or W2");
    int st = check_device();
    if (st != SWIGLU_OK) return st;
    return launched(swiglu::launch_pack(W1, W2, W_fused, K, N, (hipStream_t)stream), "pack");
}

int swiglu_workspace_size(int64_t M, int64_t N, int64_t K, int variant, uint64_t *bytes) {
    if (!bytes) return fail(SWIGLU_ERR_NULL, "bytes is required");
    *bytes = 0;
    if (variant < -1 || variant > SWIGLU_VARIANT_I)
        return fail(SWIGLU_ERR_UNSUPPORTED, "unknown variant %d", variant);
    int st = check_gemm_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    if (M == 0 || N == 0) return ok();
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    const int v = variant == SWIGLU_AUTO ? swiglu_select_variant(M, N, K) : variant;
    // variant I and the ablation (-1) run the single-accumulator GEMM
    if (v == SWIGLU_VARIANT_I || v == -1) *bytes = swiglu::workspace_bytes_for(cus);
    return ok();
}

int swiglu_describe_launch(int64_t M, int64_t N, int64_t K, int variant,
                           uint64_t workspace_bytes, char *buf, uint64_t buf_bytes) {
    if (!buf || buf_bytes == 0) return fail(SWIGLU_ERR_NULL, "buf is required");
    buf[0] = '\0';
    if (variant < kDescribeFp8 || variant > SWIGLU_VARIANT_I)
        return fail(SWIGLU_ERR_UNSUPPORTED, "unknown variant %d", variant);
    int st = variant == kDescribeDownProj ? check_down_shape(M, N, K) : check_gemm_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    if (M == 0 || N == 0) {
        std::snprintf(buf, buf_bytes, "nothing (empty problem)");
        return ok();
    }
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    // only the size of the workspace matters for the plan
    const swiglu::GemmWorkspace ws =
        make_ws(workspace_bytes ? reinterpret_cast<void *>(uintptr_t{256}) : nullptr,
                workspace_bytes, cus);
    const int v = variant == SWIGLU_AUTO ? swiglu_select_variant(M, N, K) : variant;
    if (v == kDescribeFp8) {
        swiglu::describe_gemm_fp8((int)M, (int)(2 * N), (int)K, ws, buf, buf_bytes);
    } else if (v == kDescribeDownProj) {
        swiglu::describe_gemm((int)M, (int)K, (int)N, ws, "StoreEpilogue", buf, buf_bytes);
    } else if (v == SWIGLU_VARIANT_S) {
        swiglu::describe_fused_sequential((int)M, (int)N, (int)K, ws, buf, buf_bytes);
    } else if (v == SWIGLU_VARIANT_I) {
        swiglu::describe_gemm((int)M, (int)(2 * N), (int)K, ws, "PairMulEpilogue", buf, buf_bytes,
                              true);
    } else {
        char g[256];
        swiglu::describe_gemm((int)M, (int)N, (int)K, ws, "StoreEpilogue", g, sizeof g);
        std::snprintf(buf, buf_bytes, "2 x %s + silu_mul_kernel", g);
    }
    return ok();
}

int swiglu_fused_gemm_strided(const uint16_t *A, int64_t lda, const uint16_t *W_fused,
                              uint16_t *Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                              int variant, void *workspace, uint64_t workspace_bytes,
                              void *stream) {
    if (variant != SWIGLU_AUTO && variant != SWIGLU_VARIANT_S && variant != SWIGLU_VARIANT_I)
        return fail(SWIGLU_ERR_UNSUPPORTED, "unknown variant %d", variant);
    int st = check_gemm_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    if (lda < K || lda % 8 != 0 || lda > kMaxK)
        return fail(SWIGLU_ERR_SHAPE, "lda=%lld must be a multiple of 8 in [K, 2^21]",
                    (long long)lda);
    if (ldy < N || ldy > kMaxN)
        return fail(SWIGLU_ERR_SHAPE, "ldy=%lld must lie in [N, 2^22]", (long long)ldy);
    if (M == 0 || N == 0) return ok();
    const int v = variant == SWIGLU_AUTO ? swiglu_select_variant(M, N, K) : variant;
    if (!A || !W_fused || !Y) return fail(SWIGLU_ERR_NULL, "A, W_fused and Y are required");
    if (!aligned16(A) || !aligned16(W_fused) || !aligned16(Y))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    // the memory spans of the strided views (conservative: rows interleaved
    // with another operand's count as overlapping)
    const int64_t abytes = ((M - 1) * lda + K) * 2, ybytes = ((M - 1) * ldy + N) * 2;
    const int64_t wbytes = 2 * K * N * 2;
    if (overlap(Y, ybytes, A, abytes) || overlap(Y, ybytes, W_fused, wbytes))
        return fail(SWIGLU_ERR_ALIAS, "Y overlaps an input");
    st = check_workspace(workspace, workspace_bytes);
    if (st != SWIGLU_OK) return st;
    if (workspace && workspace_bytes > 0 &&
        (overlap(workspace, (int64_t)workspace_bytes, A, abytes) ||
         overlap(workspace, (int64_t)workspace_bytes, W_fused, wbytes) ||
         overlap(workspace, (int64_t)workspace_bytes, Y, ybytes)))
        return fail(SWIGLU_ERR_ALIAS, "workspace overlaps an operand");
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    if (v == SWIGLU_VARIANT_I)
        return launched(swiglu::launch_fused_interleaved(A, (int)lda, W_fused, Y, (int)ldy,
                                                         (int)M, (int)N, (int)K,
                                                         make_ws(workspace, workspace_bytes, cus),
                                                         s),
                        "fused interleaved");
    return launched(swiglu::launch_fused_sequential(A, (int)lda, W_fused, Y, (int)ldy, (int)M,
                                                    (int)N, (int)K,
                                                    make_ws(workspace, workspace_bytes, cus), s),
                    "fused sequential");
}

int swiglu_fused_gemm(const uint16_t *A, const uint16_t *W_fused, uint16_t *Y, int64_t M,
                      int64_t N, int64_t K, int variant, void *workspace,
                      uint64_t workspace_bytes, void *stream) {
    // contiguous rows: lda = K, ldy = N (validated by the strided entry point
    // after the shape check, so the shape errors are reported first)
    return swiglu_fused_gemm_strided(A, K, W_fused, Y, N, M, N, K, variant, workspace,
                                     workspace_bytes, stream);
}

int swiglu_fused_gemm_noalloc(const uint16_t *A, const uint16_t *W_fused, uint16_t *Y,
                              int64_t M, int64_t N, int64_t K, int variant, void *stream) {
    if (variant != SWIGLU_AUTO && variant != SWIGLU_VARIANT_S && variant != SWIGLU_VARIANT_I)
        return fail(SWIGLU_ERR_UNSUPPORTED, "unknown variant %d", variant);
    int st = check_gemm_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!A || !W_fused || !Y) return fail(SWIGLU_ERR_NULL, "A, W_fused and Y are required");
    if (!aligned16(A) || !aligned16(W_fused) || !aligned16(Y))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int64_t abytes = M * K * 2, ybytes = M * N * 2, wbytes = 2 * K * N * 2;
    if (overlap(Y, ybytes, A, abytes) || overlap(Y, ybytes, W_fused, wbytes))
        return fail(SWIGLU_ERR_ALIAS, "Y overlaps an input");
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    const uint64_t need = swiglu::workspace_bytes_for(cus);
    if (need > kScratchBytes)
        return fail(SWIGLU_ERR_UNSUPPORTED,
                    "the device's %d compute units need %llu bytes of split-tail scratch; the "
                    "library's static scratch holds %llu", cus, (unsigned long long)need,
                    (unsigned long long)kScratchBytes);
    void *ptr = nullptr;
    st = scratch_on_device(&ptr);
    if (st != SWIGLU_OK) return st;
    const int v = variant == SWIGLU_AUTO ? swiglu_select_variant(M, N, K) : variant;
    const hipStream_t s = (hipStream_t)stream;
    if (v == SWIGLU_VARIANT_I)
        return launched(swiglu::launch_fused_interleaved(A, (int)K, W_fused, Y, (int)N, (int)M,
                                                         (int)N, (int)K,
                                                         make_ws(ptr, kScratchBytes, cus), s),
                        "fused interleaved (no-alloc)");
    return launched(swiglu::launch_fused_sequential(A, (int)K, W_fused, Y, (int)N, (int)M,
                                                    (int)N, (int)K,
                                                    make_ws(ptr, kScratchBytes, cus), s),
                    "fused sequential (no-alloc)");
}

int swiglu_unfused_ablation(const uint16_t *A, const uint16_t *W_fused, uint16_t *gate_ws,
                            uint16_t *up_ws, uint16_t *Y, int64_t M, int64_t N, int64_t K,
                            void *workspace, uint64_t workspace_bytes, void *stream) {
    int st = check_gemm_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    if (M == 0 || N == 0) return ok();
    if (!A || !W_fused || !gate_ws || !up_ws || !Y)
        return fail(SWIGLU_ERR_NULL, "A, W_fused, gate_ws, up_ws and Y are required");
    if (!aligned16(A) || !aligned16(W_fused) || !aligned16(gate_ws) || !aligned16(up_ws) ||
        !aligned16(Y))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int64_t abytes = M * K * 2, ybytes = M * N * 2, wbytes = 2 * K * N * 2;
    const void *outs[3] = {gate_ws, up_ws, Y};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], ybytes, A, abytes) || overlap(outs[i], ybytes, W_fused, wbytes))
            return fail(SWIGLU_ERR_ALIAS, "an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], ybytes, outs[j], ybytes))
                return fail(SWIGLU_ERR_ALIAS, "outputs overlap each other");
        if (workspace && workspace_bytes > 0 &&
            overlap(workspace, (int64_t)workspace_bytes, outs[i], ybytes))
            return fail(SWIGLU_ERR_ALIAS, "workspace overlaps an operand");
    }
    st = check_workspace(workspace, workspace_bytes);
    if (st != SWIGLU_OK) return st;
    if (workspace && workspace_bytes > 0 &&
        (overlap(workspace, (int64_t)workspace_bytes, A, abytes) ||
         overlap(workspace, (int64_t)workspace_bytes, W_fused, wbytes)))
        return fail(SWIGLU_ERR_ALIAS, "workspace overlaps an operand");
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    // the two GEMMs run in stream order, so they may share the workspace
    hipError_t e = swiglu::launch_gemm_store(A, W_fused, 0, gate_ws, (int)M, (int)N, (int)K,
                                             make_ws(workspace, workspace_bytes, cus), s);
    if (e != hipSuccess) return launched(e, "ablation gate GEMM");
    e = swiglu::launch_gemm_store(A, W_fused, 1, up_ws, (int)M, (int)N, (int)K,
                                  make_ws(workspace, workspace_bytes, cus), s);
    if (e != hipSuccess) return launched(e, "ablation up GEMM");
    return launched(swiglu::launch_silu_mul(gate_ws, up_ws, Y, M * N, s), "ablation silu_mul");
}

int swiglu_silu_mul(const uint16_t *gate, const uint16_t *up, uint16_t *Y, int64_t count,
                    void *stream) {
    if (count < 0 || count % 8 != 0)
        return fail(SWIGLU_ERR_SHAPE, "count=%lld must be a non-negative multiple of 8", (long long)count);
    if (count == 0) return ok();
    if (!gate || !up || !Y) return fail(SWIGLU_ERR_NULL, "gate, up and Y are required");
    if (!aligned16(gate) || !aligned16(up) || !aligned16(Y))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    if (overlap(Y, 2 * count, gate, 2 * count) || overlap(Y, 2 * count, up, 2 * count))
        return fail(SWIGLU_ERR_ALIAS, "Y overlaps an input");
    int st = check_device();
    if (st != SWIGLU_OK) return st;
    return launched(swiglu::launch_silu_mul(gate, up, Y, count, (hipStream_t)stream), "silu_mul");
}

int swiglu_pack_weights_nk(const uint16_t *W1t, const uint16_t *W2t, uint16_t *W_fused,
                           int64_t K, int64_t N, void *stream) {
    if (K < 0 || N < 0) return fail(SWIGLU_ERR_SHAPE, "negative size");
    // K is the row length of all three arrays
    if (K % 8 != 0) return fail(SWIGLU_ERR_SHAPE, "K=%lld must be a multiple of 8", (long long)K);
    if (K > kMaxK || N > kMaxN) return fail(SWIGLU_ERR_SHAPE, "size beyond limits");
    if (K == 0 || N == 0) return ok();
    if (!W1t || !W2t || !W_fused) return fail(SWIGLU_ERR_NULL, "W1t, W2t and W_fused are required");
    if (!aligned16(W1t) || !aligned16(W2t) || !aligned16(W_fused))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int64_t wbytes = K * N * 2;
    if (overlap(W_fused, 2 * wbytes, W1t, wbytes) || overlap(W_fused, 2 * wbytes, W2t, wbytes))
        return fail(SWIGLU_ERR_ALIAS, "W_fused overlaps W1t or W2t");
    int st = check_device();
    if (st != SWIGLU_OK) return st;
    return launched(swiglu::launch_pack_nk(W1t, W2t, W_fused, K, N, (hipStream_t)stream),
                    "pack_nk");
}

int swiglu_down_proj(const uint16_t *H, const uint16_t *W3t, uint16_t *Out, int64_t M, int64_t N,
                     int64_t D, void *workspace, uint64_t workspace_bytes, void *stream) {
    int st = check_down_shape(M, N, D);
    if (st != SWIGLU_OK) return st;
    if (M == 0 || D == 0) return ok();
    if (!H || !W3t || !Out) return fail(SWIGLU_ERR_NULL, "H, W3t and Out are required");
    if (!aligned16(H) || !aligned16(W3t) || !aligned16(Out))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int64_t hbytes = M * N * 2, wbytes = D * N * 2, obytes = M * D * 2;
    if (overlap(Out, obytes, H, hbytes) || overlap(Out, obytes, W3t, wbytes))
        return fail(SWIGLU_ERR_ALIAS, "Out overlaps an input");
    st = check_workspace(workspace, workspace_bytes);
    if (st != SWIGLU_OK) return st;
    if (workspace && workspace_bytes > 0 &&
        (overlap(workspace, (int64_t)workspace_bytes, H, hbytes) ||
         overlap(workspace, (int64_t)workspace_bytes, W3t, wbytes) ||
         overlap(workspace, (int64_t)workspace_bytes, Out, obytes)))
        return fail(SWIGLU_ERR_ALIAS, "workspace overlaps an operand");
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    return launched(swiglu::launch_down_proj(H, W3t, Out, (int)M, (int)N, (int)D,
                                             make_ws(workspace, workspace_bytes, cus),
                                             (hipStream_t)stream),
                    "down projection");
}

int swiglu_gated_mlp(const uint16_t *A, const uint16_t *W_fused, const uint16_t *W3t,
                     uint16_t *H, uint16_t *Out, int64_t M, int64_t N, int64_t K, int variant,
                     void *workspace, uint64_t workspace_bytes, void *stream) {
    if (variant != SWIGLU_AUTO && variant != SWIGLU_VARIANT_S && variant != SWIGLU_VARIANT_I)
        return fail(SWIGLU_ERR_UNSUPPORTED, "unknown variant %d", variant);
    int st = check_gemm_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    st = check_down_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    if (M == 0) return ok();   // N >= 8 and K >= 8 here (both are reduction lengths)
    const int v = variant == SWIGLU_AUTO ? swiglu_select_variant(M, N, K) : variant;
    if (!A || !W_fused || !W3t || !H || !Out)
        return fail(SWIGLU_ERR_NULL, "A, W_fused, W3t, H and Out are required");
    if (!aligned16(A) || !aligned16(W_fused) || !aligned16(W3t) || !aligned16(H) ||
        !aligned16(Out))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int64_t abytes = M * K * 2, wbytes = 2 * K * N * 2, w3bytes = K * N * 2;
    const int64_t hbytes = M * N * 2, obytes = M * K * 2;
    const void *ins[3] = {A, W_fused, W3t};
    const int64_t inb[3] = {abytes, wbytes, w3bytes};
    for (int i = 0; i < 3; ++i)
        if (overlap(H, hbytes, ins[i], inb[i]) || overlap(Out, obytes, ins[i], inb[i]))
            return fail(SWIGLU_ERR_ALIAS, "an output overlaps an input");
    if (overlap(H, hbytes, Out, obytes)) return fail(SWIGLU_ERR_ALIAS, "H overlaps Out");
    st = check_workspace(workspace, workspace_bytes);
    if (st != SWIGLU_OK) return st;
    if (workspace && workspace_bytes > 0) {
        for (int i = 0; i < 3; ++i)
            if (overlap(workspace, (int64_t)workspace_bytes, ins[i], inb[i]))
                return fail(SWIGLU_ERR_ALIAS, "workspace overlaps an operand");
        if (overlap(workspace, (int64_t)workspace_bytes, H, hbytes) ||
            overlap(workspace, (int64_t)workspace_bytes, Out, obytes))
            return fail(SWIGLU_ERR_ALIAS, "workspace overlaps an operand");
    }
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    const swiglu::GemmWorkspace ws = make_ws(workspace, workspace_bytes, cus);
    // the two launches run in stream order, so they may share the workspace
    hipError_t e = v == SWIGLU_VARIANT_I
                       ? swiglu::launch_fused_interleaved(A, (int)K, W_fused, H, (int)N, (int)M,
                                                          (int)N, (int)K, ws, s)
                       : swiglu::launch_fused_sequential(A, (int)K, W_fused, H, (int)N, (int)M,
                                                         (int)N, (int)K, ws, s);
    if (e != hipSuccess) return launched(e, "gated MLP: fused SwiGLU");
    return launched(swiglu::launch_down_proj(H, W3t, Out, (int)M, (int)N, (int)K, ws, s),
                    "gated MLP: down projection");
}

int swiglu_fp8_scale_exp(double amax) {
    if (!(amax > 0.0) || amax > 3.5e38) return 0;   // zero, negative, NaN or beyond float
    int e = -126;
    while (e < 126 && std::ldexp(amax, -e) > 448.0) ++e;   // smallest e: amax 2^-e <= 448
    return e;
}

int swiglu_quantize_fp8(const uint16_t *X, uint8_t *Q, int64_t count, int scale_exp,
                        void *stream) {
    if (count < 0 || count % 16 != 0)
        return fail(SWIGLU_ERR_SHAPE, "count=%lld must be a non-negative multiple of 16",
                    (long long)count);
    if (scale_exp < -126 || scale_exp > 126)
        return fail(SWIGLU_ERR_SHAPE, "scale_exp=%d outside [-126, 126]", scale_exp);
    if (count == 0) return ok();
    if (!X || !Q) return fail(SWIGLU_ERR_NULL, "X and Q are required");
    if (!aligned16(X) || !aligned16(Q))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    if (overlap(Q, count, X, 2 * count)) return fail(SWIGLU_ERR_ALIAS, "Q overlaps X");
    int st = check_device();
    if (st != SWIGLU_OK) return st;
    return launched(swiglu::launch_quantize_fp8(X, Q, count, scale_exp, (hipStream_t)stream),
                    "quantize_fp8");
}

int swiglu_fused_gemm_fp8(const uint8_t *A8, const uint8_t *W_fused8, uint16_t *Y, int64_t M,
                          int64_t N, int64_t K, int a_exp, int w_exp, int variant,
                          void *workspace, uint64_t workspace_bytes, void *stream) {
    if (variant != SWIGLU_AUTO && variant != SWIGLU_VARIANT_S && variant != SWIGLU_VARIANT_I)
        return fail(SWIGLU_ERR_UNSUPPORTED, "unknown variant %d", variant);
    int st = check_gemm_shape(M, N, K);
    if (st != SWIGLU_OK) return st;
    if (K % 16 != 0) return fail(SWIGLU_ERR_SHAPE, "K=%lld must be a multiple of 16", (long long)K);
    if (a_exp < -126 || a_exp > 126 || w_exp < -126 || w_exp > 126 || a_exp + w_exp < -126 ||
        a_exp + w_exp > 126)
        return fail(SWIGLU_ERR_SHAPE, "scale exponents out of range (a_exp + w_exp in [-126, 126])");
    if (M == 0 || N == 0) return ok();
    if (!A8 || !W_fused8 || !Y) return fail(SWIGLU_ERR_NULL, "A8, W_fused8 and Y are required");
    if (!aligned16(A8) || !aligned16(W_fused8) || !aligned16(Y))
        return fail(SWIGLU_ERR_ALIGN, "pointers must be 16-byte aligned");
    const int64_t abytes = M * K, ybytes = M * N * 2, wbytes = 2 * K * N;
    if (overlap(Y, ybytes, A8, abytes) || overlap(Y, ybytes, W_fused8, wbytes))
        return fail(SWIGLU_ERR_ALIAS, "Y overlaps an input");
    st = check_workspace(workspace, workspace_bytes);
    if (st != SWIGLU_OK) return st;
    if (workspace && workspace_bytes > 0 &&
        (overlap(workspace, (int64_t)workspace_bytes, A8, abytes) ||
         overlap(workspace, (int64_t)workspace_bytes, W_fused8, wbytes) ||
         overlap(workspace, (int64_t)workspace_bytes, Y, ybytes)))
        return fail(SWIGLU_ERR_ALIAS, "workspace overlaps an operand");
    int cus = 0;
    st = check_device(&cus);
    if (st != SWIGLU_OK) return st;
    const float scale = std::ldexp(1.0f, a_exp + w_exp);
    const int v = variant == SWIGLU_AUTO ? swiglu_select_variant(M, N, K) : variant;
    if (v == SWIGLU_VARIANT_S)
        return launched(swiglu::launch_fused_sequential_fp8(A8, W_fused8, Y, (int)M, (int)N,
                                                            (int)K, scale, (hipStream_t)stream),
                        "fused sequential fp8");
    return launched(swiglu::launch_fused_interleaved_fp8(A8, W_fused8, Y, (int)M, (int)N, (int)K,
                                                         scale,
                                                         make_ws(workspace, workspace_bytes, cus),
                                                         (hipStream_t)stream),
                    "fused interleaved fp8");
}

}  // extern "C"
