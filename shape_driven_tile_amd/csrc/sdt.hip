// C ABI of the MI355X fp16 / bf16 GEMM and M=1 GEMV library (declared in
// sdt.h).
// Validates arguments on the host, picks the kernel instantiation and
// enqueues it on the caller's stream.  Allocates nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <mutex>

#include "gemm_kernel.hpp"
#include "gemv_kernel.hpp"
#include "launcher.hpp"
#include "sdt.h"

namespace sdt {
namespace {

// Whether the ladder rung with this tile is built to split K across
// workgroups (only those rungs instantiate the k-split kernels).
template <int BM, int BN>
constexpr bool kLadderHasSplit() {
    for (const TileDesc& d : kLadder)
        if (d.bm == BM && d.bn == BN) return d.ksplit != 0;
    return false;
}

thread_local int g_last_hip_error = 0;

constexpr sdt_launch kAuto = {-1, -1, -1, -1, -1, -1, -1, -1};

struct DeviceInfo {
    int num_cu = 0;
    int nxcd = 1;
};
constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
DeviceInfo g_dev[kMaxDevices];

int fail_hip(hipError_t e) {
    g_last_hip_error = (int)e;
    return SDT_ERR_HIP;
}

// CU count of the current device, read once per device.  MI355X deals
// workgroups round-robin over its XCDs of 32 CUs each (8 in the single-
// partition mode); a partition with fewer CUs has proportionally fewer XCDs.
int device_info(DeviceInfo* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e);
    if (dev < 0 || dev >= kMaxDevices) return SDT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_dev[dev].num_cu <= 0) {
        int cu = 0;
        e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail_hip(e);
        if (cu <= 0) return SDT_ERR_UNSUPPORTED;
        int nxcd = (cu % 32 == 0) ? cu / 32 : 1;
        if (nxcd > 8) nxcd = 8;
        g_dev[dev].num_cu = cu;
        g_dev[dev].nxcd = nxcd < 1 ? 1 : nxcd;
    }
    *out = g_dev[dev];
    return SDT_OK;
}

// One launch of gemm_kernel; a k-split launch (splits > 1) runs the
// instantiation built for it, `splits` workgroups per tile, followed (with
// split_algo 0) by the kernel that sums the partials.
template <typename Elt, int BM, int BN, int WM, int WN, int NS, int KS, int MF = 32,
          bool HELP = false>
hipError_t launch_gemm_tile(GemmParams p, hipStream_t stream) {
    void* args[] = {&p};
    const int tiles = p.gm * p.gn;
    if constexpr (kLadderHasSplit<BM, BN>()) {
        if (p.splits > 1) {
            hipError_t e = hipLaunchKernel(
                reinterpret_cast<const void*>(&gemm_kernel<Elt, BM, BN, WM, WN, NS, KS, MF, true>),
                dim3(tiles * p.splits), dim3(WM * WN * KS * 64), args, 0, stream);
            if (e != hipSuccess || p.split_algo != 0) return e;
            return hipLaunchKernel(
                reinterpret_cast<const void*>(&gemm_splitk_reduce_kernel<Elt, BM, BN, WM, WN, MF>),
                dim3(tiles), dim3(WM * WN * 64), args, 0, stream);
        }
    }
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&gemm_kernel<Elt, BM, BN, WM, WN, NS, KS, MF, false, HELP>),
        dim3(tiles), dim3(WM * WN * KS * 64 * (HELP ? 2 : 1)), args, 0, stream);
}

// The 256 x 256 ping-pong kernel: 8 waves, 160 KB of LDS, one workgroup per
// CU; with p.persistent > 0 a grid of that many workgroups loops over the tiles.
template <typename Elt>
hipError_t launch_gemm_pp(GemmParams p, hipStream_t stream) {
    void* args[] = {&p};
    if (p.persistent > 0)
        return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_pp_kernel<Elt, true>),
                               dim3(p.persistent), dim3(512), args, 0, stream);
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_pp_kernel<Elt>),
                           dim3(p.gm * p.gn), dim3(512), args, 0, stream);
}

// Rung I with a plan check_plan accepted: its shallow (2-stage), deep or long
// pipeline with one k-group, or the deep or long pipeline with two; rung 0's
// deep pipeline is the ping-pong kernel, and a deep16 rung's deep pipeline
// with one k-group runs 16x16x32 MFMAs.
template <typename Elt, int I>
hipError_t launch_rung(GemmParams p, const Plan& pl, hipStream_t s) {
    constexpr TileDesc d = kLadder[I];
    // wave tiles that are not whole 32 x 32 MFMA tiles: 16x16x32 on every pipeline
    constexpr bool only16 = (d.bm / d.waves_m) % 32 != 0 || (d.bn / d.waves_n) % 32 != 0;
    if constexpr (only16) {
        static_assert(d.kgroups == 1 && d.long_stages == 0 && !d.pingpong && !d.ksplit,
                      "16x16x32-only rungs: one k-group, no long pipeline, no k-split");
        if (pl.stages == 2)
            return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, 2, 1, 16>(p, s);
        if constexpr (d.helpers != 0) {
            if (pl.loaders)
                return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.stages, 1, 16,
                                        true>(p, s);
        }
        return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.stages, 1, 16>(p, s);
    } else if constexpr (d.pingpong) {
        static_assert(d.bm == 256 && d.bn == 256 && d.waves_m == 2 && d.waves_n == 4 &&
                          d.stages == 3 && d.kgroups == 1,
                      "the ping-pong kernel's tile");
        if (pl.stages != 2) return launch_gemm_pp<Elt>(p, s);
        return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, 2, 1>(p, s);
    } else {
        if constexpr (d.long_stages > 0) {
            static_assert(d.kgroups == 2, "long pipelines: 32x32x16, both k-group forms");
            if (pl.stages == d.long_stages) {
                if (pl.kgroups == 2)
                    return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.long_stages, 2>(p, s);
                return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.long_stages, 1>(p, s);
            }
        }
        if constexpr (d.kgroups == 2) {
            if (pl.kgroups == 2)
                return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.stages, 2>(p, s);
        }
        if (pl.stages == 2)
            return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, 2, 1>(p, s);
        if constexpr (d.deep16 && d.helpers != 0) {
            if (pl.loaders)
                return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.stages, 1, 16,
                                        true>(p, s);
        }
        if constexpr (d.deep16)
            return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.stages, 1, 16>(p, s);
        else
            return launch_gemm_tile<Elt, d.bm, d.bn, d.waves_m, d.waves_n, d.stages, 1>(p, s);
    }
}

template <typename Elt>
hipError_t launch_gemm(const Plan& pl, GemmParams p, hipStream_t s) {
    static_assert(kNumTiles == 8, "dispatch table below lists every rung");
    switch (pl.tile) {
        case 0: return launch_rung<Elt, 0>(p, pl, s);
        case 1: return launch_rung<Elt, 1>(p, pl, s);
        case 2: return launch_rung<Elt, 2>(p, pl, s);
        case 3: return launch_rung<Elt, 3>(p, pl, s);
        case 4: return launch_rung<Elt, 4>(p, pl, s);
        case 5: return launch_rung<Elt, 5>(p, pl, s);
        case 6: return launch_rung<Elt, 6>(p, pl, s);
        default: return launch_rung<Elt, 7>(p, pl, s);
    }
}

// Zero `words` 32-bit words at `w` (the workspace's counters).
__global__ void fill_words_kernel(uint32_t* w, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        w[i] = 0u;
}

int fill_words(uint32_t* w, int64_t words, hipStream_t stream) {
    int64_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    void* args[] = {&w, &words};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fill_words_kernel),
                                   dim3((unsigned)blocks), dim3(256), args, 0, stream);
    return e == hipSuccess ? SDT_OK : fail_hip(e);
}

int fill_zero(uint16_t* C, int64_t ldc, int64_t M, int64_t N, hipStream_t stream) {
    const int64_t total = M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    int Mi = (int)M, Ni = (int)N;
    void* args[] = {&C, &ldc, &Mi, &Ni};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fill_zero_kernel),
                                   dim3((unsigned)blocks), dim3(256), args, 0, stream);
    return e == hipSuccess ? SDT_OK : fail_hip(e);
}

// GEMV instantiations.  Variant 0 (gemv_f16_m1's): four waves per column
// (gemv_m1_wsplit_kernel).  Variants 1-4: one wave streams 1, 2, 4 or 8
// columns (gemv_m1_kernel; the activations held as 8 chunks of 8 fp16 per
// lane, 4096 k per pass); among those one column per wave is the fastest on
// the decode shape (cold, 8 rotating buffers), by 15-20% over two or four:
// more waves in flight beat more loads per wave.
constexpr int kGemvRpw[] = {0, 1, 2, 4, 8};
constexpr int kGemvVariants = sizeof(kGemvRpw) / sizeof(kGemvRpw[0]);

template <typename Elt, int RPW>
hipError_t launch_gemv_rpw(GemvParams p, hipStream_t stream) {
    // one-wave workgroups for one row per wave, four waves otherwise
    constexpr int WPB = (RPW == 1) ? 1 : 4;
    const int64_t waves = (p.N + RPW - 1) / RPW;
    const int64_t blocks = (waves + WPB - 1) / WPB;
    void* args[] = {&p};
    // K a multiple of one pass (8 x 512 elements): the kernel without the
    // ragged-pass code, which needs fewer registers.
    const void* k = (p.K % (8 * 512) == 0)
                        ? reinterpret_cast<const void*>(&gemv_m1_kernel<Elt, RPW, 8, false, WPB>)
                        : reinterpret_cast<const void*>(&gemv_m1_kernel<Elt, RPW, 8, true, WPB>);
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(WPB * 64), args, 0, stream);
}

template <typename Elt>
int launch_gemv(int variant, int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                void* y, hipStream_t stream) {
    if (N > INT_MAX) return SDT_ERR_UNSUPPORTED;
    if (K == 0) return fill_zero(static_cast<uint16_t*>(y), N, 1, N, stream);
    GemvParams p;
    p.x = static_cast<const uint16_t*>(x);
    p.B = static_cast<const uint16_t*>(B);
    p.y = static_cast<uint16_t*>(y);
    p.ldb = ldb;
    p.N = (int)N;
    p.K = (int)K;
    hipError_t e;
    switch (kGemvRpw[variant]) {
        case 0: {
            void* args[] = {&p};
            e = hipLaunchKernel(reinterpret_cast<const void*>(&gemv_m1_wsplit_kernel<Elt, 4, 2>),
                                dim3((unsigned)N), dim3(256), args, 0, stream);
            break;
        }
        case 1: e = launch_gemv_rpw<Elt, 1>(p, stream); break;
        case 2: e = launch_gemv_rpw<Elt, 2>(p, stream); break;
        case 8: e = launch_gemv_rpw<Elt, 8>(p, stream); break;
        default: e = launch_gemv_rpw<Elt, 4>(p, stream); break;
    }
    return e == hipSuccess ? SDT_OK : fail_hip(e);
}

// [K][N] GEMV instantiations: (lanes per 16-byte column segment, waves per
// workgroup).  A workgroup covers 8 * SEG columns and all of K.
struct GemvKnVariant {
    int seg, waves;
};
constexpr GemvKnVariant kGemvKn[] = {{8, 16}, {8, 8}, {4, 16}, {4, 8}};
constexpr int kGemvKnVariants = sizeof(kGemvKn) / sizeof(kGemvKn[0]);

template <typename Elt, int SEG, int NW>
hipError_t launch_gemv_kn_tile(GemvKnParams p, hipStream_t stream) {
    const int64_t blocks = ((int64_t)p.N + SEG * 8 - 1) / (SEG * 8);
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_kn_kernel<Elt, SEG, NW>),
                           dim3((unsigned)blocks), dim3(NW * 64), args, 0, stream);
}

template <typename Elt>
int launch_gemv_kn(int variant, int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                   void* y, hipStream_t stream) {
    if (N > INT_MAX || K > INT_MAX) return SDT_ERR_UNSUPPORTED;
    if (K == 0) return fill_zero(static_cast<uint16_t*>(y), N, 1, N, stream);
    GemvKnParams p;
    p.x = static_cast<const uint16_t*>(x);
    p.B = static_cast<const uint16_t*>(B);
    p.y = static_cast<uint16_t*>(y);
    p.ldb = ldb;
    p.N = (int)N;
    p.K = (int)K;
    static_assert(kGemvKnVariants == 4, "dispatch below lists every variant");
    hipError_t e;
    switch (variant) {
        case 1: e = launch_gemv_kn_tile<Elt, 8, 8>(p, stream); break;
        case 2: e = launch_gemv_kn_tile<Elt, 4, 16>(p, stream); break;
        case 3: e = launch_gemv_kn_tile<Elt, 4, 8>(p, stream); break;
        default: e = launch_gemv_kn_tile<Elt, 8, 16>(p, stream); break;
    }
    return e == hipSuccess ? SDT_OK : fail_hip(e);
}

// The [K][N] GEMV split over K with the plan kn_split_plan made: the band
// kernel into the workspace's fp32 column sums, then their sum in split order.
template <typename Elt>
int launch_gemv_kn_split(const KnSplit& sp, int64_t N, int64_t K, const void* x, const void* B,
                         int64_t ldb, void* y, void* ws, hipStream_t stream) {
    GemvKnParams p;
    p.x = static_cast<const uint16_t*>(x);
    p.B = static_cast<const uint16_t*>(B);
    p.y = static_cast<uint16_t*>(y);
    p.ldb = ldb;
    p.N = (int)N;
    p.K = (int)K;
    p.part = static_cast<float*>(ws);
    p.pstride = sp.pstride;
    p.kc = sp.kc;
    int splits = sp.splits;
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void*>(&gemv_kn_kernel<Elt, kKnSplitSeg, kKnSplitWaves, true>),
        dim3((unsigned)sp.bands, (unsigned)sp.splits), dim3(kKnSplitWaves * 64), args, 0, stream);
    if (e != hipSuccess) return fail_hip(e);
    void* rargs[] = {&p, &splits};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&gemv_kn_reduce_kernel<Elt>),
                        dim3((unsigned)((N + 255) / 256)), dim3(256), rargs, 0, stream);
    return e == hipSuccess ? SDT_OK : fail_hip(e);
}

template <typename Elt>
int gemv_kn_ws_impl(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb, void* y,
                    void* ws, int64_t ws_bytes, void* stream) {
    int st = check_gemv_kn_args(N, K, x, B, ldb, y);
    if (st != SDT_OK) return st;
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws)) return SDT_ERR_INVALID_ARG;
    if (ws && (reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return SDT_ERR_UNSUPPORTED;
    if (N == 0) return SDT_OK;
    const KnSplit sp = kn_split_plan(N, K);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (sp.splits < 2 || ws_bytes < sp.bytes)
        return launch_gemv_kn<Elt>(0, N, K, x, B, ldb, y, s);
    return launch_gemv_kn_split<Elt>(sp, N, K, x, B, ldb, y, ws, s);
}

// cfg fields: -1 = the automatic choice.  route_m1: M == 1 runs the GEMV.
// ws / ws_bytes: the caller's workspace (NULL and 0: none; the plan then
// never splits K across workgroups).
template <typename Elt>
int gemm_impl(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, void* stream, const sdt_launch& cfg,
              bool route_m1, void* ws, int64_t ws_bytes) {
    int st = check_gemm_args(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SDT_OK) return st;
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws)) return SDT_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return SDT_ERR_UNSUPPORTED;
    // the configuration is checked before the sizes short-circuit
    Plan pl;
    st = resolve_plan(cfg, std::max<int64_t>(M, 1), std::max<int64_t>(N, 1), K, 256,
                      ws ? ws_bytes : 0, &pl);
    if (st != SDT_OK) return st;
    if (M == 0 || N == 0) return SDT_OK;
    if (M > INT_MAX || N > INT_MAX) return SDT_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) return fill_zero(static_cast<uint16_t*>(C), ldc, M, N, s);
    if (route_m1 && M == 1) return launch_gemv<Elt>(0, N, K, A, B, ldb, C, s);

    DeviceInfo dev;
    st = device_info(&dev);
    if (st != SDT_OK) return st;
    st = resolve_plan(cfg, M, N, K, dev.num_cu, ws ? ws_bytes : 0, &pl);
    if (st != SDT_OK) return st;
    const TileDesc& td = kLadder[pl.tile];
    const int64_t gm = ceil_div(M, td.bm);
    const int64_t gn = ceil_div(N, td.bn);
    if (gm * gn * pl.splits > INT_MAX) return SDT_ERR_UNSUPPORTED;

    GemmParams p;
    p.A = static_cast<const uint16_t*>(A);
    p.B = static_cast<const uint16_t*>(B);
    p.C = static_cast<uint16_t*>(C);
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.gm = (int)gm;
    p.gn = (int)gn;
    p.stagger = pl.stagger;
    p.nxcd = dev.nxcd;
    p.splits = pl.splits;
    p.split_algo = pl.split_algo;
    p.cnt = static_cast<int*>(ws);
    p.ws = pl.splits > 1
               ? reinterpret_cast<float*>(static_cast<char*>(ws) + counter_bytes(pl, M, N))
               : nullptr;
    p.persistent = pl.persistent;
    hipError_t e = launch_gemm<Elt>(pl, p, s);
    return e == hipSuccess ? SDT_OK : fail_hip(e);
}

// ---- the allocation-free k-split workspace ------------------------------------
// gemm_f16_noalloc takes its k-split workspace from this array instead of the
// caller: the 64 KiB counter area and the fp32 partial sums of the automatic
// plan, which splits only grids of at most one workgroup per CU, i.e. at most
// 256 x 64 KiB of partials on a 256-CU part.  Each device holds its own copy
// (zero-filled when the code object is loaded) at its own address, taken once
// per device by hipGetSymbolAddress; host code uses that address only (the
// array's name is a host-side stand-in).
constexpr int64_t kScratchBytes = kCounterBytes + (int64_t(16) << 20);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
    int st = SDT_OK;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's scratch address, set up on the first call on that
// device (the device current): its address, then its counter area cleared by
// a fill kernel on `stream` (the array starts zero-filled and every call
// leaves the counters zero; the clear makes that independent of the load).
int scratch_for_current_device(void** out, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e);
    if (dev < 0 || dev >= kMaxDevices) return SDT_ERR_UNSUPPORTED;
    ScratchSlot& sl = g_scratch[dev];
    std::call_once(sl.once, [&sl, stream] {
        void* ptr = nullptr;
        sl.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (sl.err != hipSuccess) return;
        sl.ptr = ptr;
        sl.st = fill_words(static_cast<uint32_t*>(ptr), kCounterBytes / 4, stream);
    });
    if (sl.err != hipSuccess) return fail_hip(sl.err);
    if (sl.st != SDT_OK) return sl.st;
    *out = sl.ptr;
    return SDT_OK;
}

// Does nothing: one workgroup, no memory access.  Timing it gives the
// launch floor the small shapes are measured against.
__global__ void empty_kernel() {}

// Reads memory and nothing else: one wave per 8 KB run, eight non-temporal
// 16-byte loads per lane (the decode GEMV's access pattern, without the
// activations, the arithmetic or the output), folded into one word per run so
// that no load is dead.  Timed over the decode shape's rotating weight buffers
// it gives the streaming-read ceiling the GEMV is compared with.
__global__ __launch_bounds__(64) void stream_read_kernel(const int4_t* buf, uint32_t* out) {
    const int lane = threadIdx.x;
    const int4_t* run = buf + (int64_t)blockIdx.x * 512;
    int4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(run + j * 64 + lane);
    int x = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
    if (lane == 0) out[blockIdx.x] = (uint32_t)x;
}

// Register-only MFMA loop: the MFMA phase of the 256 x 256 GEMM kernel's
// wave repeated `iters` times with no memory access, on 8 waves per
// workgroup (two per SIMD).  MF = 16: 32 accumulator tiles of 16 x 16, the
// 24 fragments of one 64-deep k-tile (two 32-deep halves of 8 A and 4 B
// fragments), 64 v_mfma_f32_16x16x32 per iteration in the kernel's order.
// MF = 32: the same 128 x 64 wave tile as 8 tiles of 32 x 32, the same 24
// fragments read as four 16-deep steps of 4 A and 2 B fragments, 32
// v_mfma_f32_32x32x16 per iteration (the same FLOPs).  Each thread then
// writes the sum of its accumulators, so no MFMA is dead.
template <typename Elt, int MF>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(const int4_t* frags, int iters,
                                                           float* out) {
    typedef typename Elt::frag8 frag8;
    const int lane = threadIdx.x & 63;
    float sum = 0.0f;
    if constexpr (MF == 16) {
        frag8 fa[2][8], fb[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                fa[h][j] = __builtin_bit_cast(frag8, frags[(h * 12 + j) * 64 + lane]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fb[h][i] = __builtin_bit_cast(frag8, frags[(h * 12 + 8 + i) * 64 + lane]);
        }
        floatx4_t acc[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[i][j] = Elt::mfma16(fb[h][i], fa[h][j], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) sum += acc[i][j][e];
    } else {
        frag8 fa[4][4], fb[4][2];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fa[h][j] = __builtin_bit_cast(frag8, frags[(h * 6 + j) * 64 + lane]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fb[h][i] = __builtin_bit_cast(frag8, frags[(h * 6 + 4 + i) * 64 + lane]);
        }
        floatx16_t acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int h = 0; h < 4; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = Elt::mfma(fb[h][i], fa[h][j], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) sum += acc[i][j][e];
    }
    out[(int64_t)blockIdx.x * 512 + threadIdx.x] = sum;
}

// Reads memory with a grid-stride loop, the access pattern of a plain
// bandwidth test rather than of any GEMV here: a fixed grid of 256-thread
// workgroups, each pass reading 4 KB per workgroup per load slot with four
// non-temporal 16-byte loads per lane in flight, striding by the whole grid.
// Folded into one word per workgroup so that no load is dead.
__global__ __launch_bounds__(256) void stream_read_grid_kernel(const int4_t* buf, int64_t n16,
                                                               uint32_t* out) {
    int x = 0;
    const int64_t stride = (int64_t)gridDim.x * 1024;
    for (int64_t base = (int64_t)blockIdx.x * 1024; base < n16; base += stride) {
        int4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            v[u] = i < n16 ? __builtin_nontemporal_load(buf + i) : int4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
    __shared__ int wx[4];
    if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = (uint32_t)(wx[0] ^ wx[1] ^ wx[2] ^ wx[3]);
}

// Rows of row_bytes read in runs of RUN bytes: workgroup w reads band
// w % nbands (RUN bytes at RUN * band) of rows [chunk * rpw, +rpw), chunk =
// w / nbands; RUN / 16 lanes per row, 16 bytes each, 8 loads per lane in flight.
template <int RUN>
__global__ __launch_bounds__(256) void stream_read_runs_kernel(const char* buf, int64_t row_bytes,
                                                               int nbands, int rpw,
                                                               uint32_t* out) {
    constexpr int LPR = RUN / 16;       // lanes per row
    constexpr int RPI = 256 / LPR;      // rows per workgroup-wide load
    const int band = blockIdx.x % nbands;
    const int chunk = blockIdx.x / nbands;
    const int t = threadIdx.x;
    const char* p = buf + ((int64_t)chunk * rpw + t / LPR) * row_bytes + (int64_t)band * RUN +
                    (t % LPR) * 16;
    int x = 0;
    for (int i = 0; i < rpw; i += 8 * RPI) {
        int4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = __builtin_nontemporal_load(
                reinterpret_cast<const int4_t*>(p + (int64_t)(i + u * RPI) * row_bytes));
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
    __shared__ int wx[4];
    if ((t & 63) == 0) wx[t >> 6] = x;
    __syncthreads();
    if (t == 0) out[blockIdx.x] = (uint32_t)(wx[0] ^ wx[1] ^ wx[2] ^ wx[3]);
}

}  // namespace
}  // namespace sdt

extern "C" int gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                        const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    return sdt::gemm_impl<sdt::F16>(M, N, K, A, lda, B, ldb, C, ldc, stream, sdt::kAuto, true,
                                    nullptr, 0);
}

extern "C" int gemm_f16_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                           const void* B, int64_t ldb, void* C, int64_t ldc, void* workspace,
                           int64_t workspace_bytes, void* stream) {
    return sdt::gemm_impl<sdt::F16>(M, N, K, A, lda, B, ldb, C, ldc, stream, sdt::kAuto, true,
                                    workspace, workspace_bytes);
}

extern "C" int gemm_f16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                           const void* B, int64_t ldb, void* C, int64_t ldc, void* stream,
                           int tile_id, int stagger) {
    return sdt::gemm_impl<sdt::F16>(M, N, K, A, lda, B, ldb, C, ldc, stream,
                                    sdt_launch{tile_id, -1, -1, stagger, -1, -1, -1, -1}, false,
                                    nullptr, 0);
}

extern "C" int gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                         const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    return sdt::gemm_impl<sdt::BF16>(M, N, K, A, lda, B, ldb, C, ldc, stream, sdt::kAuto, true,
                                     nullptr, 0);
}

extern "C" int gemm_bf16_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            const void* B, int64_t ldb, void* C, int64_t ldc, void* workspace,
                            int64_t workspace_bytes, void* stream) {
    return sdt::gemm_impl<sdt::BF16>(M, N, K, A, lda, B, ldb, C, ldc, stream, sdt::kAuto, true,
                                     workspace, workspace_bytes);
}

extern "C" int gemm_bf16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            const void* B, int64_t ldb, void* C, int64_t ldc, void* stream,
                            int tile_id, int stagger) {
    return sdt::gemm_impl<sdt::BF16>(M, N, K, A, lda, B, ldb, C, ldc, stream,
                                     sdt_launch{tile_id, -1, -1, stagger, -1, -1, -1, -1}, false,
                                     nullptr, 0);
}

extern "C" int gemm_f16_cfg(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            const void* B, int64_t ldb, void* C, int64_t ldc, void* workspace,
                            int64_t workspace_bytes, void* stream, const sdt_launch* cfg) {
    if (!cfg) return SDT_ERR_INVALID_ARG;
    return sdt::gemm_impl<sdt::F16>(M, N, K, A, lda, B, ldb, C, ldc, stream, *cfg, false,
                                    workspace, workspace_bytes);
}

extern "C" int gemm_bf16_cfg(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             const void* B, int64_t ldb, void* C, int64_t ldc, void* workspace,
                             int64_t workspace_bytes, void* stream, const sdt_launch* cfg) {
    if (!cfg) return SDT_ERR_INVALID_ARG;
    return sdt::gemm_impl<sdt::BF16>(M, N, K, A, lda, B, ldb, C, ldc, stream, *cfg, false,
                                     workspace, workspace_bytes);
}

extern "C" int gemm_f16_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    int st = sdt::check_gemm_args(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SDT_OK) return st;
    if (!sdt::sizes_supported(M, N, K)) return SDT_ERR_UNSUPPORTED;   // as gemm_f16
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the plan gemm_f16_ws makes with a workspace as large as it asks for
    int64_t need = 0;
    if (!(M <= 1 || N == 0 || K == 0)) {
        sdt::DeviceInfo dev;
        st = sdt::device_info(&dev);
        if (st != SDT_OK) return st;
        need = sdt_gemm_workspace_size(M, N, K, dev.num_cu);
        if (need < 0) return SDT_ERR_UNSUPPORTED;
    }
    if (need > sdt::kScratchBytes) return SDT_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if (need > 0) {
        st = sdt::scratch_for_current_device(&ws, s);
        if (st != SDT_OK) return st;
    }
    return sdt::gemm_impl<sdt::F16>(M, N, K, A, lda, B, ldb, C, ldc, stream, sdt::kAuto, true, ws,
                                    need > 0 ? sdt::kScratchBytes : 0);
}

extern "C" int64_t sdt_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int num_cu) {
    if (M < 0 || N < 0 || K < 0 || !sdt::sizes_supported(M, N, K)) return -1;
    if (M <= 1 || N == 0 || K == 0) return 0;   // routed to the GEMV, a no-op or a fill
    if (num_cu <= 0) {
        sdt::DeviceInfo dev;
        if (sdt::device_info(&dev) != SDT_OK) return -1;
        num_cu = dev.num_cu;
    }
    sdt::Plan p;
    if (sdt::resolve_plan(sdt::kAuto, M, N, K, num_cu, INT64_MAX, &p) != SDT_OK) return -1;
    return sdt::workspace_bytes(p, M, N);
}

extern "C" int64_t sdt_launch_workspace_size(int64_t M, int64_t N, int64_t K,
                                             const sdt_launch* cfg) {
    if (!cfg || M < 0 || N < 0 || K < 0) return -1;
    sdt::Plan p;
    if (sdt::resolve_plan(*cfg, std::max<int64_t>(M, 1), std::max<int64_t>(N, 1), K, 256,
                          INT64_MAX, &p) != SDT_OK)
        return -1;
    return (M == 0 || N == 0) ? 0 : sdt::workspace_bytes(p, M, N);
}

extern "C" int sdt_workspace_init(void* workspace, int64_t bytes, void* stream) {
    if (bytes == 0) return SDT_OK;
    if (bytes < 0 || !workspace) return SDT_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0 || bytes % 4 != 0)
        return SDT_ERR_UNSUPPORTED;
    return sdt::fill_words(static_cast<uint32_t*>(workspace), bytes / 4,
                           static_cast<hipStream_t>(stream));
}

extern "C" int gemv_f16_m1(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                           void* y, void* stream) {
    int st = sdt::check_gemm_args(1, N, K, x, K, B, ldb, y, N);
    if (st != SDT_OK) return st;
    if (N == 0) return SDT_OK;
    return sdt::launch_gemv<sdt::F16>(0, N, K, x, B, ldb, y, static_cast<hipStream_t>(stream));
}

extern "C" int gemv_bf16_m1(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                            void* y, void* stream) {
    int st = sdt::check_gemm_args(1, N, K, x, K, B, ldb, y, N);
    if (st != SDT_OK) return st;
    if (N == 0) return SDT_OK;
    return sdt::launch_gemv<sdt::BF16>(0, N, K, x, B, ldb, y, static_cast<hipStream_t>(stream));
}

extern "C" int gemv_f16_m1_ex(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                              void* y, void* stream, int variant) {
    if (variant < 0 || variant >= sdt::kGemvVariants) return SDT_ERR_INVALID_ARG;
    int st = sdt::check_gemm_args(1, N, K, x, K, B, ldb, y, N);
    if (st != SDT_OK) return st;
    if (N == 0) return SDT_OK;
    return sdt::launch_gemv<sdt::F16>(variant, N, K, x, B, ldb, y,
                                      static_cast<hipStream_t>(stream));
}

extern "C" int sdt_gemv_num_variants(void) { return sdt::kGemvVariants; }

extern "C" int gemv_f16_m1_kn(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                              void* y, void* stream) {
    int st = sdt::check_gemv_kn_args(N, K, x, B, ldb, y);
    if (st != SDT_OK || N == 0) return st;
    return sdt::launch_gemv_kn<sdt::F16>(0, N, K, x, B, ldb, y,
                                         static_cast<hipStream_t>(stream));
}

extern "C" int gemv_bf16_m1_kn(int64_t N, int64_t K, const void* x, const void* B,
                               int64_t ldb, void* y, void* stream) {
    int st = sdt::check_gemv_kn_args(N, K, x, B, ldb, y);
    if (st != SDT_OK || N == 0) return st;
    return sdt::launch_gemv_kn<sdt::BF16>(0, N, K, x, B, ldb, y,
                                          static_cast<hipStream_t>(stream));
}

extern "C" int gemv_f16_m1_kn_ws(int64_t N, int64_t K, const void* x, const void* B,
                                 int64_t ldb, void* y, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
    return sdt::gemv_kn_ws_impl<sdt::F16>(N, K, x, B, ldb, y, workspace, workspace_bytes,
                                          stream);
}

extern "C" int gemv_bf16_m1_kn_ws(int64_t N, int64_t K, const void* x, const void* B,
                                  int64_t ldb, void* y, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
    return sdt::gemv_kn_ws_impl<sdt::BF16>(N, K, x, B, ldb, y, workspace, workspace_bytes,
                                           stream);
}

extern "C" int gemv_f16_m1_kn_ex(int64_t N, int64_t K, const void* x, const void* B,
                                 int64_t ldb, void* y, void* stream, int variant) {
    if (variant < 0 || variant >= sdt::kGemvKnVariants) return SDT_ERR_INVALID_ARG;
    int st = sdt::check_gemv_kn_args(N, K, x, B, ldb, y);
    if (st != SDT_OK || N == 0) return st;
    return sdt::launch_gemv_kn<sdt::F16>(variant, N, K, x, B, ldb, y,
                                         static_cast<hipStream_t>(stream));
}

extern "C" int sdt_gemv_kn_num_variants(void) { return sdt::kGemvKnVariants; }

extern "C" int sdt_pick_tile(int64_t M, int64_t N, int64_t K, int num_cu, sdt_tile* out) {
    if (M < 0 || N < 0 || K < 0 || !out) return SDT_ERR_INVALID_ARG;
    if (!sdt::sizes_supported(M, N, K)) return SDT_ERR_UNSUPPORTED;
    if (num_cu <= 0) {
        sdt::DeviceInfo dev;
        int st = sdt::device_info(&dev);
        if (st != SDT_OK) return st;
        num_cu = dev.num_cu;
    }
    const sdt::Plan p = sdt::plan_for(sdt::pick_tile(M, N, K, num_cu), M, N, K, num_cu);
    *out = sdt::describe(p);
    return SDT_OK;
}

extern "C" int sdt_pick_tile_ws(int64_t M, int64_t N, int64_t K, int num_cu,
                                int64_t workspace_bytes, sdt_tile* out) {
    if (M < 0 || N < 0 || K < 0 || workspace_bytes < 0 || !out) return SDT_ERR_INVALID_ARG;
    if (num_cu <= 0) {
        sdt::DeviceInfo dev;
        int st = sdt::device_info(&dev);
        if (st != SDT_OK) return st;
        num_cu = dev.num_cu;
    }
    sdt::Plan p;
    int st = sdt::resolve_plan(sdt::kAuto, std::max<int64_t>(M, 1), std::max<int64_t>(N, 1), K,
                               num_cu, workspace_bytes, &p);
    if (st != SDT_OK) return st;
    *out = sdt::describe(p);
    return SDT_OK;
}

extern "C" int sdt_last_hip_error(void) { return sdt::g_last_hip_error; }

extern "C" int sdt_stream_read(const void* buf, int64_t bytes, void* out, void* stream) {
    if (bytes == 0) return SDT_OK;
    if (bytes < 0 || !buf || !out) return SDT_ERR_INVALID_ARG;
    if (bytes % 8192 != 0 || bytes / 8192 > INT_MAX ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
        return SDT_ERR_UNSUPPORTED;
    const sdt::int4_t* b = static_cast<const sdt::int4_t*>(buf);
    uint32_t* o = static_cast<uint32_t*>(out);
    void* args[] = {&b, &o};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&sdt::stream_read_kernel),
                                   dim3((unsigned)(bytes / 8192)), dim3(64), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SDT_OK : sdt::fail_hip(e);
}

extern "C" int sdt_stream_read_grid(const void* buf, int64_t bytes, void* out, int workgroups,
                                    void* stream) {
    if (bytes == 0) return SDT_OK;
    if (bytes < 0 || !buf || !out || workgroups <= 0) return SDT_ERR_INVALID_ARG;
    if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(out) & 3) != 0)
        return SDT_ERR_UNSUPPORTED;
    const sdt::int4_t* b = static_cast<const sdt::int4_t*>(buf);
    int64_t n16 = bytes / 16;
    uint32_t* o = static_cast<uint32_t*>(out);
    void* args[] = {&b, &n16, &o};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&sdt::stream_read_grid_kernel),
                                   dim3((unsigned)workgroups), dim3(256), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SDT_OK : sdt::fail_hip(e);
}

extern "C" int sdt_stream_read_runs(const void* buf, int64_t rows, int64_t row_bytes,
                                    int run_bytes, int rows_per_wg, void* out, void* stream) {
    if (rows == 0) return SDT_OK;
    if (rows < 0 || row_bytes <= 0 || !buf || !out || rows_per_wg <= 0) return SDT_ERR_INVALID_ARG;
    if (run_bytes != 64 && run_bytes != 128 && run_bytes != 256 && run_bytes != 512 &&
        run_bytes != 1024)
        return SDT_ERR_INVALID_ARG;
    const int rpi = 4096 / run_bytes;   // rows per workgroup-wide load (256 lanes x 16 bytes)
    if (row_bytes % run_bytes != 0 || rows_per_wg % (8 * rpi) != 0 || rows % rows_per_wg != 0)
        return SDT_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
        return SDT_ERR_UNSUPPORTED;
    const int64_t nbands = row_bytes / run_bytes;
    const int64_t grid = nbands * (rows / rows_per_wg);
    if (grid > INT_MAX) return SDT_ERR_UNSUPPORTED;
    const char* b = static_cast<const char*>(buf);
    int nb = (int)nbands, rpw = rows_per_wg;
    uint32_t* o = static_cast<uint32_t*>(out);
    void* args[] = {&b, &row_bytes, &nb, &rpw, &o};
    const void* k;
    switch (run_bytes) {
        case 64: k = reinterpret_cast<const void*>(&sdt::stream_read_runs_kernel<64>); break;
        case 128: k = reinterpret_cast<const void*>(&sdt::stream_read_runs_kernel<128>); break;
        case 256: k = reinterpret_cast<const void*>(&sdt::stream_read_runs_kernel<256>); break;
        case 512: k = reinterpret_cast<const void*>(&sdt::stream_read_runs_kernel<512>); break;
        default: k = reinterpret_cast<const void*>(&sdt::stream_read_runs_kernel<1024>); break;
    }
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)grid), dim3(256), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SDT_OK : sdt::fail_hip(e);
}

extern "C" int sdt_mfma_ceiling(const void* frags, int iters, void* out, int workgroups,
                                int flags, void* stream) {
    if (!frags || !out || iters <= 0 || workgroups <= 0 || (flags & ~3) != 0)
        return SDT_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(frags) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
        return SDT_ERR_UNSUPPORTED;
    const sdt::int4_t* f = static_cast<const sdt::int4_t*>(frags);
    float* o = static_cast<float*>(out);
    void* args[] = {&f, &iters, &o};
    const void* k;
    switch (flags) {
        case 0: k = reinterpret_cast<const void*>(&sdt::mfma_ceiling_kernel<sdt::F16, 16>); break;
        case 1: k = reinterpret_cast<const void*>(&sdt::mfma_ceiling_kernel<sdt::BF16, 16>); break;
        case 2: k = reinterpret_cast<const void*>(&sdt::mfma_ceiling_kernel<sdt::F16, 32>); break;
        default: k = reinterpret_cast<const void*>(&sdt::mfma_ceiling_kernel<sdt::BF16, 32>); break;
    }
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)workgroups), dim3(512), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SDT_OK : sdt::fail_hip(e);
}

extern "C" int sdt_empty_kernel(void* stream) {
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&sdt::empty_kernel), dim3(1),
                                   dim3(64), nullptr, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SDT_OK : sdt::fail_hip(e);
}
