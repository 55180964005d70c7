// Drives libsdt.so through its C ABI alone (include/sdt.h): device buffers
// from hipMalloc, no Python and no torch.  Every product is checked against
// the CPU oracle (libsdt_oracle.so, test infrastructure) on inputs generated
// here, and the error paths return their documented statuses.
//
// Build: __graft_entry__.build() (hipcc, host code only).  Run: the GPU test
// tests/test_gpu_capi.py.  Prints "CAPI OK" and exits 0 when every check
// passes; otherwise names the failing check and exits 1.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "sdt.h"

// The oracle's C entry points (its own source declares them; it shares no
// header with the library).
extern "C" {
uint16_t sdt_oracle_f16_encode_rne(double x);
double sdt_oracle_f16_decode(uint16_t h);
uint16_t sdt_oracle_bf16_encode_rne(double x);
double sdt_oracle_bf16_decode(uint16_t h);
int sdt_oracle_gemm_t(int dtype, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                      const uint16_t* B, int64_t ldb, double* C, int64_t ldc, int threads);
int sdt_oracle_gemv_m1_t(int dtype, int64_t N, int64_t K, const uint16_t* x, const uint16_t* B,
                         int64_t ldb, double* y, int threads);
int sdt_oracle_gemv_kn_t(int dtype, int64_t N, int64_t K, const uint16_t* x, const uint16_t* B,
                         int64_t ldb, double* y, int threads);
}

static int g_fail = 0;

#define CHECK(cond, ...)                                          \
    do {                                                          \
        if (!(cond)) {                                            \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);      \
            std::printf(__VA_ARGS__);                             \
            std::printf("\n");                                    \
            g_fail = 1;                                           \
        }                                                         \
    } while (0)

#define HIP_OK(x) CHECK((x) == hipSuccess, "%s", #x)

// splitmix64: a seeded stream of 64-bit values.
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

// Values k/1024 with |k| <= 1000: exact in both binary16 and, rounded by the
// oracle's encoder, in bfloat16.
static std::vector<uint16_t> draw(size_t n, uint64_t seed, int dtype) {
    Rng r{seed};
    std::vector<uint16_t> v(n);
    for (size_t i = 0; i < n; ++i) {
        const double x = ((int)(r.next() % 2001) - 1000) / 1024.0;
        v[i] = dtype == 1 ? sdt_oracle_bf16_encode_rne(x) : sdt_oracle_f16_encode_rne(x);
    }
    return v;
}

static double decode(uint16_t h, int dtype) {
    return dtype == 1 ? sdt_oracle_bf16_decode(h) : sdt_oracle_f16_decode(h);
}

// |got - ref| <= 1e-2 + rel * |ref|, rel = 2e-3 (fp16 output) or
// 2e-3 - 2^-11 + 2^-8 (bfloat16 output).
static int count_bad(const std::vector<uint16_t>& got, const std::vector<double>& ref, int dtype) {
    const double rel = dtype == 1 ? 2e-3 - std::ldexp(1.0, -11) + std::ldexp(1.0, -8) : 2e-3;
    int bad = 0;
    for (size_t i = 0; i < ref.size(); ++i) {
        const double g = decode(got[i], dtype);
        if (!(std::fabs(g - ref[i]) <= 1e-2 + rel * std::fabs(ref[i]))) ++bad;
    }
    return bad;
}

static void* dev_copy(const std::vector<uint16_t>& h) {
    void* p = nullptr;
    HIP_OK(hipMalloc(&p, h.size() * 2 + 16));
    HIP_OK(hipMemcpy(p, h.data(), h.size() * 2, hipMemcpyHostToDevice));
    return p;
}

static std::vector<uint16_t> host_copy(const void* p, size_t n) {
    std::vector<uint16_t> h(n);
    HIP_OK(hipMemcpy(h.data(), p, n * 2, hipMemcpyDeviceToHost));
    return h;
}

// C = A.B on a ragged shape with padded strides, on an explicit stream;
// use_ws: through the workspace entry point, with the workspace the library
// asks for (hipMalloc, counters zeroed by sdt_workspace_init).
static void check_gemm(int dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                       bool use_ws = false) {
    const int64_t lda = (K + 7) / 8 * 8 + 8, ldb = (K + 7) / 8 * 8 + 16, ldc = (N + 7) / 8 * 8;
    std::vector<uint16_t> A = draw((size_t)(M * lda), 11 + dtype, dtype);
    std::vector<uint16_t> B = draw((size_t)(N * ldb), 12 + dtype, dtype);
    void* dA = dev_copy(A);
    void* dB = dev_copy(B);
    void* dC = nullptr;
    HIP_OK(hipMalloc(&dC, (size_t)(M * ldc) * 2));
    void* ws = nullptr;
    int64_t ws_bytes = 0;
    if (use_ws) {
        ws_bytes = sdt_gemm_workspace_size(M, N, K, 0);
        CHECK(ws_bytes > 0, "%lldx%lldx%lld: no k-split planned", (long long)M, (long long)N,
              (long long)K);
        if (ws_bytes > 0) {
            HIP_OK(hipMalloc(&ws, (size_t)ws_bytes));
            CHECK(sdt_workspace_init(ws, ws_bytes, stream) == SDT_OK, "workspace init");
        }
    }
    int rc;
    if (use_ws)
        rc = dtype == 1 ? gemm_bf16_ws(M, N, K, dA, lda, dB, ldb, dC, ldc, ws, ws_bytes, stream)
                        : gemm_f16_ws(M, N, K, dA, lda, dB, ldb, dC, ldc, ws, ws_bytes, stream);
    else
        rc = dtype == 1 ? gemm_bf16(M, N, K, dA, lda, dB, ldb, dC, ldc, stream)
                        : gemm_f16(M, N, K, dA, lda, dB, ldb, dC, ldc, stream);
    CHECK(rc == SDT_OK, "gemm dtype %d %lldx%lldx%lld: %s", dtype, (long long)M, (long long)N,
          (long long)K, sdt_status_string(rc));
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<uint16_t> Cf = host_copy(dC, (size_t)(M * ldc));
    std::vector<uint16_t> C((size_t)(M * N));
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) C[(size_t)(m * N + n)] = Cf[(size_t)(m * ldc + n)];
    std::vector<double> ref((size_t)(M * N));
    CHECK(sdt_oracle_gemm_t(dtype, M, N, K, A.data(), lda, B.data(), ldb, ref.data(), N, 0) == 0,
          "oracle gemm");
    const int bad = count_bad(C, ref, dtype);
    CHECK(bad == 0, "gemm dtype %d %lldx%lldx%lld: %d elements outside tolerance", dtype,
          (long long)M, (long long)N, (long long)K, bad);
    HIP_OK(hipFree(dA));
    HIP_OK(hipFree(dB));
    HIP_OK(hipFree(dC));
    if (ws) HIP_OK(hipFree(ws));
}

static void check_gemv(int dtype, bool kn, int64_t N, int64_t K, bool split = false) {
    const int64_t ldb = kn ? (N + 7) / 8 * 8 : (K + 7) / 8 * 8;
    std::vector<uint16_t> x = draw((size_t)K, 21 + dtype, dtype);
    std::vector<uint16_t> B = draw((size_t)((kn ? K : N) * ldb), 22 + dtype, dtype);
    void* dx = dev_copy(x);
    void* dB = dev_copy(B);
    void* dy = nullptr;
    HIP_OK(hipMalloc(&dy, (size_t)N * 2));
    void* ws = nullptr;
    const int64_t ws_bytes = split ? sdt_gemv_kn_workspace_size(N, K) : 0;
    if (split) {
        CHECK(ws_bytes > 0, "[K][N] N=%lld K=%lld: no split planned", (long long)N, (long long)K);
        HIP_OK(hipMalloc(&ws, (size_t)ws_bytes));   // needs no initialisation
    }
    int rc;
    if (kn && split)
        rc = dtype == 1 ? gemv_bf16_m1_kn_ws(N, K, dx, dB, ldb, dy, ws, ws_bytes, nullptr)
                        : gemv_f16_m1_kn_ws(N, K, dx, dB, ldb, dy, ws, ws_bytes, nullptr);
    else if (kn)
        rc = dtype == 1 ? gemv_bf16_m1_kn(N, K, dx, dB, ldb, dy, nullptr)
                        : gemv_f16_m1_kn(N, K, dx, dB, ldb, dy, nullptr);
    else
        rc = dtype == 1 ? gemv_bf16_m1(N, K, dx, dB, ldb, dy, nullptr)
                        : gemv_f16_m1(N, K, dx, dB, ldb, dy, nullptr);
    CHECK(rc == SDT_OK, "gemv dtype %d kn %d: %s", dtype, (int)kn, sdt_status_string(rc));
    HIP_OK(hipDeviceSynchronize());
    std::vector<uint16_t> y = host_copy(dy, (size_t)N);
    std::vector<double> ref((size_t)N);
    const int orc = kn ? sdt_oracle_gemv_kn_t(dtype, N, K, x.data(), B.data(), ldb, ref.data(), 0)
                       : sdt_oracle_gemv_m1_t(dtype, N, K, x.data(), B.data(), ldb, ref.data(), 0);
    CHECK(orc == 0, "oracle gemv");
    const int bad = count_bad(y, ref, dtype);
    CHECK(bad == 0, "gemv dtype %d kn %d N=%lld K=%lld: %d outside tolerance", dtype, (int)kn,
          (long long)N, (long long)K, bad);
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dB));
    HIP_OK(hipFree(dy));
    if (ws) HIP_OK(hipFree(ws));
}

int main() {
    int dev = 0;
    HIP_OK(hipGetDevice(&dev));
    sdt_tile t;
    CHECK(sdt_pick_tile(1024, 1024, 1024, 0, &t) == SDT_OK, "pick_tile on the current device");
    std::printf("device %d: 1024^3 runs rung %d (%dx%d, %d stages, %d k-groups)\n", dev, t.id, t.bm,
                t.bn, t.stages, t.kgroups);

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    for (int dtype = 0; dtype < 2; ++dtype) {
        check_gemm(dtype, 300, 260, 1000, s);     // several tiles, ragged edges, partial k-tile
        check_gemm(dtype, 1024, 1024, 1024, s);   // two k-groups of waves
        check_gemm(dtype, 1, 500, 777 / 8 * 8, s);   // M = 1 -> the streaming GEMV
        check_gemm(dtype, 300, 260, 8200, s, true);   // K split across workgroups (ragged)
        check_gemm(dtype, 256, 256, 16384, s, true);
        check_gemv(dtype, false, 12288, 4096);
        check_gemv(dtype, true, 12288, 4096);
        check_gemv(dtype, true, 1001, 1003);
        check_gemv(dtype, true, 12288, 4096, true);   // [K][N] split over K (workspace)
        check_gemv(dtype, true, 1001, 1003, true);
    }

    // error paths: nothing is launched, the status names the cause
    void* buf = nullptr;
    HIP_OK(hipMalloc(&buf, 1 << 20));
    char* b = static_cast<char*>(buf);
    CHECK(gemm_f16(64, 64, 64, nullptr, 64, b, 64, b + 65536, 64, nullptr) == SDT_ERR_INVALID_ARG,
          "null A");
    CHECK(gemm_f16(64, 64, 64, b + 2, 64, b + 8192, 64, b + 65536, 64, nullptr) ==
              SDT_ERR_UNSUPPORTED, "misaligned A");
    CHECK(gemm_f16(64, 64, 64, b, 60, b + 8192, 64, b + 65536, 64, nullptr) == SDT_ERR_INVALID_ARG,
          "lda < K");
    sdt_launch cfg = {0, 5, -1, -1, -1, -1, -1, -1};
    CHECK(gemm_f16_cfg(64, 64, 64, b, 64, b + 8192, 64, b + 65536, 64, nullptr, 0, nullptr,
                       &cfg) == SDT_ERR_INVALID_ARG, "stage count without a kernel");
    CHECK(sdt_abi_version() == SDT_ABI_VERSION, "ABI version %d, header %d", sdt_abi_version(),
          SDT_ABI_VERSION);
    // K = 0 writes zeros (the empty sum)
    HIP_OK(hipMemset(b + 65536, 0x55, 64 * 64 * 2));
    CHECK(gemm_f16(64, 64, 0, nullptr, 0, nullptr, 0, b + 65536, 64, nullptr) == SDT_OK, "K = 0");
    HIP_OK(hipDeviceSynchronize());
    std::vector<uint16_t> z = host_copy(b + 65536, 64 * 64);
    int nz = 0;
    for (uint16_t v : z) nz += v != 0;
    CHECK(nz == 0, "K = 0 left %d nonzero outputs", nz);
    HIP_OK(hipFree(buf));
    HIP_OK(hipStreamDestroy(s));

    if (g_fail) return 1;
    std::printf("CAPI OK\n");
    return 0;
}
