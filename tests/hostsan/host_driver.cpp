// Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer: the
// launcher's planning (launcher.cpp, no HIP) over a grid of shapes, forced
// configurations and device sizes, including the extremes of the argument
// ranges, and the CPU oracle (oracle/sdt_oracle.c) on small and degenerate
// products.  Built and run by tests/test_host_sanitizers.py with g++/gcc; any
// sanitizer report makes the run fail.  Prints a checksum of every decision so
// the run cannot be optimised away.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "launcher.hpp"
#include "sdt.h"

extern "C" {
int sdt_oracle_gemm_t(int dtype, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                      const uint16_t* B, int64_t ldb, double* C, int64_t ldc, int threads);
int sdt_oracle_gemv_m1_t(int dtype, int64_t N, int64_t K, const uint16_t* x, const uint16_t* B,
                         int64_t ldb, double* y, int threads);
int sdt_oracle_gemv_kn_t(int dtype, int64_t N, int64_t K, const uint16_t* x, const uint16_t* B,
                         int64_t ldb, double* y, int threads);
uint16_t sdt_oracle_f16_encode_rne(double x);
double sdt_oracle_f16_decode(uint16_t h);
}

static uint64_t mix(uint64_t h, int64_t v) { return (h ^ (uint64_t)v) * 0x100000001b3ull; }

int main() {
    uint64_t h = 0xcbf29ce484222325ull;
    const int64_t dims[] = {0, 1, 7, 63, 64, 65, 96, 100, 255, 256, 1000, 1536, 2048, 2560,
                            3072, 4096, 8192, 12288, 65536, 1 << 20, INT32_MAX, int64_t(1) << 33};
    const int cus[] = {1, 32, 80, 256, 304};
    int plans = 0;
    for (int64_t M : dims)
        for (int64_t N : dims)
            for (int64_t K : {int64_t(0), int64_t(1), int64_t(64), int64_t(1000), int64_t(4096),
                              int64_t(16384), int64_t(1) << 20, int64_t(INT32_MAX)})
                for (int cu : cus) {
                    if (!sdt::sizes_supported(M, N, K)) {   // refused before any planning
                        sdt::Plan out;
                        sdt_launch cfg = {-1, -1, -1, -1, -1, -1, -1, -1};
                        h = mix(h, sdt::resolve_plan(cfg, M, N, K, cu, 1 << 20, &out));
                        h = mix(h, sdt_pick_rung(M, N, 64, 64, 1, &M));
                        continue;
                    }
                    const int id = sdt::pick_tile(M, N, K, cu);
                    h = mix(h, id);
                    const sdt::Plan p = sdt::plan_for(id, M, N, K, cu);
                    h = mix(mix(mix(h, p.stages), p.kgroups), p.stagger);
                    h = mix(h, sdt::check_plan(p, K));
                    for (int64_t ws : {int64_t(-1), int64_t(0), int64_t(1) << 20, int64_t(1) << 40}) {
                        sdt_launch cfg = {-1, -1, -1, -1, -1, -1, -1, -1};
                        sdt::Plan out;
                        const int st = sdt::resolve_plan(cfg, M, N, K, cu, ws, &out);
                        h = mix(mix(h, st), st == SDT_OK ? out.splits : -7);
                        if (st == SDT_OK) h = mix(h, sdt::workspace_bytes(out, M, N));
                    }
                    ++plans;
                }
    // forced configurations on one shape: every field over its range and past it
    for (int tile = -2; tile <= sdt::kNumTiles; ++tile)
        for (int stages = -2; stages <= 5; ++stages)
            for (int kg = -1; kg <= 3; ++kg)
                for (int splits : {-1, 0, 1, 2, 16, 17, 64, 65})
                    for (int algo = -1; algo <= 2; ++algo)
                        for (int pers : {-1, 0, 1, 1000}) {
                            sdt_launch cfg = {tile, stages, kg, -1, splits, algo, pers, -1};
                            sdt::Plan out;
                            h = mix(h, sdt::resolve_plan(cfg, 1000, 1000, 4160, 256, int64_t(1) << 30,
                                                         &out));
                        }
    for (int64_t N : {int64_t(-1), int64_t(0), int64_t(1), int64_t(12288), int64_t(INT32_MAX),
                      int64_t(1) << 31})
        for (int64_t K : {int64_t(-1), int64_t(0), int64_t(15), int64_t(16), int64_t(4096),
                          int64_t(INT32_MAX / 2), int64_t(INT32_MAX)}) {
            h = mix(h, sdt_gemv_kn_workspace_size(N, K));
            h = mix(h, sdt_check_gemv_kn_args(N, K, (void*)0x1000, (void*)0x2000, N + 8,
                                              (void*)0x3000));
        }
    for (int64_t K : {int64_t(0), int64_t(64), int64_t(128), int64_t(4096), int64_t(4160)})
        for (int64_t wg = 0; wg < 5; ++wg) h = mix(h, sdt_stagger_ktile(wg, 3, K / 64));
    for (int s = -1; s <= 4; ++s) h = mix(h, (int64_t)sdt_status_string(s)[0]);

    // the oracle on small and degenerate products (fp16 and bf16 tables)
    std::vector<uint16_t> A(64 * 40), B(48 * 40), x(40);
    for (size_t i = 0; i < A.size(); ++i) A[i] = sdt_oracle_f16_encode_rne(((int)(i % 7) - 3) * 0.25);
    for (size_t i = 0; i < B.size(); ++i) B[i] = sdt_oracle_f16_encode_rne(((int)(i % 5) - 2) * 0.5);
    for (size_t i = 0; i < x.size(); ++i) x[i] = sdt_oracle_f16_encode_rne(((int)(i % 3) - 1) * 1.0);
    std::vector<double> C(64 * 48), y(64);
    for (int dtype = 0; dtype < 2; ++dtype) {
        h = mix(h, sdt_oracle_gemm_t(dtype, 64, 48, 40, A.data(), 40, B.data(), 40, C.data(), 48, 2));
        h = mix(h, (int64_t)(C[5 * 48 + 7] * 1024));
        h = mix(h, sdt_oracle_gemm_t(dtype, 64, 48, 0, A.data(), 40, B.data(), 40, C.data(), 48, 1));
        h = mix(h, sdt_oracle_gemm_t(dtype, 0, 0, 40, A.data(), 40, B.data(), 40, C.data(), 48, 1));
        h = mix(h, sdt_oracle_gemm_t(dtype, 64, 48, 40, A.data(), 39, B.data(), 40, C.data(), 48, 1));
        h = mix(h, sdt_oracle_gemv_m1_t(dtype, 48, 40, x.data(), B.data(), 40, y.data(), 2));
        h = mix(h, sdt_oracle_gemv_kn_t(dtype, 48, 40, x.data(), B.data(), 48, y.data(), 2));
    }
    for (double v : {0.0, -0.0, 1.0, 65504.0, 65520.0, 1e-8, 5.9604644775390625e-8, -1e9})
        h = mix(h, sdt_oracle_f16_encode_rne(v) ^ (uint16_t)(sdt_oracle_f16_decode(
                       sdt_oracle_f16_encode_rne(v)) == v));
    std::printf("host planning and oracle: %d shape plans, checksum %016llx\n", plans,
                (unsigned long long)h);
    return 0;
}
