// gfx950 M=1 decode GEMV: y(n) = sum_k x(k) * B[n*ldb + k], fp32 accumulation,
// fp16 (round-to-nearest-even) output.
//
// The mojo-baro page ("Four rounds on the decode shape") finds this shape
// bound by how well the weight stream is coalesced (v1), by bandwidth
// efficiency rather than byte count (v2), helped by wide vector loads of
// contiguous data per thread (v3) and by a kernel specialised for one row of
// activations instead of staging eight (v4).  Here the weights are K-major,
// so each output column is one contiguous run of K fp16:
//   * one wave owns RPW consecutive columns (one, by default: 12288 waves
//     for the decode shape, every one streaming 8 KB); for each column its 64
//     lanes issue 16-byte loads at consecutive addresses (1 KB per
//     instruction), all RPW * XCH loads of a pass in flight before any
//     arithmetic;
//   * a pass that lies wholly below K (uniform across the wave) uses plain
//     loads with no per-lane bounds test -- a per-chunk test is a divergent
//     branch around every load and cost about a tenth of the bandwidth --
//     and only a ragged last pass masks element by element;
//   * the activations stay in registers (XCH chunks of 8 per lane, i.e. K up
//     to XCH * 512 per pass);
//   * products go through v_dot2_f32_f16 into fp32; one cross-lane reduction
//     per column at the end; nothing is staged in LDS.
// Weight loads are non-temporal: every byte is used once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace sdt {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct GemvParams {
    const uint16_t* x;
    const uint16_t* B;
    uint16_t* y;
    int64_t ldb;
    int N, K;
};

// Eight fp16 starting at element k of a row holding K valid elements, with
// nothing past K read.
__device__ __forceinline__ int4_t gemv_chunk(const uint16_t* row, int k, int K, bool nt) {
    if (k + 8 <= K) {
        const int4_t* p = reinterpret_cast<const int4_t*>(row + k);
        return nt ? __builtin_nontemporal_load(p) : *p;
    }
    int4_t v = {0, 0, 0, 0};
    if (k < K) {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (k + e < K) ? row[k + e] : (uint16_t)0;
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = (int)((uint32_t)h[2 * d] | ((uint32_t)h[2 * d + 1] << 16));
    }
    return v;
}

// Four v_dot2_f32_f16 over one 16-byte chunk of weights and activations.
// The chunks are reinterpreted whole and then indexed: reinterpreting a
// single element of an int vector with __builtin_bit_cast is lowered by this
// compiler as if it were always element 0.
__device__ __forceinline__ float dot8(int4_t w, int4_t x, float acc) {
    const half8_t wh = __builtin_bit_cast(half8_t, w);
    const half8_t xh = __builtin_bit_cast(half8_t, x);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const half2_t a = {wh[2 * d], wh[2 * d + 1]};
        const half2_t b = {xh[2 * d], xh[2 * d + 1]};
        acc = __builtin_amdgcn_fdot2(a, b, acc, false);
    }
    return acc;
}

template <int RPW, int XCH>
__global__ __launch_bounds__(256) void gemv_f16_m1_kernel(GemvParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n0 = wave * RPW;
    if (n0 >= p.N) return;   // whole wave leaves together
    constexpr int KP = XCH * 512;

    float acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;

    for (int kb = 0; kb < p.K; kb += KP) {
        int4_t xr[XCH];
        int4_t wv[RPW][XCH];
        if (kb + KP <= p.K) {
            // the whole pass lies below K (uniform across the wave): plain
            // 16-byte loads, activations first (cached), then the weights
#pragma unroll
            for (int j = 0; j < XCH; ++j)
                xr[j] = *reinterpret_cast<const int4_t*>(p.x + kb + (lane + 64 * j) * 8);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int64_t n = min(n0 + r, (int64_t)p.N - 1);   // clamped rows are discarded
                const uint16_t* row = p.B + n * p.ldb + kb;
#pragma unroll
                for (int j = 0; j < XCH; ++j)
                    wv[r][j] = __builtin_nontemporal_load(
                        reinterpret_cast<const int4_t*>(row + (lane + 64 * j) * 8));
            }
        } else {
            // the ragged last pass: element-exact masking, nothing past K read
#pragma unroll
            for (int j = 0; j < XCH; ++j) xr[j] = gemv_chunk(p.x, kb + (lane + 64 * j) * 8, p.K, false);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int64_t n = min(n0 + r, (int64_t)p.N - 1);
                const uint16_t* row = p.B + n * p.ldb;
#pragma unroll
                for (int j = 0; j < XCH; ++j)
                    wv[r][j] = gemv_chunk(row, kb + (lane + 64 * j) * 8, p.K, true);
            }
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int j = 0; j < XCH; ++j) acc[r] = dot8(wv[r][j], xr[j], acc[r]);
    }

#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        float v = acc[r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0 && n0 + r < p.N) {
            const _Float16 h = (_Float16)v;
            p.y[n0 + r] = __builtin_bit_cast(uint16_t, h);
        }
    }
}

}  // namespace sdt
