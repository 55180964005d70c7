// gfx950 M=1 decode GEMV: y(n) = sum_k x(k) * B[n*ldb + k] for fp16 or bf16
// operands, fp32 accumulation, output in the operand type (round-to-nearest-
// even).
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
//     instruction); a pass's weight loads go out first and the activation
//     loads interleave with them, all in flight before any arithmetic;
//   * the kernel stays at 64 VGPRs, so 8 waves per SIMD are resident: the
//     streaming rate follows the bytes in flight per CU (at 85 VGPRs, 5 waves
//     per SIMD, the decode shape took 16.4 us, at 64 15.8 us); more bytes per
//     wave do not help (two columns per wave 17.8 us);
//   * a pass that lies wholly below K (uniform across the wave) uses plain
//     loads with no per-lane bounds test -- a per-chunk test is a divergent
//     branch around every load and cost about a tenth of the bandwidth --
//     and only a ragged last pass masks element by element;
//   * the activations stay in registers (XCH chunks of 8 per lane, i.e. K up
//     to XCH * 512 per pass);
//   * products go through v_dot2_f32_f16 (v_dot2_f32_bf16) into fp32; one
//     cross-lane reduction per column at the end; nothing is staged in LDS.
// Weight loads are non-temporal: every byte is used once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace sdt {

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

// Four two-term dot products over one 16-byte chunk of weights and
// activations.  The chunks are reinterpreted whole and then indexed:
// reinterpreting a single element of an int vector with __builtin_bit_cast
// is lowered by this compiler as if it were always element 0.
template <typename Elt>
__device__ __forceinline__ float dot8(int4_t w, int4_t x, float acc) {
    typedef typename Elt::frag8 frag8;
    typedef typename Elt::vec2 vec2;
    const frag8 wh = __builtin_bit_cast(frag8, w);
    const frag8 xh = __builtin_bit_cast(frag8, x);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const vec2 a = {wh[2 * d], wh[2 * d + 1]};
        const vec2 b = {xh[2 * d], xh[2 * d + 1]};
        acc = Elt::dot2(a, b, acc);
    }
    return acc;
}

// TAIL = false: K is a multiple of XCH * 512 (no ragged pass is compiled in,
// which keeps the kernel at 64 VGPRs, 8 waves per SIMD).  WPB waves per
// workgroup: one-wave workgroups streamed the decode shape 0.6% faster than
// four-wave ones (15.85 vs 15.94 us, same box), two and eight slower.
template <typename Elt, int RPW, int XCH, bool TAIL, int WPB>
__global__ __launch_bounds__(WPB * 64) void gemv_m1_kernel(GemvParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    // Waves past N (the last workgroup's, when N is not a multiple of WPB RPW)
    // run on the clamped last row and store nothing: no early exit, whose
    // test would have the wave load N and branch before it loads the rest of
    // its arguments.
    const int64_t n0 = wave * RPW;
    constexpr int KP = XCH * 512;

    float acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;

    // Whole passes (uniform across the wave): plain 16-byte loads, the weights
    // first, then the activations (L2 hits).  The ragged last pass is a
    // separate block after this loop, compiled only with TAIL: inside the
    // loop it kept every one of a pass's loads live at once (85 VGPRs, 5
    // waves per SIMD) and the decode shape took 16.4-16.9 us; without it the
    // loop interleaves loads and dot products in fewer registers, 8 waves per
    // SIMD stay resident, and it takes 15.8 us.
    auto pass = [&](int kb) {
        int4_t xr[XCH];
        int4_t wv[RPW][XCH];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int64_t n = min(n0 + r, (int64_t)p.N - 1);   // clamped rows are discarded
            const uint16_t* row = p.B + n * p.ldb + kb;
#pragma unroll
            for (int j = 0; j < XCH; ++j) {
                wv[r][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const int4_t*>(row + (lane + 64 * j) * 8));
                // The first weight load goes out before anything else; the
                // rest interleave with the activation loads as the scheduler
                // places them.  Decode shape: every weight load first 16.4-16.6
                // us, an activation load first 15.9-16.0 us, this 15.8-15.9 us.
                if (r == 0 && j == 0) __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < XCH; ++j)
            xr[j] = *reinterpret_cast<const int4_t*>(p.x + kb + (lane + 64 * j) * 8);
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int j = 0; j < XCH; ++j) acc[r] = dot8<Elt>(wv[r][j], xr[j], acc[r]);
    };
    int kb = 0;
    if constexpr (!TAIL) {
        // K is a positive multiple of KP: at least one pass, and no test of K
        // ahead of the first loads
        do {
            pass(kb);
            kb += KP;
        } while (kb < p.K);
    } else {
        for (; kb + KP <= p.K; kb += KP) pass(kb);
    }
    if (TAIL && kb < p.K) {
        // the ragged last pass: element-exact masking, nothing past K read
        int4_t xr[XCH];
#pragma unroll
        for (int j = 0; j < XCH; ++j) xr[j] = gemv_chunk(p.x, kb + (lane + 64 * j) * 8, p.K, false);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int64_t n = min(n0 + r, (int64_t)p.N - 1);
            const uint16_t* row = p.B + n * p.ldb;
#pragma unroll
            for (int j = 0; j < XCH; ++j)
                acc[r] = dot8<Elt>(gemv_chunk(row, kb + (lane + 64 * j) * 8, p.K, true), xr[j], acc[r]);
        }
    }

#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        float v = acc[r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0 && n0 + r < p.N) {
            const typename Elt::scalar h = (typename Elt::scalar)v;
            p.y[n0 + r] = __builtin_bit_cast(uint16_t, h);
        }
    }
}

// One output column per workgroup of WPC waves.  The column's 512-element
// chunks (64 lanes x 8 fp16, 1 KB) are dealt round-robin over the waves, wave
// q taking chunks q, q + WPC, ..., XCH of them in flight per trip; each wave
// adds its chunks per lane, reduces across its lanes, and the WPC wave sums
// are added in wave order through LDS (a fixed order: deterministic).  On
// the decode shape (K = 4096) a workgroup of 4 waves reads its column's 8 KB
// as 2 KB per wave, two 16-byte loads per lane: measured against one wave
// per column (8 KB, eight loads per lane), 15.55-15.62 against 15.73-15.85 us
// on one box (cold, 8 rotating buffers), the finer workgroups keeping more
// CUs streaming while the last columns drain.
template <typename Elt, int WPC, int XCH>
__global__ __launch_bounds__(WPC * 64) void gemv_m1_wsplit_kernel(GemvParams p) {
    const int lane = threadIdx.x & 63;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n = blockIdx.x;
    const uint16_t* row = p.B + n * p.ldb;
    const int nch = p.K >> 9;                 // full chunks
    float acc = 0.0f;
    for (int c0 = q; c0 < nch; c0 += WPC * XCH) {
        int4_t w[XCH], xr[XCH];
        if (c0 + (XCH - 1) * WPC < nch) {     // a whole trip (uniform): plain loads
#pragma unroll
            for (int j = 0; j < XCH; ++j)
                w[j] = __builtin_nontemporal_load(
                    reinterpret_cast<const int4_t*>(row + (c0 + j * WPC) * 512 + lane * 8));
#pragma unroll
            for (int j = 0; j < XCH; ++j)
                xr[j] = *reinterpret_cast<const int4_t*>(p.x + (c0 + j * WPC) * 512 + lane * 8);
            // every load of the trip in flight before the first product: left
            // to itself the scheduler issued an activation load after the
            // first dot product's wait, a second memory round trip per column
            // (17.9 against 15.6 us on the decode shape)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < XCH; ++j) acc = dot8<Elt>(w[j], xr[j], acc);
        } else {
            for (int c = c0; c < nch; c += WPC)
                acc = dot8<Elt>(__builtin_nontemporal_load(
                                    reinterpret_cast<const int4_t*>(row + c * 512 + lane * 8)),
                                *reinterpret_cast<const int4_t*>(p.x + c * 512 + lane * 8), acc);
        }
    }
    if ((p.K & 511) && q == nch % WPC) {     // the ragged last chunk, element-exact
        const int k = nch * 512 + lane * 8;
        acc = dot8<Elt>(gemv_chunk(row, k, p.K, true), gemv_chunk(p.x, k, p.K, false), acc);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    __shared__ float part[WPC];
    if (lane == 0) part[q] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = part[0];
#pragma unroll
        for (int r = 1; r < WPC; ++r) v += part[r];
        const typename Elt::scalar h = (typename Elt::scalar)v;
        p.y[n] = __builtin_bit_cast(uint16_t, h);
    }
}

// ---- the same product with the weights as K rows of N ("B-layout") ---------
//
// y(n) = sum_k x(k) * B[k*ldb + n].  This is the layout the mojo-baro page
// reaches by transposing the weights at load (rounds v1-v3 of "Four rounds on
// the decode shape"), where each thread owns CPT contiguous columns so that
// its loads are wide vectors, CPT = 8 measuring best.  On MI355X:
//   * a lane owns 8 contiguous columns (one 16-byte load per weight row) and
//     SEG lanes side by side cover one SEG*8-column band, SEG*16 contiguous
//     bytes of every row; a workgroup owns one band;
//   * a band alone is too little work for a CU, so the workgroup splits K:
//     its lanes form RG row groups, and group g takes the blocks of eight
//     consecutive rows b = g, g + RG, g + 2*RG, ...; one 16-byte load gives
//     the eight activations of a block, eight loads its weights;
//   * two blocks per trip keep 18 loads per lane in flight;
//   * the RG partial sums of each column are combined in LDS in a fixed order
//     (RG/PARTS groups per partial, then the PARTS partials), so the result
//     is deterministic and needs no workspace and no second launch;
//   * only a ragged last band (N not a multiple of the band) takes the
//     element-masked loads, and a ragged last block of rows (K not a multiple
//     of 8) is taken by one row group with masking.

struct GemvKnParams {
    const uint16_t* x;
    const uint16_t* B;
    uint16_t* y;
    int64_t ldb;
    int N, K;
    // K split over workgroups (gemv_kn_kernel with SPLIT): workgroup
    // (band, blockIdx.y) sums rows [blockIdx.y * kc, +kc) (kc a multiple of 8)
    // into part[blockIdx.y * pstride + n] (fp32, pstride >= N).
    float* part;
    int64_t pstride;
    int kc;
};

// acc[c] += x(r) * w(r, c) for the first `rows` of eight rows.  The chunks are
// reinterpreted whole, then indexed (see dot8).
template <typename Elt>
__device__ __forceinline__ void kn_block(int4_t xv, const int4_t* w, int rows, float* acc) {
    typedef typename Elt::frag8 frag8;
    const frag8 xh = __builtin_bit_cast(frag8, xv);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (r < rows) {
            const frag8 wh = __builtin_bit_cast(frag8, w[r]);
            const float xr = (float)xh[r];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = __builtin_fmaf(xr, (float)wh[c], acc[c]);
        }
    }
}

// One workgroup per band of SEG * 8 columns.  Without SPLIT it sums every
// row and writes y; with SPLIT the grid's second dimension splits the rows
// (see GemvKnParams) and the workgroup writes its fp32 column sums for the
// second kernel, gemv_kn_reduce_kernel.
template <typename Elt, int SEG, int NW, bool SPLIT = false, int UB = 2>
__global__ __launch_bounds__(NW * 64) void gemv_kn_kernel(GemvKnParams p) {
    constexpr int BW = SEG * 8;          // columns per workgroup
    constexpr int RGW = 64 / SEG;        // row groups per wave
    constexpr int RG = NW * RGW;         // row groups per workgroup
    constexpr int NT = NW * 64;
    constexpr int PARTS = NT / BW;       // first-level partial sums per column
    static_assert(64 % SEG == 0 && NT % BW == 0 && RG % PARTS == 0, "reduction shape");
    __shared__ float red[RG * BW];
    __shared__ float colsum[PARTS * BW];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int seg = lane % SEG;
    const int rg = wave * RGW + lane / SEG;
    const int nb = blockIdx.x * BW;
    const int n0 = nb + seg * 8;
    // rows [kbeg, kend): blocks of eight rows b0 .. b1-1, then krem more
    const int kbeg = SPLIT ? (int)blockIdx.y * p.kc : 0;
    const int kend = SPLIT ? min(p.K, kbeg + p.kc) : p.K;
    const int b0 = kbeg / 8;
    const int b1 = kend / 8;
    const int krem = kend - b1 * 8;

    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;

    const uint16_t* col = p.B + n0;
    if (nb + BW <= p.N) {                // whole band below N (uniform)
        // UB blocks of eight rows per trip (UB * 8 loads per lane in flight),
        // the row group's blocks in increasing order
        int b = b0 + rg;
        for (; b + (UB - 1) * RG < b1; b += UB * RG) {
            int4_t xv[UB], w[UB][8];
#pragma unroll
            for (int u = 0; u < UB; ++u)
                xv[u] = *reinterpret_cast<const int4_t*>(p.x + 8 * (b + u * RG));
#pragma unroll
            for (int u = 0; u < UB; ++u)
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    w[u][r] = __builtin_nontemporal_load(reinterpret_cast<const int4_t*>(
                        col + (int64_t)(8 * (b + u * RG) + r) * p.ldb));
#pragma unroll
            for (int u = 0; u < UB; ++u) kn_block<Elt>(xv[u], w[u], 8, acc);
        }
        for (; b < b1; b += RG) {
            const int k0 = 8 * b;
            const int4_t x0 = *reinterpret_cast<const int4_t*>(p.x + k0);
            int4_t w0[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                w0[r] = __builtin_nontemporal_load(
                    reinterpret_cast<const int4_t*>(col + (int64_t)(k0 + r) * p.ldb));
            kn_block<Elt>(x0, w0, 8, acc);
        }
    } else {                             // ragged last band: masked columns
        for (int b = b0 + rg; b < b1; b += RG) {
            const int k0 = 8 * b;
            const int4_t x0 = *reinterpret_cast<const int4_t*>(p.x + k0);
            int4_t w0[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                w0[r] = gemv_chunk(p.B + (int64_t)(k0 + r) * p.ldb, n0, p.N, true);
            kn_block<Elt>(x0, w0, 8, acc);
        }
    }
    if (krem > 0 && rg == (b1 - b0) % RG) {   // ragged last block of rows
        const int k0 = 8 * b1;
        const int4_t x0 = gemv_chunk(p.x, k0, p.K, false);
        int4_t w0[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            w0[r] = (r < krem) ? gemv_chunk(p.B + (int64_t)(k0 + r) * p.ldb, n0, p.N, true)
                               : int4_t{0, 0, 0, 0};
        kn_block<Elt>(x0, w0, krem, acc);
    }

    // fixed-order reduction of the RG partial sums of each column
#pragma unroll
    for (int c = 0; c < 8; ++c) red[rg * BW + seg * 8 + c] = acc[c];
    __syncthreads();
    {
        const int c = t % BW, q = t / BW;
        constexpr int PER = RG / PARTS;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < PER; ++j) s += red[(q * PER + j) * BW + c];
        colsum[q * BW + c] = s;
    }
    __syncthreads();
    if (t < BW) {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < PARTS; ++q) s += colsum[q * BW + t];
        if (nb + t < p.N) {
            if constexpr (SPLIT) {
                p.part[(int64_t)blockIdx.y * p.pstride + nb + t] = s;
            } else {
                const typename Elt::scalar h = (typename Elt::scalar)s;
                p.y[nb + t] = __builtin_bit_cast(uint16_t, h);
            }
        }
    }
}

// Second kernel of a split [K][N] product: y(n) = the `splits` partial sums of
// column n added in split order, rounded once to the element type.  The
// partials are loaded eight splits at a time, all eight in flight before the
// adds (a load-then-add loop waits one memory round trip per split).
template <typename Elt>
__global__ __launch_bounds__(256) void gemv_kn_reduce_kernel(GemvKnParams p, int splits) {
    constexpr int G = 8;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= p.N) return;
    float s = 0.0f;
    for (int q0 = 0; q0 < splits; q0 += G) {
        float v[G];
#pragma unroll
        for (int j = 0; j < G; ++j)
            v[j] = q0 + j < splits ? p.part[(int64_t)(q0 + j) * p.pstride + n] : 0.0f;
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (q0 + j < splits) s = q0 + j == 0 ? v[j] : s + v[j];
    }
    const typename Elt::scalar h = (typename Elt::scalar)s;
    p.y[n] = __builtin_bit_cast(uint16_t, h);
}

}  // namespace sdt
