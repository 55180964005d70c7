// gfx950 fp16 GEMM kernel family: C = A.B, fp32 accumulation on MFMA, fp16
// (round-to-nearest-even) output.
//
// Design, after "Beating hipBLASLt on a Gaming GPU" (section "The result":
// two LDS buffers, one barrier per K-step, a two-deep global prefetch, A
// XOR-swizzled, B stored transposed) and "The part that actually mattered"
// (the tile is a compile-time parameter with its own wave layout),
// re-designed for CDNA4:
//   * wave64 and v_mfma_f32_32x32x16_f16: each wave owns a (BM/WM) x (BN/WN)
//     block of 32x32 accumulator tiles;
//   * both operands are K-contiguous rows (A row-major, B "K-major"), so both
//     are staged the same way: a k-tile is BM (or BN) rows of 64 fp16 =
//     128 bytes, eight 16-byte chunks per row;
//   * LDS: two stages; chunk c of row r lives at chunk c ^ swz(r), so the
//     16-byte fragment reads of 16 consecutive rows hit distinct bank groups;
//   * prefetch: while tile i is multiplied out of one LDS stage, tile i+1 is
//     written from registers into the other and tile i+2 is in flight in
//     registers -- one barrier per k-tile;
//   * stagger (FlyDSL PR "Speed up the RDNA3 GEMM up to 1.85x by choosing the
//     tile from the shape", Changes): workgroup w visits k-tiles in the order
//     (w + i) & (nkt - 1) when nkt is a power of two;
//   * edges: operand rows come through a buffer descriptor clipped to the
//     valid rows, so rows past M or N read as zero; the k tail is masked; the
//     store is masked.  One code path serves every shape.
//   * MI355X has 8 XCDs with private L2s and the dispatcher deals workgroup
//     ids round-robin over them; ids are remapped so each XCD works on a
//     contiguous, GROUP_M-grouped band of output tiles.
//
// The MFMA is issued as D = B_tile . A_tile^T (operand "A" of the instruction
// takes rows of B), so each lane's four consecutive accumulator rows are four
// consecutive n of one output row m and leave as one 8-byte store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdt {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef unsigned int uint2_t __attribute__((ext_vector_type(2)));

// Byte offset used for a row that does not exist: past the end of every
// descriptor (whose byte count stays below 2^31), so the load returns zero.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Raw-buffer descriptor word 3 for gfx9-family parts (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kGroupM = 8;

struct GemmParams {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int gm, gn;    // output tiles along M and N
    int nkt;       // k-tiles, ceil(K / 64)
    int stagger;   // 1: (w + i) & (nkt - 1) order
    int nxcd;      // XCDs the dispatcher deals workgroups over
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// A chunk of eight fp16 at byte offset `off` whose k range [k, k+8) straddles
// K: read the valid elements one by one so nothing past K is touched.
__device__ __noinline__ int4_t load_partial_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                  int soff, int valid) {
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        h[e] = (e < valid && off != kOutOfRange)
                   ? __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * e, soff, 0)
                   : (uint16_t)0;
    int4_t v;
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = (int)((uint32_t)h[2 * d] | ((uint32_t)h[2 * d + 1] << 16));
    return v;
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_kernel(GemmParams p) {
    constexpr int BK = 64;
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM;
    constexpr int WTN = BN / WN;
    constexpr int FM = WTM / 32;
    constexpr int FN = WTN / 32;
    constexpr int RPP = NT / 8;        // operand rows covered by one load pass
    constexpr int A_LD = BM / RPP;     // 16-byte chunks per thread per k-tile
    constexpr int B_LD = BN / RPP;
    constexpr int A_UNITS = BM * 8;    // 16-byte LDS units per stage
    constexpr int STAGE = (BM + BN) * 8;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BM % RPP == 0 && BN % RPP == 0, "rows must split evenly over passes");
    static_assert(RPP % 16 == 0, "swizzle assumes 16-row periodicity per pass");

    __shared__ int4_t smem[2 * STAGE];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wave_m = wave % WM;
    const int wave_n = wave / WM;

    // ---- workgroup -> output tile (XCD-aware, grouped) -------------------
    const int nwg = p.gm * p.gn;
    const int w = blockIdx.x;
    int logical = w;
    if (p.nxcd > 1) {
        const int xcd = w % p.nxcd;
        const int q = nwg / p.nxcd;
        const int r = nwg % p.nxcd;
        logical = xcd * q + min(xcd, r) + w / p.nxcd;
    }
    const int group_span = kGroupM * p.gn;
    const int g = logical / group_span;
    const int first_m = g * kGroupM;
    const int gsz = min(p.gm - first_m, kGroupM);
    const int within = logical - g * group_span;
    const int tm = first_m + within % gsz;
    const int tn = within / gsz;
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    // ---- operand descriptors and per-thread row offsets ------------------
    const int rows_a = min((int64_t)BM, (int64_t)p.M - m0);
    const int rows_b = min((int64_t)BN, (int64_t)p.N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.A + m0 * p.lda, (uint32_t)((int64_t)rows_a * p.lda * 2));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.B + n0 * p.ldb, (uint32_t)((int64_t)rows_b * p.ldb * 2));
    const int lrow = t >> 3;   // row within a pass
    const int lchk = t & 7;    // 16-byte chunk within the 128-byte k-slice
    uint32_t off_a[A_LD], off_b[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int row = lrow + i * RPP;
        off_a[i] = row < rows_a ? (uint32_t)(row * p.lda * 2 + lchk * 16) : kOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int row = lrow + i * RPP;
        off_b[i] = row < rows_b ? (uint32_t)(row * p.ldb * 2 + lchk * 16) : kOutOfRange;
    }
    // LDS unit this thread writes for pass i: row (lrow + i*RPP), chunk lchk.
    const int st_unit = lrow * 8 + (lchk ^ swz(lrow));

    const int nkt = p.nkt;
    const int k_tail = p.K - (nkt - 1) * BK;   // valid k in the last tile, 1..64
    const int k0 = p.stagger ? (w & (nkt - 1)) : 0;

    int4_t rga[A_LD], rgb[B_LD];

    auto load_tile = [&](int i) {
        const int kt = p.stagger ? ((k0 + i) & (nkt - 1)) : i;
        const int soff = kt * BK * 2;
        if (kt == nkt - 1 && k_tail < BK) {
            const int valid = k_tail - lchk * 8;   // elements of this chunk below K
#pragma unroll
            for (int j = 0; j < A_LD; ++j) {
                if (valid >= 8)
                    rga[j] = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, off_a[j], soff, 0));
                else if (valid <= 0)
                    rga[j] = (int4_t){0, 0, 0, 0};
                else
                    rga[j] = load_partial_chunk(ra, off_a[j], soff, valid);
            }
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                if (valid >= 8)
                    rgb[j] = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, off_b[j], soff, 0));
                else if (valid <= 0)
                    rgb[j] = (int4_t){0, 0, 0, 0};
                else
                    rgb[j] = load_partial_chunk(rb, off_b[j], soff, valid);
            }
        } else {
#pragma unroll
            for (int j = 0; j < A_LD; ++j)
                rga[j] = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, off_a[j], soff, 0));
#pragma unroll
            for (int j = 0; j < B_LD; ++j)
                rgb[j] = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, off_b[j], soff, 0));
        }
    };

    auto store_tile = [&](int stage) {
        int4_t* base = smem + stage * STAGE;
#pragma unroll
        for (int j = 0; j < A_LD; ++j) base[st_unit + j * RPP * 8] = rga[j];
#pragma unroll
        for (int j = 0; j < B_LD; ++j) base[A_UNITS + st_unit + j * RPP * 8] = rgb[j];
    };

    floatx16_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Fragment addressing: lane reads row (lane % 32) of a 32-row block,
    // 16-byte chunk 2*kk + lane/32 of the k-tile.
    const int frow = lane & 31;
    const int fsw = swz(frow);
    const int fhalf = lane >> 5;
    const int a_row0 = wave_m * WTM + frow;
    const int b_row0 = wave_n * WTN + frow;

    auto compute = [&](int stage, int kk) {
        const int4_t* base = smem + stage * STAGE;
        const int chunk = (2 * kk + fhalf) ^ fsw;
        half8_t fa[FM], fb[FN];
#pragma unroll
        for (int j = 0; j < FM; ++j)
            fa[j] = __builtin_bit_cast(half8_t, base[(a_row0 + j * 32) * 8 + chunk]);
#pragma unroll
        for (int i = 0; i < FN; ++i)
            fb[i] = __builtin_bit_cast(half8_t, base[A_UNITS + (b_row0 + i * 32) * 8 + chunk]);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[i], fa[j], acc[i][j], 0, 0, 0);
    };

    // ---- prologue: tile 0 into stage 0, tile 1 in flight -----------------
    load_tile(0);
    store_tile(0);
    if (nkt > 1) load_tile(1);
    __syncthreads();

    // ---- main loop: one barrier per k-tile -------------------------------
    for (int i = 0; i < nkt; ++i) {
        const int s = i & 1;
        compute(s, 0);
        compute(s, 1);
        if (i + 1 < nkt) {
            store_tile(s ^ 1);
            if (i + 2 < nkt) load_tile(i + 2);
        }
        compute(s, 2);
        compute(s, 3);
        __syncthreads();
    }

    // ---- epilogue: fp32 -> fp16 (RNE), masked 8-byte stores --------------
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int64_t m = m0 + wave_m * WTM + j * 32 + frow;
            if (m >= p.M) continue;
            uint16_t* crow = p.C + m * p.ldc;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int64_t n = n0 + wave_n * WTN + i * 32 + 8 * gq + 4 * fhalf;
                half4_t h;
                h[0] = (_Float16)acc[i][j][4 * gq + 0];
                h[1] = (_Float16)acc[i][j][4 * gq + 1];
                h[2] = (_Float16)acc[i][j][4 * gq + 2];
                h[3] = (_Float16)acc[i][j][4 * gq + 3];
                if (n + 3 < p.N) {
                    *reinterpret_cast<uint2_t*>(crow + n) = __builtin_bit_cast(uint2_t, h);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const _Float16 v = h[e];   // element first, then reinterpret
                        if (n + e < p.N) crow[n + e] = __builtin_bit_cast(uint16_t, v);
                    }
                }
            }
        }
    }
}

// C = 0 for K == 0 (the empty sum), M x N with stride ldc.
__global__ void fill_zero_kernel(uint16_t* C, int64_t ldc, int M, int N) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)M * N;
    for (int64_t e = idx; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = e / N;
        const int64_t n = e - m * N;
        C[m * ldc + n] = 0;
    }
}

}  // namespace sdt
