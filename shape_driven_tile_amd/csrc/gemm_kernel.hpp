// gfx950 GEMM kernel family: C = A.B for fp16 or bf16 operands, fp32
// accumulation on MFMA, output in the operand type (round-to-nearest-even).
//
// After "Beating hipBLASLt on a Gaming GPU" (section "The result": two LDS
// buffers, one barrier per K-step, prefetch of the next tiles while the
// current one is consumed, an XOR swizzle, B stored transposed) and "The part
// that actually mattered" (the tile is a compile-time parameter with its own
// wave layout), re-designed for CDNA4:
//   * wave64, each wave owning a (BM/WM) x (BN/WN) block of accumulator
//     tiles: MF = 32 runs v_mfma_f32_32x32x16_f16 (_bf16 for the bf16
//     variant) on 32x32 tiles, MF = 16 v_mfma_f32_16x16x32 on 16x16 tiles,
//     which costs less energy per FLOP where the part runs at its power
//     limit (the one-k-group deep pipelines of the 256 x 128 and 128 x 128
//     rungs, every pipeline of the 96, 160 and 192 rungs; the 256 x 256
//     ping-pong kernel at the end of this file also uses 16x16x32, with its
//     own schedule);
//   * both operands are K-contiguous rows (A row-major, B "K-major"), staged
//     the same way: a k-tile is BM (or BN) rows of 64 fp16 = 128 bytes, eight
//     16-byte chunks per row; chunk c of row r is stored at chunk c ^ swz(r),
//     which keeps the 16-byte fragment reads of 16 consecutive rows on
//     distinct LDS bank groups;
//   * global -> LDS without registers: buffer_load_dwordx4 ... lds writes a
//     wave's 64 lanes to 1 KB of consecutive LDS, so each lane fetches the
//     global chunk that belongs at its swizzled LDS slot;
//   * NS LDS stages (a compile-time parameter of the rung: as many as fit):
//     while tile i is multiplied out of its stage, tiles i+1 .. i+NS-1 are
//     landing in the others; right after the single barrier of step i the
//     loads of tile i+NS are issued into the stage tile i just freed, so the
//     global prefetch runs NS-1 tiles deep;
//   * MFMA fragments are double-buffered in registers across the sub-steps
//     of a k-tile (four 16 deep with MF = 32, two 32 deep with MF = 16), so
//     the LDS reads of sub-step kk+1 are in flight under the MFMAs of
//     sub-step kk, and the first reads of tile i+1 go out under the last
//     MFMAs of tile i, past the barrier;
//   * KS = 2 k-groups (MF = 32): a second set of waves takes sub-steps 1
//     and 3 of every k-tile while the first takes 0 and 2, halving each
//     wave's dependent MFMA chain per k-tile and doubling the waves a small
//     grid keeps in flight;
//     the second group's partial sums are added to the first's through LDS
//     (a fixed order: the result is deterministic) before the epilogue;
//   * k-loop stagger (FlyDSL PR "Speed up the RDNA3 GEMM up to 1.85x by
//     choosing the tile from the shape", Changes), when the launch plan
//     enables it (the automatic plan on every rung except the ping-pong one,
//     for the shapes launcher.cpp's stagger_auto names) or a caller forces it:
//     with a power-of-two number of full k-tiles, workgroup w visits them in
//     the order (w + i) & (nfull - 1);
//   * edges: operand rows come through buffer descriptors clipped to the
//     valid rows, so rows past M or N read as zero; a partial last k-tile is
//     loaded through registers with per-element masking; stores are masked;
//     wave tiles 64 columns wide, and every MF = 16 wave tile, pass their
//     output through LDS so that each lane stores 16 contiguous bytes;
//   * MI355X deals workgroup ids round-robin over its XCDs, each with a
//     private L2; ids are remapped so every XCD works through a contiguous,
//     GROUP_M-grouped band of output tiles.
//
// The MFMA is issued as D = B_frag . A_frag^T (the instruction's first
// operand takes rows of B), so each lane's four consecutive accumulator rows
// are four consecutive n of one output row m (one 8-byte store where a wave
// tile 32 columns wide stores them directly).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launcher.hpp"

namespace sdt {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef unsigned int uint2_t __attribute__((ext_vector_type(2)));
typedef unsigned int uint4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

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
    int stagger;   // 1: full k-tiles in (w + i) & (K/64 - 1) order
    int nxcd;      // XCDs the dispatcher deals workgroups over
    int splits;    // workgroups per output tile along K (1: none; see gemm_kernel)
    int split_algo;  // splits > 1: 0 a second kernel reduces, 1 the tile's last workgroup does
    float* ws;     // splits > 1: fp32 partial sums, tiles x splits slots of BM x BN
    int* cnt;      // split_algo 1: one arrival counter per (tile, wave), zero between launches
    int persistent;  // ping-pong kernel: 0 one workgroup per tile, else the grid size
};

// Dealing order of workgroup ids over the XCDs: MI355X hands workgroup w to
// XCD w % nxcd.  Returns a logical index such that every XCD works through a
// contiguous range of [0, nwg) (a bijection for any nwg).
__device__ __forceinline__ int xcd_remap(int w, int nwg, int nxcd) {
    if (nxcd <= 1) return w;
    const int xcd = w % nxcd, q = nwg / nxcd, r = nwg % nxcd;
    return xcd * q + min(xcd, r) + w / nxcd;
}

// Output tile `tile` (a logical index in [0, gm * gn)) in the grouped order:
// kGroupM tile rows at a time, column by column inside a group, so that
// consecutive tiles share B rows and a group shares A rows.
__device__ __forceinline__ void grouped_origin(const GemmParams& p, int tile, int BM, int BN,
                                               int64_t& m0, int64_t& n0) {
    const int group_span = kGroupM * p.gn;
    const int g = tile / group_span;
    const int first_m = g * kGroupM;
    const int gsz = min(p.gm - first_m, kGroupM);
    const int within = tile - g * group_span;
    m0 = (int64_t)(first_m + within % gsz) * BM;
    n0 = (int64_t)(within / gsz) * BN;
}

// Element types.  Each names its vector types, the 32x32x16 and 16x16x32 MFMAs, the
// two-term dot product into fp32 used by the GEMV kernels, and (through
// `scalar`) the fp32 -> 16-bit conversion of the epilogues, which rounds to
// nearest even (v_cvt_f16_f32 / v_cvt_pk_bf16_f32 under the default mode).
struct F16 {
    typedef half8_t frag8;
    typedef half4_t vec4;
    typedef half2_t vec2;
    typedef _Float16 scalar;
    static __device__ __forceinline__ floatx16_t mfma(frag8 a, frag8 b, floatx16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ floatx4_t mfma16(frag8 a, frag8 b, floatx4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(vec2 a, vec2 b, float c) {
        return __builtin_amdgcn_fdot2(a, b, c, false);
    }
};
struct BF16 {
    typedef bf16x8_t frag8;
    typedef bf16x4_t vec4;
    typedef bf16x2_t vec2;
    typedef __bf16 scalar;
    static __device__ __forceinline__ floatx16_t mfma(frag8 a, frag8 b, floatx16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ floatx4_t mfma16(frag8 a, frag8 b, floatx4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(vec2 a, vec2 b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
    }
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// The ping-pong kernel's 16x16x32 fragment reads put 16 consecutive rows
// and one 16-byte chunk on each group of 16 lanes (four chunks per read).
// With swz() above those reads run at half the LDS rate (SQ_LDS_BANK_CONFLICT
// at 8192^3: 102M cycles).  Chunk c of row r is stored at c ^ swz_pp(r), an
// XOR-linear map of the row's three low bits (bit 0 -> 4, bit 1 -> 5,
// bit 2 -> 3) chosen by timing every such map on MI355X: the reads then run
// at the rate of contiguous 16-byte reads (245 B/clk per CU).
__device__ __forceinline__ int swz_pp(int row) {
    return ((row & 1) ? 4 : 0) ^ ((row & 2) ? 5 : 0) ^ ((row & 4) ? 3 : 0);
}

// Buffer descriptor over `bytes` bytes from `base`.  Both are workgroup-
// uniform; readfirstlane says so to the compiler, which keeps the descriptor
// in scalar registers (in vector registers every load would become a
// waterfall loop).  Offsets at or past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)n, kRsrcWord3);
}

// 16 bytes per lane from global memory straight into LDS at
// lds_wave_base + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int4_t* lds_wave_base,
                                      uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds_wave_base, 16, voff, soff, 0, 0);
}

// Eight fp16 at byte offset `off` of which only the first `valid` lie below K
// (valid >= 8: all; valid <= 0: none, zero returned).  Nothing at or past K
// is read.
__device__ __forceinline__ int4_t load16_tail(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff,
                                              int valid) {
    if (valid >= 8)
        return __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
    int4_t v = {0, 0, 0, 0};
    if (valid > 0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t lo = (2 * d < valid)
                ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * d, soff, 0) : 0u;
            const uint32_t hi = (2 * d + 1 < valid)
                ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * d + 2, soff, 0) : 0u;
            v[d] = (int)(lo | (hi << 16));
        }
    }
    return v;
}

// s_waitcnt vmcnt(N) (at most N global loads of this wave still in flight),
// leaving the LDS and export counters alone.  gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int N>
__device__ __forceinline__ void wait_global_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Epilogue of one wave: its FN x FM accumulator tiles of 32 x 32 (tile (i, j)
// covers rows mb + 32 j .., columns nb + 32 i ..) rounded to the output type
// (nearest even) and stored with 8-byte stores, masked at the M and N edges.
// Lane l holds row (l % 32) of each tile, columns 8 g + 4 (l / 32) + 0..3 in
// accumulator elements 4 g .. 4 g + 3.
template <typename Elt, int FM, int FN>
__device__ __forceinline__ void store_block(const GemmParams& p, const floatx16_t (&acc)[FN][FM],
                                            int64_t mb, int64_t nb, int frow, int fhalf) {
    typedef typename Elt::vec4 vec4;
    typedef typename Elt::scalar scalar;
#pragma unroll
    for (int i2 = 0; i2 < FN; ++i2) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int64_t m = mb + j * 32 + frow;
            if (m >= p.M) continue;
            uint16_t* crow = p.C + m * p.ldc;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int64_t n = nb + i2 * 32 + 8 * gq + 4 * fhalf;
                vec4 h;
                h[0] = (scalar)acc[i2][j][4 * gq + 0];
                h[1] = (scalar)acc[i2][j][4 * gq + 1];
                h[2] = (scalar)acc[i2][j][4 * gq + 2];
                h[3] = (scalar)acc[i2][j][4 * gq + 3];
                if (n + 3 < p.N) {
                    *reinterpret_cast<uint2_t*>(crow + n) = __builtin_bit_cast(uint2_t, h);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const scalar v = h[e];   // element first, then reinterpret
                        if (n + e < p.N) crow[n + e] = __builtin_bit_cast(uint16_t, v);
                    }
                }
            }
        }
    }
}

// Epilogue of one wave of the ping-pong kernel (128 x 64 outputs held as
// FM = 8 row blocks x FN = 4 column blocks of 16 x 16 MFMA tiles; lane l has
// row 16 j + l % 16, columns 16 i + 4 (l / 16) .. + 3 of tile (i, j)) through
// 4 KB of LDS owned by the wave, 32 rows at a time.  Stored directly, each
// 8-byte store would touch 16 rows; staged, every lane stores 16 contiguous
// bytes and 8 lanes cover a row's 128 bytes.  Row r of the stage keeps its
// 16-byte chunk c at c ^ ((r >> 1) & 7): the 8-byte writes (16 rows x one
// chunk per 16 lanes) and the 16-byte reads (an even and an odd row x 8
// chunks per 16 lanes served together) both fall on distinct banks.  Masked
// at the M and N edges.
template <typename Elt, int FM = 8>
__device__ __forceinline__ void store_block_staged(const GemmParams& p,
                                                   const floatx4_t (&acc)[4][FM], int64_t mb,
                                                   int64_t nb, int lane, int4_t* stage) {
    typedef typename Elt::vec4 vec4;
    typedef typename Elt::scalar scalar;
    char* lds = reinterpret_cast<char*>(stage);
    const int wq = lane >> 4;          // write: column group 4 (l / 16) of a 16-wide tile
    // read: rows 8 k + rr, chunk lane % 8; lanes 0-31 take the even rows and
    // 32-63 the odd ones, so lanes l and l + 32 (served together) hit
    // different halves of the banks
    const int rr = 2 * ((lane >> 3) & 3) + (lane >> 5);
    const int rc = lane & 7;
#pragma unroll
    for (int q = 0; q < FM / 2; ++q) { // rows 32 q .. 32 q + 31: tiles j = 2 q, 2 q + 1
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int r = 16 * jj + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const floatx4_t& a = acc[i][2 * q + jj];
                vec4 h;
                h[0] = (scalar)a[0];
                h[1] = (scalar)a[1];
                h[2] = (scalar)a[2];
                h[3] = (scalar)a[3];
                const int chunk = 2 * i + (wq >> 1);
                *reinterpret_cast<uint2_t*>(lds + r * 128 + ((chunk ^ ((r >> 1) & 7)) * 16) +
                                            (wq & 1) * 8) = __builtin_bit_cast(uint2_t, h);
            }
        }
        // Other lanes of this wave read what these wrote: LDS runs a wave's
        // accesses in order; the fence keeps the compiler from reordering them.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 8 * k + rr;
            const int4_t v = *reinterpret_cast<const int4_t*>(
                lds + r * 128 + ((rc ^ ((r >> 1) & 7)) * 16));
            const int64_t m = mb + q * 32 + r;
            const int64_t n = nb + 8 * rc;
            if (m < p.M) {
                uint16_t* dst = p.C + m * p.ldc + n;
                if (n + 7 < p.N) {
                    // non-temporal: C goes out to memory as it is written
                    // instead of staying dirty in L2 until the end-of-kernel
                    // writeback (4096^3: 98.9 -> 98.1 us, 8192^3: 759 ->
                    // 750 us).  The 8-byte stores of store_block, each
                    // covering part of a line, measured 8-32% slower this way.
                    __builtin_nontemporal_store(v, reinterpret_cast<int4_t*>(dst));
                } else {
                    const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < p.N) dst[e] = e16[e];
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
}

// Epilogue of one wave of gemm_kernel whose wave tile is 64 columns wide
// (FN = 2 tiles of 32 x 32, FM row blocks; lane l holds row l % 32 of a tile,
// columns 8 g + 4 (l / 32) .. + 3 in accumulator elements 4 g .. 4 g + 3)
// through 4 KB of LDS owned by the wave, 32 rows at a time, so that every
// lane stores 16 contiguous bytes and 8 lanes a row's 128 bytes (the 8-byte
// stores of store_block touch 32 rows per instruction).  Same stage layout as
// store_block_staged: row r keeps its 16-byte chunk c at c ^ ((r >> 1) & 7);
// the 8-byte writes (32 rows x one chunk, both halves) fall on every bank
// exactly twice.  Masked at the M and N edges.
template <typename Elt, int FM>
__device__ __forceinline__ void store_block_staged32(const GemmParams& p,
                                                     const floatx16_t (&acc)[2][FM], int64_t mb,
                                                     int64_t nb, int lane, int4_t* stage) {
    typedef typename Elt::vec4 vec4;
    typedef typename Elt::scalar scalar;
    char* lds = reinterpret_cast<char*>(stage);
    const int wr = lane & 31;          // write: row of the 32-row block
    const int wh = lane >> 5;          // write: which 8-byte half of the chunk
    const int rr = 2 * ((lane >> 3) & 3) + (lane >> 5);
    const int rc = lane & 7;
#pragma unroll
    for (int j = 0; j < FM; ++j) {     // rows 32 j .. 32 j + 31
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                vec4 h;
                h[0] = (scalar)acc[i][j][4 * g + 0];
                h[1] = (scalar)acc[i][j][4 * g + 1];
                h[2] = (scalar)acc[i][j][4 * g + 2];
                h[3] = (scalar)acc[i][j][4 * g + 3];
                const int chunk = 4 * i + g;
                *reinterpret_cast<uint2_t*>(lds + wr * 128 + ((chunk ^ ((wr >> 1) & 7)) * 16) +
                                            wh * 8) = __builtin_bit_cast(uint2_t, h);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 8 * k + rr;
            const int4_t v = *reinterpret_cast<const int4_t*>(
                lds + r * 128 + ((rc ^ ((r >> 1) & 7)) * 16));
            const int64_t m = mb + j * 32 + r;
            const int64_t n = nb + 8 * rc;
            if (m < p.M) {
                uint16_t* dst = p.C + m * p.ldc + n;
                if (n + 7 < p.N) {
                    *reinterpret_cast<int4_t*>(dst) = v;
                } else {
                    const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < p.N) dst[e] = e16[e];
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
}

// ---- k-split partial sums -------------------------------------------------------
// A wave's fp32 accumulators (FN x FM tiles of ACC values per lane) leave and
// return in 16-byte pieces: piece q = (i * FM + j) * (ACC / 4) + e of the
// wave's slot holds accumulator elements 4e .. 4e + 3 of tile (i, j) for all
// 64 lanes, lane l at byte 16 (64 q + l), so every store or load instruction
// of a wave covers 1 KB of consecutive memory.  AUX is the buffer
// instruction's cache-policy field: 0, or kScopeDevice for the single-kernel
// reduction (see splitk_arrive).
constexpr int kScopeDevice = 16;   // sc1: coherent at device scope, across XCDs

template <int AUX, int FN, int FM, typename acc_t>
__device__ __forceinline__ void store_partial(const acc_t (&acc)[FN][FM], __amdgpu_buffer_rsrc_t r,
                                              int lane) {
    constexpr int E = sizeof(acc_t) / 16;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                // element first, then reinterpret: a bit cast applied to a
                // vector-element expression reads element 0 of the vector
                uint4_t v;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const float x = acc[i][j][4 * e + d];
                    v[d] = __builtin_bit_cast(uint32_t, x);
                }
                __builtin_amdgcn_raw_buffer_store_b128(v, r, (((i * FM + j) * E + e) * 64 + lane) * 16,
                                                       0, AUX);
            }
}

// acc = partial (ADD false) or acc += partial (ADD true), element by element.
template <int AUX, bool ADD, int FN, int FM, typename acc_t>
__device__ __forceinline__ void load_partial(acc_t (&acc)[FN][FM], __amdgpu_buffer_rsrc_t r, int lane) {
    constexpr int E = sizeof(acc_t) / 16;
    uint4_t v[FN][FM][E];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[i][j][e] = __builtin_amdgcn_raw_buffer_load_b128(
                    r, (((i * FM + j) * E + e) * 64 + lane) * 16, 0, AUX);
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t u = v[i][j][e][d];   // element first (see store_partial)
                    const float x = __builtin_bit_cast(float, u);
                    if constexpr (ADD)
                        acc[i][j][4 * e + d] += x;
                    else
                        acc[i][j][4 * e + d] = x;
                }
}

// Slot of (tile, split, wave) in the partial-sum area: tiles x splits x
// waves slots of `slot_floats` each.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_slot(const GemmParams& p, int tile, int split,
                                                               int wave, int nwaves, int slot_floats) {
    const int64_t idx = ((int64_t)tile * p.splits + split) * nwaves + wave;
    return make_rsrc(p.ws + idx * slot_floats, (uint32_t)slot_floats * 4);
}

// The single-kernel k-split reduction, per workgroup.  Every wave of the
// workgroup has stored its part of this split's partial sums (with the
// device-scope bit: written through to memory).  A workgroup barrier (each
// wave waits for its stores first), then one thread makes them visible at
// agent scope (a release fence: the XCDs' L2s are separate caches, so the
// XCD's dirty lines are written back) and counts the arrival on the tile's
// counter with an agent-scope atomic.  The workgroup that arrives last owns
// the tile: its counting thread takes an acquire fence (which invalidates
// what the CU and XCD caches hold of the other splits' slots) and clears the
// counter for the next launch; after a second barrier its waves form
//   acc = ((P_0 + P_1) + P_2) + ... + P_{splits-1}
// in that order, whichever split they hold (fp32 addition is commutative, so
// adding their own P_split to the running sum of P_0 .. P_{split-1} gives
// the same bits as the opposite operand order): the result does not depend
// on the order of arrival.  The other workgroups are done.  No workgroup
// waits for another: nothing spins.  `active` = false for waves that hold
// no accumulators (a second k-group): they take the two barriers only.
// Returns whether the calling wave owns its block.
template <int FN, int FM, typename acc_t>
__device__ __forceinline__ bool splitk_arrive(const GemmParams& p, acc_t (&acc)[FN][FM], int tile,
                                              int split, int wave, int nwaves, int lane,
                                              bool active, int* flag) {
    constexpr int SLOT = FN * FM * (int)(sizeof(acc_t) / 4) * 64;
    if (active)
        store_partial<kScopeDevice>(acc, partial_slot(p, tile, split, wave, nwaves, SLOT), lane);
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        int* counter = p.cnt + tile;
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == p.splits - 1;
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *flag = last;
    }
    __syncthreads();
    if (!active || !*flag) return false;
    if (split == 0) {
        for (int s = 1; s < p.splits; ++s)
            load_partial<kScopeDevice, true>(acc, partial_slot(p, tile, s, wave, nwaves, SLOT), lane);
    } else {
        acc_t run[FN][FM];
        load_partial<kScopeDevice, false>(run, partial_slot(p, tile, 0, wave, nwaves, SLOT), lane);
        for (int s = 1; s < split; ++s)
            load_partial<kScopeDevice, true>(run, partial_slot(p, tile, s, wave, nwaves, SLOT), lane);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = run[i][j] + acc[i][j];
        for (int s = split + 1; s < p.splits; ++s)
            load_partial<kScopeDevice, true>(acc, partial_slot(p, tile, s, wave, nwaves, SLOT), lane);
    }
    return true;
}

// Epilogue of one wave whose 16 x 16 accumulator tiles (FN column tiles x FM
// row tiles, MF = 16) span a width other than 64 columns: 16 rows at a time
// through the wave's LDS (rows FN * 32 bytes, padded by 16 so consecutive rows
// start on different banks), then 16 contiguous bytes per lane, a row's FN * 32
// bytes stored by 2 FN lanes side by side.  Masked at the M and N edges.
template <typename Elt, int FN, int FM>
__device__ __forceinline__ void store_block_staged16(const GemmParams& p,
                                                     const floatx4_t (&acc)[FN][FM], int64_t mb,
                                                     int64_t nb, int lane, int4_t* stage) {
    typedef typename Elt::vec4 vec4;
    typedef typename Elt::scalar scalar;
    constexpr int RB = FN * 32 + 16;   // staged row stride, bytes
    constexpr int CPR = 2 * FN;        // 16-byte chunks per row
    static_assert(16 * RB <= 4096, "16 staged rows fit the wave's 4 KB");
    char* lds = reinterpret_cast<char*>(stage);
    const int wr = lane & 15, wq = lane >> 4;
#pragma unroll
    for (int j = 0; j < FM; ++j) {     // rows 16 j .. 16 j + 15
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const floatx4_t& a = acc[i][j];
            vec4 h;
            h[0] = (scalar)a[0];
            h[1] = (scalar)a[1];
            h[2] = (scalar)a[2];
            h[3] = (scalar)a[3];
            *reinterpret_cast<uint2_t*>(lds + wr * RB + i * 32 + wq * 8) =
                __builtin_bit_cast(uint2_t, h);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int c = lane; c < 16 * CPR; c += 64) {
            const int r = c / CPR, cc = c - (c / CPR) * CPR;
            const int4_t v = *reinterpret_cast<const int4_t*>(lds + r * RB + cc * 16);
            const int64_t m = mb + j * 16 + r;
            const int64_t n = nb + 8 * cc;
            if (m < p.M) {
                uint16_t* dst = p.C + m * p.ldc + n;
                if (n + 7 < p.N) {
                    *reinterpret_cast<int4_t*>(dst) = v;
                } else {
                    const uint16_t* e16 = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < p.N) dst[e] = e16[e];
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
}

// Epilogue of one wave of gemm_kernel (and of the k-split reduction kernel):
// rounds the accumulators to the output type and stores them, through the
// wave's 4 KB of LDS at `stage` when its tile is 64 columns wide.
template <typename Elt, int MF, int FN, int FM, typename acc_t>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, const acc_t (&acc)[FN][FM],
                                              int64_t mb, int64_t nb, int lane, int4_t* stage) {
    if constexpr (MF == 16 && FN == 4) {
        store_block_staged<Elt, FM>(p, acc, mb, nb, lane, stage);
    } else if constexpr (MF == 16) {
        store_block_staged16<Elt, FN, FM>(p, acc, mb, nb, lane, stage);
    } else if constexpr (FN == 2) {
        store_block_staged32<Elt, FM>(p, acc, mb, nb, lane, stage);
    } else {
        store_block<Elt, FM, FN>(p, acc, mb, nb, lane & 31, lane >> 5);
    }
}

// HELP (one k-group, no k-split): the workgroup also holds one loader wave
// per compute wave.  The loader waves issue every global -> LDS load, with
// the same slabs, waits and barriers the compute waves would have used, and
// exit after the k-loop; the compute waves then issue nothing but fragment
// reads and MFMAs.  With one compute wave per SIMD each 1 KB direct-to-LDS
// load otherwise takes about 17 cycles of the wave's issue (the CU's 64 B/clk)
// between its MFMAs.
template <typename Elt, int BM, int BN, int WM, int WN, int NS, int KS, int MF = 32, bool SK = false,
          bool HELP = false>
__global__ __launch_bounds__(WM * WN * KS * 64 * (HELP ? 2 : 1)) void gemm_kernel(GemmParams p) {
    typedef typename Elt::frag8 frag8;
    constexpr int BK = kBK;
    constexpr int NMN = WM * WN;       // waves per k-group (one output block each)
    constexpr int NW = NMN * KS;       // waves per workgroup
    static_assert(KS == 1 || KS == 2, "k-groups: 1 or 2");
    // MF = 32: v_mfma_f32_32x32x16 on 32 x 32 tiles, four 16-deep sub-steps per
    // k-tile.  MF = 16: v_mfma_f32_16x16x32 on 16 x 16 tiles, two 32-deep
    // sub-steps, one k-group.
    static_assert(MF == 32 || (MF == 16 && KS == 1), "MFMA shape");
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int A_UNITS = BM * 8, B_UNITS = BN * 8;   // 16-byte LDS units per stage
    constexpr int STAGE = A_UNITS + B_UNITS;
    constexpr int A_DMA = A_UNITS / (64 * NW);         // 1 KB loads per wave per k-tile
    constexpr int B_DMA = B_UNITS / (64 * NW);
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be whole MFMA tiles");
    static_assert(A_UNITS % (64 * NW) == 0 && B_UNITS % (64 * NW) == 0,
                  "each wave loads whole 8-row slabs");
    static_assert(NS >= 2 && NS * STAGE * 16 <= 160 * 1024, "stages must fit the LDS");
    static_assert(KS == 1 || BM * BN * 4 <= NS * STAGE * 16, "k-group partials fit the LDS");
    static_assert(WM * WN * (KS > 1 && MF == 32 ? (BM / WM / MF) * (BN / WN / MF) : 1) * 256 <
                      NS * STAGE && (KS == 1 || BM * BN / 4 < NS * STAGE),
                  "the last LDS unit is free after the k-loop");
    constexpr int L = A_DMA + B_DMA;   // global loads per wave per k-tile

    __shared__ int4_t smem[NS * STAGE];
    // The k-split arrival's verdict for the workgroup, in the last LDS unit:
    // by then every k-step's reads are done, and neither the k-group sums nor
    // the staged epilogue reach that far.
    int* const splitk_flag = reinterpret_cast<int*>(smem + NS * STAGE - 1);

    const int t = threadIdx.x;
    const int lane = t & 63;
    // Wave-uniform, and said so: the per-wave LDS destinations of the
    // direct-to-LDS loads (M0) then come from scalar arithmetic instead of a
    // v_readfirstlane per load (8192^3: 909 -> 894 us).
    const int wave_id = __builtin_amdgcn_readfirstlane(t >> 6);
    static_assert(!HELP || (KS == 1 && !SK), "loader waves: one k-group, no k-split");
    const bool loader = HELP && wave_id >= NW;
    const int wave = HELP ? wave_id % NW : wave_id;   // a loader wave takes its compute wave's slabs
    const int kg = wave / NMN;         // k-group: sub-steps kg, kg + KS, ... of each k-tile
    const int wmn = wave % NMN;
    const int wave_m = wmn % WM;
    const int wave_n = wmn / WM;

    // ---- workgroup -> (k-split, output tile), XCD-aware and grouped ----------
    // With splits > 1 the grid holds `splits` workgroups per tile; logical
    // index l takes split l / tiles of tile l % tiles, so each XCD's range is
    // neighbouring tiles over one k-range (shared A and B rows in its L2).
    const int ntile = p.gm * p.gn;
    const int w = blockIdx.x;
    const int logical = xcd_remap(w, SK ? ntile * p.splits : ntile, p.nxcd);
    const int split = SK ? logical / ntile : 0;
    const int tile = logical - split * ntile;
    int64_t m0, n0;
    grouped_origin(p, tile, BM, BN, m0, n0);

    // ---- operand descriptors: only this tile's valid rows are addressable ----
    const int rows_a = (int)min((int64_t)BM, (int64_t)p.M - m0);
    const int rows_b = (int)min((int64_t)BN, (int64_t)p.N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.A + m0 * p.lda, (uint32_t)((int64_t)rows_a * p.lda * 2));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.B + n0 * p.ldb, (uint32_t)((int64_t)rows_b * p.ldb * 2));

    // Load j of this wave fills LDS units [(wave*X + j)*64, +64): 8 rows of
    // the stage; lane l lands in unit +l, i.e. row l/8 at swizzled position
    // l%8, which holds logical chunk (l%8) ^ swz(row).  A row past the valid
    // ones has an offset past the descriptor and reads as zero.
    uint32_t voff_a[A_DMA], voff_b[B_DMA];
    int chk_a[A_DMA], chk_b[B_DMA];
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int row = (wave * A_DMA + j) * 8 + (lane >> 3);
        chk_a[j] = (lane & 7) ^ (MF == 32 ? swz(row) : swz_pp(row));
        voff_a[j] = (uint32_t)(row * p.lda * 2 + chk_a[j] * 16);
    }
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int row = (wave * B_DMA + j) * 8 + (lane >> 3);
        chk_b[j] = (lane & 7) ^ (MF == 32 ? swz(row) : swz_pp(row));
        voff_b[j] = (uint32_t)(row * p.ldb * 2 + chk_b[j] * 16);
    }

    // ---- k-tile sequence: the full tiles (staggered), then a partial one ------
    // A k-split takes a contiguous run of the full k-tiles (the first
    // nfull % splits splits one more than the others); the last split also
    // takes the partial one.  Splits are never staggered.
    const int nfull_all = p.K / BK;
    int kbeg = 0, nfull = nfull_all, ktail = p.K - nfull_all * BK;
    if (SK && p.splits > 1) {
        const int q = nfull_all / p.splits, r = nfull_all % p.splits;
        kbeg = split * q + min(split, r);
        nfull = q + (split < r ? 1 : 0);
        if (split != p.splits - 1) ktail = 0;
    }
    const int nseq = nfull + (ktail > 0 ? 1 : 0);
    const int kmask = p.stagger ? (nfull - 1) : 0x7fffffff;
    const int k0 = p.stagger ? (w & (nfull - 1)) : 0;

    auto dma_tile = [&](int step, int stage) {   // a full k-tile, straight into LDS
        const int soff = (kbeg + ((k0 + step) & kmask)) * (BK * 2);
        int4_t* base = smem + stage * STAGE;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) dma16(ra, base + (wave * A_DMA + j) * 64, voff_a[j], soff);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j)
            dma16(rb, base + A_UNITS + (wave * B_DMA + j) * 64, voff_b[j], soff);
    };
    auto tail_tile = [&](int stage) {            // the partial k-tile, masked
        const int soff = nfull_all * (BK * 2);
        int4_t* base = smem + stage * STAGE;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j)
            base[(wave * A_DMA + j) * 64 + lane] =
                load16_tail(ra, voff_a[j], soff, ktail - chk_a[j] * 8);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j)
            base[A_UNITS + (wave * B_DMA + j) * 64 + lane] =
                load16_tail(rb, voff_b[j], soff, ktail - chk_b[j] * 8);
    };
    auto load_step = [&](int step, int stage) {
        if (step < nfull) dma_tile(step, stage); else tail_tile(stage);
    };

    // ---- accumulators and fragments ----------------------------------------------
    typedef std::conditional_t<MF == 32, floatx16_t, floatx4_t> acc_t;
    constexpr int ACC = MF == 32 ? 16 : 4;
    acc_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < ACC; ++e) acc[i][j][e] = 0.0f;

    // MF = 32: lane reads row (lane % 32) of a 32-row block, chunk 2*kk +
    // lane/32.  MF = 16: row (lane % 16) of a 16-row block, chunk 4*kk +
    // lane/16.  Rows of one lane differ by multiples of MF: same swizzle.
    const int frow = lane & (MF - 1);
    const int fsw = MF == 32 ? swz(frow) : swz_pp(frow);
    const int fhalf = lane / MF;
    const int a_row0 = wave_m * WTM + frow;
    const int b_row0 = wave_n * WTN + frow;
    frag8 fa[2][FM], fb[2][FN];
    auto read_frags = [&](int stage, int kk, int set) {
        const int4_t* base = smem + stage * STAGE;
        const int chunk = ((64 / MF) * kk + fhalf) ^ fsw;
#pragma unroll
        for (int j = 0; j < FM; ++j)
            fa[set][j] = __builtin_bit_cast(frag8, base[(a_row0 + j * MF) * 8 + chunk]);
#pragma unroll
        for (int i = 0; i < FN; ++i)
            fb[set][i] = __builtin_bit_cast(frag8, base[A_UNITS + (b_row0 + i * MF) * 8 + chunk]);
    };
    auto mfmas = [&](int set) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                if constexpr (MF == 32)
                    acc[i][j] = Elt::mfma(fb[set][i], fa[set][j], acc[i][j]);
                else
                    acc[i][j] = Elt::mfma16(fb[set][i], fa[set][j], acc[i][j]);
    };
    // One MFMA, then one fragment read and one global load while any remain
    // (scheduling-group masks: 0x008 MFMA, 0x100 LDS read, 0x020 global read).
    auto interleave = [&](auto n_reads, auto n_loads) {
        constexpr int R = decltype(n_reads)::value, V = decltype(n_loads)::value;
#pragma unroll
        for (int m = 0; m < FM * FN; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (m < V) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };
    using Reads = std::integral_constant<int, FM + FN>;
    using Loads = std::integral_constant<int, A_DMA + B_DMA>;
    using None = std::integral_constant<int, 0>;

    // ---- prologue: tiles 0 .. NS-1 issued, tile 0 landed ------------------------
    const int npro = min(nseq, NS);
    if (!HELP || loader) {
        for (int j = 0; j < npro; ++j) load_step(j, j);
        if (nseq > NS)
            wait_global_loads<(NS - 1) * L>();   // all NS prologue tiles are full ones
        else
            wait_global_loads<0>();
    }
    __syncthreads();
    if constexpr (HELP) {
        if (loader) {
            // The compute waves' k-loop below without the fragment reads and
            // MFMAs: the same waits before the same barriers, the same loads
            // after them.
            int sl = 0;
            int il = 0;
            for (; il + NS < nfull; ++il) {
                wait_global_loads<(NS - 2) * L>();
                __syncthreads();
                dma_tile(il + NS, sl);
                sl = (sl + 1 == NS) ? 0 : sl + 1;
            }
            for (; il < nseq; ++il) {
                wait_global_loads<0>();
                __syncthreads();
                if (il + NS < nseq) load_step(il + NS, sl);
                sl = (sl + 1 == NS) ? 0 : sl + 1;
            }
            return;
        }
    }
    read_frags(0, kg, 0);

    // ---- steady state: one basic block per k-tile ----------------------------------
    // (A) kk1 reads under kk0 MFMAs, (B) kk2 reads under kk1, (C) kk3 reads
    // under kk2; then tile i+1 must have landed (at most NS-2 younger tiles of
    // this wave still in flight) and every wave must be done with stage s:
    // wait, barrier; (D) tile i+NS's loads into stage s and the next stage's
    // kk0 reads under the kk3 MFMAs.  MF = 16 has two sub-steps: (A), then the
    // wait and barrier, then (D) under the kk1 MFMAs.
    int i = 0;
    int s = 0;                               // stage of tile i
    for (; i + NS < nfull; ++i) {
        const int sn = (s + 1 == NS) ? 0 : s + 1;
        if constexpr (KS == 1 && MF == 16) {
            read_frags(s, 1, 1);
            mfmas(0);
            interleave(Reads{}, None{});
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (KS == 1) {
            read_frags(s, 1, 1);
            mfmas(0);
            interleave(Reads{}, None{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(s, 2, 0);
            mfmas(1);
            interleave(Reads{}, None{});
            __builtin_amdgcn_sched_barrier(0);
            read_frags(s, 3, 1);
            mfmas(0);
            interleave(Reads{}, None{});
            __builtin_amdgcn_sched_barrier(0);
        } else {
            read_frags(s, kg + 2, 1);
            mfmas(0);
            interleave(Reads{}, None{});
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!HELP) wait_global_loads<(NS - 2) * L>();
        __syncthreads();
        if constexpr (!HELP) dma_tile(i + NS, s);
        read_frags(sn, kg, 0);
        mfmas(1);
        if constexpr (HELP)
            interleave(Reads{}, None{});
        else
            interleave(Reads{}, Loads{});
        __builtin_amdgcn_sched_barrier(0);
        s = sn;
    }
    // ---- the last steps (every condition spelled out, full waits) -------------------
    for (; i < nseq; ++i) {
        const int sn = (s + 1 == NS) ? 0 : s + 1;
        if constexpr (KS == 1 && MF == 16) {
            read_frags(s, 1, 1);
            mfmas(0);
        } else if constexpr (KS == 1) {
            read_frags(s, 1, 1);
            mfmas(0);
            read_frags(s, 2, 0);
            mfmas(1);
            read_frags(s, 3, 1);
            mfmas(0);
        } else {
            read_frags(s, kg + 2, 1);
            mfmas(0);
        }
        if constexpr (!HELP) wait_global_loads<0>();
        __syncthreads();
        if constexpr (!HELP) {
            if (i + NS < nseq) load_step(i + NS, s);
        }
        if (i + 1 < nseq) read_frags(sn, kg, 0);
        mfmas(1);
        s = sn;
    }

    // ---- k-groups: group 1 hands its partial sums to group 0 through LDS ----------
    if constexpr (KS > 1) {
        __syncthreads();                 // every wave is done reading the stages
        float* red = reinterpret_cast<float*>(smem);
        if (kg == 1) {
#pragma unroll
            for (int i2 = 0; i2 < FN; ++i2)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        red[((wmn * FN * FM + i2 * FM + j) * 16 + e) * 64 + lane] = acc[i2][j][e];
        }
        __syncthreads();
        if (kg == 1) {
            // the single-kernel k-split reduction's barriers are taken by every wave
            if constexpr (SK) {
                if (p.splits > 1 && p.split_algo != 0)
                    splitk_arrive(p, acc, 0, 0, 0, NMN, lane, false, splitk_flag);
            }
            return;
        }
#pragma unroll
        for (int i2 = 0; i2 < FN; ++i2)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[i2][j][e] += red[((wmn * FN * FM + i2 * FM + j) * 16 + e) * 64 + lane];
    }

    // ---- k-split: partial sums out; the split that completes a block sums them --------
    if constexpr (SK) {
        if (p.splits > 1) {
            constexpr int SLOT = FN * FM * ACC * 64;
            if (p.split_algo == 0) {   // a second kernel sums the partials
                store_partial<0>(acc, partial_slot(p, tile, split, wmn, NMN, SLOT), lane);
                return;
            }
            if (!splitk_arrive(p, acc, tile, split, wmn, NMN, lane, true, splitk_flag)) return;
        }
    }

    // ---- epilogue: fp32 -> fp16 / bf16 (RNE), masked stores ---------------------------
    // A 64-column wave tile goes through 4 KB of LDS per wave: with k-groups
    // in the wave's own part of the partial-sum area (which only it reads),
    // otherwise at the start of the stages, which no wave reads any more
    // after the last k-step's barrier.
    int4_t* stage = (KS > 1 && MF == 32) ? smem + wmn * (FN * FM * 256) : smem + wmn * 256;
    gemm_epilogue<Elt, MF>(p, acc, m0 + wave_m * WTM, n0 + wave_n * WTN, lane, stage);
}

// The second kernel of a k-split launch with split_algo 0: one workgroup per
// output tile, laid out as gemm_kernel's k-group 0 (WM x WN waves), sums the
// tile's `splits` partials in split order, ((P_0 + P_1) + P_2) + ..., and
// stores the block with gemm_kernel's epilogue.  The slots are loaded G at a
// time (G * FN * FM * ACC floats per lane: 128 for every tile), all G in
// flight before their adds: a load-then-add loop waits one memory round trip
// per split.  A slot past the last split is loaded through an empty buffer
// descriptor (zeros, no memory access) and not added.
template <typename Elt, int BM, int BN, int WM, int WN, int MF>
__global__ __launch_bounds__(WM * WN * 64) void gemm_splitk_reduce_kernel(GemmParams p) {
    constexpr int NMN = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int ACC = MF == 32 ? 16 : 4;
    constexpr int SLOT = FN * FM * ACC * 64;
    constexpr int G = 128 / (FN * FM * ACC) > 8 ? 8 : 128 / (FN * FM * ACC);
    static_assert(G >= 1, "a slot fits the registers");
    typedef std::conditional_t<MF == 32, floatx16_t, floatx4_t> acc_t;
    __shared__ int4_t smem[NMN * 256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave_m = wave % WM, wave_n = wave / WM;
    const int tile = blockIdx.x;
    int64_t m0, n0;
    grouped_origin(p, tile, BM, BN, m0, n0);
    acc_t acc[FN][FM];
    load_partial<0, false>(acc, partial_slot(p, tile, 0, wave, NMN, SLOT), lane);
    for (int s0 = 1; s0 < p.splits; s0 += G) {
        acc_t v[G][FN][FM];
#pragma unroll
        for (int g = 0; g < G; ++g)
            load_partial<0, false>(v[g],
                                   s0 + g < p.splits ? partial_slot(p, tile, s0 + g, wave, NMN, SLOT)
                                                     : make_rsrc(p.ws, 0),
                                   lane);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (s0 + g < p.splits) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j) acc[i][j] += v[g][i][j];
            }
        }
    }
    gemm_epilogue<Elt, MF>(p, acc, m0 + wave_m * WTM, n0 + wave_n * WTN, lane, smem + wave * 256);
}

// The 256 x 256 rung with a ping-pong schedule (8 waves, 2 per SIMD).
//
// Same staging as above (swizzled K-contiguous rows, direct global -> LDS
// loads), but the two waves that share a SIMD never compete for the MFMA
// pipe: waves 0-3 (group 0, columns 0-127 of the tile) and waves 4-7 (group
// 1, columns 128-255) run the same loop one phase apart.  A phase is one
// barrier interval; in every phase one group issues the 32 MFMAs of a whole
// k-tile from fragments already in registers while the other reads the 24
// fragments of its next k-tile from LDS and issues global -> LDS loads.  On
// MI355X a CU's global -> LDS writes take LDS cycles that fragment reads then
// wait for, and a CU takes in 64 bytes per clock, so issuing a k-tile's 64 KB
// stalls the issuing wave for about a phase; here neither delay reaches the
// MFMA pipe, and each group's barrier falls inside the other's MFMA stream.
//
// The LDS (160 KB) holds A in two 32 KB stages and B in three, so that every
// load goes into a stage that is already free when it is issued and overlaps
// the issuing group's fragment reads; each group issues half a k-tile per
// read phase.  Timeline (P = barrier interval; A of tile t in A stage t % 2,
// B in B stage t % 3):
//   group 0: P 2t   loads A(t+1), reads tile t    | P 2t+1 MFMAs of tile t,
//                                                    then waits for A(t+1)
//   group 1: P 2t+1 loads B(t+2), reads tile t,   | P 2t+2 MFMAs of tile t
//                   then waits for B(t+1)
// A(t+1) goes into the stage of A(t-1) and B(t+2) into that of B(t-1), whose
// last reads (group 1's) ended with P 2t-1; both are complete before group 0
// reads tile t+1 in P 2t+2.  Group 1 takes one extra barrier before its loop
// and group 0 one after it, so every wave executes the same number of
// barriers.
constexpr int kPpLdsUnits = 2 * 256 * 8 + 3 * 256 * 8;   // 160 KB of 16-byte units

// One 256 x 256 output tile of the ping-pong kernel: w is the tile's
// workgroup index in a one-workgroup-per-tile launch (the persistent form
// passes each tile it visits in turn).
template <typename Elt>
__device__ __forceinline__ void gemm_pp_tile(const GemmParams& p, const int w, int4_t* smem) {
    typedef typename Elt::frag8 frag8;
    constexpr int BM = 256, BN = 256, BK = kBK;
    constexpr int WTM = 128, WTN = 64;          // per wave: 2 x 4 waves
    constexpr int FM = WTM / 16, FN = WTN / 16;   // 16 x 16 MFMA tiles per wave
    constexpr int A_UNITS = BM * 8, B_UNITS = BN * 8;   // 16-byte LDS units per stage
    constexpr int B_BASE = 2 * A_UNITS;                 // A stages first, then B stages
    constexpr int DMA = 8;                      // loads per operand k-tile per wave: 64 rows
    static_assert(2 * A_UNITS + 3 * B_UNITS == kPpLdsUnits, "LDS layout");

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 2;
    const int wave_m = wave & 1;
    const int wave_n = wave >> 1;
    const int lw = wave & 3;                    // loader index within the group

    // ---- workgroup -> output tile ---------------------------------------------------
    // The dispatcher deals workgroup ids round-robin over the XCDs (32 CUs
    // each), one workgroup per CU at a time.  When the tile grid is made of
    // 16 x 16 blocks and there are 8 XCDs, the 256 workgroups in flight at once
    // cover one such block: XCD x takes its 4 x 8 part (x % 4, x / 4), so each
    // XCD's L2 serves 4 A and 8 B row bands and every band is shared by 2 or 4
    // XCDs through the Infinity Cache; blocks are visited row by row.  Other
    // grids use the grouped order of gemm_kernel.
    const int nwg = p.gm * p.gn;
    int64_t m0, n0;
    if (p.nxcd == 8 && (p.gm & 15) == 0 && (p.gn & 15) == 0) {
        const int x = w & 7, idx = w >> 3;      // idx-th workgroup of XCD x
        const int blk = idx >> 5, k = idx & 31;
        const int bn = p.gn >> 4;
        const int bm_ = blk / bn, bn_ = blk - bm_ * bn;
        m0 = (int64_t)(bm_ * 16 + (x & 3) * 4 + (k & 3)) * BM;
        n0 = (int64_t)(bn_ * 16 + (x >> 2) * 8 + (k >> 2)) * BN;
    } else {
        int logical = w;
        if (p.nxcd > 1) {
            const int xcd = w % p.nxcd, q = nwg / p.nxcd, r = nwg % p.nxcd;
            logical = xcd * q + min(xcd, r) + w / p.nxcd;
        }
        const int group_span = kGroupM * p.gn;
        const int g = logical / group_span;
        const int first_m = g * kGroupM;
        const int gsz = min(p.gm - first_m, kGroupM);
        const int within = logical - g * group_span;
        m0 = (int64_t)(first_m + within % gsz) * BM;
        n0 = (int64_t)(within / gsz) * BN;
    }

    const int rows_a = (int)min((int64_t)BM, (int64_t)p.M - m0);
    const int rows_b = (int)min((int64_t)BN, (int64_t)p.N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.A + m0 * p.lda, (uint32_t)((int64_t)rows_a * p.lda * 2));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.B + n0 * p.ldb, (uint32_t)((int64_t)rows_b * p.ldb * 2));

    // Load j of loader lw fills LDS units [(8 lw + j) * 64, +64): rows
    // 64 lw + 8 j + lane/8 at swizzled position lane % 8.  The row offset
    // stays in the lane offset (vaddr), which the buffer range check covers,
    // so rows past M or N read as zero.
    uint32_t voff_a[DMA], voff_b[DMA];
    int chk[DMA];
#pragma unroll
    for (int j = 0; j < DMA; ++j) {
        const int row = lw * 64 + j * 8 + (lane >> 3);
        chk[j] = (lane & 7) ^ swz_pp(row);
        voff_a[j] = (uint32_t)(row * p.lda * 2 + chk[j] * 16);
        voff_b[j] = (uint32_t)(row * p.ldb * 2 + chk[j] * 16);
    }

    const int nfull = p.K / BK;
    const int ktail = p.K - nfull * BK;
    const int kmask = p.stagger ? (nfull - 1) : 0x7fffffff;
    const int k0 = p.stagger ? (w & (nfull - 1)) : 0;

    floatx4_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;

    // v_mfma_f32_16x16x32: lane l supplies row l % 16 of a 16-row block, k
    // 8 (l / 16) .. + 7 of a 32-deep half k-tile: chunk 4 h + l / 16 of the row.
    // Rows of one lane differ by multiples of 16, so their swizzle is the same.
    const int frow = lane & 15;
    const int fsw = swz_pp(frow);
    const int fq = lane >> 4;
    const int a_row0 = wave_m * WTM + frow;
    const int b_row0 = wave_n * WTN + frow;
    frag8 fa[2][FM], fb[2][FN];                 // both 32-deep halves of one k-tile
    // Fragments of one k-tile from A stage sa and B stage sb.
    auto read_tile = [&](int sa, int sb) {
        const int4_t* abase = smem + sa * A_UNITS;
        const int4_t* bbase = smem + B_BASE + sb * B_UNITS;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int chunk = (4 * h + fq) ^ fsw;
#pragma unroll
            for (int j = 0; j < FM; ++j)
                fa[h][j] = __builtin_bit_cast(frag8, abase[(a_row0 + j * 16) * 8 + chunk]);
#pragma unroll
            for (int i = 0; i < FN; ++i)
                fb[h][i] = __builtin_bit_cast(frag8, bbase[(b_row0 + i * 16) * 8 + chunk]);
        }
    };
    // One group's loads of one operand's full k-tile (8 per wave) into a stage.
    auto dma_a = [&](int step, int sa) {
        int4_t* base = smem + sa * A_UNITS;
        const int soff = ((k0 + step) & kmask) * (BK * 2);
#pragma unroll
        for (int j = 0; j < DMA; ++j) dma16(ra, base + (lw * DMA + j) * 64, voff_a[j], soff);
    };
    auto dma_b = [&](int step, int sb) {
        int4_t* base = smem + B_BASE + sb * B_UNITS;
        const int soff = ((k0 + step) & kmask) * (BK * 2);
#pragma unroll
        for (int j = 0; j < DMA; ++j) dma16(rb, base + (lw * DMA + j) * 64, voff_b[j], soff);
    };
    // The 64 MFMAs of one k-tile.  D = B_frag . A_frag^T: lane l's four
    // accumulators are four consecutive n of output row m.
    auto mfma_tile = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[i][j] = Elt::mfma16(fb[h][i], fa[h][j], acc[i][j]);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- prologue: A(0), B(0), B(1) --------------------------------------------------
    if (grp == 1) {
        if (nfull > 0) {
            dma_a(0, 0);
            dma_b(0, 0);
        }
        if (nfull > 1) dma_b(1, 1);
        wait_global_loads<0>();
    }
    __syncthreads();
    if (grp == 1) __syncthreads();            // one phase behind group 0

    // ---- one full k-tile per iteration: read phase, then MFMA phase ---------------
    int sb = 0;                               // B stage of tile i (i % 3)
    for (int i = 0; i < nfull; ++i) {
        const int sa = i & 1;
        const int sb2 = (sb == 0) ? 2 : sb - 1;   // (i + 2) % 3
        if (grp == 0) {
            if (i + 1 < nfull) dma_a(i + 1, sa ^ 1);
        } else {
            if (i + 2 < nfull) dma_b(i + 2, sb2);
        }
        read_tile(sa, sb);
        // 8 loads and 24 fragment reads per wave, interleaved (masks: 0x020
        // global read, 0x100 LDS read).
#pragma unroll
        for (int m = 0; m < DMA; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
        if (grp == 1) {
            // B(i+1) (issued in the previous read phase) must be in LDS before
            // group 0 reads tile i+1 in the next phase; B(i+2) may stay in flight.
            if (i + 2 < nfull)
                wait_global_loads<DMA>();
            else
                wait_global_loads<0>();
        }
        // A __syncthreads here would be a release, which on this target also
        // waits for every direct-to-LDS load in flight.
        wait_lds();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        mfma_tile();
        if (grp == 0) wait_global_loads<0>();  // A(i+1), read by both groups next
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        sb = (sb == 2) ? 0 : sb + 1;
    }
    // Group 1 has taken one barrier more than group 0 (its extra one).  A
    // partial k-tile needs both groups in step: group 0 catches up first.
    // Otherwise group 0 stores while group 1 runs its last MFMA phase and
    // takes the matching barrier at the very end.
    if (grp == 0 && ktail > 0) __syncthreads();

    // ---- a partial last k-tile: every wave loads an eighth, masked, through
    // registers into A stage 0 and B stage 0 (all reads of the full tiles are
    // done and no load is in flight) -------------------------------------------------
    if (ktail > 0) {
        const int soff = nfull * (BK * 2);
#pragma unroll
        for (int r = 0; r < (A_UNITS + B_UNITS) / 512; ++r) {
            const int u = r * 512 + t;
            const bool is_a = u < A_UNITS;
            const int ul = is_a ? u : u - A_UNITS;
            const int row = ul >> 3;
            const int c = (ul & 7) ^ swz_pp(row);
            const uint32_t voff = (uint32_t)(row * (is_a ? p.lda : p.ldb) * 2 + c * 16);
            smem[is_a ? ul : B_BASE + ul] = is_a ? load16_tail(ra, voff, soff, ktail - c * 8)
                                                 : load16_tail(rb, voff, soff, ktail - c * 8);
        }
        __syncthreads();
        read_tile(0, 0);
        mfma_tile();
    }

    // ---- epilogue through 4 KB of LDS per wave, in A stage 1 (not used by the
    // partial k-tile; every read of the full k-tiles has completed) ----------------
    store_block_staged<Elt>(p, acc, m0 + wave_m * WTM, n0 + wave_n * WTN, lane,
                            smem + A_UNITS + wave * 256);
    if (grp == 0 && ktail == 0) __syncthreads();   // matches group 1's extra barrier
}

// The ping-pong kernel.  PERSIST = false: one workgroup per output tile.
// PERSIST = true (persistent workgroups, the FlyDSL PR's Changes): a grid of
// p.persistent workgroups, workgroup w taking tiles w, w + grid, w + 2 grid,
// ... in turn.  Each tile's barriers pair up between the two wave groups
// (above); a barrier between tiles lets every wave finish the previous
// tile's epilogue (in A stage 1) before group 1's prologue loads and group
// 0's first A load of the next tile go into the stages.
template <typename Elt, bool PERSIST = false>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmParams p) {
    __shared__ int4_t smem[kPpLdsUnits];   // 160 KB
    if constexpr (PERSIST) {
        const int ntile = p.gm * p.gn;
        for (int v = blockIdx.x; v < ntile; v += gridDim.x) {
            if (v != (int)blockIdx.x) __syncthreads();
            // The strides pass through an empty asm each tile, so the tile's
            // stride-derived load offsets are recomputed per tile instead of
            // hoisted out of the loop and held across it: 27 spilled VGPRs
            // instead of 34 (the per-tile code alone takes 250 of the 256 a
            // wave has at two waves per SIMD, so the loop's state spills).
            GemmParams q = p;
            asm volatile("" : "+s"(q.lda), "+s"(q.ldb));
            gemm_pp_tile<Elt>(q, v, smem);
        }
    } else {
        gemm_pp_tile<Elt>(p, blockIdx.x, smem);
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
