// Host-side launch decisions for the fp16 GEMM: the tile ladder, pick_tile,
// the k-loop stagger rule and argument validation.  Pure C++ (no HIP headers)
// so that every decision can be tested on a machine without a GPU.
#pragma once

#include <cstdint>

#include "sdt.h"

namespace sdt {

// k-tile depth shared by every rung: 64 fp16 = one 128-byte row segment.
constexpr int kBK = 64;

// A rung of the ladder.  waves_m x waves_n wavefronts split the bm x bn block;
// each wave owns a (bm/waves_m) x (bn/waves_n) sub-block of 32x32 (or, on the
// 16x16x32 pipelines, 16x16) MFMA tiles.
// A launch uses 2 (forced plans only), `stages` or `long_stages` LDS stages
// of (bm + bn) x 64 elements each (see plan_for); the global prefetch runs
// stages - 1 k-tiles deep.  A ping-pong
// rung's deep pipeline is its own kernel (gemm_pp_kernel): two wave groups
// one phase apart, A in two LDS stages and B in `stages` (three).
struct TileDesc {
    int bm, bn, waves_m, waves_n, stages;
    int kgroups;    // 2: also built with two k-groups of waves (see kgroups_for)
    int pingpong;   // 1: the deep pipeline is the ping-pong kernel
    int deep16;     // 1: the deep pipeline with one k-group runs 16x16x32 MFMAs
    int long_stages;  // > 0: a deeper pipeline for long k-loops (see kLongMinKTiles)
    int ksplit;     // 1: every pipeline also built to split K across workgroups
    // When the automatic plan runs two k-groups (kgroups == 2 only; see
    // kgroups_for_grid): with CUs left idle, a grid below kg2_grid8 / 8 of
    // the CUs and at least kg2_min_ktiles k-tiles; with one workgroup on
    // every CU, at least kg2_full_ktiles k-tiles (0: never).
    int kg2_min_ktiles, kg2_grid8, kg2_full_ktiles;
    // 1: the deep one-k-group 16x16x32 pipeline (the automatic plan's usual
    // pick on the rung) runs with a loader wave beside each compute wave,
    // which issues the global -> LDS loads (gemm_kernel's HELP); only where
    // both waves fit on a SIMD (at most 256 registers each).
    int helpers;
};

// Largest tile first.  The indices are the ABI's tile ids.  `stages` is the
// deep pipeline of the rung.  Below the largest rung, whose deep pipeline
// (2 A + 3 B stages) fills all 160 KB, 3 stages measured 1-6% faster than 4 or
// 6 on the squares up to 2048 (the longer prologue costs more than the deeper
// prefetch gains).  The two smallest rungs also have a 4-stage pipeline for
// long k-loops, where one k-tile's few MFMAs cannot cover the operand latency
// two tiles ahead (64x64 with two k-groups: 512x512x8192 24.2 against 30.2 us,
// 768x768x4096 14.5 against 17.5, 1024x1024x3072 13.2 against 15.2; 128x64
// at 1280x1280x4096: 22.1 against 23.1).
// The three smallest rungs can also split K across workgroups (the larger
// ones are picked when the grid already fills the CUs, and the 256 x 128
// wave tile has no registers left for the k-split sum).
//
// Two k-groups against one k-group of 16x16x32 MFMAs, fitted on MI355X
// (graph-timed, us, one k-group / two).  With loader waves (the one-k-group
// pipeline from 12 k-tiles on 256 x 128, 128 x 128 and 64 x 64) one k-group
// wins on the two larger rungs wherever two could run, CUs idle or not
// (2048x2560x4096 41.48 / 47.68, 3072x1536x4096 40.50 / 45.70, 2240^3
// 27.28 / 30.62, 1536x1792x4096 26.82 / 29.31, 1920^3 16.38 / 17.64,
// 1792^3 14.86 / 15.50, 1664^3 13.69 / 14.23, 1536x2048x1536 13.92 /
// 14.61), so they never plan two (kg2_grid8 = 0); before them, two won
// with CUs idle (1536^3 on 128 x 128, 144 workgroups: 14.8 / 13.7).  On
// 64 x 64 one k-group wins up to 24 k-tiles (768^2 x 1536 6.39 / 7.13,
// 512^2 x 1536 6.22 / 6.94) and two from 40 (1024^2 x 2560 11.44 / 10.58,
// 512^2 x 4096 17.07 / 14.70, 768^2 x 4096 17.05 / 14.60, 1024^2 x 4096
// 17.86 / 15.68), CUs idle or not.  On 128 x 64 one k-group wins
// up to 80 k-tiles (1280^3 9.34 / 10.32, 2048 x 1024 x 2048 13.52 / 14.82,
// 1152^2 x 5120 26.78 / 27.83) and two only on longer loops with a quarter
// of the CUs idle (1152^2 x 6144, 162 workgroups: 31.07 / 30.49; with 200
// workgroups one k-group still wins at 128 k-tiles, 39.68 / 40.38).
constexpr TileDesc kLadder[] = {
    // 8 waves, 128x64 per wave; 2 x 64 KB, or ping-pong 160 KB
    {256, 256, 2, 4, 3, 1, 1, 0, 0, 0, 0, 0, 0, 0},
    // 4 waves, 128x64 per wave, 3 x 48 KB
    {256, 128, 2, 2, 3, 2, 0, 1, 0, 0, 12, 0, 0, 1},
    // 4 waves, 64x64 per wave, 3 x 32 KB
    {128, 128, 2, 2, 3, 2, 0, 1, 0, 1, 12, 0, 0, 1},
    // 4 waves, 64x32 per wave, 3 (long: 4) x 24 KB (loaders measured mixed:
    // 4096x512x1024 7.93 / 7.49 us, 1280^3 9.30 / 9.62, 1152x1152x5120
    // 26.80 / 27.10)
    {128, 64, 2, 2, 3, 2, 0, 1, 4, 1, 96, 6, 0, 0},
    // 4 waves, 32x32 per wave, 3 (long: 4) x 16 KB
    {64, 64, 2, 2, 3, 2, 0, 1, 4, 1, 40, 8, 40, 1},
    // Off the ladder (see kNumLadder), 16x16x32 MFMAs on every pipeline (48
    // and 80 are no multiples of 32): 4 waves of 48x48, 3 x 24 KB; 8 waves of
    // 96x48, 3 x 48 KB; 4 waves of 80x80, 3 x 40 KB (loaders: 96 x 96 measured
    // even, 1536^3 11.18 / 11.18 us, 1440x1440x1000 10.64 / 10.79; the other
    // two have too many registers for them).
    {96, 96, 2, 2, 3, 1, 0, 1, 0, 0, 0, 0, 0, 0},
    {192, 192, 2, 4, 3, 1, 0, 1, 0, 0, 0, 0, 0, 0},
    {160, 160, 2, 2, 3, 1, 0, 1, 0, 0, 0, 0, 0, 0},
};

// Fewest full k-tiles at which a rung with a long pipeline uses it in place
// of its deep one (with two k-groups, which themselves need 12).  Fitted on
// MI355X with the operands in HBM (caches flushed before each launch, as in a
// benchmark step that streams other products in between, or for weights read
// once): 4 stages against 3, kernel-trace medians, 384x384x768 (12 k-tiles)
// 7.50 against 7.78 us, 768^3 7.56 / 8.12, 1024^3 8.72 / 9.24,
// 1024x1024x2048 13.28 / 14.92, 128x8192x1024 10.02 / 10.84.  Repeated on
// operands already in L2 the two tie within 4% either way (768^3 6.32 /
// 6.32, 1024^3 7.64 / 7.50, 384x384x768 6.12 / 5.88).
constexpr int kLongMinKTiles = 12;

// Shortest k-loop (in 64-deep k-tiles) that a second k-group of waves pays
// on: a grid resident all at once spends each k-tile on one chain of
// barrier, fragment reads and dependent MFMAs; splitting every tile's four
// sub-steps over two wave groups halves that chain (on 32x32x16 MFMAs,
// 1024^3: 7.05 -> 6.21 us, 1536^3: 15.8 -> 14.8 us) but costs a reduction
// through LDS that loops of 8 k-tiles or fewer do not earn back (256^3: 3.69
// -> 3.85 us).  Each rung's own thresholds (kLadder) sit at or above it.
constexpr int kSplitMinKTiles = 12;

// Largest operand footprint, 2*K*(M+N) bytes, and fewest full k-tiles at
// which the automatic plan staggers the k-loop (rungs other than the ping-pong
// kernel, power-of-two k-tile count).  Fitted on MI355X: with A and B within
// 16 MiB the stagger spreads the workgroups' concurrent row reads over
// different k-offsets and buys 2-5% (2048^3 19.5 against 20.6 us,
// 1024x1024x4096 17.5 against 18.2); past it it breaks the workgroups' shared
// k-window in L2 and costs up to 49% (2048x2048x8192), and on the ping-pong
// kernel 9% at 4096^3.  Below 16 k-tiles it measured neutral.
constexpr int64_t kStaggerMaxOperandBytes = int64_t(16) << 20;
constexpr int kStaggerMinKTiles = 16;

// Most workgroups one output tile's k-loop is split over.
constexpr int kMaxSplits = 64;
// Fewest full k-tiles per split the automatic plan keeps.  Fitted on MI355X
// (graph-timed sweep of every k-split rung, count, reduction and pipeline):
// a split pays only where each workgroup's k-loop is long -- 128x128x65536
// 162 -> 20 us, 256x256x16384 43.8 -> 13-16, 384x384x12288 36.8 -> 15.5,
// 512x512x8192 24.5 -> 13.3 -- and loses everywhere with shorter loops
// (1024^3 6.0 -> 11.6 at best, 1536^3 13.8 -> 22.6, 512^3 4.5 -> 6.9): the
// partial sums make a second round trip through memory and the reduction
// a second launch or a fence, which only a long k-loop earns back.
constexpr int kSplitAutoMinKTiles = 16;
// Most splits the automatic plan takes: the second kernel sums a tile's
// partials in one workgroup, so its time grows with the count
// (128x128x65536: 16 splits 24 us, 64 splits 32 us).
constexpr int kMaxSplitsAuto = 16;
// How the automatic plan reduces a k-split: 0, a second kernel.  The
// single-kernel reduction (1) measured slower at the grid sizes the plan
// makes (512x512x8192 split 4: 16.0 against 13.3 us; 256x256x16384 split 16:
// 16.2 against 14.3): its agent-scope release fence writes back the XCD's L2
// once per workgroup.
constexpr int kSplitAlgoAuto = 0;
// Bytes at the start of a k-split workspace that hold the arrival counters
// (one int per output tile: at most 16384 tiles).
constexpr int64_t kCounterBytes = 64 * 1024;

// How one product is launched: rung, LDS stages, k-groups of waves, k-loop
// stagger; k-split across workgroups (splits per tile and how the partial
// sums are reduced: 0 a second kernel, 1 the last workgroup of each tile);
// persistent workgroups (ping-pong rung: 0 off, else the grid size).
struct Plan {
    int tile, stages, kgroups, stagger;
    int splits = 1, split_algo = 0, persistent = 0;
    int loaders = 0;   // 1: the rung's loader-wave pipeline (gemm_kernel's HELP)
};

// Fewest full k-tiles at which the automatic plan runs a loader-wave rung's
// deep one-k-group pipeline with its loader waves.  Fitted on MI355X
// (graph-timed, us, without / with loaders, same bits, three boxes): from 12
// k-tiles they win on the three rungs built with them -- 256 x 128:
// 4096x2048x2048 36.88 / 32.20, 4096x2048x4096 66.70 / 57.35, 8192x1024x1024
// 21.33 / 20.12, 2048x4096x1024 21.62 / 19.54; 128 x 128: 2048^3
// 21.36 / 18.61, 2048x2048x1920 21.00 / 18.44, x2304 24.26 / 20.90,
// 1024x4096x4096 38.45 / 33.09, 4096x1024x1024 11.93 / 10.83; 64 x 64:
// 768^3 5.00 / 4.85, 1024^3 5.97 / 5.64, 384x384x768 4.84 / 4.63,
// 256x4096x1024 5.85 / 5.49, 768x768x1280 6.48 / 5.88 -- and on shorter
// loops the extra waves cost more than they take off the compute waves
// (256^3 3.33 / 3.52, 512x2048x512 4.45 / 4.53).
constexpr int kLoaderMinKTiles = 12;

// Fewest full k-tiles at which pick_tile takes the 256 x 128 rung (with loader
// waves) in place of the ping-pong kernel when the latter's grid is between
// one and one and a half waves of workgroups, and between two and two and a
// quarter (see pick_tile).
constexpr int kPastOneWaveMinKTiles = 32;
constexpr int kPastTwoWavesMinKTiles = 64;
constexpr int kNumTiles = sizeof(kLadder) / sizeof(kLadder[0]);
// Rungs 0 .. kNumLadder-1 form the ladder pick_rung walks (largest first).
// The rungs after them are off the ladder: pick_tile takes one in place of the
// ladder's pick when its smaller tile turns a grid that leaves CUs idle into
// more workgroups that still fit one per CU (see pick_tile).
constexpr int kNumLadder = 5;

// Largest leading dimension accepted: a workgroup addresses its operand rows
// through one buffer descriptor with 32-bit byte offsets below 2^31.
constexpr int64_t kMaxLd = (int64_t(1) << 22) - 64;

// The [K][N] decode GEMV split over K (gemv_f16_m1_kn_ws): bands of
// kKnSplitSeg * 8 columns (512-byte runs of every weight row) read by
// workgroups of kKnSplitWaves waves, each over kc rows, until about
// kKnSplitTargetWgs workgroups stream at once; a second kernel adds the
// splits' fp32 column sums in split order.  Fitted on MI355X at the decode
// shape (K = 4096, N = 12288, weights in HBM): runs of 128 bytes per row, the
// one-launch kernel's, read at most 5.46 TB/s however many workgroups read
// them, runs of 512 bytes 6.29 TB/s; the split kernel alone streams in
// 16.2 us with 768 workgroups (384: 17.9, 1536: 20.9), 18.6 us with the sum.
constexpr int kKnSplitSeg = 32;
constexpr int kKnSplitWaves = 8;
constexpr int kKnSplitTargetWgs = 768;
struct KnSplit {
    int splits;        // 1: no split (the one-launch kernel)
    int kc;            // rows per split, a multiple of 8
    int64_t bands;     // workgroups along N
    int64_t pstride;   // floats per split in the workspace (bands * band width)
    int64_t bytes;     // workspace bytes (0 without a split)
};
KnSplit kn_split_plan(int64_t N, int64_t K);

// Whether a plan runs its rung's pipeline with loader waves (the rung's
// `helpers`, its deep pipeline, one k-group, no k-split, no long pipeline).
sdt_tile describe(const Plan& p);
sdt_tile describe_rung(int id);
int64_t workspace_bytes(const Plan& p, int64_t M, int64_t N);
int64_t counter_bytes(const Plan& p, int64_t M, int64_t N);
int splits_for(const Plan& p, int64_t M, int64_t N, int64_t K, int num_cu);
bool stagger_auto(int id, int64_t M, int64_t N, int64_t K);
int long_for(int id, int stages, int kgroups, int64_t K);
int kgroups_for(int id, int64_t M, int64_t N, int64_t K, int num_cu);
int kgroups_for_grid(int id, int64_t wgs, int64_t nkt, int num_cu);
int kgroups_for_split(int id, int64_t wgs, int64_t nkt, int num_cu);
int resolve_plan(const sdt_launch& cfg, int64_t M, int64_t N, int64_t K, int num_cu,
                 int64_t ws_bytes, Plan* out);
Plan plan_for(int id, int64_t M, int64_t N, int64_t K, int num_cu);
int check_plan(const Plan& p, int64_t K);
int pick_rung(int64_t M, int64_t N, int ref_bm, int ref_bn, int rungs,
              const int64_t* min_blocks);
int pick_tile(int64_t M, int64_t N, int64_t K, int num_cu);
bool stagger_eligible(int64_t K);
int check_gemv_kn_args(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                       const void* y);
bool is_pow2(int64_t v);
int64_t ceil_div(int64_t a, int64_t b);
bool sizes_supported(int64_t M, int64_t N, int64_t K);
int check_gemm_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                    const void* B, int64_t ldb, const void* C, int64_t ldc);

}  // namespace sdt
