// Host-side launch decisions (see launcher.hpp).  No HIP dependency.
#include "launcher.hpp"

#include <algorithm>
#include <climits>
#include <cstdint>

namespace sdt {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Every size a kernel takes is an int, and block counts are products of two
// of them: M, N and K up to 2^31 - 1 keep those within int64_t.
bool sizes_supported(int64_t M, int64_t N, int64_t K) {
    return M <= INT_MAX && N <= INT_MAX && K <= INT_MAX;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Whether a plan's pipeline can run with loader waves: a rung built with
// them, its deep pipeline, one k-group, no k-split.
bool loaders_possible(const Plan& p) {
    const TileDesc& d = kLadder[p.tile];
    return d.helpers && p.kgroups == 1 && p.stages == d.stages && p.splits <= 1;
}

bool loaders_auto(const Plan& p, int64_t K) {
    return loaders_possible(p) && K / kBK >= kLoaderMinKTiles;
}

sdt_tile describe(const Plan& p) {
    const TileDesc& d = kLadder[p.tile];
    sdt_tile t;
    t.id = p.tile;
    t.bm = d.bm;
    t.bn = d.bn;
    t.bk = kBK;
    t.waves_m = d.waves_m;
    t.waves_n = d.waves_n;
    t.threads = 64 * d.waves_m * d.waves_n * p.kgroups * (p.loaders ? 2 : 1);
    t.kgroups = p.kgroups;
    t.stages = p.stages;
    t.lds_bytes = (d.pingpong && p.stages == d.stages)
                      ? (2 * d.bm + d.stages * d.bn) * kBK * 2   // A in 2 stages, B in `stages`
                      : p.stages * (d.bm + d.bn) * kBK * 2;
    t.stagger = p.stagger;
    t.long_stages = d.long_stages;
    t.splits = p.splits;
    t.split_algo = p.splits > 1 ? p.split_algo : 0;
    t.persistent = p.persistent;
    t.ksplit = d.ksplit;
    t.loaders = p.loaders;
    return t;
}

// The rung as built: its deep pipeline and the most k-groups it has.
sdt_tile describe_rung(int id) {
    Plan p;
    p.tile = id;
    p.stages = kLadder[id].stages;
    p.kgroups = kLadder[id].kgroups;
    p.stagger = 0;
    sdt_tile t = describe(p);
    t.loaders = kLadder[id].helpers;
    return t;
}

// Workspace of a k-split launch: the arrival-counter area (a fixed
// kCounterBytes at the start, whatever the shape, so that no launch's partial
// sums ever land where another keeps counters: counters stay zero between
// launches), then the fp32 partial sums (splits slots of bm x bn per tile).
// Zero without a split.
int64_t counter_bytes(const Plan& p, int64_t, int64_t) {
    return p.splits <= 1 ? 0 : kCounterBytes;
}

int64_t workspace_bytes(const Plan& p, int64_t M, int64_t N) {
    if (p.splits <= 1) return 0;
    const TileDesc& d = kLadder[p.tile];
    const int64_t tiles = ceil_div(M, d.bm) * ceil_div(N, d.bn);
    return kCounterBytes + tiles * p.splits * int64_t(d.bm) * d.bn * 4;
}

// k-split of the automatic plan when a workspace is available: on a rung
// built for it, while the grid leaves CUs idle, as many splits as keep the
// grid within the CU count, each with at least kSplitAutoMinKTiles full
// k-tiles (at most kMaxSplitsAuto).  1 = no split.
int splits_for(const Plan& p, int64_t M, int64_t N, int64_t K, int num_cu) {
    const TileDesc& d = kLadder[p.tile];
    if (!d.ksplit || p.stagger) return 1;
    if (num_cu <= 0) num_cu = 256;
    const int64_t tiles = ceil_div(M, d.bm) * ceil_div(N, d.bn);
    if (tiles <= 0) return 1;   // an empty product (M or N zero): nothing to split
    const int64_t nfull = K / kBK;
    int64_t s = num_cu / tiles;
    if (s > nfull / kSplitAutoMinKTiles) s = nfull / kSplitAutoMinKTiles;
    if (s > kMaxSplitsAuto) s = kMaxSplitsAuto;
    return s >= 2 ? (int)s : 1;
}

// Two k-groups on a rung built with them, when its grid is resident all at
// once (at most one workgroup per CU) and the k-loop is long enough.
int kgroups_for(int id, int64_t M, int64_t N, int64_t K, int num_cu) {
    const TileDesc& d = kLadder[id];
    return kgroups_for_grid(id, ceil_div(M, d.bm) * ceil_div(N, d.bn), ceil_div(K, kBK), num_cu);
}

// The same rule for a grid of `wgs` workgroups each running `nkt` k-tiles.
int kgroups_for_grid(int id, int64_t wgs, int64_t nkt, int num_cu) {
    const TileDesc& d = kLadder[id];
    if (d.kgroups < 2) return 1;
    if (num_cu <= 0) num_cu = 256;
    if (nkt < kSplitMinKTiles) return 1;
    // The one-k-group pipeline runs 16x16x32 MFMAs, whose lower energy per
    // FLOP wins where the part runs at its power limit and whose shorter
    // dependent chain per k-tile (two 32-deep MFMAs per accumulator instead
    // of four 16-deep ones) wins on short loops; the second k-group halves
    // the chain, which pays on long loops with CUs left idle.  The rung's
    // thresholds (kLadder) are fitted per rung.
    if (wgs == num_cu) return d.kg2_full_ktiles > 0 && nkt >= d.kg2_full_ktiles ? 2 : 1;
    return 8 * wgs < int64_t(d.kg2_grid8) * num_cu && nkt >= d.kg2_min_ktiles ? 2 : 1;
}

// The k-group rule for a k-split grid, whose workgroups store partial sums
// instead of C: two k-groups whenever the grid fits the CUs (on the 256 x 128
// and 128 x 128 rungs, leaves some idle) and each split runs 12 k-tiles or
// more.  On the 64 x 64 rung the one-k-group 16x16x32 pipeline that wins
// unsplit lost here (512^2 x 8192 in 4 splits of 32 k-tiles, 256 workgroups:
// 15.24 against 14.06 us with two k-groups).
int kgroups_for_split(int id, int64_t wgs, int64_t nkt, int num_cu) {
    const TileDesc& d = kLadder[id];
    if (d.kgroups < 2 || nkt < kSplitMinKTiles) return 1;
    if (num_cu <= 0) num_cu = 256;
    return (d.long_stages > 0 ? wgs <= num_cu : wgs < num_cu) ? 2 : 1;
}

// The rung's long pipeline in place of its deep one when it has one, the
// launch runs two k-groups and the k-loop holds at least kLongMinKTiles full
// k-tiles; otherwise `stages`.  Only the two-k-group form was measured
// faster: one k-group is planned when the grid exceeds the CU count, where the
// fourth stage's LDS costs a co-resident workgroup per CU (128 x 64: 72 ->
// 96 KB, two workgroups per CU -> one).
int long_for(int id, int stages, int kgroups, int64_t K) {
    const TileDesc& d = kLadder[id];
    if (kgroups == 2 && stages == d.stages && d.long_stages > 0 && K / kBK >= kLongMinKTiles)
        return d.long_stages;
    return stages;
}

// The automatic plan on rung `id`: the rung's deep pipeline, which long_for
// swaps for its long one when two k-groups run a long k-loop.  The 2-stage
// pipeline is never planned: it never measured faster by more than 2% (256^3
// on operands in L2), and with the operands in HBM it lost by up to 38% even
// where they fit in one XCD's L2 (kernel-trace medians with caches flushed
// before each launch, 2 against 3 stages: 512^3 7.92 / 6.48 us, 640^3
// 9.36 / 7.34, 2048x2048x512 11.84 / 10.24, 4096x4096x256 16.76 / 14.68 with
// the ping-pong kernel; on operands in L2 5.44 / 5.44, 5.92 / 6.00,
// 9.68 / 9.20, 16.12 / 14.00).
Plan plan_for(int id, int64_t M, int64_t N, int64_t K, int num_cu) {
    const TileDesc& d = kLadder[id];
    Plan p;
    p.tile = id;
    p.kgroups = kgroups_for(id, M, N, K, num_cu);
    p.stages = long_for(id, d.stages, p.kgroups, K);
    p.stagger = stagger_auto(id, M, N, K) ? 1 : 0;
    p.loaders = loaders_auto(p, K) ? 1 : 0;
    return p;
}

bool stagger_auto(int id, int64_t M, int64_t N, int64_t K) {
    // the ladder's rungs other than the ping-pong kernel (the off-ladder rungs
    // were measured without it)
    if (id < 0 || id >= kNumLadder || kLadder[id].pingpong) return false;
    if (!stagger_eligible(K) || K / kBK < kStaggerMinKTiles) return false;
    return 2 * K * (M + N) <= kStaggerMaxOperandBytes;
}

// A plan the library has a kernel for: stages 2, the rung's deep count or its
// long count; two k-groups only on rungs built with them, and with the deep
// or long pipeline.
int check_plan(const Plan& p, int64_t K) {
    if (p.tile < 0 || p.tile >= kNumTiles) return SDT_ERR_INVALID_ARG;
    const TileDesc& d = kLadder[p.tile];
    const bool is_long = d.long_stages > 0 && p.stages == d.long_stages;
    if (p.stages != 2 && p.stages != d.stages && !is_long) return SDT_ERR_INVALID_ARG;
    if (p.kgroups != 1 && p.kgroups != 2) return SDT_ERR_INVALID_ARG;
    if (p.kgroups == 2 && (d.kgroups < 2 || (p.stages != d.stages && !is_long)))
        return SDT_ERR_INVALID_ARG;
    // k-split: rungs built for it, at most one split per full k-tile (and
    // kMaxSplits), never with the stagger
    if (p.splits < 1 || p.splits > kMaxSplits) return SDT_ERR_INVALID_ARG;
    if (p.splits > 1 && (!d.ksplit || p.splits > K / kBK || p.stagger)) return SDT_ERR_INVALID_ARG;
    if (p.split_algo != 0 && p.split_algo != 1) return SDT_ERR_INVALID_ARG;
    // persistent workgroups: the ping-pong kernel only
    if (p.persistent < 0 || (p.persistent > 0 && (!d.pingpong || p.stages != d.stages)))
        return SDT_ERR_INVALID_ARG;
    // loader waves: the pipelines built with them
    if (p.loaders != 0 && (p.loaders != 1 || !loaders_possible(p))) return SDT_ERR_INVALID_ARG;
    return SDT_OK;
}

// The plan a launch runs: gemm_f16's automatic plan (pick_tile, plan_for),
// with every field of cfg that is not -1 forced, and a k-split (splits_for)
// when the caller offers ws_bytes >= 0 bytes of workspace and it fits.
int resolve_plan(const sdt_launch& cfg, int64_t M, int64_t N, int64_t K, int num_cu,
                 int64_t ws_bytes, Plan* out) {
    if (!sizes_supported(M, N, K)) return SDT_ERR_UNSUPPORTED;
    if (cfg.tile_id < -1 || cfg.tile_id >= kNumTiles) return SDT_ERR_INVALID_ARG;
    if (cfg.stagger < -1 || cfg.stagger > 1) return SDT_ERR_INVALID_ARG;
    if (cfg.stages < -1 || cfg.kgroups < -1) return SDT_ERR_INVALID_ARG;
    if (cfg.splits < -1 || cfg.splits == 0 || cfg.splits > kMaxSplits) return SDT_ERR_INVALID_ARG;
    if (cfg.split_algo < -1 || cfg.split_algo > 1 || cfg.persistent < -1) return SDT_ERR_INVALID_ARG;
    if (cfg.loaders < -1 || cfg.loaders > 1) return SDT_ERR_INVALID_ARG;
    if (cfg.tile_id >= 0) {   // a forced rung: its forced fields must name a kernel it has
        const TileDesc& d = kLadder[cfg.tile_id];
        if (cfg.stages >= 0 && cfg.stages != 2 && cfg.stages != d.stages &&
            !(d.long_stages > 0 && cfg.stages == d.long_stages))
            return SDT_ERR_INVALID_ARG;
        if (cfg.kgroups >= 0 && cfg.kgroups != 1 && !(cfg.kgroups == 2 && d.kgroups == 2))
            return SDT_ERR_INVALID_ARG;
        if (cfg.kgroups == 2 && cfg.stages == 2 && d.stages != 2) return SDT_ERR_INVALID_ARG;
    } else if (cfg.stages >= 0 || cfg.kgroups >= 0) {
        if (cfg.stages > 4 || cfg.kgroups > 2) return SDT_ERR_INVALID_ARG;
    }
    if (cfg.stagger == 1 && !stagger_eligible(K)) return SDT_ERR_UNSUPPORTED;
    if (num_cu <= 0) num_cu = 256;
    const int id = cfg.tile_id >= 0 ? cfg.tile_id : pick_tile(M, N, K, num_cu);
    const TileDesc& d = kLadder[id];
    Plan pl = plan_for(id, M, N, K, num_cu);
    if (cfg.stagger != -1) pl.stagger = cfg.stagger;

    // k-split: forced, or taken by the automatic plan when the workspace holds it
    if (cfg.splits >= 1) {
        pl.splits = cfg.splits;
    } else if (ws_bytes > 0 && cfg.stagger != 1) {
        Plan t = pl;
        t.stagger = 0;
        t.splits = splits_for(t, M, N, K, num_cu);
        const int64_t counters = ceil_div(M, d.bm) * ceil_div(N, d.bn);
        if (t.splits > 1 && workspace_bytes(t, M, N) <= ws_bytes && counters <= kCounterBytes / 4)
            pl = t;
    }
    if (pl.splits > 1) {
        pl.stagger = cfg.stagger == 1 ? 1 : 0;
        // the split grid decides the k-groups and stages, as for any grid
        const int64_t wgs = ceil_div(M, d.bm) * ceil_div(N, d.bn) * pl.splits;
        const int64_t nkt = (K / kBK) / pl.splits;   // full k-tiles of the shortest split
        pl.kgroups = kgroups_for_split(id, wgs, nkt, num_cu);
        pl.stages = long_for(id, d.stages, pl.kgroups, K / pl.splits);
        pl.split_algo = cfg.split_algo >= 0 ? cfg.split_algo : kSplitAlgoAuto;
    }
    if (cfg.kgroups >= 0) {
        pl.kgroups = cfg.kgroups;
        if (cfg.stages < 0)
            pl.stages = long_for(id, d.stages, pl.kgroups, pl.splits > 1 ? K / pl.splits : K);
    }
    if (cfg.stages >= 0) pl.stages = cfg.stages;
    if (cfg.split_algo >= 0) pl.split_algo = cfg.split_algo;
    if (cfg.persistent >= 0) pl.persistent = cfg.persistent;
    // loader waves: forced, or the automatic rule on the plan as it now stands
    pl.loaders = cfg.loaders >= 0 ? cfg.loaders : (loaders_auto(pl, K) ? 1 : 0);
    int st = check_plan(pl, K);
    if (st != SDT_OK) return st;
    if (pl.persistent > ceil_div(M, d.bm) * ceil_div(N, d.bn)) return SDT_ERR_INVALID_ARG;
    // one arrival counter per tile must fit the counter area
    if (pl.splits > 1 && ceil_div(M, d.bm) * ceil_div(N, d.bn) > kCounterBytes / 4)
        return SDT_ERR_UNSUPPORTED;
    if (pl.splits > 1 && workspace_bytes(pl, M, N) > (ws_bytes < 0 ? 0 : ws_bytes))
        return SDT_ERR_INVALID_ARG;
    *out = pl;
    return SDT_OK;
}

// "Beating hipBLASLt on a Gaming GPU", section "The part that actually
// mattered": count how many reference-sized output blocks the grid produces
// (ceil division on both sides) and take the first rung whose threshold that
// count reaches; the last rung is the fallback.
int pick_rung(int64_t M, int64_t N, int ref_bm, int ref_bn, int rungs,
              const int64_t* min_blocks) {
    if (M < 0 || N < 0 || ref_bm <= 0 || ref_bn <= 0 || rungs <= 0 || !min_blocks ||
        !sizes_supported(M, N, 0))
        return -1;
    const int64_t blocks = ceil_div(M, ref_bm) * ceil_div(N, ref_bn);
    for (int r = 0; r < rungs; ++r)
        if (blocks >= min_blocks[r]) return r;
    return rungs - 1;
}

// MI355X rule, in the pages' form (thresholds on the count of reference-
// sized blocks, largest tile first).  Blocks are counted in units of the
// smallest rung (64x64), so a rung of area a*64*64 yields blocks/a
// workgroups on a shape its tile divides.  A rung qualifies once it yields
// more workgroups than half the CUs: on MI355X a large tile does about twice
// the work per CU of the next smaller ones (fewer L2 and LDS bytes per
// MFMA), so it stays ahead while it occupies over half the machine.  Fitted to
// a sweep of every rung over square shapes 256..8192 at 256 CUs; the larger
// rung is picked at 3072 (144 WGs of 256x256), 2560 (200 WGs of 256x128) and
// 1536 (144 WGs of 128x128), and the smaller at 2560 / 2048 / 1024, where the
// larger would leave half the CUs or more idle.
int pick_tile(int64_t M, int64_t N, int64_t K, int num_cu) {
    if (num_cu <= 0) num_cu = 256;
    int64_t thresholds[kNumLadder];
    for (int r = 0; r < kNumLadder; ++r) {
        const int64_t area = int64_t(kLadder[r].bm / 64) * (kLadder[r].bn / 64);
        thresholds[r] = area * (num_cu / 2 + 1);
    }
    thresholds[kNumLadder - 1] = 0;
    const int r = pick_rung(M, N, 64, 64, kNumLadder, thresholds);
    // The ping-pong grid just past one wave (more workgroups than CUs, at most
    // one and a half times as many): its second wave leaves most CUs idle,
    // while the 256 x 128 rung with loader waves, whose workgroup takes about
    // 0.55 of a ping-pong workgroup's time (8192^3: 98.7 against 179.4 us per
    // wave; 4096^3: 51.5 against 94.2), runs three waves of its twice as many
    // workgroups in less.  Fitted on MI355X (graph-timed, us, 256 x 256 /
    // 256 x 128 with loaders): 4352^3 (289 workgroups) 171.2 / 155.4, 4608^3
    // (324) 184.4 / 169.0, 4096x5120x4096 (320) 163.2 / 150.9, 8192x2560x4096
    // 162.8 / 150.3, 4096x6144x4096 (384) 169.4 / 162.6, 6144x4096x2048 93.0 /
    // 90.9; with 16 k-tiles a tie (4096x5120x1024: 51.05 / 51.11).  Nearer two
    // waves it loses (5120^3, 400: 210.3 / 242.5).  Just past two waves, up to
    // 2.25, it pays from 64 k-tiles (5888^2 x 8192, 529: 492.3 / 470.9,
    // 6656x5120x6144, 520: 375.7 / 360.5, 6144x5632x6144 376.4 / 363.2, 6144^3,
    // 576: 376.1 / 362.9, 6144^2 x 4096 260.2 / 257.1, 8192x4608x6144 378.0 /
    // 370.3) but not on 32 (6144^2 x 2048 139.2 / 142.8), and from about 2.4
    // waves it is even (6400^2 x 6144, 625: 388.1 / 386.5; x 8192 503.3 /
    // 505.4; x 4096 260.9 / 264.6).
    if (r == 0 && kLadder[1].helpers) {
        const int64_t b0 = ceil_div(M, kLadder[0].bm) * ceil_div(N, kLadder[0].bn);
        const int64_t nkt = K / kBK, cu = num_cu;
        if ((b0 > cu && 2 * b0 <= 3 * cu && nkt >= kPastOneWaveMinKTiles) ||
            (b0 > 2 * cu && 4 * b0 <= 9 * cu && nkt >= kPastTwoWavesMinKTiles))
            return 1;
    }
    // An off-ladder rung with a smaller tile whose grid is larger than the
    // pick's but still at most one workgroup per CU: every CU then runs one
    // smaller tile instead of some CUs idling while the others run a larger
    // one (the first such rung in id order).  Fitted on MI355X: the 96 x 96
    // rung in place of 128 x 128 at 1536^3 14.5 -> 11.0 us, 1440^3 15.9 ->
    // 13.7, 1152x1920x2048 16.3 -> 13.8, 768x3072x4096 26.6 -> 23.4,
    // 1536x1536x12288 74.7 -> 62.2; with more workgroups than CUs it lost
    // (1664^3: 17.7 against 14.9, 1536x2048x1536: 17.0 against 14.9), and
    // in place of 128 x 64 (a smaller tile already) it did not pay.  The
    // 192 x 192 rung in place of the 256 x 256 ping-pong kernel: 3072^3
    // 54.2 -> 48.6, 2944^3 53.9 -> 46.8, 3072x3072x1024 23.4 -> 21.0,
    // 3072x3072x8192 131.9 -> 121.2, 3072x2816x4096 69.9 -> 61.3; with
    // 272 workgroups (3000x3104x1000) 41.2 against 28.1.  The 160 x 160 rung
    // in place of 256 x 128: 2560^3 36.7 -> 33.7, 2496^3 37.2 -> 33.8,
    // 2560x2560x1024 19.5 -> 17.1, 2560x2560x8192 101.3 -> 94.5,
    // 1280x5120x4096 52.1 -> 49.9; it lost 4% at 2304^3 (30.3 -> 31.5),
    // where the 256 x 128 grid has no ragged edge and the 160 x 160 one
    // does: at the power limit the extra padded work costs clock.
    //
    // The replacement's grid must also fill at least 7/8 of the CUs: below
    // that the measured outcomes of the 160 x 160 rung scattered by +-5% on
    // rectangular shapes (768x6144x4096, 195 workgroups: 46.1 against 44.0;
    // 3072x1536x4096, 200: 47.0 against 44.6; 2048x2560x4096, 208: 45.4
    // against 48.1), while from 7/8 up every shape measured gained or tied
    // but 2304^3 (225 workgroups: 31.5 against 30.3).
    //
    // Where the pick runs its loader-wave pipeline (K of at least
    // kLoaderMinKTiles full k-tiles on a rung built with them), a replacement
    // must also cut a workgroup's tile by a third: the 96 x 96 rung in place of
    // 128 x 128 still pays (1536^3 10.66 against 13.57 us, 1456x1456x2048
    // 13.71 against 16.16), the 160 x 160 one in place of 256 x 128 no longer
    // does (2560^3 33.42 against 30.78, 2304^3 30.53 against 26.93, 2496^3
    // 34.24 against 32.75, 2560x2560x1024 17.85 against 16.55, 2560x2560x8192
    // 95.44 against 86.72, 1280x5120x4096 52.00 against 46.09), with one shape
    // measured the other way (3000x2000x2000 35.14 against 36.51).
    const bool loaders = kLadder[r].helpers && K / kBK >= kLoaderMinKTiles;
    const int64_t br = ceil_div(M, kLadder[r].bm) * ceil_div(N, kLadder[r].bn);
    for (int c = kNumLadder; c < kNumTiles; ++c) {
        const int64_t bc = ceil_div(M, kLadder[c].bm) * ceil_div(N, kLadder[c].bn);
        const int64_t ac = int64_t(kLadder[c].bm) * kLadder[c].bn;
        const int64_t ar = int64_t(kLadder[r].bm) * kLadder[r].bn;
        if (ac < ar && br < bc && bc <= num_cu && 8 * bc >= 7 * int64_t(num_cu) &&
            (!loaders || 3 * ac <= 2 * ar))
            return c;
    }
    return r;
}

// FlyDSL PR, Changes: the k-loop stagger wraps with a mask over the full
// k-tiles, so it exists only when their count is a power of two (a partial
// last tile always runs last, outside the wrap).
bool stagger_eligible(int64_t K) { return K >= kBK && is_pow2(K / kBK); }

static bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int check_gemm_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                    const void* B, int64_t ldb, const void* C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return SDT_ERR_INVALID_ARG;
    if (lda < K || ldb < K || ldc < N) return SDT_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return SDT_OK;  // nothing to compute or write
    if (!C) return SDT_ERR_INVALID_ARG;
    if (K > 0 && (!A || !B)) return SDT_ERR_INVALID_ARG;
    // 16-byte vector loads and stores: aligned rows.  A stride only matters
    // when there is more than one row to step over.
    if (!aligned16(C) || (M > 1 && ldc % 8 != 0)) return SDT_ERR_UNSUPPORTED;
    if (K > 0) {
        if (!aligned16(A) || !aligned16(B)) return SDT_ERR_UNSUPPORTED;
        if ((M > 1 && lda % 8 != 0) || (N > 1 && ldb % 8 != 0)) return SDT_ERR_UNSUPPORTED;
        if (lda > kMaxLd || ldb > kMaxLd) return SDT_ERR_UNSUPPORTED;
    }
    return SDT_OK;
}

// The [K][N] decode product: K rows of ldb >= N weights.  Rows are read with
// 16-byte loads at column offsets that are multiples of 8, so B must be
// 16-byte aligned with ldb a multiple of 8 whenever there is a second row;
// the activations are read 8 at a time from a 16-byte aligned x.
KnSplit kn_split_plan(int64_t N, int64_t K) {
    KnSplit s{1, 0, 0, 0, 0};
    // (K at most INT_MAX / 2: a range's end, start + kc, stays an int)
    if (N <= 0 || K < 16 || N > INT_MAX || K > INT_MAX / 2) return s;
    const int64_t bw = int64_t(kKnSplitSeg) * 8;
    const int64_t bands = ceil_div(N, bw);
    int64_t splits = std::min(ceil_div(kKnSplitTargetWgs, bands), K / 8);
    if (splits < 2) return s;
    const int64_t kc = ceil_div(ceil_div(K, splits), 8) * 8;
    splits = ceil_div(K, kc);
    if (splits < 2) return s;
    s.splits = (int)splits;
    s.kc = (int)kc;
    s.bands = bands;
    s.pstride = bands * bw;
    s.bytes = splits * s.pstride * 4;
    return s;
}

int check_gemv_kn_args(int64_t N, int64_t K, const void* x, const void* B, int64_t ldb,
                       const void* y) {
    if (N < 0 || K < 0) return SDT_ERR_INVALID_ARG;
    if (K > 0 && ldb < N) return SDT_ERR_INVALID_ARG;
    if (N == 0) return SDT_OK;
    if (!y) return SDT_ERR_INVALID_ARG;
    if (K > 0 && (!x || !B)) return SDT_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(y) & 1u) != 0) return SDT_ERR_UNSUPPORTED;
    if (K > 0) {
        if (!aligned16(x) || !aligned16(B)) return SDT_ERR_UNSUPPORTED;
        if (K > 1 && ldb % 8 != 0) return SDT_ERR_UNSUPPORTED;
    }
    return SDT_OK;
}

}  // namespace sdt

// ---- host-only C ABI --------------------------------------------------------

extern "C" int sdt_pick_rung(int64_t M, int64_t N, int ref_bm, int ref_bn, int rungs,
                             const int64_t* min_blocks) {
    return sdt::pick_rung(M, N, ref_bm, ref_bn, rungs, min_blocks);
}

extern "C" int sdt_num_tiles(void) { return sdt::kNumTiles; }

extern "C" int sdt_abi_version(void) { return SDT_ABI_VERSION; }

extern "C" int sdt_tile_info(int tile_id, sdt_tile* out) {
    if (tile_id < 0 || tile_id >= sdt::kNumTiles || !out) return SDT_ERR_INVALID_ARG;
    *out = sdt::describe_rung(tile_id);
    return SDT_OK;
}

extern "C" int sdt_plan_tile(int tile_id, int64_t M, int64_t N, int64_t K, int num_cu,
                             sdt_tile* out) {
    if (tile_id < 0 || tile_id >= sdt::kNumTiles || M < 0 || N < 0 || K < 0 || !out)
        return SDT_ERR_INVALID_ARG;
    if (!sdt::sizes_supported(M, N, K)) return SDT_ERR_UNSUPPORTED;
    if (num_cu <= 0) num_cu = 256;
    *out = sdt::describe(sdt::plan_for(tile_id, M, N, K, num_cu));
    return SDT_OK;
}

extern "C" int sdt_stagger_eligible(int64_t K) { return sdt::stagger_eligible(K) ? 1 : 0; }

// FlyDSL PR, Changes: each workgroup starts at its own k-tile and wraps with
// a mask, one add and one and per trip.
extern "C" int64_t sdt_stagger_ktile(int64_t wg, int64_t i, int64_t nkt) {
    if (!sdt::is_pow2(nkt) || wg < 0 || i < 0) return -1;
    return (wg + i) & (nkt - 1);
}

extern "C" int64_t sdt_gemv_kn_workspace_size(int64_t N, int64_t K) {
    if (N < 0 || K < 0) return -1;
    return sdt::kn_split_plan(N, K).bytes;
}

extern "C" int sdt_check_gemv_kn_args(int64_t N, int64_t K, const void* x, const void* B,
                                      int64_t ldb, const void* y) {
    return sdt::check_gemv_kn_args(N, K, x, B, ldb, y);
}

extern "C" int sdt_check_gemm_args(int64_t M, int64_t N, int64_t K, const void* A,
                                   int64_t lda, const void* B, int64_t ldb,
                                   const void* C, int64_t ldc) {
    return sdt::check_gemm_args(M, N, K, A, lda, B, ldb, C, ldc);
}

extern "C" const char* sdt_status_string(int status) {
    switch (status) {
        case SDT_OK: return "SDT_OK";
        case SDT_ERR_INVALID_ARG: return "SDT_ERR_INVALID_ARG: invalid argument";
        case SDT_ERR_UNSUPPORTED:
            return "SDT_ERR_UNSUPPORTED: misaligned pointer/stride or size limit";
        case SDT_ERR_HIP: return "SDT_ERR_HIP: HIP runtime error (see sdt_last_hip_error)";
        default: return "unknown sdt status";
    }
}
