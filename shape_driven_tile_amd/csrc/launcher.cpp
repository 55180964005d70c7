// Host-side launch decisions (see launcher.hpp).  No HIP dependency.
#include "launcher.hpp"

#include <cstdint>

namespace sdt {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

sdt_tile describe(int id, int stages, int kgroups, int stagger) {
    const TileDesc& d = kLadder[id];
    sdt_tile t;
    t.id = id;
    t.bm = d.bm;
    t.bn = d.bn;
    t.bk = kBK;
    t.waves_m = d.waves_m;
    t.waves_n = d.waves_n;
    t.threads = 64 * d.waves_m * d.waves_n * kgroups;
    t.kgroups = kgroups;
    t.stages = stages;
    t.lds_bytes = (d.pingpong && stages == d.stages)
                      ? (2 * d.bm + d.stages * d.bn) * kBK * 2   // A in 2 stages, B in `stages`
                      : stages * (d.bm + d.bn) * kBK * 2;
    t.stagger = stagger;
    t.long_stages = d.long_stages;
    return t;
}

// 2 stages while A and B (2 bytes per element) fit in one XCD's L2, else the
// rung's deep pipeline.
int stages_for(int id, int64_t M, int64_t N, int64_t K) {
    const int64_t operand_bytes = 2 * K * (M + N);
    return operand_bytes <= kShallowOperandBytes ? 2 : kLadder[id].stages;
}

// Two k-groups on a rung built with them, when its grid is resident all at
// once (at most one workgroup per CU) and the k-loop is long enough.
int kgroups_for(int id, int64_t M, int64_t N, int64_t K, int num_cu) {
    const TileDesc& d = kLadder[id];
    if (d.kgroups < 2) return 1;
    if (num_cu <= 0) num_cu = 256;
    const int64_t wgs = ceil_div(M, d.bm) * ceil_div(N, d.bn);
    const int64_t nkt = ceil_div(K, kBK);
    if (nkt < kSplitMinKTiles) return 1;
    // A rung whose one-k-group pipeline runs 16x16x32 MFMAs keeps it once the
    // grid fills every CU: there the part runs at its power limit and that
    // MFMA's lower energy per FLOP wins (128x128 at 2048^3: 20.0 us against
    // 21.5 with two k-groups; 256x128 at 4096x2048x2048: 35.8 against 37.4);
    // with CUs left idle the second k-group's shorter dependent chain wins
    // (1536^3: 13.7 against 14.8; 256x128 at 2304^3: 31.8 against 34.6).
    if (d.deep16) return wgs < num_cu ? 2 : 1;
    return wgs <= num_cu ? 2 : 1;
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

// The automatic plan on rung `id`: two k-groups always run the deep
// pipeline, one k-group the pipeline stages_for picks; long_for then swaps a
// two-k-group deep pipeline for the rung's long one on a long k-loop.
Plan plan_for(int id, int64_t M, int64_t N, int64_t K, int num_cu) {
    const TileDesc& d = kLadder[id];
    Plan p;
    p.tile = id;
    p.kgroups = kgroups_for(id, M, N, K, num_cu);
    p.stages = long_for(id, p.kgroups == 2 ? d.stages : stages_for(id, M, N, K), p.kgroups, K);
    p.stagger = stagger_auto(id, M, N, K) ? 1 : 0;
    return p;
}

bool stagger_auto(int id, int64_t M, int64_t N, int64_t K) {
    if (id < 0 || id >= kNumTiles || kLadder[id].pingpong) return false;
    if (!stagger_eligible(K) || K / kBK < kStaggerMinKTiles) return false;
    return 2 * K * (M + N) <= kStaggerMaxOperandBytes;
}

// A plan the library has a kernel for: stages 2, the rung's deep count or its
// long count; two k-groups only on rungs built with them, and with the deep
// or long pipeline.
int check_plan(const Plan& p) {
    if (p.tile < 0 || p.tile >= kNumTiles) return SDT_ERR_INVALID_ARG;
    const TileDesc& d = kLadder[p.tile];
    const bool is_long = d.long_stages > 0 && p.stages == d.long_stages;
    if (p.stages != 2 && p.stages != d.stages && !is_long) return SDT_ERR_INVALID_ARG;
    if (p.kgroups != 1 && p.kgroups != 2) return SDT_ERR_INVALID_ARG;
    if (p.kgroups == 2 && (d.kgroups < 2 || (p.stages != d.stages && !is_long)))
        return SDT_ERR_INVALID_ARG;
    return SDT_OK;
}

// "Beating hipBLASLt on a Gaming GPU", section "The part that actually
// mattered": count how many reference-sized output blocks the grid produces
// (ceil division on both sides) and take the first rung whose threshold that
// count reaches; the last rung is the fallback.
int pick_rung(int64_t M, int64_t N, int ref_bm, int ref_bn, int rungs,
              const int64_t* min_blocks) {
    if (M < 0 || N < 0 || ref_bm <= 0 || ref_bn <= 0 || rungs <= 0 || !min_blocks)
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
int pick_tile(int64_t M, int64_t N, int64_t /*K*/, int num_cu) {
    if (num_cu <= 0) num_cu = 256;
    int64_t thresholds[kNumTiles];
    for (int r = 0; r < kNumTiles; ++r) {
        const int64_t area = int64_t(kLadder[r].bm / 64) * (kLadder[r].bn / 64);
        thresholds[r] = area * (num_cu / 2 + 1);
    }
    thresholds[kNumTiles - 1] = 0;
    return pick_rung(M, N, 64, 64, kNumTiles, thresholds);
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

extern "C" int sdt_tile_info(int tile_id, sdt_tile* out) {
    if (tile_id < 0 || tile_id >= sdt::kNumTiles || !out) return SDT_ERR_INVALID_ARG;
    *out = sdt::describe(tile_id, sdt::kLadder[tile_id].stages, sdt::kLadder[tile_id].kgroups);
    return SDT_OK;
}

extern "C" int sdt_plan_tile(int tile_id, int64_t M, int64_t N, int64_t K, int num_cu,
                             sdt_tile* out) {
    if (tile_id < 0 || tile_id >= sdt::kNumTiles || M < 0 || N < 0 || K < 0 || !out)
        return SDT_ERR_INVALID_ARG;
    if (num_cu <= 0) num_cu = 256;
    const sdt::Plan p = sdt::plan_for(tile_id, M, N, K, num_cu);
    *out = sdt::describe(p.tile, p.stages, p.kgroups, p.stagger);
    return SDT_OK;
}

extern "C" int sdt_stagger_eligible(int64_t K) { return sdt::stagger_eligible(K) ? 1 : 0; }

// FlyDSL PR, Changes: each workgroup starts at its own k-tile and wraps with
// a mask, one add and one and per trip.
extern "C" int64_t sdt_stagger_ktile(int64_t wg, int64_t i, int64_t nkt) {
    if (!sdt::is_pow2(nkt) || wg < 0 || i < 0) return -1;
    return (wg + i) & (nkt - 1);
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
