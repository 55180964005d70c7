"""Host-side tests of the C ABI (no GPU): the library loads and exports every
declared symbol, argument validation, the tile ladder and pick_tile, and the
k-loop stagger arithmetic.  No compute call reaches a device here: every
gemm_f16 call below is rejected (or is a no-op) before the HIP runtime is
touched."""
import ctypes
import os
import re

import pytest

from shape_driven_tile_amd import binding as sdt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdt.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "gfx1100_tile_ladder.tsv")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert "gemm_f16" in names and "gemv_f16_m1" in names
    assert sorted(sdt.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = sdt.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"libsdt.so does not export {name}"


def test_status_strings():
    for code in (0, 1, 2, 3):
        assert sdt.status_string(code).startswith(["SDT_OK", "SDT_ERR_INVALID_ARG",
                                                   "SDT_ERR_UNSUPPORTED", "SDT_ERR_HIP"][code])
    assert "unknown" in sdt.status_string(99)
    assert sdt.last_hip_error() == 0


# ---- argument validation ------------------------------------------------------

A16 = 0x10000   # fake, 16-byte aligned addresses: never dereferenced here
B16 = 0x20000
C16 = 0x30000


@pytest.mark.parametrize("args,want", [
    ((64, 64, 64, A16, 64, B16, 64, C16, 64), sdt.SDT_OK),
    ((-1, 64, 64, A16, 64, B16, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),
    ((64, -1, 64, A16, 64, B16, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),
    ((64, 64, -1, A16, 64, B16, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),
    ((64, 64, 64, A16, 56, B16, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),   # lda < K
    ((64, 64, 64, A16, 64, B16, 56, C16, 64), sdt.SDT_ERR_INVALID_ARG),   # ldb < K
    ((64, 64, 64, A16, 64, B16, 64, C16, 56), sdt.SDT_ERR_INVALID_ARG),   # ldc < N
    ((64, 64, 64, None, 64, B16, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),
    ((64, 64, 64, A16, 64, None, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),
    ((64, 64, 64, A16, 64, B16, 64, None, 64), sdt.SDT_ERR_INVALID_ARG),
    ((0, 64, 64, None, 64, None, 64, None, 64), sdt.SDT_OK),             # empty: no-op
    ((64, 0, 64, None, 64, None, 64, None, 0), sdt.SDT_OK),
    ((64, 64, 0, None, 0, None, 0, C16, 64), sdt.SDT_OK),                # K = 0: zeros
    ((64, 64, 64, A16 + 8, 64, B16, 64, C16, 64), sdt.SDT_ERR_UNSUPPORTED),
    ((64, 64, 64, A16, 64, B16 + 2, 64, C16, 64), sdt.SDT_ERR_UNSUPPORTED),
    ((64, 64, 64, A16, 64, B16, 64, C16 + 4, 64), sdt.SDT_ERR_UNSUPPORTED),
    ((64, 64, 60, A16, 60, B16, 64, C16, 64), sdt.SDT_ERR_UNSUPPORTED),  # lda % 8
    ((64, 64, 60, A16, 64, B16, 60, C16, 64), sdt.SDT_ERR_UNSUPPORTED),  # ldb % 8
    ((64, 60, 64, A16, 64, B16, 64, C16, 60), sdt.SDT_ERR_UNSUPPORTED),  # ldc % 8
    ((1, 64, 61, A16, 61, B16, 64, C16, 64), sdt.SDT_OK),                # one row: lda free
    ((64, 1, 61, A16, 64, B16, 61, C16, 8), sdt.SDT_OK),                 # one column: ldb free
    ((8, 8, 8, A16, (1 << 22), B16, 8, C16, 8), sdt.SDT_ERR_UNSUPPORTED),  # ld limit
])
def test_check_gemm_args(args, want):
    assert sdt.check_gemm_args(*args) == want


@pytest.mark.parametrize("args,want", [
    ((-1, 64, 64, A16, 64, B16, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),
    ((64, 64, 64, None, 64, B16, 64, C16, 64), sdt.SDT_ERR_INVALID_ARG),
    ((64, 64, 64, A16 + 8, 64, B16, 64, C16, 64), sdt.SDT_ERR_UNSUPPORTED),
    ((0, 64, 64, None, 64, None, 64, None, 64), sdt.SDT_OK),
])
def test_gemm_f16_rejects_before_launch(args, want):
    """The entry point returns the validation status and launches nothing."""
    assert sdt.gemm_f16_raw(*args) == want


def test_gemm_f16_ex_rejects_bad_choices():
    L = sdt.lib()
    base = (64, 64, 64, A16, 64, B16, 64, C16, 64, None)
    assert L.gemm_f16_ex(*base, sdt.num_tiles(), -1) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemm_f16_ex(*base, -2, -1) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemm_f16_ex(*base, 0, 2) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemv_f16_m1_ex(64, 64, A16, B16, 64, C16, None, -1) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemv_f16_m1_ex(64, 64, A16, B16, 64, C16, None,
                            sdt.gemv_num_variants()) == sdt.SDT_ERR_INVALID_ARG


KN_OK = (0x10000, 0x20000, 0x30000)   # fake 16-byte aligned x, B, y


@pytest.mark.parametrize("args,want", [
    ((12288, 4096, *KN_OK[:2], 12288, KN_OK[2]), 0),
    ((-1, 4, *KN_OK[:2], 8, KN_OK[2]), 1),
    ((8, -1, *KN_OK[:2], 8, KN_OK[2]), 1),
    ((16, 4, *KN_OK[:2], 8, KN_OK[2]), 1),            # ldb < N
    ((0, 4, None, None, 0, None), 0),                  # nothing to do
    ((16, 4, None, KN_OK[1], 16, KN_OK[2]), 1),        # null x
    ((16, 4, KN_OK[0], KN_OK[1], 16, None), 1),        # null y
    ((16, 0, None, None, 0, KN_OK[2]), 0),             # K=0: only y is touched
    ((16, 4, KN_OK[0] + 2, KN_OK[1], 16, KN_OK[2]), 2),
    ((16, 4, KN_OK[0], KN_OK[1] + 8, 16, KN_OK[2]), 2),
    ((16, 4, KN_OK[0], KN_OK[1], 20, KN_OK[2]), 2),    # ldb % 8
    ((16, 1, KN_OK[0], KN_OK[1], 20, KN_OK[2]), 0),    # one row: ldb unconstrained
    ((16, 4, KN_OK[0], KN_OK[1], 16, KN_OK[2] + 1), 2),  # y odd address
    ((16, 4, KN_OK[0], KN_OK[1], 16, KN_OK[2] + 2), 0),
])
def test_check_gemv_kn_args(args, want):
    assert sdt.check_gemv_kn_args(*args) == want


def test_gemv_kn_rejects_before_launch():
    """Every invalid call returns its status without touching a device."""
    L = sdt.lib()
    assert L.gemv_f16_m1_kn(16, 4, KN_OK[0] + 2, KN_OK[1], 16, KN_OK[2], None) == 2
    assert L.gemv_f16_m1_kn(16, 4, KN_OK[0], KN_OK[1], 8, KN_OK[2], None) == 1
    assert L.gemv_f16_m1_kn(0, 4, None, None, 0, None, None) == 0
    assert L.gemv_f16_m1_kn_ex(16, 4, *KN_OK[:2], 16, KN_OK[2], None, -1) == 1
    assert L.gemv_f16_m1_kn_ex(16, 4, *KN_OK[:2], 16, KN_OK[2], None,
                               sdt.gemv_kn_num_variants()) == 1
    assert sdt.gemv_kn_num_variants() >= 1


def test_gemv_rejects_before_launch():
    assert sdt.gemv_f16_m1_raw(-1, 64, A16, B16, 64, C16) == sdt.SDT_ERR_INVALID_ARG
    assert sdt.gemv_f16_m1_raw(64, 64, A16, B16, 60, C16) == sdt.SDT_ERR_INVALID_ARG
    assert sdt.gemv_f16_m1_raw(64, 64, A16 + 2, B16, 64, C16) == sdt.SDT_ERR_UNSUPPORTED
    assert sdt.gemv_f16_m1_raw(0, 64, None, None, 64, None) == sdt.SDT_OK


# ---- the tile ladder and pick_tile -------------------------------------------

# Rungs 0-4 are the ladder pick_rung walks; the rungs after them are taken
# only in place of the ladder's pick (the header's sdt_pick_tile rule).
NUM_LADDER = 5
# rungs whose deep one-k-group pipeline runs a loader wave beside each
# compute wave (256 x 128, 128 x 128 and 64 x 64)
LOADER_RUNGS = (1, 2, 4)


def ladder():
    return [sdt.tile_info(i) for i in range(sdt.num_tiles())]


def blocks(t, M, N):
    return -(-M // t["bm"]) * -(-N // t["bn"])


def ladder_pick(M, N, num_cu):
    """The ladder's own pick: the first rung whose 64 x 64 block count reaches
    (bm/64)(bn/64)(num_cu/2 + 1), else the smallest."""
    tiles = ladder()
    b64 = -(-M // 64) * -(-N // 64)
    area = [(r["bm"] // 64) * (r["bn"] // 64) for r in tiles[:NUM_LADDER]]
    return next((i for i, a in enumerate(area[:-1]) if b64 >= a * (num_cu // 2 + 1)),
                NUM_LADDER - 1)


def past_wave_band(b0, K, num_cu):
    """A ping-pong grid of b0 workgroups just past one or two waves."""
    return ((num_cu < b0 and 2 * b0 <= 3 * num_cu and K // 64 >= 32) or
            (2 * num_cu < b0 and 4 * b0 <= 9 * num_cu and K // 64 >= 64))


def expected_pick(M, N, num_cu, K=4096):
    """The header's rule, restated: the ladder's pick from the 64 x 64 block
    count, then an off-ladder rung with a smaller tile whose grid is larger
    than the pick's, at most num_cu and at least 7/8 of it, and at most 2/3
    of the pick's area where the pick runs loader waves (from 12 k-tiles);
    256 x 128 in place of a 256 x 256 grid of more than num_cu and at most
    3/2 num_cu workgroups from 32 k-tiles, or of more than 2 num_cu and at
    most 9/4 num_cu from 64."""
    tiles = ladder()
    r = ladder_pick(M, N, num_cu)
    if r == 0 and past_wave_band(blocks(tiles[0], M, N), K, num_cu):
        return 1
    loaders = r in LOADER_RUNGS and K // 64 >= 12
    ar = tiles[r]["bm"] * tiles[r]["bn"]
    for c in tiles[NUM_LADDER:]:
        ac = c["bm"] * c["bn"]
        if (ac < ar and blocks(tiles[r], M, N) < blocks(c, M, N) <= num_cu
                and 8 * blocks(c, M, N) >= 7 * num_cu and (not loaders or 3 * ac <= 2 * ar)):
            return c["id"]
    return r


def lds_bytes(t, stages):
    """LDS of a launch: `stages` x (bm + bn) x 64 fp16, except rung 0's deep
    pipeline, the ping-pong kernel, which keeps A in 2 stages and B in 3."""
    if t["id"] == 0 and stages == 3:
        return (2 * t["bm"] + 3 * t["bn"]) * 64 * 2
    return stages * (t["bm"] + t["bn"]) * 64 * 2


def test_ladder_is_well_formed():
    tiles = ladder()
    assert len(tiles) == NUM_LADDER + 3
    areas = [t["bm"] * t["bn"] for t in tiles[:NUM_LADDER]]
    assert areas == sorted(areas, reverse=True), "largest tile first"
    # the off-ladder 96 x 96, 192 x 192 and 160 x 160 rungs: 16x16x32 MFMAs
    # only, one k-group, no k-split
    shapes = [(t["bm"], t["bn"], t["waves_m"], t["waves_n"]) for t in tiles[NUM_LADDER:]]
    assert shapes == [(96, 96, 2, 2), (192, 192, 2, 4), (160, 160, 2, 2)]
    for off in tiles[NUM_LADDER:]:
        assert off["kgroups"] == 1 and off["ksplit"] == 0 and off["long_stages"] == 0
    for t in tiles:
        assert t["bk"] == 64
        assert t["kgroups"] in (1, 2)
        # the rung as built: its deep pipeline with its most k-groups, and
        # whether it is built with loader waves
        assert t["loaders"] == int(t["id"] in LOADER_RUNGS)
        assert t["threads"] == 64 * t["waves_m"] * t["waves_n"] * t["kgroups"]
        mf = 32 if t["id"] < NUM_LADDER else 16
        assert t["bm"] % (mf * t["waves_m"]) == 0 and t["bn"] % (mf * t["waves_n"]) == 0
        assert 2 <= t["stages"] <= 4
        assert t["lds_bytes"] == lds_bytes(t, t["stages"])
        assert t["lds_bytes"] <= 160 * 1024, "fits MI355X LDS"
    with pytest.raises(sdt.SdtError):
        sdt.tile_info(len(tiles))


# Two k-groups on the rungs built with them, per rung: (k-tiles needed with
# CUs left idle, the grid's bound in eighths of the CUs, k-tiles needed with
# one workgroup on every CU (0: never)).
KG2_RULE = {1: (12, 0, 0), 2: (12, 0, 0), 3: (96, 6, 0), 4: (40, 8, 40)}


def expected_kgroups(tile_id, wgs, nkt, num_cu):
    if tile_id not in KG2_RULE or nkt < 12:
        return 1
    least, grid8, full = KG2_RULE[tile_id]
    if wgs == num_cu:
        return 2 if full and nkt >= full else 1
    return 2 if 8 * wgs < grid8 * num_cu and nkt >= least else 1


def test_launch_plan_rules():
    """k-groups: 2 on rungs built with them by each rung's thresholds (256x128
    and 128x128: never, their one-k-group pipeline runs loader waves; 128x64:
    fewer than 3/4 of the CUs and at least 96 k-tiles; 64x64: at most one
    workgroup per CU and at least 40), else the one-k-group pipeline, 16x16x32
    on every ladder rung below 256x256.  Stages: the deep
    count, never the 2-stage pipeline; a two-k-group deep pipeline becomes the
    rung's long one (if it has one) from 12 full k-tiles.  Stagger: on ladder
    rungs 1-4, a power-of-two count of at least 16 full k-tiles and A and B
    within 16 MiB."""
    tiles = ladder()
    shapes = [(256, 256, 256), (512, 512, 512), (768, 768, 768), (1024, 1024, 1024),
              (512, 512, 2048), (1024, 1024, 1025), (512, 512, 4096), (2048, 2048, 2048),
              (2048, 2048, 4096), (1536, 1536, 2048), (1024, 1024, 4096),
              (4096, 4096, 4096), (8192, 8192, 8192), (1, 1, 1), (100, 3000, 700),
              (512, 512, 3008), (512, 512, 3072), (1024, 1024, 8192), (64, 64, 8192),
              (2048, 1024, 4096), (384, 384, 768), (384, 384, 704), (640, 640, 640),
              (768, 768, 1472), (768, 768, 1536), (1024, 1024, 2496), (1024, 1024, 2560),
              (1152, 1152, 6080), (1152, 1152, 6144), (1280, 1280, 8192), (960, 960, 2560)]
    for num_cu in (80, 256):
        for t in tiles:
            for (M, N, K) in shapes:
                p = sdt.plan_tile(t["id"], M, N, K, num_cu)
                wgs = -(-M // t["bm"]) * -(-N // t["bn"])
                kg = expected_kgroups(t["id"], wgs, -(-K // 64), num_cu)
                assert kg == 1 or t["kgroups"] == 2
                st = t["stages"]
                if kg == 2 and t["long_stages"] and K // 64 >= 12:
                    st = t["long_stages"]
                assert (p["kgroups"], p["stages"]) == (kg, st), (num_cu, t["id"], M, N, K)
                nkt = K // 64
                stg = int(0 < t["id"] < NUM_LADDER and nkt >= 16 and nkt & (nkt - 1) == 0
                          and 2 * K * (M + N) <= 16 << 20)
                assert p["stagger"] == stg, (num_cu, t["id"], M, N, K)
                ld = int(t["id"] in LOADER_RUNGS and kg == 1 and st == t["stages"] and K // 64 >= 12)
                assert p["loaders"] == ld, (num_cu, t["id"], M, N, K)
                assert p["threads"] == 64 * t["waves_m"] * t["waves_n"] * kg * (2 if ld else 1)
                assert p["lds_bytes"] == lds_bytes(t, st)
    with pytest.raises(sdt.SdtError):
        sdt.plan_tile(len(tiles), 1, 1, 1)
    with pytest.raises(sdt.SdtError):
        sdt.plan_tile(0, -1, 1, 1)
    # pick_tile reports the plan of the rung it picks
    for (M, N, K) in shapes:
        p = sdt.pick_tile(M, N, K, 256)
        assert p == sdt.plan_tile(p["id"], M, N, K, 256)
    assert sdt.pick_tile(1024, 1024, 1024, 256)["kgroups"] == 1   # 256 x 64x64, 16 k-tiles
    assert sdt.pick_tile(1024, 1024, 4096, 256)["kgroups"] == 2   # 64 k-tiles
    assert sdt.pick_tile(768, 768, 768, 256)["kgroups"] == 1      # 144 workgroups, 12 k-tiles
    assert sdt.pick_tile(768, 768, 2048, 256)["kgroups"] == 1     # 32 k-tiles: loader waves
    assert sdt.pick_tile(768, 768, 2560, 256)["kgroups"] == 2     # 40 k-tiles
    assert sdt.pick_tile(1280, 1280, 4096, 256)["kgroups"] == 1   # 128x64, 200 workgroups
    assert sdt.pick_tile(1152, 1152, 8192, 256)["kgroups"] == 2   # 128x64, 162, 128 k-tiles
    assert sdt.pick_tile(256, 256, 256, 256)["kgroups"] == 1
    assert sdt.pick_tile(8192, 8192, 8192, 256)["kgroups"] == 1
    for (M, N, K), rung in [((4608, 4608, 4608), 1), ((4352, 4352, 2048), 1),
                            ((4096, 6144, 4096), 1), ((4096, 5120, 1984), 0),
                            ((5120, 5120, 5120), 0), ((6144, 6144, 6144), 1),
                            ((6144, 6144, 2048), 0), ((6400, 6400, 8192), 0),
                            ((5888, 5888, 4096), 1), ((5888, 5888, 4032), 0),
                            ((4096, 4096, 4096), 0), ((8192, 8192, 8192), 0)]:
        p = sdt.pick_tile(M, N, K, 256)             # ping-pong grid past one wave
        assert (p["id"], p["loaders"]) == (rung, rung), (M, N, K)
    p = sdt.pick_tile(1664, 1664, 1664, 256)                      # 169 workgroups
    assert (p["kgroups"], p["loaders"]) == (1, 1)
    # 1536^3: 96 x 96 in place of 128 x 128 (256 workgroups instead of 144)
    p = sdt.pick_tile(1536, 1536, 1536, 256)
    assert (p["id"], p["bm"], p["kgroups"], p["stages"], p["stagger"]) == (5, 96, 1, 3, 0)
    assert sdt.pick_tile(2048, 2048, 2048, 256)["kgroups"] == 1   # 256: the 16x16x32 pipeline
    # stagger: eligible, at least 16 k-tiles, operands within 16 MiB, not the ping-pong rung
    assert sdt.pick_tile(2048, 2048, 2048, 256)["stagger"] == 1
    assert sdt.pick_tile(2048, 2048, 4096, 256)["stagger"] == 0     # 32 MiB of operands
    assert sdt.pick_tile(2048, 2048, 1984, 256)["stagger"] == 0     # 31 k-tiles
    assert sdt.pick_tile(512, 512, 512, 256)["stagger"] == 0        # 8 k-tiles
    assert sdt.pick_tile(4096, 4096, 1024, 256)["stagger"] == 0     # ping-pong rung
    assert sdt.tile_info(2)["stagger"] == 0


def test_gemm_cfg_rejects_kernels_that_do_not_exist():
    """Forced combinations without a kernel are refused before any device
    call (fake aligned pointers, null stream)."""
    L = sdt.lib()
    args = (512, 512, 512, 0x10000, 512, 0x20000, 512, 0x30000, 512, None, 0, None)
    tiles = ladder()
    def cfg(*v):
        return ctypes.byref(sdt.launch_cfg(*v))
    assert L.gemm_f16_cfg(*args, None) == sdt.SDT_ERR_INVALID_ARG
    for t in tiles:
        assert L.gemm_f16_cfg(*args, cfg(t["id"], 5, -1, -1)) == sdt.SDT_ERR_INVALID_ARG
        assert L.gemm_f16_cfg(*args, cfg(t["id"], -1, 3, -1)) == sdt.SDT_ERR_INVALID_ARG
        if t["kgroups"] == 1:
            assert L.gemm_f16_cfg(*args, cfg(t["id"], -1, 2, -1)) == sdt.SDT_ERR_INVALID_ARG
        if t["stages"] != 2:
            assert L.gemm_bf16_cfg(*args, cfg(t["id"], 2, 2, -1)) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemm_f16_cfg(*args, cfg(len(tiles), -1, -1, -1)) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemm_f16_cfg(*args, cfg(-1, -2, -1, -1)) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemm_f16_cfg(*args, cfg(-1, -1, -1, 2)) == sdt.SDT_ERR_INVALID_ARG


def test_pick_rung_reproduces_printed_gfx1100_ladder():
    """The pages' rule with gfx1100 constants reproduces the printed tile,
    warp layout and grid of all ten measured sizes."""
    rungs = [((128, 128), "4x2"), ((64, 128), "2x4"), ((64, 64), "2x2")]
    thresholds = [96, 64, 0]           # in 128x128-equivalent blocks
    rows = [l.split("\t") for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 10
    for size, tile, warps, grid in rows:
        n = int(size)
        r = sdt.pick_rung(n, n, 128, 128, thresholds)
        (bm, bn), w = rungs[r]
        assert tile == f"{bm}x{bn}x32", (n, tile)
        assert warps == w
        gx, gy = (int(v) for v in grid.split("x"))
        assert sorted((gx, gy)) == sorted((n // bm, n // bn))


def test_pick_rung_edges():
    assert sdt.pick_rung(0, 0, 128, 128, [96, 64, 0]) == 2
    assert sdt.pick_rung(100, 100, 128, 128, [1, 0]) == 0     # ceil division
    assert sdt.pick_rung(10, 10, 0, 128, [1]) == -1
    assert sdt.pick_rung(10, 10, 128, 128, []) == -1


def test_pick_tile_properties():
    tiles = ladder()
    for num_cu in (32, 80, 256, 304):
        prev_area = 0
        for n in [64 * i for i in range(1, 200)]:
            t = sdt.pick_tile(n, n, n, num_cu)
            assert 0 <= t["id"] < len(tiles)
            assert t == sdt.pick_tile(n, n, n, num_cu), "deterministic"
            # the ladder's pick grows with the square size; an off-ladder rung
            # only ever stands in for it with a smaller tile
            r = ladder_pick(n, n, num_cu)
            area = tiles[r]["bm"] * tiles[r]["bn"]
            assert area >= prev_area, "the ladder's tile grows with the square size"
            prev_area = area
            assert t["id"] == r or t["bm"] * t["bn"] < area
            # never off the largest tile while its grid alone fills the
            # machine, but for 256 x 128 just past one wave on long k-loops
            big = tiles[0]
            if (n // big["bm"]) * (n // big["bn"]) >= num_cu:
                band = past_wave_band(blocks(big, n, n), n, num_cu)
                assert t["id"] == (1 if band else 0), (num_cu, n)
    # the largest ladder rung whose grid, counted in 64x64 blocks scaled by
    # the rung's area, exceeds half the CUs (exactly its workgroup count when
    # the tile divides the shape), or the off-ladder rung in its place
    for num_cu in (80, 256, 304):
        for n in [64 * i for i in range(1, 200)]:
            t = sdt.pick_tile(n, n, n, num_cu)
            assert t["id"] == expected_pick(n, n, num_cu, n), (num_cu, n)
            if n % 256 == 0 and t["id"] < NUM_LADDER:
                wgs = (n // t["bm"]) * (n // t["bn"])
                assert t["id"] == NUM_LADDER - 1 or wgs > num_cu // 2
            if t["id"] >= NUM_LADDER:   # more workgroups than the ladder's pick, one per CU
                assert 7 * num_cu <= 8 * blocks(t, n, n) <= 8 * num_cu
    for (M, N) in [(1536, 1536), (1440, 1440), (1152, 1920), (768, 3072), (1664, 1664),
                   (1536, 2048), (1280, 1280), (100, 30000), (30000, 100)]:
        for num_cu in (80, 256, 304):
            assert sdt.pick_tile(M, N, 4096, num_cu)["id"] == expected_pick(M, N, num_cu)
            assert sdt.pick_tile(M, N, 512, num_cu)["id"] == expected_pick(M, N, num_cu, 512)
    assert sdt.pick_tile(1536, 2048, 1536, 256)["id"] == 2      # 352 > 256 workgroups of 96 x 96
    assert sdt.pick_tile(1152, 1920, 2048, 256)["id"] == 5      # 135 -> 240 workgroups
    assert sdt.pick_tile(3072, 3072, 3072, 256)["id"] == 6      # 144 -> 256 workgroups
    assert sdt.pick_tile(3000, 3104, 1000, 256)["id"] == 0      # 272 > 256 of 192 x 192
    assert sdt.pick_tile(2816, 2816, 2816, 256)["id"] == 1      # 225 < 242 of 256 x 128
    assert sdt.pick_tile(2560, 2560, 2560, 256)["id"] == 1      # 256 x 128 with loader waves
    assert sdt.pick_tile(2560, 2560, 640, 256)["id"] == 7       # 10 k-tiles: 200 -> 256 workgroups
    assert sdt.pick_tile(2048, 4096, 2048, 256)["id"] == 1      # 256 x 128 fills the CUs
    assert sdt.pick_tile(2048, 2560, 4096, 256)["id"] == 1      # 208 < 7/8 of 256 of 160 x 160
    assert sdt.pick_tile(768, 11008, 4096, 256)["id"] == 6      # 232 of 192 x 192
    assert sdt.pick_tile(1440, 1440, 1440, 256)["id"] == 5      # 225 of 96 x 96
    # any shape, even degenerate ones, gets a valid rung
    for (M, N) in [(1, 1), (1, 100000), (100000, 1), (0, 5), (7, 3)]:
        assert 0 <= sdt.pick_tile(M, N, 64, 256)["id"] < len(tiles)


def test_pick_tile_on_mi355x_square_sweep():
    """The rungs a sweep of every rung over square shapes measured fastest on
    MI355X (256 CUs); 1280 is a tie between 128x64 and 64x64."""
    want = {256: (64, 64), 512: (64, 64), 768: (64, 64), 1024: (64, 64), 1280: (128, 64),
            1536: (96, 96), 1664: (128, 128), 1792: (128, 128), 1920: (128, 128),
            2048: (128, 128), 2304: (256, 128), 2560: (256, 128), 3072: (192, 192),
            3584: (256, 256), 4096: (256, 256), 4352: (256, 128), 4608: (256, 128),
            5120: (256, 256), 5376: (256, 256), 5632: (256, 256), 6144: (256, 128),
            8192: (256, 256)}
    for n, (bm, bn) in want.items():
        t = sdt.pick_tile(n, n, n, 256)
        assert (t["bm"], t["bn"]) == (bm, bn), n
    # the K sweep keeps one tile for every K
    assert len({sdt.pick_tile(2048, 2048, K, 256)["id"]
                for K in (1920, 1984, 2048, 2112, 2176, 2304)}) == 1


# ---- k-loop stagger -----------------------------------------------------------

def test_stagger_eligibility_on_k_sweep():
    """On the K sweep (M=N=2048) only K=2048 has a power-of-two k-tile count,
    the one K where the FlyDSL PR (Motivation) wires the stagger up."""
    for K in (1920, 1984, 2048, 2112, 2176, 2304):
        assert sdt.stagger_eligible(K) == (K == 2048), K


def test_stagger_eligibility_details():
    assert not sdt.stagger_eligible(0) and not sdt.stagger_eligible(63)
    assert sdt.stagger_eligible(64) and sdt.stagger_eligible(65)  # 1 full k-tile (+ a partial)
    assert sdt.stagger_eligible(129)                               # 2 full k-tiles + a partial
    assert not sdt.stagger_eligible(192)                           # 3 full k-tiles
    assert sdt.stagger_eligible(8192) and not sdt.stagger_eligible(8192 + 64)
    assert not sdt.stagger_eligible(-64)


def test_forced_stagger_needs_eligibility():
    """gemm_f16_ex(stagger=1) on a K whose k-tile count is not a power of two
    is rejected before anything is launched (null stream, fake pointers)."""
    rc = sdt.lib().gemm_f16_ex(256, 256, 192, 4096, 192, 8192, 192, 16384, 256, None, -1, 1)
    assert rc == sdt.SDT_ERR_UNSUPPORTED


def test_stagger_is_a_permutation():
    nkt = 1
    while nkt <= 4096:
        wgs = range(nkt) if nkt <= 64 else (0, 1, 2, 3, nkt // 2, nkt - 1, nkt, 12345)
        for wg in wgs:
            seq = [sdt.stagger_ktile(wg, i, nkt) for i in range(nkt)]
            assert sorted(seq) == list(range(nkt)), (nkt, wg)
            assert seq[0] == wg % nkt
        nkt *= 2
    assert sdt.stagger_ktile(0, 0, 3) == -1


def test_decode_shape_bytes():
    """The decode weights are 4096 x 12288 fp16 = 100,663,296 bytes ("100.7 MB" on
    the mojo-baro page, section "Four rounds on the decode shape")."""
    from shape_driven_tile_amd import inputs
    assert inputs.DECODE_K * inputs.DECODE_N * 2 == 100_663_296


def test_capi_program_links_only_the_c_abi():
    """The C-ABI test program needs nothing but libsdt.so, the CPU oracle and
    the HIP runtime (no Python, no torch)."""
    import subprocess
    binp = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi", "capi_check")
    if not os.path.exists(binp):
        pytest.skip("tests/capi/capi_check not built")
    out = subprocess.run(["readelf", "-d", binp], capture_output=True, text=True).stdout
    needed = set(re.findall(r"NEEDED\)\s+Shared library: \[([^\]]+)\]", out))
    assert "libsdt.so" in needed and "libsdt_oracle.so" in needed
    assert not any("torch" in n or "python" in n for n in needed), needed


def test_bench_refuses_more_than_one_gpu():
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from shape_driven_tile_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libsdt.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


def test_one_hip_runtime_when_the_library_loads_first():
    """Loading the library before anything has imported torch must not leave
    two HIP runtimes in the process (libsdt.so's own dependency on the system
    one, then torch's bundled copy): the second to open the GPU would find no
    device.  The binding imports torch before it loads libsdt.so."""
    import subprocess
    import sys
    code = ("from shape_driven_tile_amd import binding as b; b.lib(); import torch; "
            "m = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in m if 'libamdhip64' in l}), "
            "len({l.split()[-1] for l in m if 'libhsa-runtime64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == ["1", "1"], r.stdout


_REFUSAL_PROBE = r"""
import sys
sys.path.insert(0, sys.argv[1])
from shape_driven_tile_amd import binding as sdt
A, B, C = 0x10000, 0x20000, 0x30000   # never dereferenced: the runtime refuses first
out = []
out.append(sdt.gemm_f16_raw(64, 64, 64, A, 64, B, 64, C, 64))
out.append(sdt.last_hip_error())
out.append(sdt.gemm_f16_raw(64, 64, 0, A, 64, B, 64, C, 64))      # K = 0: the zero fill
out.append(sdt.gemv_f16_m1_raw(128, 64, A, B, 64, C))
out.append(sdt.lib().sdt_empty_kernel(None))
out.append(sdt.last_hip_error())
print(" ".join(str(v) for v in out))
"""


def test_runtime_refusal_maps_to_sdt_err_hip():
    """A launch the HIP runtime refuses before any GPU work (here: a process
    in which no device is visible, so the runtime reports hipErrorNoDevice,
    100) comes back as SDT_ERR_HIP from every launching entry point, with the
    runtime's code kept for sdt_last_hip_error().  Run in a child process with
    every device hidden, so the outcome does not depend on the machine."""
    import subprocess
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, "-c", _REFUSAL_PROBE, ROOT], env=env,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    vals = [int(v) for v in res.stdout.split()[-6:]]
    hip_err = sdt.SDT_ERR_HIP
    assert vals == [hip_err, 100, hip_err, hip_err, hip_err, 100], vals


def test_abi_version():
    assert sdt.lib().sdt_abi_version() == sdt.ABI_VERSION
    text = open(HEADER).read()
    assert f"#define SDT_ABI_VERSION {sdt.ABI_VERSION}" in text


def test_ksplit_plan_rules():
    """gemm_f16_ws's plan: without a workspace (or one too small) it is
    gemm_f16's; with room it splits K on the rungs built for it while the
    grid leaves CUs idle: the most splits that keep tiles x splits within the
    CU count, each with at least 16 full k-tiles, at most 16, reduced by a
    second kernel; the stagger is then off.  The workspace it reports is the fixed 64 KiB counter area plus
    the fp32 partial tiles."""
    tiles = ladder()
    shapes = [(256, 256, 256), (512, 512, 512), (768, 768, 768), (1024, 1024, 1024),
              (1536, 1536, 1536), (2048, 2048, 2048), (4096, 4096, 4096), (300, 260, 1000),
              (64, 64, 64), (100, 3000, 700), (512, 512, 8192), (128, 128, 65536),
              (256, 256, 16384), (384, 384, 12288), (768, 768, 8192), (64, 128, 1 << 20)]
    for num_cu in (80, 256):
        for (M, N, K) in shapes:
            plain = sdt.pick_tile(M, N, K, num_cu)
            assert sdt.pick_tile_ws(M, N, K, num_cu, 0) == plain
            big = sdt.pick_tile_ws(M, N, K, num_cu, 1 << 40)
            t = tiles[plain["id"]]
            ntile = -(-M // t["bm"]) * -(-N // t["bn"])
            s = min(num_cu // ntile, (K // 64) // 16, 16) if t["ksplit"] else 1
            s = s if s >= 2 else 1
            assert big["id"] == plain["id"] and big["splits"] == s, (num_cu, M, N, K, big)
            need = sdt.gemm_workspace_size(M, N, K, num_cu)
            if s == 1:
                assert need == 0 and big == plain
                continue
            assert big["stagger"] == 0 and big["split_algo"] == 0
            assert need == 65536 + ntile * s * t["bm"] * t["bn"] * 4
            assert sdt.pick_tile_ws(M, N, K, num_cu, need) == big
            assert sdt.pick_tile_ws(M, N, K, num_cu, need - 1)["splits"] == 1


def test_loader_waves_plan_and_refusals():
    """Loader waves: the automatic plan takes them on rungs 2-5's deep
    one-k-group pipeline from 12 full k-tiles and reports twice the threads;
    forcing them is accepted on those pipelines only (checked before any
    device call, fake aligned pointers)."""
    t = sdt.pick_tile(2048, 2048, 2048, 256)
    assert (t["id"], t["kgroups"], t["loaders"], t["threads"]) == (2, 1, 1, 512)
    t = sdt.pick_tile(256, 256, 256, 256)
    assert (t["id"], t["loaders"], t["threads"]) == (4, 0, 256)
    t = sdt.pick_tile(768, 768, 768, 256)
    assert (t["id"], t["loaders"], t["threads"]) == (4, 1, 512)
    for n in (4096, 8192):    # the ping-pong rung has none
        assert sdt.pick_tile(n, n, n, 256)["loaders"] == 0
    t = sdt.pick_tile_ws(512, 512, 8192, 256, 1 << 24)   # a k-split plan: none
    assert t["splits"] > 1 and t["loaders"] == 0
    L = sdt.lib()
    args = (512, 512, 512, 0x10000, 512, 0x20000, 512, 0x30000, 512, None, 0, None)
    def cfg(**kw):
        return ctypes.byref(sdt.launch_cfg(**kw))
    def check(expect, **kw):
        # refused by the planner (sdt_launch_workspace_size: -1) and by
        # gemm_f16_cfg before it touches the device
        assert L.sdt_launch_workspace_size(512, 512, 512, cfg(**kw)) == -1, kw
        assert L.gemm_f16_cfg(*args, cfg(**kw)) == expect, kw
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=0, loaders=1)               # the ping-pong rung
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=2, kgroups=2, loaders=1)    # two k-groups
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=2, stages=2, loaders=1)     # the 2-stage pipeline
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=6, loaders=1)               # 192 x 192: none built
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=2, loaders=2)
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=2, loaders=-2)
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=3, loaders=1)               # 128 x 64: none built
    check(sdt.SDT_ERR_INVALID_ARG, tile_id=5, loaders=1)               # 96 x 96: none built
    for tile in (1, 2, 4):
        for ld in (0, 1):
            c = sdt.launch_cfg(tile_id=tile, kgroups=1, loaders=ld)
            assert L.sdt_launch_workspace_size(512, 512, 512, ctypes.byref(c)) == 0


def test_ksplit_and_persistent_cfg_refusals():
    """Forced k-split and persistent configurations the library has no kernel
    for, or without the workspace they need, are refused before any device
    call (fake aligned pointers)."""
    L = sdt.lib()
    ws, big = 0x40000, 1 << 40
    def call(M, N, K, w, wbytes, **kw):
        c = sdt.launch_cfg(**kw)
        return L.gemm_f16_cfg(M, N, K, 0x10000, K, 0x20000, K, 0x30000, N, w, wbytes, None,
                              ctypes.byref(c))
    bad = sdt.SDT_ERR_INVALID_ARG
    assert call(512, 512, 1024, None, 0, tile_id=4, splits=2) == bad            # no workspace
    need = sdt.launch_workspace_size(512, 512, 1024, tile_id=4, splits=2)
    assert need > 0
    assert call(512, 512, 1024, ws, need - 16, tile_id=4, splits=2) == bad      # too small
    assert call(512, 512, 1024, ws, big, tile_id=0, splits=2) == bad            # rung 0: no split
    assert call(512, 512, 1024, ws, big, tile_id=1, splits=2) == bad
    assert call(512, 512, 1024, ws, big, tile_id=4, splits=65) == bad
    assert call(512, 512, 1024, ws, big, tile_id=4, splits=17) == bad          # 16 full k-tiles
    assert call(512, 512, 1024, ws, big, tile_id=4, splits=0) == bad
    assert call(512, 512, 1024, ws, big, tile_id=4, splits=-2) == bad
    assert call(512, 512, 960, ws, big, tile_id=4, splits=16) == bad            # 15 full k-tiles
    assert call(512, 512, 1024, ws, big, tile_id=4, splits=2, stagger=1) == bad
    assert call(512, 512, 1024, ws, big, tile_id=4, splits=2, split_algo=2) == bad
    assert call(512, 512, 1024, ws + 8, big, tile_id=4, splits=2) == sdt.SDT_ERR_UNSUPPORTED
    assert call(512, 512, 1024, None, 8, tile_id=4) == bad                      # bytes, no pointer
    assert call(512, 512, 1024, None, -1, tile_id=4) == bad
    # persistent workgroups: the ping-pong kernel only, at most one per tile
    assert call(4096, 4096, 4096, None, 0, tile_id=2, persistent=64) == bad
    assert call(4096, 4096, 4096, None, 0, tile_id=0, stages=2, persistent=64) == bad
    assert call(4096, 4096, 4096, None, 0, tile_id=0, persistent=257) == bad    # 256 tiles
    assert call(4096, 4096, 4096, None, 0, tile_id=0, persistent=-2) == bad
    with pytest.raises(sdt.SdtError):
        sdt.launch_workspace_size(512, 512, 1024, tile_id=4, splits=65)


# ---- the [K][N] GEMV split over K ------------------------------------------------

def test_gemv_kn_split_plan():
    """gemv_f16_m1_kn_ws's split: 256-column bands, K cut into ranges of a
    multiple of 8 rows so that about 768 workgroups stream at once (at least
    2 ranges, each of at least 8 rows); the workspace holds one fp32 row of
    bands * 256 column sums per range.  No split below 16 rows or when the
    bands alone make 768 workgroups."""
    def plan(N, K):
        if N <= 0 or K < 16 or N > 2 ** 31 - 1 or K > (2 ** 31 - 1) // 2:
            return 0
        bands = -(-N // 256)
        s = min(-(-768 // bands), K // 8)
        if s < 2:
            return 0
        kc = -(-(-(-K // s)) // 8) * 8
        s = -(-K // kc)
        return 0 if s < 2 else s * bands * 256 * 4
    for N in (1, 8, 255, 256, 257, 1000, 4096, 12288, 65536, 196608, 196609, 1 << 20):
        for K in (0, 1, 15, 16, 17, 20, 64, 1000, 4096, 4100, 65536):
            assert sdt.gemv_kn_workspace_size(N, K) == plan(N, K), (N, K)
    assert sdt.gemv_kn_workspace_size(12288, 4096) == 16 * 48 * 256 * 4
    assert sdt.gemv_kn_workspace_size(1024, 2 ** 30 - 8) > 0
    assert sdt.gemv_kn_workspace_size(1024, 2 ** 30) == 0     # past INT_MAX / 2 rows
    assert sdt.gemv_kn_workspace_size(2 ** 31, 4096) == 0
    assert sdt.gemv_kn_workspace_size(-1, 5) == -1 and sdt.gemv_kn_workspace_size(5, -1) == -1


def test_gemv_kn_ws_argument_checks():
    """Refusals before any device call (fake aligned pointers, null stream)."""
    L = sdt.lib()
    x, B, y, ws = 0x10000, 0x20000, 0x30000, 0x40000
    assert L.gemv_f16_m1_kn_ws(-1, 8, x, B, 16, y, None, 0, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemv_f16_m1_kn_ws(16, 8, x, B, 8, y, None, 0, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemv_f16_m1_kn_ws(16, 8, x, B, 16, y, None, 64, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemv_f16_m1_kn_ws(16, 8, x, B, 16, y, ws, -1, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.gemv_f16_m1_kn_ws(16, 8, x, B, 16, y, ws + 4, 64, None) == sdt.SDT_ERR_UNSUPPORTED
    assert L.gemv_f16_m1_kn_ws(16, 8, x, B + 2, 16, y, ws, 64, None) == sdt.SDT_ERR_UNSUPPORTED
    assert L.gemv_bf16_m1_kn_ws(16, 8, x + 2, B, 16, y, ws, 64, None) == sdt.SDT_ERR_UNSUPPORTED
    assert L.gemv_f16_m1_kn_ws(0, 8, x, B, 16, y, ws, 64, None) == sdt.SDT_OK   # N == 0: no-op


def test_stream_read_runs_argument_checks():
    """Refusals of the run-length read kernel before any device call."""
    L = sdt.lib()
    b, o = 0x10000, 0x20000
    ok_args = (1024, 4096, 128, 256)
    assert L.sdt_stream_read_runs(b, 0, 4096, 128, 256, o, None) == sdt.SDT_OK
    assert L.sdt_stream_read_runs(None, *ok_args, o, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_runs(b, *ok_args, None, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_runs(b, -1, 4096, 128, 256, o, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_runs(b, 1024, 4096, 96, 256, o, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_runs(b, 1024, 4000, 128, 256, o, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_runs(b, 1024, 4096, 128, 128, o, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_runs(b, 1000, 4096, 512, 64, o, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_runs(b + 8, *ok_args, o, None) == sdt.SDT_ERR_UNSUPPORTED
    assert L.sdt_stream_read_runs(b, *ok_args, o + 2, None) == sdt.SDT_ERR_UNSUPPORTED


def test_mfma_ceiling_argument_checks():
    """Refusals of the register-only MFMA loop before any device call."""
    L = sdt.lib()
    f, o = 0x10000, 0x20000
    assert L.sdt_mfma_ceiling(None, 10, o, 256, 0, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_mfma_ceiling(f, 10, None, 256, 0, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_mfma_ceiling(f, 0, o, 256, 0, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_mfma_ceiling(f, 10, o, 0, 1, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_mfma_ceiling(f, 10, o, 256, 4, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_mfma_ceiling(f, 10, o, 256, -1, None) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_mfma_ceiling(f + 8, 10, o, 256, 0, None) == sdt.SDT_ERR_UNSUPPORTED
    assert L.sdt_mfma_ceiling(f, 10, o + 2, 256, 1, None) == sdt.SDT_ERR_UNSUPPORTED


def test_sizes_past_int_range_refused():
    """M, N or K past 2^31 - 1: every kernel size is an int, and the planner's
    block counts (products of two sizes) must not overflow.  Refused before
    any device call."""
    big = 2 ** 40
    for (M, N, K) in [(big, 64, 64), (64, big, 64), (64, 64, big), (big, big, 64)]:
        with pytest.raises(sdt.SdtError) as e:
            sdt.pick_tile(M, N, K, 256)
        assert e.value.status == sdt.SDT_ERR_UNSUPPORTED
        with pytest.raises(sdt.SdtError):
            sdt.plan_tile(0, M, N, K, 256)
        with pytest.raises(sdt.SdtError):
            sdt.pick_tile_ws(M, N, K, 256, 1 << 30)
        assert sdt.lib().sdt_gemm_workspace_size(M, N, K, 256) == -1
    assert sdt.pick_rung(big, big, 1, 1, [1, 0]) == -1
    assert sdt.pick_rung(2 ** 31 - 1, 2 ** 31 - 1, 1, 1, [1, 0]) == 0
    L = sdt.lib()
    # lda = ldb = K = 64 and ldc = N: the sizes alone decide
    assert L.gemm_f16(big, 64, 64, 0x10000, 64, 0x20000, 64, 0x30000, 64, None) == \
        sdt.SDT_ERR_UNSUPPORTED
    assert L.gemm_f16_ws(64, big, 64, 0x10000, 64, 0x20000, 64, 0x30000, big, None, 0, None) == \
        sdt.SDT_ERR_UNSUPPORTED
    assert L.gemm_f16_noalloc(big, 64, 64, 0x10000, 64, 0x20000, 64, 0x30000, 64, None) == \
        sdt.SDT_ERR_UNSUPPORTED
