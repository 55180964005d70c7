"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element
by element, on the same seeded inputs.

Tolerance for uniform inputs: |C_gpu - C_ref| <= 1e-2 + 2e-3*|C_ref| with C_ref
the unrounded fp64 oracle.  Exact regimes (small integers, all-ones, identity,
K=1, overflow) are compared bit for bit with the oracle's RNE fp16 rounding.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (assert_bitexact, assert_close, run_gemm, run_gemv, sample_positions,
                         say, seeded_rows, to_dev)
from shape_driven_tile_amd import inputs

pytestmark = pytest.mark.gpu


def _ntiles():
    from shape_driven_tile_amd import binding as sdt
    return sdt.num_tiles()


# ---- the five workloads -------------------------------------------------------

def test_square_256():
    say("square 256^3 uniform, auto tile")
    A, B = inputs.square_operands(256, 0)
    C, _ = run_gemm(A, B)
    assert_close(C, oracle.gemm(A, B))


@pytest.mark.parametrize("n", inputs.SQUARE_SWEEP)
def test_square_sweep(n):
    say(f"square {n}^3 uniform, auto tile, full oracle")
    A, B = inputs.square_operands(n, 1)
    C, _ = run_gemm(A, B)
    assert_close(C, oracle.gemm(A, B))


def test_square_4096_full():
    """4096^3 (the automatic plan: the 256 x 256 ping-pong kernel with its 16 x
    16-block XCD order on a 256-CU part): every element of C against the oracle."""
    say("square 4096^3 uniform, auto tile, full oracle")
    A, B = inputs.square_operands(4096, 2)
    C, _ = run_gemm(A, B)
    assert_close(C, oracle.gemm(A, B))


def test_square_8192_full():
    """8192^3: every element of C against the oracle (1.1e12 fp64
    multiply-adds on the host's cores, about 15 s with 16 threads)."""
    say("square 8192^3 uniform, auto tile, full C")
    n = 8192
    A, B = inputs.square_operands(n, 2)
    C, pad_ok = run_gemm(A, B)
    assert pad_ok
    assert_close(C, oracle.gemm(A, B))


@pytest.mark.parametrize("shape", [(4096, 4096, 1024), (8192, 8192, 512), (4096, 4096, 4096)])
def test_integer_exact_large_auto(shape):
    """Integer inputs in [-2, 2] (every fp32 partial sum exact, so any order
    gives the same bits) through gemm_f16's automatic plan at the large-square
    grids: the ping-pong kernel and, on a part with 8 XCDs, its 16 x 16-block
    tile order.  Every element of C, bit for bit against the oracle's RNE
    rounding."""
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    p = sdt.pick_tile(M, N, K, 0)
    assert (p["id"], p["stages"]) == (0, 3), p   # the ping-pong kernel
    A = inputs.integer_f16((M, K), 21)
    B = inputs.integer_f16((N, K), 22)
    say(f"integer {shape} automatic plan (ping-pong), full C")
    C, pad_ok = run_gemm(A, B)
    assert pad_ok
    assert_bitexact(C, oracle.gemm(A, B))


def test_integer_exact_8192_rows_auto():
    """8192^3 on integer inputs through the automatic plan: 512 seeded whole
    rows and 16 whole columns bit for bit."""
    n = 8192
    A = inputs.integer_f16((n, n), 23)
    B = inputs.integer_f16((n, n), 24)
    say("integer 8192^3 automatic plan, 512 full rows + 16 full columns")
    C, _ = run_gemm(A, B)
    rows = seeded_rows(n, 512, seed=5)
    assert_bitexact(C[rows], oracle.gemm(np.ascontiguousarray(A[rows]), B))
    cols = seeded_rows(n, 16, seed=6)
    r = np.repeat(np.arange(n), len(cols))
    c = np.tile(cols, n)
    assert_bitexact(C[r, c], oracle.gemm_sample(A, B, r, c))


@pytest.mark.parametrize("shape,rung", [((1536, 1536, 1536), 5), ((1440, 1440, 1000), 5),
                                        ((3072, 3072, 1024), 6), ((768, 11008, 512), 6),
                                        ((2560, 2560, 640), 7), ((1280, 5120, 704), 7)])
def test_integer_exact_off_ladder_auto(shape, rung):
    """Shapes whose automatic plan takes an off-ladder rung (96 x 96, 192 x 192,
    160 x 160) at their real grids (one workgroup per CU, XCD-aware order,
    ragged edges where the tile does not divide), every element bit for bit
    on integer inputs, then uniform inputs within the tolerance."""
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    assert sdt.pick_tile(M, N, K, 256)["id"] == rung
    A = inputs.integer_f16((M, K), 31)
    B = inputs.integer_f16((N, K), 32)
    say(f"integer {shape} automatic plan (rung {rung}), full C")
    C, pad_ok = run_gemm(A, B)
    assert pad_ok
    assert_bitexact(C, oracle.gemm(A, B))
    Au = inputs.uniform_f16((M, K), 33)
    Bu = inputs.uniform_f16((N, K), 34)
    say(f"uniform {shape} automatic plan (rung {rung}), full C")
    C, _ = run_gemm(Au, Bu)
    assert_close(C, oracle.gemm(Au, Bu))


@pytest.mark.parametrize("shape", [(4352, 4352, 2048), (4200, 4504, 2104), (5800, 5880, 4104)])
def test_integer_exact_past_one_wave_auto(shape):
    """Shapes whose 256 x 256 grid is just past one or two waves of
    workgroups (289, 306 and 529 on 256 CUs), where the automatic plan takes
    the 256 x 128 rung with loader waves: every element bit for bit on
    integer inputs (the last two ragged in M, N and K)."""
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    p = sdt.pick_tile(M, N, K, 256)
    assert (p["id"], p["loaders"]) == (1, 1), p
    A = inputs.integer_f16((M, K), 41)
    B = inputs.integer_f16((N, K), 42)
    say(f"integer {shape} automatic plan (256x128, loader waves), full C")
    C, pad_ok = run_gemm(A, B)
    assert pad_ok
    assert_bitexact(C, oracle.gemm(A, B))


def test_integer_exact_pingpong_short_k_block_order():
    """The ping-pong kernel (forced, and the automatic plan) at 4096 x 4096 x
    128: two k-tiles, fewer than its stages, the 16 x 16-block tile order,
    every element bit for bit."""
    from shape_driven_tile_amd import binding as sdt
    p = sdt.pick_tile(4096, 4096, 128, 256)
    assert (p["id"], p["stages"]) == (0, 3), p
    A = inputs.integer_f16((4096, 128), 25)
    B = inputs.integer_f16((4096, 128), 26)
    say("integer 4096x4096x128 ping-pong forced, full C")
    C, pad_ok = run_gemm(A, B, tile=0, stagger=0, stages=3, kgroups=1)
    assert pad_ok
    assert_bitexact(C, oracle.gemm(A, B))


@pytest.mark.parametrize("K", inputs.K_SWEEP_K)
def test_k_sweep(K):
    say(f"K sweep M=N=2048 K={K}, auto tile/stagger, full oracle")
    A, B = inputs.square_operands(2048, 3, k=K)
    C, _ = run_gemm(A, B)
    assert_close(C, oracle.gemm(A, B))


def test_k_sweep_stagger_arms_at_2048():
    """K=2048 is the one sweep point with a power-of-two k-tile count: both
    stagger arms match the oracle and agree bit for bit on integer inputs."""
    say("K=2048 stagger on/off")
    A, B = inputs.square_operands(2048, 3, k=2048)
    ref = oracle.gemm(A, B)
    for st in (0, 1):
        C, _ = run_gemm(A, B, tile=2, stagger=st)
        assert_close(C, ref)
    Ai = inputs.integer_f16((2048, 2048), 7)
    Bi = inputs.integer_f16((2048, 2048), 8)
    ref_i = oracle.gemm(Ai, Bi)
    for st in (0, 1):
        C, _ = run_gemm(Ai, Bi, tile=2, stagger=st)
        assert_bitexact(C, ref_i)


def test_decode_gemv_all_buffers():
    say("decode GEMV N=12288 K=4096, 8 weight buffers")
    x = inputs.decode_activations()
    for r in range(inputs.DECODE_BUFFERS):
        W = inputs.decode_weights(r)
        y = run_gemv(x, W)
        assert_close(y, oracle.gemv_m1(x, W))


# ---- exact regimes (bit for bit) ---------------------------------------------

@pytest.mark.parametrize("shape", [(300, 200, 1024), (257, 129, 1000), (64, 64, 64),
                                   (513, 771, 520)])
def test_integer_exact_every_tile(shape):
    M, N, K = shape
    A = inputs.integer_f16((M, K), 11)
    B = inputs.integer_f16((N, K), 12)
    ref = oracle.gemm(A, B)
    nfull = K // 64
    staggers = (0, 1) if nfull > 0 and nfull & (nfull - 1) == 0 else (0,)
    for tile in range(_ntiles()):
        for st in staggers:
            say(f"integer {shape} tile={tile} stagger={st}")
            C, _ = run_gemm(A, B, tile=tile, stagger=st)
            assert_bitexact(C, ref)


@pytest.mark.parametrize("shape", [(257, 259, 4160), (300, 260, 4104)])
def test_integer_exact_every_tile_deep_pipeline(shape):
    """The automatic plan is every rung's deep pipeline (on the rungs with a
    long pipeline it takes that one when it runs two k-groups, which the
    assertion checks; the long pipelines themselves run in
    test_long_pipeline_every_rung_with_one).  Here each rung's deep pipeline
    is forced: exact integer sums, bit for bit, with a ragged last k-tile in
    the second shape and ragged M/N in both; one k-group and, where built,
    two."""
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    A = inputs.integer_f16((M, K), 13)
    B = inputs.integer_f16((N, K), 14)
    ref = oracle.gemm(A, B)
    for tile in range(_ntiles()):
        info = sdt.tile_info(tile)
        plan = sdt.plan_tile(tile, M, N, K, 1 << 20)
        long_ = info["long_stages"] and plan["kgroups"] == 2 and K // 64 >= 12
        assert plan["stages"] == (info["long_stages"] if long_ else info["stages"])
        for kg in ((1, 2) if info["kgroups"] == 2 else (1,)):
            say(f"integer deep {shape} tile={tile} stages={info['stages']} kgroups={kg}")
            C, pad_ok = run_gemm(A, B, tile=tile, stagger=0, stages=info["stages"], kgroups=kg)
            assert pad_ok
            assert_bitexact(C, ref)


LOADER_RUNGS = (1, 2, 4)


@pytest.mark.parametrize("K", [8, 64, 200, 768, 1032, 2048])
def test_loader_waves_exact_every_rung(K):
    """Loader waves forced on and off on every rung built with them (256 x
    128, 128 x 128 and 64 x 64), one k-group, the deep pipeline: exact
    integer sums bit for bit against the oracle with ragged M and N, k-loops
    of 0 to 32 full k-tiles (a partial one after them at K = 8, 200 and
    1032), staggered where the k-tile count allows.  The loader waves issue
    the same loads the compute waves would, so both forms give the same bits."""
    M, N = 300, 260
    A = inputs.integer_f16((M, K), 60 + K)
    B = inputs.integer_f16((N, K), 61 + K)
    ref = oracle.gemm(A, B)
    nfull = K // 64
    staggers = (0, 1) if nfull >= 2 and nfull & (nfull - 1) == 0 and K % 64 == 0 else (0,)
    for tile in LOADER_RUNGS:
        for st in staggers:
            for ld in (0, 1):
                say(f"loaders={ld} K={K} tile={tile} stagger={st}")
                C, pad_ok = run_gemm(A, B, tile=tile, stagger=st, stages=3, kgroups=1, loaders=ld)
                assert pad_ok
                assert_bitexact(C, ref)


@pytest.mark.parametrize("shape", [(2048, 2048, 2048), (2048, 2048, 1920), (768, 768, 768),
                                   (1024, 1024, 1024), (4096, 1024, 1024), (4096, 2048, 2048)])
def test_loader_waves_same_bits_uniform(shape):
    """On uniform inputs the automatic plan (loader waves here) and the same
    plan without them give identical bits, and both are within tolerance of
    the oracle on sampled rows and columns."""
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    A, B = inputs.square_operands(M, 70, k=K) if M == N else (inputs.uniform_f16((M, K), 71),
                                                              inputs.uniform_f16((N, K), 72))
    plan = sdt.pick_tile(M, N, K, 0)
    assert plan["loaders"] == 1 and plan["threads"] == 512, plan
    say(f"uniform {shape} automatic plan (loaders) and loaders forced off")
    C_on, _ = run_gemm(A, B)
    C_off, _ = run_gemm(A, B, tile=plan["id"], stagger=plan["stagger"], stages=plan["stages"],
                        kgroups=plan["kgroups"], loaders=0)
    assert np.array_equal(C_on.view(np.uint16), C_off.view(np.uint16))
    rows = sorted(set([0, 1, M // 2, M - 1] + list(np.random.default_rng(M).integers(0, M, 12))))
    ref_rows = oracle.gemm(np.ascontiguousarray(A[rows]), B)
    assert_close(C_on[rows], ref_rows)


@pytest.mark.parametrize("K", [8, 64, 104, 128, 192])
def test_short_k_every_pipeline(K):
    """k-loops of 0 to 3 full k-tiles (with and without a partial one) on every
    rung's 2-stage and deep pipeline, two k-groups where built: the ping-pong
    kernel's prologue, barrier pairing and tail then run with fewer tiles than
    it has stages.  Exact integer sums, bit for bit, ragged M and N."""
    from shape_driven_tile_amd import binding as sdt
    M, N = 300, 260
    A = inputs.integer_f16((M, K), 40 + K)
    B = inputs.integer_f16((N, K), 41 + K)
    ref = oracle.gemm(A, B)
    for tile in range(_ntiles()):
        info = sdt.tile_info(tile)
        plans = [(2, 1), (info["stages"], 1)] + ([(info["stages"], 2)] if info["kgroups"] == 2
                                                 else [])
        for stages, kg in plans:
            say(f"short K={K} tile={tile} stages={stages} kgroups={kg}")
            C, pad_ok = run_gemm(A, B, tile=tile, stagger=0, stages=stages, kgroups=kg)
            assert pad_ok
            assert_bitexact(C, ref)


@pytest.mark.parametrize("shape", [(300, 260, 3136), (257, 129, 3112)])
def test_long_pipeline_every_rung_with_one(shape):
    """The 4-stage pipeline of the rungs that have one, with one and two
    k-groups, on 49 and 48 full k-tiles (the second with a partial one after
    them), bit for bit on integer inputs; then the automatic plan, which takes
    it here."""
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    A = inputs.integer_f16((M, K), 70)
    B = inputs.integer_f16((N, K), 71)
    ref = oracle.gemm(A, B)
    tried = 0
    for tile in range(_ntiles()):
        info = sdt.tile_info(tile)
        if not info["long_stages"]:
            continue
        for kg in (1, 2):
            say(f"long pipeline {shape} tile={tile} stages={info['long_stages']} kgroups={kg}")
            C, pad_ok = run_gemm(A, B, tile=tile, stagger=0, stages=info["long_stages"], kgroups=kg)
            assert pad_ok
            assert_bitexact(C, ref)
            tried += 1
    assert tried >= 4
    auto = sdt.pick_tile(M, N, K, 256)
    assert auto["stages"] == sdt.tile_info(auto["id"])["long_stages"] > 0
    say(f"long pipeline {shape} automatic plan")
    C, pad_ok = run_gemm(A, B)
    assert pad_ok
    assert_bitexact(C, ref)


def test_long_pipeline_uniform_512x512x8192():
    """The automatic plan at 512 x 512 x 8192 (64 x 64, two k-groups, 4
    stages) against the oracle within the stated tolerance."""
    from shape_driven_tile_amd import binding as sdt
    A = inputs.uniform_f16((512, 8192), 72)
    B = inputs.uniform_f16((512, 8192), 73)
    p = sdt.pick_tile(512, 512, 8192, 256)
    assert (p["id"], p["kgroups"], p["stages"]) == (4, 2, 4)
    say("long pipeline 512x512x8192 uniform, automatic plan")
    C, pad_ok = run_gemm(A, B)
    assert pad_ok
    assert_close(C, oracle.gemm(A, B))


def test_offsets_past_4gib():
    """Operand and output rows more than 4 GiB from their base pointers (lda =
    ldc = 131072, M = 16448): every rung, both pipelines, reaches them with
    64-bit row offsets and writes nothing past N.  Exact integer sums."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    M, N, K, ld = 16448, 256, 64, 131072
    assert (M - 1) * ld * 2 > (1 << 32)
    A = inputs.integer_f16((M, K), 60)
    B = inputs.integer_f16((N, K), 61)
    ref = oracle.gemm(A, B)
    say(f"offsets past 4 GiB: M={M} N={N} K={K} lda=ldb=ldc={ld}")
    dA = torch.empty((M, ld), dtype=torch.float16, device="cuda:0")
    dB = torch.empty((N, ld), dtype=torch.float16, device="cuda:0")
    dA[:, :K].copy_(torch.from_numpy(A))
    dB[:, :K].copy_(torch.from_numpy(B))
    dC = torch.empty((M, ld), dtype=torch.float16, device="cuda:0")
    for tile in range(_ntiles()):
        info = sdt.tile_info(tile)
        for stages in (2, info["stages"]):
            say(f"offsets past 4 GiB tile={tile} stages={stages}")
            dC.fill_(float("nan"))
            sdt.gemm_f16_cfg(dA[:, :K], dB[:, :K], dC[:, :N], tile_id=tile, stages=stages,
                             kgroups=1, stagger=0)
            torch.cuda.synchronize()
            assert bool(torch.isnan(dC[:, N:N + 64]).all().item())
            assert bool(torch.isnan(dC[-1, -64:]).all().item())
            assert_bitexact(dC[:, :N].cpu().numpy(), ref)
    del dA, dB, dC
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape", [(200, 136, 136), (64, 64, 64), (513, 771, 520), (1, 700, 1000)])
def test_two_kgroups_every_rung(shape):
    """Two k-groups of waves (the second takes sub-steps 1 and 3 of every
    k-tile, its partial sums added through LDS) on every rung built with
    them: integer inputs bit for bit, uniform inputs within tolerance, ragged
    M/N/K (K = 136 and 520 end in a partial k-tile), NaN-padded C."""
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    Ai = inputs.integer_f16((M, K), 15)
    Bi = inputs.integer_f16((N, K), 16)
    refi = oracle.gemm(Ai, Bi)
    Au = inputs.uniform_f16((M, K), 17)
    Bu = inputs.uniform_f16((N, K), 18)
    refu = oracle.gemm(Au, Bu)
    for tile in range(_ntiles()):
        info = sdt.tile_info(tile)
        if info["kgroups"] != 2:
            continue
        say(f"two k-groups {shape} tile={tile}")
        C, pad_ok = run_gemm(Ai, Bi, tile=tile, stagger=0, kgroups=2)
        assert pad_ok
        assert_bitexact(C, refi)
        C, pad_ok = run_gemm(Au, Bu, tile=tile, stagger=0, kgroups=2)
        assert pad_ok
        assert_close(C, refu)


def test_two_kgroups_auto_plan_matches_oracle():
    """Shapes whose automatic plan uses two k-groups (each rung's grid and
    k-loop thresholds) against the oracle, and bit-identical to the forced
    plan."""
    from shape_driven_tile_amd import binding as sdt
    for (M, N, K) in [(1024, 1024, 4096), (768, 768, 2560), (896, 896, 3072),
                      (1152, 1152, 8192)]:
        p = sdt.pick_tile(M, N, K, 256)
        assert p["kgroups"] == 2, (M, N, K)
        say(f"auto two k-groups {M}x{N}x{K} tile={p['id']}")
        A = inputs.uniform_f16((M, K), 19)
        B = inputs.uniform_f16((N, K), 20)
        C, _ = run_gemm(A, B)
        C2, _ = run_gemm(A, B, tile=p["id"], stagger=p["stagger"], stages=p["stages"], kgroups=2)
        assert (C.view(np.uint16) == C2.view(np.uint16)).all()
        r, c = sample_positions(M, N, rows=8, cols=8, extra=2048, seed=M)
        assert_close(C[r, c], oracle.gemm_sample(A, B, r, c))


@pytest.mark.parametrize("K", [1, 8, 256, 1920, 2048, 2304, 4096, 8192, 16384])
def test_all_ones(K):
    say(f"all-ones K={K}")
    A = np.ones((96, max(K, 8)), np.float16)
    B = np.ones((160, max(K, 8)), np.float16)
    C, _ = run_gemm(A, B, K=K)
    assert (C.astype(np.float64) == K).all()


def test_identity():
    say("identity B, M != K")
    A = inputs.uniform_f16((384, 256), 13)
    B = np.eye(256, dtype=np.float16)
    C, _ = run_gemm(A, B)
    assert (C.view(np.uint16) == A.view(np.uint16)).all()


def test_k1_outer_product():
    say("K=1 outer product, padded rows")
    a = inputs.padded(inputs.uniform_f16((70, 1), 14), 8)
    b = inputs.padded(inputs.uniform_f16((90, 1), 15), 8)
    C, _ = run_gemm(a, b, K=1)
    assert_bitexact(C, oracle.gemm(a, b, K=1))


def test_overflow_rounds_to_inf():
    say("overflow to inf")
    A = np.full((64, 64), 255.0, np.float16)
    B = np.full((64, 64), 255.0, np.float16)
    B[::2] = -255.0
    C, _ = run_gemm(A, B)
    ref = oracle.gemm(A, B)
    assert ((oracle.f16_encode_rne(ref) & 0x7FFF) == 0x7C00).all(), "every fp16 result is +-inf"
    assert_bitexact(C, ref)


# ---- ragged shapes, strides and padding --------------------------------------

@pytest.mark.parametrize("M,N,K,pa,pb,pc", [
    (1, 1, 1, 7, 7, 7), (3, 5, 7, 1, 9, 3), (65, 129, 72, 8, 0, 8), (257, 511, 8, 0, 8, 0),
    (100, 90, 37, 3, 11, 6), (300, 200, 1000, 24, 0, 40), (129, 1025, 200, 64, 64, 64),
    (520, 260, 4100, 0, 0, 0), (2, 3000, 300, 4, 4, 8), (300, 1, 520, 8, 8, 7),
    (2, 1, 16384, 0, 0, 7), (3000, 3100, 1000, 8, 0, 8)])
def test_ragged_and_padded(M, N, K, pa, pb, pc):
    """Ragged M, N, K with padded leading dimensions full of NaN: the padding
    never reaches C, and nothing past column N of C is written."""
    say(f"ragged M={M} N={N} K={K} pads={pa},{pb},{pc}")
    ka = -(-(K + pa) // 8) * 8
    kb = -(-(K + pb) // 8) * 8
    A = inputs.padded(inputs.uniform_f16((M, K), 21), ka)
    B = inputs.padded(inputs.uniform_f16((N, K), 22), kb)
    C, pad_ok = run_gemm(A, B, K=K, ldc_pad=pc)
    assert_close(C, oracle.gemm(A, B, K=K))
    assert pad_ok, "kernel wrote past column N"


def _random_shapes(count, seed=2024, max_work=2 ** 33):
    """Seeded shapes for the automatic plan: K log-uniform in [1, 4096]; M and
    N log-uniform in [1, 4096] for a quarter of the shapes and in [256, 4096]
    for the rest (so the larger rungs come up too); M * N * K kept under
    max_work so the oracle stays quick; leading dimensions padded by 0-40
    elements, rounded up to multiples of 8."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        lo = 0 if len(out) < count // 4 else 8
        M, N = (int(round(2 ** rng.uniform(lo, 12))) for _ in range(2))
        K = int(round(2 ** rng.uniform(0, 12)))
        if M * N * K > max_work:
            continue
        pads = [int(rng.integers(0, 41)) for _ in range(3)]
        out.append((M, N, K, *pads))
    return out


@pytest.mark.parametrize("M,N,K,pa,pb,pc", _random_shapes(40))
def test_integer_exact_random_shapes_auto(M, N, K, pa, pb, pc):
    """Seeded random shapes through gemm_f16's automatic plan (whatever rung,
    pipeline, k-group count and stagger it picks), integer inputs with
    NaN-filled padding: C equals the oracle's RNE result bit for bit and
    nothing past column N is written."""
    from shape_driven_tile_amd import binding as sdt
    plan = sdt.pick_tile(M, N, K, 256)
    say(f"random auto M={M} N={N} K={K} pads={pa},{pb},{pc} rung={plan['id']} "
        f"stages={plan['stages']} kgroups={plan['kgroups']} stagger={plan['stagger']}")
    ka = -(-(K + pa) // 8) * 8
    kb = -(-(K + pb) // 8) * 8
    A = inputs.padded(inputs.integer_f16((M, K), 1000 + M), ka)
    B = inputs.padded(inputs.integer_f16((N, K), 2000 + N), kb)
    C, pad_ok = run_gemm(A, B, K=K, ldc_pad=pc)
    assert_bitexact(C, oracle.gemm(A, B, K=K))
    assert pad_ok, "kernel wrote past column N"


def test_random_shapes_reach_every_rung():
    """The random-shape set above reaches at least five rungs (a host-side
    check of what it covers)."""
    from shape_driven_tile_amd import binding as sdt
    rungs = {sdt.pick_tile(M, N, K, 256)["id"] for M, N, K, *_ in _random_shapes(40) if M > 1}
    assert len(rungs) >= 5, rungs


def test_every_tile_forced_uniform():
    A, B = inputs.square_operands(520, 4)
    ref = oracle.gemm(A, B)
    for tile in range(_ntiles()):
        say(f"uniform 520^3 tile={tile}")
        C, _ = run_gemm(A, B, tile=tile, stagger=0)
        assert_close(C, ref)


def test_padded_and_tight_same_shape():
    """A padded slice and a tight operand of one shape give the same result
    (strides are runtime arguments, so no kernel is shared at the wrong pitch;
    FlyDSL PR, Changes: the resolve-cache stride key)."""
    say("padded vs tight same shape")
    A, B = inputs.square_operands(512, 5)
    Ct, _ = run_gemm(A, B)
    Cp, _ = run_gemm(inputs.padded(A, 512 + 64), inputs.padded(B, 512 + 32), K=512)
    assert (Ct.view(np.uint16) == Cp.view(np.uint16)).all()


# ---- M = 1 and the GEMV -------------------------------------------------------

def test_m1_routes_to_gemv():
    say("gemm_f16 M=1 == gemv_f16_m1; gemm_f16_ex M=1 via the MFMA kernel")
    x = inputs.decode_activations()
    W = inputs.decode_weights(0)
    y = run_gemv(x, W)
    C, _ = run_gemm(x[None, :], W)
    assert (C[0].view(np.uint16) == y.view(np.uint16)).all()
    C2, _ = run_gemm(x[None, :], W, tile=-1, stagger=0)
    assert_close(C2[0], oracle.gemv_m1(x, W))


@pytest.mark.parametrize("N,K", [(12288, 4096), (12289, 1000), (100, 37), (77, 5000),
                                 (4096, 8), (33, 1)])
def test_gemv_variants_agree(N, K):
    from shape_driven_tile_amd import binding as sdt
    x = inputs.uniform_f16((K,), 31)
    W = inputs.padded(inputs.normal_f16((N, K), 32), -(-K // 8) * 8 + 8)
    ref = oracle.gemv_m1(x, W, K=K)
    base = None
    for v in range(sdt.gemv_num_variants()):
        say(f"gemv N={N} K={K} variant={v}")
        y = run_gemv(x, W, K=K, variant=v)
        assert_close(y, ref)
        if v == 0:
            continue          # four waves per column: the same products, another order
        if base is None:
            base = y
        assert (y.view(np.uint16) == base.view(np.uint16)).all(), "variants differ"
    # exact inputs: every variant gives the oracle's rounding bit for bit
    xi = inputs.integer_f16((K,), 33)
    Wi = inputs.padded(inputs.integer_f16((N, K), 34), -(-K // 8) * 8 + 8)
    refi = oracle.gemv_m1(xi, Wi, K=K)
    for v in range(sdt.gemv_num_variants()):
        say(f"gemv integer N={N} K={K} variant={v}")
        assert_bitexact(run_gemv(xi, Wi, K=K, variant=v), refi)


def test_gemv_exact_cases():
    say("gemv one-hot and integer inputs")
    K, N = 4096, 12288
    W = inputs.normal_f16((N, K), 41)
    for j in (0, 4095, 1234):
        e = np.zeros(K, np.float16)
        e[j] = 1
        y = run_gemv(e, W)
        assert (y.view(np.uint16) == W[:, j].view(np.uint16)).all()
    xi = inputs.integer_f16((K,), 42)
    Wi = inputs.integer_f16((N, K), 43)
    assert_bitexact(run_gemv(xi, Wi), oracle.gemv_m1(xi, Wi))


# ---- degenerate calls, errors, streams, determinism ---------------------------

def test_k0_writes_zeros_and_empty_is_noop():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("K=0 zeros, M=0/N=0 no-op")
    A = torch.empty((70, 0), dtype=torch.float16, device="cuda:0")
    B = torch.empty((50, 0), dtype=torch.float16, device="cuda:0")
    C = torch.full((70, 56), 7.0, dtype=torch.float16, device="cuda:0")[:, :50]
    sdt.gemm_f16(A, B, C)
    torch.cuda.synchronize()
    assert (C == 0).all().item()
    C2 = torch.full((0, 50), 7.0, dtype=torch.float16, device="cuda:0")
    sdt.gemm_f16(torch.empty((0, 64), dtype=torch.float16, device="cuda:0"),
                 torch.ones((50, 64), dtype=torch.float16, device="cuda:0"), C2)
    y = torch.full((12,), 7.0, dtype=torch.float16, device="cuda:0")
    sdt.gemv_f16_m1(torch.empty((0,), dtype=torch.float16, device="cuda:0"),
                    torch.empty((12, 0), dtype=torch.float16, device="cuda:0"), y)
    torch.cuda.synchronize()
    assert (y == 0).all().item()


def test_misaligned_operands_are_rejected():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("misaligned operands rejected before launch")
    buf = torch.zeros((64, 72), dtype=torch.float16, device="cuda:0")
    B = torch.zeros((64, 64), dtype=torch.float16, device="cuda:0")
    C = torch.full((64, 64), 3.0, dtype=torch.float16, device="cuda:0")
    with pytest.raises(sdt.SdtError) as e:
        sdt.gemm_f16(buf[:, 1:65], B, C)
    assert e.value.status == sdt.SDT_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (C == 3.0).all().item()


def test_nondefault_stream():
    import torch
    say("non-default stream")
    A, B = inputs.square_operands(640, 6)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C, _ = run_gemm(A, B, stream=s)
    assert_close(C, oracle.gemm(A, B))


def test_concurrent_host_threads_own_streams():
    """The entry points are reentrant: four host threads, each enqueueing on
    its own stream (ctypes drops the GIL for the call), produce bit for bit
    what the same calls give one after another on the default stream.  The
    shapes differ per thread so different rungs, plans and the GEMV run at
    the same time; every output is allocated before the threads start."""
    import threading

    import torch
    from shape_driven_tile_amd import binding as sdt
    cases = [(512, 512, 512), (1000, 1104, 520), (2048, 2048, 2048), (1, 12288, 4096)]
    ops = []
    for i, (M, N, K) in enumerate(cases):
        A = to_dev(inputs.uniform_f16((M, K), 900 + i))
        B = to_dev(inputs.uniform_f16((N, K), 950 + i))
        ops.append((A, B, [torch.empty((M, N), dtype=torch.float16, device="cuda:0")
                           for _ in range(5)]))

    def call(A, B, C, stream=None):
        if A.shape[0] == 1:
            sdt.gemv_f16_m1(A[0], B, C[0], stream=stream)
        else:
            sdt.gemm_f16(A, B, C, stream=stream)

    say("concurrent host threads: sequential reference")
    refs = []
    for A, B, outs in ops:
        R = torch.empty_like(outs[0])
        call(A, B, R)
        refs.append(R)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in ops]
    errors = []

    def worker(j):
        try:
            A, B, outs = ops[j]
            for C in outs:
                call(A, B, C, stream=streams[j])
        except Exception as e:          # reported after the join
            errors.append((j, repr(e)))

    say("concurrent host threads: 4 threads x 5 calls")
    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(ops))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a host thread did not return"
    torch.cuda.synchronize()
    assert not errors, errors
    assert sdt.last_hip_error() == 0
    for (A, B, outs), R in zip(ops, refs):
        for C in outs:
            assert torch.equal(C.view(torch.int16), R.view(torch.int16))


def test_determinism_repeated_launches():
    """No atomics on the path: repeated launches are bit-identical (a missing
    barrier or an LDS race would show up as run-to-run differences)."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    A, B = inputs.square_operands(1536, 7)
    dA, dB = to_dev(A), to_dev(B)
    outs = []
    for tile in range(_ntiles()):
        say(f"determinism 1536^3 tile={tile}")
        first = None
        for _ in range(10):
            C = torch.empty((1536, 1536), dtype=torch.float16, device="cuda:0")
            sdt.gemm_f16_ex(dA, dB, C, tile_id=tile)
            torch.cuda.synchronize()
            if first is None:
                first = C
            else:
                assert torch.equal(first.view(torch.int16), C.view(torch.int16))
        outs.append(first)
    x = to_dev(inputs.decode_activations())
    W = to_dev(inputs.decode_weights(1))
    ys = []
    for _ in range(10):
        y = torch.empty((inputs.DECODE_N,), dtype=torch.float16, device="cuda:0")
        sdt.gemv_f16_m1(x, W, y)
        ys.append(y)
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))


def test_graph_capture_replays_match_eager():
    """Calls captured in a HIP graph (the library allocates nothing and
    records no memset, so a caller may capture it) replay bit for bit like
    eager launches, several times in a row with eager work and syncs between
    replays: a 2-stage, a deep and a two-k-group GEMM, the K = 0 fill, and
    both decode GEMVs."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    dev = "cuda:0"
    shapes = [(256, 256, 256), (1000, 1000, 1000), (300, 260, 4104), (64, 48, 0)]
    ops = []
    for i, (M, N, K) in enumerate(shapes):
        A = torch.from_numpy(inputs.uniform_f16((M, K), 40 + i)).to(dev)
        B = torch.from_numpy(inputs.uniform_f16((N, K), 50 + i)).to(dev)
        ldc = -(-N // 8) * 8
        C = torch.empty((M, ldc), dtype=torch.float16, device=dev)[:, :N]
        ops.append((A, B, C))
    x = torch.from_numpy(inputs.decode_activations()).to(dev)
    W = torch.from_numpy(inputs.decode_weights(2)).to(dev)
    Wkn = torch.from_numpy(inputs.decode_weights_kn(2)).to(dev)
    y1 = torch.empty((inputs.DECODE_N,), dtype=torch.float16, device=dev)
    y2 = torch.empty_like(y1)

    def work():
        for i, (A, B, C) in enumerate(ops):
            if i == 0:   # the automatic plan never takes the 2-stage pipeline: forced
                sdt.gemm_f16_cfg(A, B, C, stages=2)
            else:
                sdt.gemm_f16(A, B, C)
        sdt.gemv_f16_m1(x, W, y1)
        sdt.gemv_f16_m1_kn(x, Wkn, y2)

    say("graph capture: eager reference")
    work()
    torch.cuda.synchronize()
    ref = [C.clone() for _, _, C in ops] + [y1.clone(), y2.clone()]
    outs = [C for _, _, C in ops] + [y1, y2]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"graph capture: replay {rep}")
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.contiguous().view(torch.int16), r.contiguous().view(torch.int16)), rep
        work()                       # eager work between replays
        torch.cuda.synchronize()
