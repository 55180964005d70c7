"""GPU parity of the k-split launches (gemm_f16_ws / gemm_bf16_ws and forced
split configurations through gemm_f16_cfg) against the CPU oracle.

A k-split divides each output tile's full k-tiles into contiguous runs, one
workgroup each (the last also takes a partial k-tile), and adds the fp32
partial sums in split order before the one rounding to the output type
("Iteratively Tuning hipBLASLt TensileLite Kernels", The Six Rounds, 2:
Split-K, with the partials reduced either by a second kernel or inside the
same kernel).  Integer inputs in [-2, 2] make every fp32 partial and total
exact, so every split count, boundary, reduction and pipeline must give the
oracle's RNE rounding bit for bit; uniform inputs are held to the stated
tolerance, and both reductions must agree bit for bit (same order of sums).
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (DEV, assert_bitexact, assert_bitexact_bf16, assert_close, bits_to_dev_bf16,
                         dev_bf16_to_bits, say, to_dev)
from shape_driven_tile_amd import inputs

pytestmark = pytest.mark.gpu


def _sdt():
    from shape_driven_tile_amd import binding as sdt
    return sdt


def _ws(nbytes):
    return _sdt().Workspace(nbytes, device=DEV)


def _counters_zero(ws, nbytes):
    import torch
    torch.cuda.synchronize()
    return bool((ws.tensor[:nbytes] == 0).all().item())


def _launch(A, B, ws, **cfg):
    """A: (M, K), B: (N, K) device float16; returns C (M, N) on the host and
    whether the NaN padding past N stayed untouched."""
    import torch
    sdt = _sdt()
    M, N = A.shape[0], B.shape[0]
    ldc = -(-N // 8) * 8 + 8
    full = torch.full((M, ldc), float("nan"), dtype=torch.float16, device=DEV)
    C = full[:, :N]
    if cfg:
        sdt.gemm_f16_cfg(A, B, C, workspace=ws, **cfg)
    else:
        sdt.gemm_f16_ws(A, B, C, workspace=ws)
    torch.cuda.synchronize()
    return C.cpu().numpy(), bool(torch.isnan(full[:, N:]).all().item())


def _split_counts(K):
    nfull = K // 64
    return sorted({s for s in (2, 3, 4, 5, 7, 8, 16) if s <= nfull} | ({nfull} if nfull <= 16 else set()))


@pytest.mark.parametrize("shape", [(300, 260, 1000), (257, 129, 4160), (64, 64, 320),
                                   (130, 70, 136)])
def test_integer_exact_every_split(shape):
    """Every k-split rung, split count (up to one per full k-tile, so a split
    of a single k-tile and splits of unequal length occur), both reductions,
    and the 2-stage, deep and two-k-group pipelines: bit for bit on integer
    inputs, ragged M, N and K (a partial k-tile on the last split)."""
    sdt = _sdt()
    M, N, K = shape
    A = inputs.integer_f16((M, K), 301)
    B = inputs.integer_f16((N, K), 302)
    ref = oracle.gemm(A, B)
    dA, dB = to_dev(A), to_dev(B)
    ws = _ws(64 << 20)
    tried = 0
    for tile in range(sdt.num_tiles()):
        info = sdt.tile_info(tile)
        if not info["ksplit"]:
            continue
        pipes = [(2, 1), (info["stages"], 1), (info["stages"], 2)]
        if info["long_stages"]:
            pipes.append((info["long_stages"], 2))
        for sp in _split_counts(K):
            for stages, kg in pipes:
                for algo in (0, 1):
                    say(f"k-split integer {shape} tile={tile} splits={sp} algo={algo} "
                        f"stages={stages} kgroups={kg}")
                    C, pad_ok = _launch(dA, dB, ws, tile_id=tile, stagger=0, splits=sp,
                                        split_algo=algo, stages=stages, kgroups=kg)
                    assert pad_ok
                    assert_bitexact(C, ref)
                    tried += 1
    assert tried >= 3 * 3 * 2 * len(_split_counts(K))   # 3 rungs x 3+ pipelines x 2 reductions
    assert _counters_zero(ws, 65536), "arrival counters not left at zero"


def _random_long_k(count, seed=77, max_work=2 ** 33):
    """Seeded long-K shapes for gemm_f16_ws's automatic plan: M and N
    log-uniform in [1, 2048], K log-uniform in [1024, 49152], M * N * K under
    max_work (the oracle stays quick)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        M, N = (int(round(2 ** rng.uniform(0, 11))) for _ in range(2))
        K = int(round(2 ** rng.uniform(10, np.log2(49152))))
        if M * N * K <= max_work:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("shape", _random_long_k(24))
def test_integer_exact_random_long_k_ws(shape):
    """Seeded random long-K shapes through gemm_f16_ws with the workspace its
    plan asks for (split or not, whatever the plan picks): integer inputs, C
    equal to the oracle's RNE result bit for bit, nothing written past column
    N, and the arrival counters left at zero."""
    sdt = _sdt()
    M, N, K = shape
    plan = sdt.pick_tile_ws(M, N, K, 0, 1 << 40)
    need = sdt.gemm_workspace_size(M, N, K)
    assert (need > 0) == (plan["splits"] > 1)
    say(f"random long-K ws {shape} rung={plan['id']} splits={plan['splits']} "
        f"algo={plan['split_algo']} kgroups={plan['kgroups']} stages={plan['stages']}")
    ld = -(-K // 8) * 8                  # rows padded (NaN) to the 8-element pitch
    A = inputs.padded(inputs.integer_f16((M, K), 500 + M), ld)
    B = inputs.padded(inputs.integer_f16((N, K), 600 + N), ld)
    ws = _ws(max(need, 65536))
    C, pad_ok = _launch(to_dev(A)[:, :K], to_dev(B)[:, :K], ws)
    assert pad_ok
    assert_bitexact(C, oracle.gemm(A, B, K=K))
    assert _counters_zero(ws, 65536 if need else 0), "arrival counters not left at zero"


def test_random_long_k_set_splits():
    """Host-side: the random long-K set above has split and unsplit plans."""
    sdt = _sdt()
    splits = [sdt.pick_tile_ws(M, N, K, 256, 1 << 40)["splits"] for M, N, K in _random_long_k(24)]
    assert sum(s > 1 for s in splits) >= 6 and sum(s == 1 for s in splits) >= 2, splits


@pytest.mark.parametrize("shape", [(256, 256, 256), (512, 512, 512), (1024, 1024, 1024),
                                   (1536, 1536, 1536), (256, 256, 16384), (128, 128, 65536),
                                   (512, 512, 8192), (384, 384, 12288), (200, 300, 20000)])
def test_uniform_automatic_plan(shape):
    """gemm_f16_ws's automatic plan (uniform [-1, 1]) on square workloads,
    where it does not split, and on long-K ones, where it does: every element
    against the oracle; with a workspace too small for its split it runs
    gemm_f16's plan, bit for bit."""
    import torch
    sdt = _sdt()
    M, N, K = shape
    A = inputs.uniform_f16((M, K), 361)
    B = inputs.uniform_f16((N, K), 362)
    dA, dB = to_dev(A), to_dev(B)
    need = sdt.gemm_workspace_size(M, N, K)
    plan = sdt.pick_tile_ws(M, N, K, 0, 1 << 40)
    assert (need > 0) == (plan["splits"] > 1)
    assert (plan["splits"] > 1) == (K >= 8192), plan
    ws = _ws(max(need, 16))
    say(f"k-split automatic plan {shape} (splits={plan['splits']} algo={plan['split_algo']})")
    C, pad_ok = _launch(dA, dB, ws)
    assert pad_ok
    assert_close(C, oracle.gemm(A, B))
    # no workspace (or too small): the unsplit plan, the same bits as gemm_f16
    small = _ws(16)
    C2, _ = _launch(dA, dB, small)
    ldc = -(-N // 8) * 8
    C3 = torch.empty((M, ldc), dtype=torch.float16, device=DEV)[:, :N]
    sdt.gemm_f16(dA, dB, C3)
    torch.cuda.synchronize()
    assert np.array_equal(C2.view(np.uint16), C3.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("shape", [(1536, 1536, 1536), (1000, 1000, 3000), (640, 384, 4096)])
def test_uniform_both_reductions_agree(shape):
    """Uniform inputs: the two reductions add the same partials in the same
    order, so they agree bit for bit, and both match the oracle within the
    tolerance; repeated launches give identical bits (no arrival-order
    dependence in the single-kernel reduction)."""
    sdt = _sdt()
    M, N, K = shape
    A = inputs.uniform_f16((M, K), 311)
    B = inputs.uniform_f16((N, K), 312)
    ref = oracle.gemm(A, B)
    dA, dB = to_dev(A), to_dev(B)
    ws = _ws(64 << 20)
    for tile in (2, 3, 4):
        for sp in (2, 3, 5):
            outs = []
            for algo in (0, 1, 1, 1):
                say(f"k-split uniform {shape} tile={tile} splits={sp} algo={algo}")
                C, _ = _launch(dA, dB, ws, tile_id=tile, splits=sp, split_algo=algo)
                outs.append(C.view(np.uint16).copy())
            assert_close(outs[0].view(np.float16), ref)
            for o in outs[1:]:
                assert np.array_equal(o, outs[0])


def test_forced_split_needs_workspace_and_a_split_rung():
    """A forced split is refused (SDT_ERR_INVALID_ARG, nothing launched)
    without a workspace, with one smaller than it needs, on a rung not built
    for it, with more splits than full k-tiles, or with the stagger on."""
    import torch
    sdt = _sdt()
    A = torch.zeros((512, 1024), dtype=torch.float16, device=DEV)
    B = torch.zeros((512, 1024), dtype=torch.float16, device=DEV)
    C = torch.zeros((512, 512), dtype=torch.float16, device=DEV)
    need = sdt.launch_workspace_size(512, 512, 1024, tile_id=4, splits=4, split_algo=1,
                                     stages=-1, kgroups=-1, stagger=0, persistent=-1)
    assert need == 65536 + 64 * 4 * 64 * 64 * 4   # the counter area + 64 tiles x 4 splits
    bad = [dict(tile_id=4, splits=4, workspace=None),
           dict(tile_id=4, splits=4, workspace=_ws(need - 16)),
           dict(tile_id=0, splits=2, workspace=_ws(64 << 20)),
           dict(tile_id=1, splits=2, workspace=_ws(64 << 20)),
           dict(tile_id=5, splits=2, workspace=_ws(64 << 20)),
           dict(tile_id=6, splits=2, workspace=_ws(64 << 20)),
           dict(tile_id=7, splits=2, workspace=_ws(64 << 20)),
           dict(tile_id=4, splits=17, workspace=_ws(64 << 20)),   # 16 full k-tiles
           dict(tile_id=4, splits=65, workspace=_ws(64 << 20)),
           dict(tile_id=4, splits=16, stagger=1, workspace=_ws(64 << 20))]
    for kw in bad:
        with pytest.raises(sdt.SdtError) as e:
            sdt.gemm_f16_cfg(A, B, C, **kw)
        assert e.value.status == sdt.SDT_ERR_INVALID_ARG, kw
    # 1024 / 64 = 16 full k-tiles: 16 splits is the most
    sdt.gemm_f16_cfg(A, B, C, tile_id=4, splits=16, workspace=_ws(64 << 20))
    with pytest.raises(sdt.SdtError):
        sdt.gemm_f16_cfg(A[:, :960], B[:, :960], C, tile_id=4, splits=16, workspace=_ws(64 << 20))
    torch.cuda.synchronize()


def test_graph_replays_match_eager():
    """gemm_f16_ws captured in a HIP graph (the single-kernel reduction with
    its arrival counters, and the two-kernel one), replayed four times with
    eager launches between the replays: every replay bit-identical to the
    eager result, and the counters back at zero."""
    import torch
    sdt = _sdt()
    M = N = 768
    K = 2048
    A = to_dev(inputs.uniform_f16((M, K), 321))
    B = to_dev(inputs.uniform_f16((N, K), 322))
    for algo in (1, 0):
        ws = _ws(64 << 20)
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        sdt.gemm_f16_cfg(A, B, C, tile_id=4, splits=4, split_algo=algo, workspace=ws)
        torch.cuda.synchronize()
        eager = C.clone()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                sdt.gemm_f16_cfg(A, B, C, tile_id=4, splits=4, split_algo=algo, workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for r in range(4):
            say(f"k-split graph replay algo={algo} #{r}")
            C.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(C.view(torch.int16), eager.view(torch.int16))
            sdt.gemm_f16_cfg(A, B, C, tile_id=4, splits=3, split_algo=algo, workspace=ws)
            torch.cuda.synchronize()
        assert _counters_zero(ws, 4096)
        del g


def test_two_streams_own_workspaces():
    """Two streams, each with its own workspace, running single-kernel
    k-split launches at the same time: both results bit for bit equal to
    sequential launches."""
    import torch
    sdt = _sdt()
    M, N, K = 512, 384, 2048
    A = to_dev(inputs.integer_f16((M, K), 331))
    B = to_dev(inputs.integer_f16((N, K), 332))
    ref = oracle.gemm(A.cpu().numpy(), B.cpu().numpy())
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    w1, w2 = _ws(32 << 20), _ws(32 << 20)
    C1 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    C2 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    torch.cuda.synchronize()
    say("k-split on two streams, own workspaces")
    for _ in range(20):
        sdt.gemm_f16_cfg(A, B, C1, tile_id=4, splits=4, split_algo=1, workspace=w1, stream=s1)
        sdt.gemm_f16_cfg(A, B, C2, tile_id=3, splits=8, split_algo=1, workspace=w2, stream=s2)
    torch.cuda.synchronize()
    assert_bitexact(C1.cpu().numpy(), ref)
    assert_bitexact(C2.cpu().numpy(), ref)


def test_bf16_split_integer_and_uniform():
    """gemm_bf16 through the same k-split kernels: integer inputs bit for bit
    with both reductions, uniform inputs within the bf16 tolerance."""
    import torch
    sdt = _sdt()
    M, N, K = 300, 260, 1000
    A = inputs.integer_bf16((M, K), 341)
    B = inputs.integer_bf16((N, K), 342)
    ref = oracle.gemm(A, B, dtype="bf16")
    dA, dB = bits_to_dev_bf16(A), bits_to_dev_bf16(B)
    ws = _ws(64 << 20)
    for tile in (2, 3, 4):
        for algo in (0, 1):
            say(f"bf16 k-split integer tile={tile} algo={algo}")
            C = torch.full((M, -(-N // 8) * 8), float("nan"), dtype=torch.bfloat16,
                           device=DEV)[:, :N]
            sdt.gemm_bf16_cfg(dA, dB, C, tile_id=tile, splits=3, split_algo=algo, workspace=ws)
            torch.cuda.synchronize()
            assert_bitexact_bf16(dev_bf16_to_bits(C), ref)
    Au, Bu = inputs.square_operands_bf16(768, 1)
    C = torch.empty((768, 768), dtype=torch.bfloat16, device=DEV)
    wsu = _ws(max(sdt.gemm_workspace_size(768, 768, 768), 16))
    sdt.gemm_bf16_ws(bits_to_dev_bf16(Au), bits_to_dev_bf16(Bu), C, workspace=wsu)
    torch.cuda.synchronize()
    got = oracle.bf16_decode(dev_bf16_to_bits(C))
    refu = oracle.gemm(Au, Bu, dtype="bf16")
    assert (np.abs(got - refu) <= oracle.tolerance(refu, "bf16")).all()


def test_workspace_reused_across_shapes():
    """One workspace serving k-split launches of different shapes in turn
    (few tiles, then many, then few): the partial sums of one launch never
    land in the counter area another relies on, so every launch is bit for
    bit right and the counters end at zero."""
    sdt = _sdt()
    ws = _ws(64 << 20)
    for (M, N, K, tile, sp) in [(128, 128, 1024, 3, 8), (700, 650, 1000, 4, 7),
                                (256, 128, 2048, 2, 16), (900, 1000, 768, 4, 3),
                                (64, 64, 512, 4, 8)]:
        A = inputs.integer_f16((M, K), 351 + M)
        B = inputs.integer_f16((N, K), 352 + N)
        say(f"workspace reuse {M}x{N}x{K} tile={tile} splits={sp}")
        C, pad_ok = _launch(to_dev(A), to_dev(B), ws, tile_id=tile, splits=sp, split_algo=1)
        assert pad_ok
        assert_bitexact(C, oracle.gemm(A, B))
    assert _counters_zero(ws, 65536)
