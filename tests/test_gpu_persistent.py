"""GPU parity of persistent workgroups on the ping-pong kernel (the FlyDSL
pull request's Changes: persistent workgroups, where the grid is a fixed
number of workgroups and each loops over output tiles): a grid of P
workgroups, workgroup w taking tiles w, w + P, w + 2P, ...  Every tile is
computed exactly as in the one-workgroup-per-tile launch (same per-element
sums), so the two agree bit for bit; integer inputs are exact against the
oracle on ragged grids of every size relation between P and the tile count.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import DEV, assert_bitexact, assert_close, say, to_dev
from shape_driven_tile_amd import inputs

pytestmark = pytest.mark.gpu


def _run(dA, dB, **cfg):
    import torch
    from shape_driven_tile_amd import binding as sdt
    M, N = dA.shape[0], dB.shape[0]
    ldc = -(-N // 8) * 8 + 8
    full = torch.full((M, ldc), float("nan"), dtype=torch.float16, device=DEV)
    sdt.gemm_f16_cfg(dA, dB, full[:, :N], **cfg)
    torch.cuda.synchronize()
    return full[:, :N].cpu().numpy(), bool(torch.isnan(full[:, N:]).all().item())


@pytest.mark.parametrize("shape", [(1000, 1100, 520), (3000, 3100, 1000), (4224, 4096, 264)])
def test_integer_exact_persistent_grids(shape):
    """P = 1, 7, 64, 255, 256 and the tile count (the pull request's only
    non-zero value), on ragged M, N and K: bit for bit."""
    M, N, K = shape
    A = inputs.integer_f16((M, K), 401)
    B = inputs.integer_f16((N, K), 402)
    ref = oracle.gemm(A, B)
    dA, dB = to_dev(A), to_dev(B)
    tiles = -(-M // 256) * -(-N // 256)
    for P in sorted({1, 7, 64, 255, 256, tiles}):
        if P > tiles:
            continue
        say(f"persistent {shape} P={P} of {tiles} tiles")
        C, pad_ok = _run(dA, dB, tile_id=0, stages=3, kgroups=1, stagger=0, persistent=P)
        assert pad_ok
        assert_bitexact(C, ref)


def test_uniform_persistent_matches_per_tile_launch():
    """3072^3 uniform (144 tiles): persistent grids of 144, 128 and 96
    workgroups give the bits of the one-workgroup-per-tile launch, which
    matches the oracle within the tolerance."""
    n = 3072
    A = inputs.uniform_f16((n, n), 411)
    B = inputs.uniform_f16((n, n), 412)
    dA, dB = to_dev(A), to_dev(B)
    say("persistent 3072^3 uniform, per-tile launch")
    base, _ = _run(dA, dB, tile_id=0, stages=3, kgroups=1, persistent=0)
    assert_close(base, oracle.gemm(A, B))
    for P in (144, 128, 96):
        say(f"persistent 3072^3 uniform P={P}")
        C, _ = _run(dA, dB, tile_id=0, stages=3, kgroups=1, persistent=P)
        assert np.array_equal(C.view(np.uint16), base.view(np.uint16))
