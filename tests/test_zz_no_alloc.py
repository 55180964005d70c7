"""The allocation-free entry point gemm_f16_noalloc, through the C ABI,
against gemm_f16_ws (the entry point it is a variant of) with a workspace of
the size the library asks for: the same plan, so the same bits, on two calls
in a row, the second with a smaller input (the library's scratch array then
holds the first call's partial sums and counters), and both within the
tolerance of the oracle.  The shapes are ones whose plan splits K, so the
scratch array is used."""
import numpy as np
import pytest

import oracle
from gpu_helpers import DEV, assert_close, say, to_dev
from shape_driven_tile_amd import inputs

pytestmark = pytest.mark.gpu

SHAPES = [(256, 256, 16384), (128, 192, 8200)]   # the second smaller


def _nan_out(M, N):
    import torch
    ldc = -(-N // 8) * 8
    return torch.full((M, ldc), float("nan"), dtype=torch.float16, device=DEV)[:, :N]


def test_noalloc_matches_workspace_entry_point():
    import torch
    from shape_driven_tile_amd import binding as sdt
    for i, (M, N, K) in enumerate(SHAPES):
        plan = sdt.pick_tile_ws(M, N, K, 0, 1 << 40)
        assert plan["splits"] > 1, "the shape must use the k-split scratch"
        A = inputs.uniform_f16((M, K), 601 + i)
        B = inputs.uniform_f16((N, K), 611 + i)
        dA, dB = to_dev(A), to_dev(B)
        say(f"gemm_f16_noalloc {M}x{N}x{K} (splits {plan['splits']}), call {i + 1}")
        C1 = _nan_out(M, N)
        sdt.gemm_f16_noalloc(dA, dB, C1)
        torch.cuda.synchronize()
        say(f"gemm_f16_ws {M}x{N}x{K}")
        ws = sdt.Workspace(sdt.gemm_workspace_size(M, N, K), device=DEV)
        C2 = _nan_out(M, N)
        sdt.gemm_f16_ws(dA, dB, C2, workspace=ws)
        torch.cuda.synchronize()
        got, want = C1.cpu().numpy(), C2.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
        assert_close(got, oracle.gemm(A, B))


def test_noalloc_unsplit_and_degenerate():
    """Without a split (a square whose plan is gemm_f16's), M = 1 (the GEMV)
    and K = 0 (zeros) it behaves as gemm_f16, bit for bit."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    for (M, N, K) in [(512, 512, 512), (1, 700, 1000), (64, 64, 0)]:
        A = to_dev(inputs.uniform_f16((M, K), 621)) if K else \
            torch.empty((M, 0), dtype=torch.float16, device=DEV)
        B = to_dev(inputs.uniform_f16((N, K), 622)) if K else \
            torch.empty((N, 0), dtype=torch.float16, device=DEV)
        say(f"gemm_f16_noalloc {M}x{N}x{K} against gemm_f16")
        C1, C2 = _nan_out(M, N), _nan_out(M, N)
        sdt.gemm_f16_noalloc(A, B, C1)
        sdt.gemm_f16(A, B, C2)
        torch.cuda.synchronize()
        assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
