"""GPU parity of the [K][N] decode GEMV split over K through a workspace
(gemv_f16_m1_kn_ws, gemv_bf16_m1_kn_ws) against the CPU oracle, through the
C ABI.

The split path reads 256-column bands with K cut into ranges, writes fp32
column sums to the workspace and adds them in split order in a second kernel.
Cases: the decode shape on all 8 rotating buffers (tolerance) and bit for bit
on integer inputs; ragged N, ragged K (a partial last split and a partial last
block of eight rows), NaN-filled row padding, y untouched past N; repeated
calls bit-identical; a workspace that is too small (or none) gives the
one-launch kernel's bits; K below the split's minimum; graph replays; bf16.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (DEV, assert_bitexact, assert_bitexact_bf16, assert_close,
                         bits_to_dev_bf16, dev_bf16_to_bits, run_gemv_kn, say, to_dev)
from shape_driven_tile_amd import inputs

pytestmark = pytest.mark.gpu


def _sdt():
    from shape_driven_tile_amd import binding as sdt
    return sdt


def run_kn_ws(x, W, N=None, ws_bytes=None, y_pad=8):
    """gemv_f16_m1_kn_ws with a fresh workspace of ws_bytes (default: what the
    split needs).  Returns y (N,) and whether the y_pad elements past N stayed
    NaN."""
    import torch
    sdt = _sdt()
    K, ldb = W.shape
    N = ldb if N is None else N
    need = sdt.gemv_kn_workspace_size(N, K)
    ws = sdt.Workspace(need if ws_bytes is None else ws_bytes, device=DEV)
    dx = to_dev(x[:K])
    dW = to_dev(W)[:, :N]
    full = torch.full((N + y_pad,), float("nan"), dtype=torch.float16, device=DEV)
    sdt.gemv_f16_m1_kn_ws(dx, dW, full[:N], workspace=ws)
    torch.cuda.synchronize()
    return full[:N].cpu().numpy(), bool(torch.isnan(full[N:]).all().item())


def test_split_plan_at_the_decode_shape():
    sdt = _sdt()
    # 48 bands of 256 columns x 16 splits of 256 rows: 768 workgroups
    assert sdt.gemv_kn_workspace_size(12288, 4096) == 16 * 48 * 256 * 4


def test_decode_kn_ws_all_buffers():
    x = inputs.decode_activations()
    for r in range(inputs.DECODE_BUFFERS):
        say(f"gemv_kn_ws decode K=4096 N=12288 buffer {r}")
        W = inputs.decode_weights_kn(r)
        y, pad_ok = run_kn_ws(x, W)
        assert pad_ok
        assert_close(y, oracle.gemv_kn(x, W))


@pytest.mark.parametrize("N,K", [(12288, 4096), (1000, 4100), (777, 1029), (300, 20),
                                 (257, 16), (8, 4096), (4096, 17), (5000, 3001)])
def test_kn_ws_integer_exact(N, K):
    """Integer inputs: every partial sum is exact in fp32, so the split sum is
    the correctly rounded exact sum, bit for bit, whatever the split."""
    sdt = _sdt()
    assert sdt.gemv_kn_workspace_size(N, K) > 0, "the case must take the split path"
    ldb = -(-(N + 5) // 8) * 8
    x = inputs.integer_f16((K,), 91)
    W = inputs.padded(inputs.integer_f16((K, N), 92), ldb)   # NaN past column N
    say(f"gemv_kn_ws integer N={N} K={K} ldb={ldb}")
    y, pad_ok = run_kn_ws(x, W, N=N)
    assert pad_ok, "wrote past N"
    assert_bitexact(y, oracle.gemv_kn(x, W, N=N))


@pytest.mark.parametrize("N,K", [(1000, 4100), (517, 1000), (33, 4096), (12288, 64)])
def test_kn_ws_uniform_ragged(N, K):
    ldb = -(-(N + 5) // 8) * 8
    x = inputs.uniform_f16((K,), 93)
    W = inputs.padded(inputs.normal_f16((K, N), 94, std=0.5), ldb)
    say(f"gemv_kn_ws uniform N={N} K={K}")
    y, pad_ok = run_kn_ws(x, W, N=N)
    assert pad_ok
    assert_close(y, oracle.gemv_kn(x, W, N=N))


def test_kn_ws_small_or_no_workspace_is_the_one_launch_kernel():
    """Without a workspace large enough the call runs gemv_f16_m1_kn: the same
    bits; with none needed (K < 16) likewise."""
    sdt = _sdt()
    for (N, K) in [(12288, 4096), (1000, 4096), (296, 15)]:   # ldb = N, a multiple of 8
        x = inputs.uniform_f16((K,), 95)
        W = inputs.normal_f16((K, N), 96, std=0.5)
        need = sdt.gemv_kn_workspace_size(N, K)
        assert (need == 0) == (K < 16)
        ref, _ = run_gemv_kn(x, W)
        for nb in (0, max(need - 16, 0)):
            say(f"gemv_kn_ws N={N} K={K} workspace {nb} of {need} bytes")
            y, pad_ok = run_kn_ws(x, W, ws_bytes=nb)
            assert pad_ok
            assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))


def test_kn_ws_deterministic_and_reusable():
    """Repeated calls on one workspace give identical bits (the split sum is in
    a fixed order); the workspace needs no clearing between calls or shapes."""
    import torch
    sdt = _sdt()
    x = torch.from_numpy(inputs.decode_activations()).to(DEV)
    W = torch.from_numpy(inputs.decode_weights_kn(5)).to(DEV)
    ws = sdt.Workspace(sdt.gemv_kn_workspace_size(12288, 4096), device=DEV)
    y0 = torch.empty((12288,), dtype=torch.float16, device=DEV)
    say("gemv_kn_ws repeated calls bit-identical")
    sdt.gemv_f16_m1_kn_ws(x, W, y0, workspace=ws)
    y = torch.empty_like(y0)
    xs = torch.from_numpy(inputs.uniform_f16((1029,), 97)).to(DEV)
    Ws = torch.from_numpy(inputs.normal_f16((1029, 776), 98, std=0.5)).to(DEV)
    ys = torch.empty((776,), dtype=torch.float16, device=DEV)
    for i in range(10):
        sdt.gemv_f16_m1_kn_ws(x, W, y, workspace=ws)
        sdt.gemv_f16_m1_kn_ws(xs, Ws, ys, workspace=ws)   # another shape in between
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), i


def test_kn_ws_graph_replays_match_eager():
    import torch
    sdt = _sdt()
    x = torch.from_numpy(inputs.decode_activations()).to(DEV)
    W = torch.from_numpy(inputs.decode_weights_kn(6)).to(DEV)
    ws = sdt.Workspace(sdt.gemv_kn_workspace_size(12288, 4096), device=DEV)
    y_eager = torch.empty((12288,), dtype=torch.float16, device=DEV)
    sdt.gemv_f16_m1_kn_ws(x, W, y_eager, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("gemv_kn_ws captured in a graph, replayed 5 times")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sdt.gemv_f16_m1_kn_ws(x, W, y, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(5):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), i


def test_kn_ws_bf16_integer_exact():
    import torch
    sdt = _sdt()
    N, K = 1000, 4100
    xb = inputs.integer_bf16((K,), 99)
    Wb = inputs.integer_bf16((K, N), 100)
    ref = oracle.gemv_kn(xb, Wb, dtype="bf16")
    ws = sdt.Workspace(sdt.gemv_kn_workspace_size(N, K), device=DEV)
    y = torch.empty((N,), dtype=torch.bfloat16, device=DEV)
    say("gemv_bf16_m1_kn_ws integer N=1000 K=4100")
    sdt.gemv_bf16_m1_kn_ws(bits_to_dev_bf16(xb), bits_to_dev_bf16(Wb), y, workspace=ws)
    torch.cuda.synchronize()
    assert_bitexact_bf16(dev_bf16_to_bits(y), ref)
