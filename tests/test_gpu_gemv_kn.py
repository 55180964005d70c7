"""GPU parity of the [K][N] decode GEMV (gemv_f16_m1_kn) against the CPU
oracle, through the C ABI.

The weights are K rows of N contiguous values, the layout the mojo-baro page
reaches by transposing the weights at load ("Four rounds on the decode
shape").  Cases: the decode shape on all 8 rotating buffers; every variant on
ragged N and K with NaN-filled row padding; exact integer and one-hot inputs
bit for bit; agreement with the [N][K] kernel on the same matrix; K=0, N=0,
K=1; misaligned operands rejected before launch.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import assert_bitexact, assert_close, run_gemv, run_gemv_kn, say
from shape_driven_tile_amd import inputs

pytestmark = pytest.mark.gpu


def test_decode_kn_all_buffers():
    x = inputs.decode_activations()
    for r in range(inputs.DECODE_BUFFERS):
        say(f"gemv_kn decode K=4096 N=12288 buffer {r}")
        W = inputs.decode_weights_kn(r)
        y, pad_ok = run_gemv_kn(x, W)
        assert pad_ok
        assert_close(y, oracle.gemv_kn(x, W))


@pytest.mark.parametrize("N,K", [(12288, 4096), (1000, 4099), (64, 8), (65, 7), (5, 1),
                                 (517, 1000), (33, 4096), (4096, 16)])
def test_kn_variants_ragged_padded(N, K):
    from shape_driven_tile_amd import binding as sdt
    ldb = -(-(N + 5) // 8) * 8
    x = inputs.uniform_f16((K,), 81)
    W = inputs.padded(inputs.normal_f16((K, N), 82, std=0.5), ldb)   # NaN past column N
    ref = oracle.gemv_kn(x, W, N=N)
    for v in range(sdt.gemv_kn_num_variants()):
        say(f"gemv_kn N={N} K={K} ldb={ldb} variant={v}")
        y, pad_ok = run_gemv_kn(x, W, N=N, variant=v)
        assert pad_ok, "wrote past N"
        assert_close(y, ref)


@pytest.mark.parametrize("N,K", [(12288, 4096), (777, 1029)])
def test_kn_exact_integer_every_variant(N, K):
    """Integer inputs: every partial sum is exact in fp32, so each variant's
    output is the correctly rounded exact sum, bit for bit."""
    from shape_driven_tile_amd import binding as sdt
    x = inputs.integer_f16((K,), 83)
    W = inputs.padded(inputs.integer_f16((K, N), 84), -(-N // 8) * 8)   # ldb % 8 == 0
    ref = oracle.gemv_kn(x, W, N=N)
    for v in range(sdt.gemv_kn_num_variants()):
        say(f"gemv_kn integer N={N} K={K} variant={v}")
        y, _ = run_gemv_kn(x, W, N=N, variant=v)
        assert_bitexact(y, ref)


def test_kn_one_hot_selects_a_row():
    K, N = 4096, 12288
    W = inputs.decode_weights_kn(0)
    for j in (0, 7, 8, 2047, 4095):
        say(f"gemv_kn one-hot row {j}")
        e = np.zeros(K, np.float16)
        e[j] = 1
        y, _ = run_gemv_kn(e, W)
        assert (y.view(np.uint16) == W[j].view(np.uint16)).all(), j


def test_kn_matches_nk_layout():
    """The same matrix stored either way round gives results within the
    acceptance bound of each other's oracle (the orders of the fp32 sums
    differ)."""
    say("gemv_kn vs gemv_f16_m1 on the same matrix")
    x = inputs.decode_activations()
    Wnk = inputs.decode_weights(3)
    Wkn = inputs.decode_weights_kn(3)
    ref = oracle.gemv_m1(x, Wnk)
    assert (ref == oracle.gemv_kn(x, Wkn)).all()
    y1 = run_gemv(x, Wnk)
    y2, _ = run_gemv_kn(x, Wkn)
    assert_close(y1, ref)
    assert_close(y2, ref)


def test_kn_degenerate_sizes():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("gemv_kn K=0 writes zeros, N=0 is a no-op, K=1")
    y = torch.full((100,), float("nan"), dtype=torch.float16, device="cuda:0")
    x = torch.empty((0,), dtype=torch.float16, device="cuda:0")
    W = torch.empty((0, 100), dtype=torch.float16, device="cuda:0")
    sdt.gemv_f16_m1_kn(x, W, y)
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == 0).all()
    x1 = torch.ones((3,), dtype=torch.float16, device="cuda:0")
    sdt.gemv_f16_m1_kn(x1, torch.empty((3, 0), dtype=torch.float16, device="cuda:0"),
                       torch.empty((0,), dtype=torch.float16, device="cuda:0"))
    torch.cuda.synchronize()
    xs = inputs.uniform_f16((1,), 85)
    Ws = inputs.uniform_f16((1, 300), 86)
    ys, _ = run_gemv_kn(xs, Ws)
    assert_bitexact(ys, oracle.gemv_kn(xs, Ws))


def test_kn_misaligned_rejected():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("gemv_kn misaligned operands rejected")
    buf = torch.zeros((4096 * 16 + 64,), dtype=torch.float16, device="cuda:0")
    y = torch.zeros((16,), dtype=torch.float16, device="cuda:0")
    L = sdt.lib()
    base = buf.data_ptr()
    # B shifted by one element: not 16-byte aligned
    rc = L.gemv_f16_m1_kn(16, 8, base, base + 2, 16, y.data_ptr(), None)
    assert rc == sdt.SDT_ERR_UNSUPPORTED
    # ldb not a multiple of 8
    rc = L.gemv_f16_m1_kn(16, 8, base, base + 256, 20, y.data_ptr(), None)
    assert rc == sdt.SDT_ERR_UNSUPPORTED
    # x not 16-byte aligned
    rc = L.gemv_f16_m1_kn(16, 8, base + 2, base + 256, 16, y.data_ptr(), None)
    assert rc == sdt.SDT_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_kn_deterministic():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("gemv_kn repeated launches bit-identical")
    x = torch.from_numpy(inputs.decode_activations()).to("cuda:0")
    W = torch.from_numpy(inputs.decode_weights_kn(5)).to("cuda:0")
    y0 = torch.empty((12288,), dtype=torch.float16, device="cuda:0")
    sdt.gemv_f16_m1_kn(x, W, y0)
    y = torch.empty_like(y0)
    for _ in range(20):
        sdt.gemv_f16_m1_kn(x, W, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
