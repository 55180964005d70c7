"""GPU parity of the bfloat16 entry points (gemm_bf16, gemv_bf16_m1,
gemv_bf16_m1_kn) against the CPU oracle's bfloat16 definition, through the C
ABI.

Acceptance bound |C_gpu - C_ref| <= 1e-2 + 5.42e-3 |C_ref| against the
unrounded fp64 reference: the fp16 path's allowance for fp32 accumulation
with half a bfloat16 ulp (2^-8 relative) in place of half an fp16 ulp
(oracle.tolerance).  Exact regimes (integer inputs) are compared bit for bit
with the correctly rounded reference.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (assert_bitexact_bf16, assert_close_bf16, bits_to_dev_bf16,
                         dev_bf16_to_bits, run_gemm_bf16, say, seeded_rows)
from shape_driven_tile_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [256, 512, 768, 1024, 1536, 2048])
def test_bf16_square_full(n):
    say(f"bf16 square {n}^3, full oracle")
    A, B = inputs.square_operands_bf16(n, 1)
    C, _ = run_gemm_bf16(A, B)
    assert_close_bf16(C, oracle.gemm(A, B, dtype="bf16"))


def test_bf16_square_4096_full():
    say("bf16 square 4096^3, full oracle")
    A, B = inputs.square_operands_bf16(4096, 2)
    C, _ = run_gemm_bf16(A, B)
    assert_close_bf16(C, oracle.gemm(A, B, dtype="bf16"))


def test_bf16_square_8192_rows():
    """512 seeded whole rows (both edges of every 256-row band) and 16 whole
    columns of the 8192^3 product."""
    n = 8192
    say("bf16 square 8192^3, 512 full rows + 16 full columns")
    A, B = inputs.square_operands_bf16(n, 2)
    C, _ = run_gemm_bf16(A, B)
    rows = seeded_rows(n, 512, seed=n)
    assert_close_bf16(C[rows], oracle.gemm(np.ascontiguousarray(A[rows]), B, dtype="bf16"))
    cols = seeded_rows(n, 16, seed=n + 1)
    r = np.repeat(np.arange(n), len(cols))
    c = np.tile(cols, n)
    assert_close_bf16(C[r, c], oracle.gemm_sample(A, B, r, c, dtype="bf16"))


def test_bf16_integer_exact_4096_auto():
    """Integer inputs through gemm_bf16's automatic plan at 4096^3 (the
    ping-pong kernel and its 16 x 16-block tile order), every element bit for
    bit."""
    A = inputs.integer_bf16((4096, 4096), 103)
    B = inputs.integer_bf16((4096, 4096), 104)
    say("bf16 integer 4096^3 automatic plan, full C")
    C, pad_ok = run_gemm_bf16(A, B)
    assert pad_ok
    assert_bitexact_bf16(C, oracle.gemm(A, B, dtype="bf16"))


@pytest.mark.parametrize("shape", [(200, 136, 136), (257, 129, 200), (64, 64, 4096),
                                   (257, 259, 4160)])
def test_bf16_integer_exact_every_tile(shape):
    from shape_driven_tile_amd import binding as sdt
    M, N, K = shape
    A = inputs.integer_bf16((M, K), 101)
    B = inputs.integer_bf16((N, K), 102)
    ref = oracle.gemm(A, B, dtype="bf16")
    for tile in range(sdt.num_tiles()):
        say(f"bf16 integer {shape} tile={tile}")
        C, pad_ok = run_gemm_bf16(A, B, tile=tile)
        assert pad_ok
        assert_bitexact_bf16(C, ref)


def _random_shapes_bf16(count, seed=4049, max_work=2 ** 33):
    """Seeded shapes: M and N log-uniform in [1, 4096] (a quarter) or
    [256, 4096], K log-uniform in [1, 4096], M * N * K under max_work, row
    pitches padded by 0-40 elements and rounded up to multiples of 8."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        lo = 0 if len(out) < count // 4 else 8
        M, N = (int(round(2 ** rng.uniform(lo, 12))) for _ in range(2))
        K = int(round(2 ** rng.uniform(0, 12)))
        if M * N * K <= max_work:
            out.append((M, N, K, int(rng.integers(0, 41)), int(rng.integers(0, 41))))
    return out


@pytest.mark.parametrize("M,N,K,pa,pb", _random_shapes_bf16(16))
def test_bf16_integer_exact_random_shapes_auto(M, N, K, pa, pb):
    """gemm_bf16's automatic plan on seeded random shapes with NaN-padded
    rows: integer inputs, bit for bit against the oracle's bf16 rounding."""
    from shape_driven_tile_amd import binding as sdt
    say(f"bf16 random auto M={M} N={N} K={K} pads={pa},{pb} "
        f"rung={sdt.pick_tile(M, N, K, 256)['id']}")
    ka = -(-(K + pa) // 8) * 8
    kb = -(-(K + pb) // 8) * 8
    A = inputs.padded_bits(inputs.integer_bf16((M, K), 3000 + M), ka)
    B = inputs.padded_bits(inputs.integer_bf16((N, K), 4000 + N), kb)
    C, pad_ok = run_gemm_bf16(A, B, K=K)
    assert pad_ok
    assert_bitexact_bf16(C, oracle.gemm(A, B, K=K, dtype="bf16"))


def test_bf16_two_kgroups_integer():
    from shape_driven_tile_amd import binding as sdt
    M, N, K = 257, 259, 4160
    A = inputs.integer_bf16((M, K), 107)
    B = inputs.integer_bf16((N, K), 108)
    ref = oracle.gemm(A, B, dtype="bf16")
    for tile in range(sdt.num_tiles()):
        if sdt.tile_info(tile)["kgroups"] != 2:
            continue
        say(f"bf16 two k-groups integer tile={tile}")
        C, pad_ok = run_gemm_bf16(A, B, tile=tile, stagger=0, kgroups=2)
        assert pad_ok
        assert_bitexact_bf16(C, ref)


@pytest.mark.parametrize("M,N,K", [(77, 91, 65), (300, 260, 1000), (129, 255, 8)])
def test_bf16_ragged_padded(M, N, K):
    from shape_driven_tile_amd import binding as sdt
    lda = -(-K // 8) * 8 + 8
    ldb = -(-K // 8) * 8 + 16
    A = inputs.padded_bits(inputs.uniform_bf16((M, K), 103), lda)
    B = inputs.padded_bits(inputs.uniform_bf16((N, K), 104), ldb)
    ref = oracle.gemm(A, B, K=K, dtype="bf16")
    for tile in range(sdt.num_tiles()):
        say(f"bf16 ragged M={M} N={N} K={K} tile={tile}")
        C, pad_ok = run_gemm_bf16(A, B, K=K, tile=tile)
        assert pad_ok
        assert_close_bf16(C, ref)


def test_bf16_decode_all_buffers_and_routing():
    import torch
    from shape_driven_tile_amd import binding as sdt
    x = inputs.decode_activations_bf16()
    dx = bits_to_dev_bf16(x)
    y = torch.empty((inputs.DECODE_N,), dtype=torch.bfloat16, device="cuda:0")
    for r in range(inputs.DECODE_BUFFERS):
        say(f"bf16 decode GEMV buffer {r}")
        W = inputs.decode_weights_bf16(r)
        sdt.gemv_bf16_m1(dx, bits_to_dev_bf16(W), y)
        torch.cuda.synchronize()
        got = dev_bf16_to_bits(y)
        assert_close_bf16(got, oracle.gemv_m1(x, W, dtype="bf16"))
        if r == 0:
            say("bf16 gemm M=1 routes to the GEMV")
            C = torch.empty((1, inputs.DECODE_N), dtype=torch.bfloat16, device="cuda:0")
            sdt.gemm_bf16(dx.view(1, -1), bits_to_dev_bf16(W), C)
            torch.cuda.synchronize()
            assert (dev_bf16_to_bits(C)[0] == got).all()


def test_bf16_decode_kn():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("bf16 [K][N] decode GEMV")
    x = inputs.decode_activations_bf16()
    W = np.ascontiguousarray(inputs.decode_weights_bf16(1).T)
    y = torch.empty((inputs.DECODE_N,), dtype=torch.bfloat16, device="cuda:0")
    sdt.gemv_bf16_m1_kn(bits_to_dev_bf16(x), bits_to_dev_bf16(W), y)
    torch.cuda.synchronize()
    assert_close_bf16(dev_bf16_to_bits(y), oracle.gemv_kn(x, W, dtype="bf16"))
    # exact integers, bit for bit
    xi = inputs.integer_bf16((1000,), 105)
    Wi = inputs.integer_bf16((1000, 520), 106)
    yi = torch.empty((520,), dtype=torch.bfloat16, device="cuda:0")
    sdt.gemv_bf16_m1_kn(bits_to_dev_bf16(xi), bits_to_dev_bf16(Wi), yi)
    torch.cuda.synchronize()
    assert_bitexact_bf16(dev_bf16_to_bits(yi), oracle.gemv_kn(xi, Wi, dtype="bf16"))


def test_bf16_k0_and_rejections():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("bf16 K=0 writes zeros; misaligned rejected")
    A = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda:0")
    B = torch.empty((7, 0), dtype=torch.bfloat16, device="cuda:0")
    C = torch.full((5, 8), float("nan"), dtype=torch.bfloat16, device="cuda:0")[:, :7]
    sdt.gemm_bf16(A, B, C)
    torch.cuda.synchronize()
    assert (C.float().cpu().numpy() == 0).all()
    buf = torch.zeros((4096,), dtype=torch.bfloat16, device="cuda:0")
    L = sdt.lib()
    p = buf.data_ptr()
    assert L.gemm_bf16(8, 8, 8, p + 2, 8, p + 256, 8, p + 512, 8, None) == sdt.SDT_ERR_UNSUPPORTED
    with pytest.raises(TypeError):
        sdt.gemm_bf16(buf.half().view(64, 64), buf.view(64, 64), buf.view(64, 64))
    torch.cuda.synchronize()
