"""Shared helpers for the GPU parity tests: move seeded host operands to the
device, run the library through its C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle

DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case before any GPU step, so a failed run points at it."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_gemm(A, B, K=None, tile=None, stagger=-1, ldc_pad=0, stream=None, stages=-1,
             kgroups=-1, loaders=-1):
    """A: (M, lda) float16, B: (N, ldb) float16 host buffers (K-contiguous rows).
    Returns the (M, N) float16 result and whether the C padding was untouched."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    M, lda = A.shape
    N, ldb = B.shape
    K = lda if K is None else K
    dA = to_dev(A)[:, :K]
    dB = to_dev(B)[:, :K]
    # ldc: N plus ldc_pad, rounded up to the 8-element multiple the ABI needs
    # for more than one row
    ldc = N + ldc_pad if M == 1 else -(-(N + ldc_pad) // 8) * 8
    full = torch.full((M, ldc), float("nan"), dtype=torch.float16, device=DEV)
    dC = full[:, :N]
    if stages != -1 or kgroups != -1 or loaders != -1:
        sdt.gemm_f16_cfg(dA, dB, dC, tile_id=-1 if tile is None else tile, stages=stages,
                         kgroups=kgroups, stagger=stagger, stream=stream, loaders=loaders)
    elif tile is None and stagger == -1:
        sdt.gemm_f16(dA, dB, dC, stream=stream)
    else:
        sdt.gemm_f16_ex(dA, dB, dC, tile_id=-1 if tile is None else tile, stagger=stagger,
                        stream=stream)
    torch.cuda.synchronize()
    pad_ok = bool(torch.isnan(full[:, N:]).all().item()) if ldc > N else True
    return dC.cpu().numpy(), pad_ok


def run_gemv(x, W, K=None, variant=None):
    import torch
    from shape_driven_tile_amd import binding as sdt
    N, ldb = W.shape
    K = x.shape[0] if K is None else K
    dx = to_dev(x[:K])
    dW = to_dev(W)[:, :K]
    dy = torch.full((N,), float("nan"), dtype=torch.float16, device=DEV)
    sdt.gemv_f16_m1(dx, dW, dy, variant=variant)
    torch.cuda.synchronize()
    return dy.cpu().numpy()


def tol_report(gpu16: np.ndarray, ref: np.ndarray) -> tuple[bool, str]:
    """The acceptance bound |C_gpu - C_ref| <= 1e-2 + 2e-3 |C_ref| per element
    (NaN or inf where the reference is finite fails)."""
    g = gpu16.astype(np.float64)
    tol = oracle.tolerance(ref)
    err = np.abs(g - ref)
    ok = err <= tol
    bad = int((~ok).sum())
    worst = float(np.nanmax(np.where(np.isfinite(err), err / tol, np.inf))) if err.size else 0.0
    return bad == 0, f"{bad} of {g.size} outside tolerance, worst |d|/tol = {worst:.3g}"


def assert_close(gpu16, ref):
    ok, msg = tol_report(gpu16, ref)
    assert ok, msg


def assert_bitexact(gpu16, ref):
    want = oracle.f16_encode_rne(ref)
    got = np.ascontiguousarray(gpu16).view(np.uint16)
    diff = got != want
    if diff.any():
        g = np.ascontiguousarray(gpu16).astype(np.float64)
        nan = int(np.isnan(g[diff]).sum())
        idx = np.argwhere(diff)
        raise AssertionError(f"{int(diff.sum())} of {got.size} differ from the RNE oracle "
                             f"({nan} NaN, i.e. never written); first at {idx[0].tolist()}, "
                             f"last at {idx[-1].tolist()}")


def sample_positions(M, N, rows=32, cols=32, extra=4096, seed=0):
    """Whole rows and columns (first, last, tile seams, random) plus random
    elements, as (row, col) index arrays."""
    rng = np.random.default_rng(seed)
    rs = sorted(set([0, 1, M // 2, M - 1] + list(rng.integers(0, M, rows))))
    cs = sorted(set([0, 1, N // 2, N - 1] + list(rng.integers(0, N, cols))))
    r = [np.full(N, i) for i in rs] + [np.arange(M) for _ in cs] + [rng.integers(0, M, extra)]
    c = [np.arange(N) for _ in rs] + [np.full(M, j) for j in cs] + [rng.integers(0, N, extra)]
    return np.concatenate(r).astype(np.int64), np.concatenate(c).astype(np.int64)


def seeded_rows(n, count, seed, band=256):
    """`count` distinct sorted indices in [0, n): 0 and n - 1, the first and
    last index of every `band`-wide tile band when count covers them all, the
    rest drawn from a seeded generator."""
    rng = np.random.default_rng(seed)
    pick = {0, n - 1}
    if count >= 2 * (-(-n // band)):
        for b in range(0, n, band):
            pick.update((b, min(b + band, n) - 1))
    while len(pick) < min(count, n):
        pick.update(int(v) for v in rng.integers(0, n, count - len(pick)))
    return np.array(sorted(pick)[:count], dtype=np.int64)


def run_gemv_kn(x, W, N=None, variant=None, y_pad=8):
    """x: (K,) float16; W: (K, ldb) float16 host buffer, the N of a row
    contiguous.  Returns y (N,) and whether the y_pad elements past N stayed
    untouched."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    K, ldb = W.shape
    N = ldb if N is None else N
    dx = to_dev(x[:K])
    dW = to_dev(W)[:, :N]
    full = torch.full((N + y_pad,), float("nan"), dtype=torch.float16, device=DEV)
    dy = full[:N]
    sdt.gemv_f16_m1_kn(dx, dW, dy, variant=variant)
    torch.cuda.synchronize()
    pad_ok = bool(torch.isnan(full[N:]).all().item())
    return dy.cpu().numpy(), pad_ok


# ---- bfloat16 (uint16 bit patterns on the host) -----------------------------------

def bits_to_dev_bf16(a: np.ndarray):
    import torch
    b = np.ascontiguousarray(np.asarray(a, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_bf16_to_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_gemm_bf16(A, B, K=None, tile=None, stagger=-1, stages=-1, kgroups=-1):
    """A: (M, lda), B: (N, ldb) uint16 bfloat16 bit arrays.  Returns C's bits
    (M, N) and whether the C padding (NaN) stayed untouched."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    M, lda = A.shape
    N, ldb = B.shape
    K = lda if K is None else K
    dA = bits_to_dev_bf16(A)[:, :K]
    dB = bits_to_dev_bf16(B)[:, :K]
    ldc = N if M == 1 else -(-N // 8) * 8 + 8
    full = torch.full((M, ldc), float("nan"), dtype=torch.bfloat16, device=DEV)
    dC = full[:, :N]
    if stages != -1 or kgroups != -1:
        sdt.gemm_bf16_cfg(dA, dB, dC, tile_id=-1 if tile is None else tile, stages=stages,
                          kgroups=kgroups, stagger=stagger)
    elif tile is None and stagger == -1:
        sdt.gemm_bf16(dA, dB, dC)
    else:
        sdt.gemm_bf16_ex(dA, dB, dC, tile_id=-1 if tile is None else tile, stagger=stagger)
    torch.cuda.synchronize()
    pad_ok = bool(torch.isnan(full[:, N:]).all().item()) if ldc > N else True
    return dev_bf16_to_bits(dC), pad_ok


def assert_close_bf16(bits, ref):
    ok, msg = tol_report_values(oracle.bf16_decode(bits), ref, "bf16")
    assert ok, msg


def tol_report_values(got64: np.ndarray, ref: np.ndarray, dtype: str) -> tuple[bool, str]:
    tol = oracle.tolerance(ref, dtype)
    err = np.abs(got64 - ref)
    ok = err <= tol
    bad = int((~ok).sum())
    worst = float(np.nanmax(np.where(np.isfinite(err), err / tol, np.inf))) if err.size else 0.0
    return bad == 0, f"{bad} of {got64.size} outside tolerance, worst |d|/tol = {worst:.3g}"


def assert_bitexact_bf16(bits, ref):
    want = oracle.bf16_encode_rne(ref)
    diff = np.ascontiguousarray(bits) != want
    assert not diff.any(), f"{int(diff.sum())} of {want.size} differ from the RNE oracle"
