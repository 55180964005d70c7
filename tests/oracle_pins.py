"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes an :class:`oracle.Oracle` and raises AssertionError when
the oracle disagrees with something the mathematics or an independent library
routine fixes: the IEEE binary16 definition (checked exhaustively against
numpy's float16), exact rational arithmetic on tiny inputs, closed forms
(all-ones, identity, K=1), exact integer arithmetic, an exact fixed-point sum
with the fp64 recursive-summation error bound, and invariants (transpose,
padding, thread count, sampled vs full).  The same pins run against
deliberately broken builds of the oracle (tests/test_oracle_mutants.py) to
show that a plausible mistake anywhere in it is caught.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from shape_driven_tile_amd import inputs

ALL_BITS = np.arange(65536, dtype=np.uint16)
U = 2.0 ** -53  # unit roundoff of fp64


def _np_dec(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---- binary16 codec -------------------------------------------------------

def pin_decode_exhaustive(o):
    d = o.f16_decode(ALL_BITS)
    ref = _np_dec(ALL_BITS)
    same = (d == ref) | (np.isnan(d) & np.isnan(ref))
    assert same.all(), f"decode differs at {np.flatnonzero(~same)[:8]}"
    # sign of zero survives
    assert np.signbit(d[0x8000]) and not np.signbit(d[0])


def pin_encode_roundtrip(o):
    d = _np_dec(ALL_BITS)
    fin = ~np.isnan(d)
    e = o.f16_encode_rne(d)
    assert (e[fin] == ALL_BITS[fin]).all(), "encode(decode(h)) != h"
    nan_out = e[~fin]
    assert ((nan_out & 0x7C00) == 0x7C00).all() and ((nan_out & 0x3FF) != 0).all()


def pin_encode_rne_ties(o):
    """Every midpoint between neighbouring finite binary16 values rounds to the
    neighbour with an even encoding; one fp64 ulp either side goes to the
    nearer neighbour."""
    h = np.arange(0, 0x7BFF, dtype=np.uint16)          # pairs (h, h+1), both finite
    lo = _np_dec(h)
    hi = _np_dec(h + 1)
    mid = (lo + hi) / 2.0                               # exact in fp64
    want = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    for sgn, sbit in ((1.0, 0), (-1.0, 0x8000)):
        got = o.f16_encode_rne(sgn * mid)
        assert (got == (want | sbit)).all(), "tie not rounded to even"
        below = o.f16_encode_rne(sgn * np.nextafter(mid, 0.0))
        above = o.f16_encode_rne(sgn * np.nextafter(mid, np.inf))
        assert (below == (h | sbit)).all(), "value below a midpoint not rounded down"
        assert (above == ((h + 1) | sbit)).all(), "value above a midpoint not rounded up"


def pin_encode_vs_numpy(o):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(400_000) * np.exp2(rng.uniform(-27.0, 17.0, 400_000))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert (o.f16_encode_rne(x) == ref).all()


def pin_encode_special_values(o):
    cases = [
        (65504.0, 0x7BFF), (np.nextafter(65520.0, 0.0), 0x7BFF), (65520.0, 0x7C00),
        (-65520.0, 0xFC00), (np.inf, 0x7C00), (-np.inf, 0xFC00), (0.0, 0x0000),
        (-0.0, 0x8000), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000),
        (np.nextafter(2.0 ** -25, 1.0), 0x0001), (3 * 2.0 ** -25, 0x0002),
        (2.0 ** -14, 0x0400), (1.0, 0x3C00), (-2.0, 0xC000), (1.0 + 2.0 ** -11, 0x3C00),
        (1.0 + 3 * 2.0 ** -11, 0x3C02),
    ]
    xs = np.array([c[0] for c in cases], dtype=np.float64)
    want = np.array([c[1] for c in cases], dtype=np.uint16)
    got = o.f16_encode_rne(xs)
    assert (got == want).all(), f"{xs[got != want]} -> {got[got != want]}"


# ---- GEMM -----------------------------------------------------------------

def pin_bruteforce_fraction(o):
    """Tiny shapes: the oracle equals the exact rational sum up to the fp64
    recursive-summation bound (K-1)*u*sum|ab|."""
    for (M, N, K, seed) in [(1, 1, 1, 1), (2, 3, 5, 2), (3, 2, 8, 3), (5, 5, 3, 4),
                            (8, 1, 2, 5), (1, 8, 7, 6)]:
        A = inputs.uniform_f16((M, K), 100 + seed)
        B = inputs.uniform_f16((N, K), 200 + seed)
        C = o.gemm(A, B)
        a = A.astype(np.float64)
        b = B.astype(np.float64)
        for m in range(M):
            for n in range(N):
                exact = sum((Fraction(a[m, k]) * Fraction(b[n, k]) for k in range(K)),
                            Fraction(0))
                mag = sum(abs(Fraction(a[m, k]) * Fraction(b[n, k])) for k in range(K))
                err = abs(Fraction(C[m, n]) - exact)
                assert err <= Fraction(max(K - 1, 0)) * Fraction(U) * mag, (M, N, K, m, n)


def pin_all_ones(o):
    """A = B = 1 gives K in every element, exactly."""
    for K in (1, 7, 256, 1920, 1984, 2048, 2112, 2176, 2304, 4096, 8192, 16384):
        A = np.ones((3, K), np.float16)
        B = np.ones((5, K), np.float16)
        C = o.gemm(A, B)
        assert (C == K).all(), K


def pin_identity(o):
    """B = I gives C = A exactly (one non-zero product per sum), M != K."""
    A = inputs.uniform_f16((40, 24), 11)
    B = np.eye(24, dtype=np.float16)
    C = o.gemm(A, B)
    assert (C == A.astype(np.float64)).all()
    assert (o.f16_encode_rne(C) == A.view(np.uint16)).all()


def pin_k1_outer(o):
    """K = 1: C(m, n) = a_m * b_n, exact in fp64; its fp16 rounding equals
    numpy's correctly rounded cast of the same product."""
    a = inputs.uniform_f16((17, 1), 12)
    b = inputs.uniform_f16((9, 1), 13)
    C = o.gemm(a, b)
    ref = np.outer(a[:, 0].astype(np.float64), b[:, 0].astype(np.float64))
    assert (C == ref).all()
    assert (o.f16_encode_rne(C) == ref.astype(np.float16).view(np.uint16)).all()


def pin_integer_exact(o):
    """Small-integer inputs: every sum is an exact integer; compare with exact
    int64 matrix products (rectangular shapes, so a transposed operand fails)."""
    for (M, N, K, seed) in [(33, 17, 2304, 1), (5, 9, 1, 2), (64, 48, 130, 3)]:
        A = inputs.integer_f16((M, K), 300 + seed)
        B = inputs.integer_f16((N, K), 400 + seed)
        ref = A.astype(np.int64) @ B.astype(np.int64).T
        C = o.gemm(A, B)
        assert (C == ref).all(), (M, N, K)


def pin_fixed_point_bound(o):
    """Inputs in [-1, 1] are integer multiples of 2^-24, so the exact sum is an
    integer multiple of 2^-48 computed exactly in int64; the oracle must be
    within the fp64 bound (K-1)*u*sum|ab| of it."""
    for (M, N, K, seed) in [(24, 20, 300, 1), (6, 40, 1000, 2)]:
        A = inputs.uniform_f16((M, K), 500 + seed)
        B = inputs.uniform_f16((N, K), 600 + seed)
        ia = (A.astype(np.float64) * 2.0 ** 24).astype(np.int64)
        ib = (B.astype(np.float64) * 2.0 ** 24).astype(np.int64)
        assert (ia.astype(np.float64) == A.astype(np.float64) * 2.0 ** 24).all()
        exact = (ia @ ib.T).astype(object)                    # units of 2^-48
        mag = (np.abs(ia) @ np.abs(ib).T).astype(object)
        C = o.gemm(A, B)
        c48 = (C * 2.0 ** 48).astype(np.int64).astype(object)  # exact: C is a multiple of 2^-48
        assert ((C * 2.0 ** 48) == np.floor(C * 2.0 ** 48)).all()
        err = np.abs(c48 - exact)
        bound = [(K - 1) * Fraction(int(s)) / 2 ** 53 for s in mag.ravel()]
        for e, bnd in zip(err.ravel(), bound):
            assert Fraction(int(e)) <= bnd


def pin_transpose(o):
    """gemm(B, A) is gemm(A, B) transposed, bit for bit (both K-contiguous)."""
    A = inputs.uniform_f16((13, 40), 21)
    B = inputs.uniform_f16((7, 40), 22)
    assert (o.gemm(B, A) == o.gemm(A, B).T).all()


def pin_numpy_crosscheck(o):
    """Against numpy's fp64 matmul (a different summation order)."""
    A = inputs.uniform_f16((50, 70), 31)
    B = inputs.uniform_f16((60, 70), 32)
    a = A.astype(np.float64)
    b = B.astype(np.float64)
    ref = a @ b.T
    mag = np.abs(a) @ np.abs(b).T
    assert (np.abs(o.gemm(A, B) - ref) <= 2 * 70 * U * mag).all()


def pin_padding_ignored(o):
    """Row padding past K (filled with NaN) never reaches the result."""
    A = inputs.uniform_f16((19, 72), 41)
    B = inputs.uniform_f16((23, 72), 42)
    tight = o.gemm(A, B)
    padded = o.gemm(inputs.padded(A, 80), inputs.padded(B, 96), K=72)
    assert (tight == padded).all()


def pin_k0(o):
    """K = 0 is the empty sum."""
    A = np.full((4, 8), np.nan, np.float16)
    B = np.full((3, 8), np.nan, np.float16)
    assert (o.gemm(A, B, K=0) == 0.0).all()


def pin_sample(o):
    A = inputs.uniform_f16((37, 90), 51)
    B = inputs.uniform_f16((29, 90), 52)
    full = o.gemm(A, B)
    rng = np.random.default_rng(5)
    r = rng.integers(0, 37, 200)
    c = rng.integers(0, 29, 200)
    assert (o.gemm_sample(A, B, r, c) == full[r, c]).all()


def pin_threads(o):
    A = inputs.uniform_f16((64, 257), 61)
    B = inputs.uniform_f16((48, 257), 62)
    assert (o.gemm(A, B, threads=1) == o.gemm(A, B, threads=max(2, o.max_threads()))).all()


# ---- M=1 decode GEMV ------------------------------------------------------

def pin_gemv(o):
    K, N = 300, 50
    x = inputs.uniform_f16((K,), 71)
    W = inputs.normal_f16((N, K), 72)
    Wp = inputs.padded(W, 304)
    y = o.gemv_m1(x, Wp, K=K)
    # the same definition as a one-row GEMM
    assert (y == o.gemm(x[None, :], W)[0]).all()
    # one-hot activations select one weight per column
    for j in (0, 1, 150, K - 1):
        e = np.zeros(K, np.float16)
        e[j] = 1
        assert (o.gemv_m1(e, Wp, K=K) == W[:, j].astype(np.float64)).all(), j
    # all-ones
    assert (o.gemv_m1(np.ones(K, np.float16), np.ones((N, K), np.float16)) == K).all()
    # fp64 cross-check
    ref = W.astype(np.float64) @ x.astype(np.float64)
    mag = np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64))
    assert (np.abs(y - ref) <= 2 * K * U * mag).all()


def pin_gemv_kn(o):
    """The [K][N] weight layout: the same products summed in the same ascending
    k order as the [N][K] form, so the two agree bit for bit on transposed
    copies; plus closed forms that do not go through the other function."""
    K, N = 300, 50
    x = inputs.uniform_f16((K,), 73)
    W = inputs.normal_f16((K, N), 74)          # K rows, N contiguous
    Wp = inputs.padded(W, 56)
    y = o.gemv_kn(x, Wp, N=N)
    assert (y == o.gemv_m1(x, np.ascontiguousarray(W.T))).all()
    # one-hot activations select row k of the weights
    for j in (0, 1, 150, K - 1):
        e = np.zeros(K, np.float16)
        e[j] = 1
        assert (o.gemv_kn(e, Wp, N=N) == W[j].astype(np.float64)).all(), j
    # a single nonzero weight column n sees only its own column
    Z = np.zeros((K, N), np.float16)
    Z[:, 7] = 1
    z = o.gemv_kn(np.ones(K, np.float16), Z)
    assert z[7] == K and (np.delete(z, 7) == 0).all()
    # exact rationals on a tiny case
    xs = inputs.uniform_f16((5,), 75)
    Ws = inputs.uniform_f16((5, 3), 76)
    ys = o.gemv_kn(xs, Ws)
    for n in range(3):
        exact = sum(Fraction(float(xs[k])) * Fraction(float(Ws[k, n])) for k in range(5))
        assert abs(Fraction(ys[n]) - exact) <= Fraction(4 * U) * sum(
            abs(Fraction(float(xs[k])) * Fraction(float(Ws[k, n]))) for k in range(5))


# ---- bfloat16 -------------------------------------------------------------------

def _torch_bf16_dec(bits):
    import torch
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def pin_bf16_decode_exhaustive(o):
    got = o.bf16_decode(ALL_BITS)
    want = _torch_bf16_dec(ALL_BITS)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == want[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(want[~nan])).all()


def pin_bf16_encode_roundtrip(o):
    v = _torch_bf16_dec(ALL_BITS)
    fin = np.isfinite(v)
    assert (o.bf16_encode_rne(v[fin]) == ALL_BITS[fin]).all()


def pin_bf16_encode_rne_ties(o):
    """Every midpoint between adjacent positive finite values rounds to the
    even pattern; one fp64 ulp either side rounds to the nearer neighbour."""
    lo = np.arange(0, 0x7F7F, dtype=np.uint16)
    a = _torch_bf16_dec(lo)
    b = _torch_bf16_dec(lo + 1)
    mid = (a + b) / 2                        # exact in fp64
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert (o.bf16_encode_rne(mid) == even).all()
    assert (o.bf16_encode_rne(np.nextafter(mid, 0)) == lo).all()
    assert (o.bf16_encode_rne(np.nextafter(mid, np.inf)) == lo + 1).all()
    assert (o.bf16_encode_rne(-mid) == (even | 0x8000)).all()


def pin_bf16_encode_vs_torch(o):
    """fp32 values over the whole range, rounded by torch's float -> bfloat16."""
    import torch
    rng = np.random.default_rng(91)
    m = rng.uniform(1.0, 2.0, 400_000)
    e = rng.integers(-140, 128, 400_000)
    x = (np.where(rng.integers(0, 2, 400_000) == 1, -1.0, 1.0) * np.ldexp(m, e)).astype(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (o.bf16_encode_rne(x.astype(np.float64)) == want).all()


def pin_bf16_encode_special_values(o):
    cases = [(1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
             (255 * 2.0 ** 120, 0x7F7F), (255.5 * 2.0 ** 120, 0x7F80),
             (np.nextafter(255.5 * 2.0 ** 120, 0), 0x7F7F), (np.inf, 0x7F80),
             (-np.inf, 0xFF80), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),
             (3 * 2.0 ** -134, 0x0002), (2.0 ** -126, 0x0080), (1.0 + 2.0 ** -8, 0x3F80),
             (1.0 + 3 * 2.0 ** -8, 0x3F82)]
    for x, bits in cases:
        assert int(o.bf16_encode_rne(np.array([x]))[0]) == bits, (x, hex(bits))
    n = int(o.bf16_encode_rne(np.array([np.nan]))[0])
    assert (n & 0x7F80) == 0x7F80 and (n & 0x7F) != 0


def pin_bf16_gemm(o):
    """The bfloat16 entry points: the same sums over the bfloat16 decode."""
    # exact integers
    A = inputs.integer_bf16((13, 70), 92)
    B = inputs.integer_bf16((11, 70), 93)
    Ai = _torch_bf16_dec(A).astype(np.int64)
    Bi = _torch_bf16_dec(B).astype(np.int64)
    assert (o.gemm(A, B, dtype="bf16") == (Ai @ Bi.T).astype(np.float64)).all()
    # 0x3F80 is 1.0 in bfloat16 (and 1.875 in binary16): all-ones -> K
    ones = np.full((3, 257), 0x3F80, np.uint16)
    assert (o.gemm(ones, ones, dtype="bf16") == 257).all()
    # exact rationals
    a = inputs.uniform_bf16((2, 6), 94)
    b = inputs.uniform_bf16((3, 6), 95)
    C = o.gemm(a, b, dtype="bf16")
    fa, fb = _torch_bf16_dec(a), _torch_bf16_dec(b)
    for i in range(2):
        for j in range(3):
            terms = [Fraction(float(fa[i, k])) * Fraction(float(fb[j, k])) for k in range(6)]
            assert abs(Fraction(C[i, j]) - sum(terms)) <= Fraction(6 * U) * sum(abs(t) for t in terms)
    # fp64 cross-check with a bound, padding ignored, sampled = full
    A = inputs.uniform_bf16((40, 300), 96)
    B = inputs.uniform_bf16((30, 300), 97)
    Cf = o.gemm(inputs.padded_bits(A, 312), inputs.padded_bits(B, 304), K=300, dtype="bf16")
    fa, fb = _torch_bf16_dec(A), _torch_bf16_dec(B)
    assert (np.abs(Cf - fa @ fb.T) <= 2 * 300 * U * (np.abs(fa) @ np.abs(fb).T)).all()
    r = np.array([0, 39, 7, 21])
    c = np.array([0, 29, 3, 17])
    assert (o.gemm_sample(A, B, r, c, dtype="bf16") == Cf[r, c]).all()
    # GEMV in both layouts = the one-row GEMM
    x = inputs.uniform_bf16((300,), 98)
    y = o.gemv_m1(x, inputs.padded_bits(B, 304), K=300, dtype="bf16")
    assert (y == o.gemm(x[None, :], B, dtype="bf16")[0]).all()
    assert (o.gemv_kn(x, np.ascontiguousarray(B.T), dtype="bf16") == y).all()
    e = np.zeros(300, np.uint16)
    e[123] = 0x3F80
    assert (o.gemv_m1(e, B, dtype="bf16") == fb[:, 123]).all()


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
