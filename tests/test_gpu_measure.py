"""GPU tests of the library's measurement kernels (not part of the product's
math): the empty kernel behind the launch floor, the read-only streaming
kernels behind the decode shape's read ceilings and the register-only MFMA loop
behind the matrix-core ceiling.  The streaming kernel's output words are exact
(XOR of each 8 KB run's 32-bit words), so the test checks that every byte was
read, in bounds, and nothing else was written; the MFMA loop's sums are exact
integers on operands in {-1, 0, 1}."""
import numpy as np
import pytest

from gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu


def _xor_words(buf_u8: np.ndarray) -> np.ndarray:
    return np.bitwise_xor.reduce(buf_u8.view(np.int32).reshape(-1, 2048), axis=1)


def test_empty_kernel_runs():
    import torch
    from shape_driven_tile_amd import binding as sdt
    say("sdt_empty_kernel x 10")
    for _ in range(10):
        sdt.empty_kernel()
    torch.cuda.synchronize()


@pytest.mark.parametrize("runs", [1, 3, 257, 12288])
def test_stream_read_words_exact(runs):
    import torch
    from shape_driven_tile_amd import binding as sdt
    rng = np.random.default_rng(7000 + runs)
    host = rng.integers(0, 256, size=runs * 8192, dtype=np.uint8)
    buf = to_dev(host)
    out = torch.full((runs + 4,), -1, dtype=torch.int32, device=buf.device)   # 4 guard words
    say(f"sdt_stream_read runs={runs}")
    sdt.stream_read(buf, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got[:runs], _xor_words(host))
    assert (got[runs:] == -1).all(), "words past the last run were written"


def test_stream_read_arguments():
    import ctypes

    import torch
    from shape_driven_tile_amd import binding as sdt
    L = sdt.lib()
    buf = torch.zeros(2 * 8192, dtype=torch.uint8, device="cuda:0")
    out = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    say("sdt_stream_read argument checks (nothing enqueued)")
    assert L.sdt_stream_read(buf.data_ptr(), 0, out.data_ptr(), s) == sdt.SDT_OK
    assert L.sdt_stream_read(buf.data_ptr(), -8192, out.data_ptr(), s) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read(None, 8192, out.data_ptr(), s) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read(buf.data_ptr(), 8192, None, s) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read(buf.data_ptr(), 4096, out.data_ptr(), s) == sdt.SDT_ERR_UNSUPPORTED
    assert L.sdt_stream_read(buf.data_ptr() + 8, 8192, out.data_ptr(), s) == \
        sdt.SDT_ERR_UNSUPPORTED
    assert L.sdt_stream_read(buf.data_ptr(), 8192, out.data_ptr() + 2, s) == \
        sdt.SDT_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 0).all()


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096 * 16 + 48, 3), (8192 * 12288, 8192),
                                        (1 << 20, 4096)])
def test_stream_read_grid_words_exact(nbytes, wgs):
    """The grid-stride read: the XOR of its per-workgroup words is the XOR of
    every 32-bit word of the buffer (every byte read once, none past the
    end: a 16-byte tail past a whole pass included), and nothing past the
    last workgroup's word is written."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    rng = np.random.default_rng(7100 + wgs)
    host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = to_dev(host)
    out = torch.full((wgs + 4,), -1, dtype=torch.int32, device=buf.device)
    say(f"sdt_stream_read_grid bytes={nbytes} workgroups={wgs}")
    sdt.stream_read_grid(buf, out, wgs)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.bitwise_xor.reduce(got[:wgs]) == np.bitwise_xor.reduce(host.view(np.int32))
    assert (got[wgs:] == -1).all()


def test_stream_read_grid_arguments():
    import ctypes

    import torch
    from shape_driven_tile_amd import binding as sdt
    L = sdt.lib()
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    out = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p, o = buf.data_ptr(), out.data_ptr()
    say("sdt_stream_read_grid argument checks (nothing enqueued)")
    assert L.sdt_stream_read_grid(p, 0, o, 1, s) == sdt.SDT_OK
    assert L.sdt_stream_read_grid(p, -16, o, 1, s) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_grid(None, 16, o, 1, s) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_grid(p, 16, None, 1, s) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_grid(p, 16, o, 0, s) == sdt.SDT_ERR_INVALID_ARG
    assert L.sdt_stream_read_grid(p, 24, o, 1, s) == sdt.SDT_ERR_UNSUPPORTED
    assert L.sdt_stream_read_grid(p + 8, 16, o, 1, s) == sdt.SDT_ERR_UNSUPPORTED
    assert L.sdt_stream_read_grid(p, 16, o + 2, 1, s) == sdt.SDT_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 0).all()


@pytest.mark.parametrize("run,rpw", [(64, 512), (128, 256), (256, 128), (512, 64), (1024, 32),
                                     (128, 1024)])
def test_stream_read_runs_words_exact(run, rpw):
    """The run-length read kernel: workgroup w's word is the XOR of every
    32-bit word of its band of its rows, so every byte was read, in bounds."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    rows, row_bytes = 1024, 4096
    rng = np.random.default_rng(7100 + run)
    host = rng.integers(0, 256, size=rows * row_bytes, dtype=np.uint8)
    buf = to_dev(host)
    nbands = row_bytes // run
    grid = nbands * (rows // rpw)
    out = torch.full((grid + 4,), -1, dtype=torch.int32, device=buf.device)   # 4 guard words
    say(f"sdt_stream_read_runs run={run} rows_per_wg={rpw} grid={grid}")
    sdt.stream_read_runs(buf, rows, row_bytes, run, rpw, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    words = host.view(np.int32).reshape(rows, row_bytes // 4)
    want = np.empty(grid, np.int32)
    for w in range(grid):
        band, chunk = w % nbands, w // nbands
        blk = words[chunk * rpw:(chunk + 1) * rpw, band * run // 4:(band + 1) * run // 4]
        want[w] = np.bitwise_xor.reduce(blk.ravel())
    np.testing.assert_array_equal(got[:grid], want)
    assert (got[grid:] == -1).all(), "words past the grid were written"


@pytest.mark.parametrize("mfma32", [False, True])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("iters", [1, 5])
def test_mfma_ceiling_counts_every_product(bf16, iters, mfma32):
    """The register-only MFMA loop behind the matrix-core ceiling: with operand
    values in {-1, 0, 1} every sum is an exact integer, and the sum of a
    wave's 64 outputs is iters x sum over every k step and every k of (the
    column sum of its B fragments) x (that of its A fragments), however the
    instruction maps rows and columns to lanes.  So every MFMA the FLOP count
    assumes was issued and accumulated."""
    import torch
    from shape_driven_tile_amd import binding as sdt
    rng = np.random.default_rng(9100 + iters + 10 * bf16 + 100 * mfma32)
    vals = rng.integers(-1, 2, size=(24, 64, 8)).astype(np.float32)   # [fragment][lane][elt]
    if bf16:
        bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    else:
        bits = vals.astype(np.float16).view(np.uint16)
    frags = to_dev(np.ascontiguousarray(bits))
    wgs = 4
    out = torch.full((wgs * 512 + 16,), float("nan"), dtype=torch.float32, device=frags.device)
    say(f"sdt_mfma_ceiling iters={iters} bf16={bf16} mfma32={mfma32}")
    sdt.mfma_ceiling(frags, iters, out, wgs, bf16=bf16, mfma32=mfma32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[wgs * 512:]).all(), "values past the last workgroup were written"
    if mfma32:
        # 32 rows per fragment, k = 8 (lane // 32) + elt of a 16-deep step;
        # step s: fragments 6 s .. 6 s + 3 A, 6 s + 4 .. 6 s + 5 B
        colsum = vals.reshape(24, 2, 32, 8).sum(axis=2).reshape(24, 16)
        steps = [(range(6 * h, 6 * h + 4), range(6 * h + 4, 6 * h + 6)) for h in range(4)]
    else:
        # 16 rows per fragment, k = 8 (lane // 16) + elt of a 32-deep half;
        # half h: fragments 12 h .. 12 h + 7 A, 12 h + 8 .. 12 h + 11 B
        colsum = vals.reshape(24, 4, 16, 8).sum(axis=2).reshape(24, 32)
        steps = [(range(12 * h, 12 * h + 8), range(12 * h + 8, 12 * h + 12)) for h in range(2)]
    expect = 0.0
    for fa, fb in steps:
        a = colsum[list(fa)].sum(axis=0)
        b = colsum[list(fb)].sum(axis=0)
        expect += float((a * b).sum())
    expect *= iters
    per_wave = got[:wgs * 512].astype(np.float64).reshape(wgs * 8, 64).sum(axis=1)
    np.testing.assert_array_equal(per_wave, np.full(wgs * 8, expect))
    again = torch.full_like(out, float("nan"))
    sdt.mfma_ceiling(frags, iters, again, wgs, bf16=bf16, mfma32=mfma32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(again.cpu().numpy()[:wgs * 512], got[:wgs * 512])
