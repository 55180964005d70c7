"""Thin ctypes binding over ``libsdt.so`` (C ABI in ``include/sdt.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Tensors are torch tensors on a ROCm device, used for
device memory and streams; the library is handed raw pointers, strides in
elements, and the current stream.  A missing library raises immediately: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdt.so")

SDT_OK = 0
SDT_ERR_INVALID_ARG = 1
SDT_ERR_UNSUPPORTED = 2
SDT_ERR_HIP = 3

# Every function include/sdt.h declares.
EXPORTS = (
    "gemm_f16", "gemv_f16_m1", "gemm_f16_ex", "gemv_f16_m1_ex", "sdt_gemv_num_variants",
    "gemv_f16_m1_kn", "gemv_f16_m1_kn_ex", "sdt_gemv_kn_num_variants", "sdt_check_gemv_kn_args",
    "gemm_bf16", "gemm_bf16_ex", "gemv_bf16_m1", "gemv_bf16_m1_kn",
    "sdt_pick_tile", "sdt_pick_rung", "sdt_num_tiles", "sdt_tile_info",
    "sdt_stagger_eligible", "sdt_stagger_ktile", "sdt_check_gemm_args",
    "sdt_status_string", "sdt_last_hip_error", "sdt_empty_kernel", "sdt_stream_read",
    "sdt_plan_tile",
    "gemm_f16_cfg", "gemm_bf16_cfg",
    "gemm_f16_ws", "gemm_bf16_ws", "sdt_gemm_workspace_size", "sdt_launch_workspace_size",
    "sdt_workspace_init", "sdt_pick_tile_ws", "sdt_abi_version", "sdt_stream_read_grid",
    "gemm_f16_noalloc", "gemv_f16_m1_kn_ws", "gemv_bf16_m1_kn_ws", "sdt_gemv_kn_workspace_size",
    "sdt_stream_read_runs", "sdt_mfma_ceiling",
)

# The include/sdt.h version these structures and signatures follow.
ABI_VERSION = 5


class SdtTile(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int), ("bm", ctypes.c_int), ("bn", ctypes.c_int),
                ("bk", ctypes.c_int), ("waves_m", ctypes.c_int), ("waves_n", ctypes.c_int),
                ("threads", ctypes.c_int), ("stages", ctypes.c_int),
                ("lds_bytes", ctypes.c_int), ("kgroups", ctypes.c_int),
                ("stagger", ctypes.c_int), ("long_stages", ctypes.c_int),
                ("splits", ctypes.c_int), ("split_algo", ctypes.c_int),
                ("persistent", ctypes.c_int), ("ksplit", ctypes.c_int),
                ("loaders", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class SdtLaunch(ctypes.Structure):
    """sdt_launch: -1 in a field = the automatic choice."""
    _fields_ = [("tile_id", ctypes.c_int), ("stages", ctypes.c_int),
                ("kgroups", ctypes.c_int), ("stagger", ctypes.c_int),
                ("splits", ctypes.c_int), ("split_algo", ctypes.c_int),
                ("persistent", ctypes.c_int), ("loaders", ctypes.c_int)]


class SdtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status)
        if status == SDT_ERR_HIP:
            msg += f" (hipError {last_hip_error()})"
        super().__init__(f"{where}: {msg}")


_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int


def lib():
    """Load libsdt.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m shape_driven_tile_amd.build`")
    # torch first: it loads its own HIP and HSA runtimes, whose sonames then
    # satisfy libsdt.so's dependencies, so the process holds one runtime.
    # Loaded the other way round, libsdt.so pulls in the system runtime and
    # torch adds its copy; the second to touch the GPU finds no device.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    L.gemm_f16.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
    L.gemm_f16_ex.argtypes = L.gemm_f16.argtypes + [_int, _int]
    L.gemv_f16_m1.argtypes = [_i64, _i64, _vp, _vp, _i64, _vp, _vp]
    L.gemv_f16_m1_ex.argtypes = L.gemv_f16_m1.argtypes + [_int]
    L.sdt_gemv_num_variants.argtypes = []
    L.gemv_f16_m1_kn.argtypes = [_i64, _i64, _vp, _vp, _i64, _vp, _vp]
    L.gemm_bf16.argtypes = L.gemm_f16.argtypes
    L.gemm_bf16_ex.argtypes = L.gemm_f16_ex.argtypes
    L.gemv_bf16_m1.argtypes = L.gemv_f16_m1.argtypes
    L.gemv_bf16_m1_kn.argtypes = L.gemv_f16_m1_kn.argtypes
    L.gemv_f16_m1_kn_ex.argtypes = L.gemv_f16_m1_kn.argtypes + [_int]
    L.sdt_gemv_kn_num_variants.argtypes = []
    L.sdt_check_gemv_kn_args.argtypes = [_i64, _i64, _vp, _vp, _i64, _vp]
    L.sdt_pick_tile.argtypes = [_i64, _i64, _i64, _int, ctypes.POINTER(SdtTile)]
    L.sdt_pick_rung.argtypes = [_i64, _i64, _int, _int, _int, ctypes.POINTER(_i64)]
    L.sdt_num_tiles.argtypes = []
    L.sdt_tile_info.argtypes = [_int, ctypes.POINTER(SdtTile)]
    L.sdt_plan_tile.argtypes = [_int, _i64, _i64, _i64, _int, ctypes.POINTER(SdtTile)]
    L.gemm_f16_ws.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
    L.gemm_bf16_ws.argtypes = L.gemm_f16_ws.argtypes
    L.gemm_f16_cfg.argtypes = L.gemm_f16_ws.argtypes + [ctypes.POINTER(SdtLaunch)]
    L.gemm_bf16_cfg.argtypes = L.gemm_f16_cfg.argtypes
    L.sdt_gemm_workspace_size.argtypes = [_i64, _i64, _i64, _int]
    L.sdt_gemm_workspace_size.restype = _i64
    L.sdt_launch_workspace_size.argtypes = [_i64, _i64, _i64, ctypes.POINTER(SdtLaunch)]
    L.sdt_launch_workspace_size.restype = _i64
    L.sdt_workspace_init.argtypes = [_vp, _i64, _vp]
    L.sdt_pick_tile_ws.argtypes = [_i64, _i64, _i64, _int, _i64, ctypes.POINTER(SdtTile)]
    L.sdt_abi_version.argtypes = []
    L.gemm_f16_noalloc.argtypes = L.gemm_f16.argtypes
    L.sdt_stream_read_grid.argtypes = [_vp, _i64, _vp, _int, _vp]
    L.gemv_f16_m1_kn_ws.argtypes = [_i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp]
    L.gemv_bf16_m1_kn_ws.argtypes = L.gemv_f16_m1_kn_ws.argtypes
    L.sdt_gemv_kn_workspace_size.argtypes = [_i64, _i64]
    L.sdt_gemv_kn_workspace_size.restype = _i64
    L.sdt_stream_read_runs.argtypes = [_vp, _i64, _i64, _int, _int, _vp, _vp]
    L.sdt_mfma_ceiling.argtypes = [_vp, _int, _vp, _int, _int, _vp]
    L.sdt_stagger_eligible.argtypes = [_i64]
    L.sdt_stagger_ktile.argtypes = [_i64, _i64, _i64]
    L.sdt_stagger_ktile.restype = _i64
    L.sdt_check_gemm_args.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
    L.sdt_status_string.argtypes = [_int]
    L.sdt_status_string.restype = ctypes.c_char_p
    L.sdt_last_hip_error.argtypes = []
    L.sdt_empty_kernel.argtypes = [_vp]
    L.sdt_stream_read.argtypes = [_vp, _i64, _vp, _vp]
    for name in ("gemm_f16", "gemm_f16_ex", "gemv_f16_m1", "gemv_f16_m1_ex",
                 "gemv_f16_m1_kn", "gemv_f16_m1_kn_ex", "sdt_gemv_kn_num_variants",
                 "gemm_bf16", "gemm_bf16_ex", "gemv_bf16_m1", "gemv_bf16_m1_kn",
                 "sdt_check_gemv_kn_args",
                 "sdt_gemv_num_variants", "sdt_pick_tile", "sdt_pick_rung", "sdt_num_tiles",
                 "sdt_tile_info", "sdt_stagger_eligible", "sdt_plan_tile", "sdt_check_gemm_args",
                 "gemm_f16_cfg", "gemm_bf16_cfg", "gemm_f16_ws", "gemm_bf16_ws",
                 "sdt_workspace_init", "sdt_pick_tile_ws", "sdt_abi_version",
                 "sdt_stream_read_grid", "gemm_f16_noalloc", "sdt_last_hip_error", "sdt_empty_kernel", "sdt_stream_read",
                 "gemv_f16_m1_kn_ws", "gemv_bf16_m1_kn_ws", "sdt_stream_read_runs",
                 "sdt_mfma_ceiling"):
        getattr(L, name).restype = _int
    if L.sdt_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.sdt_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild the library")
    _lib = L
    return L


# ---- host-only helpers ------------------------------------------------------

def status_string(status: int) -> str:
    return lib().sdt_status_string(int(status)).decode()


def last_hip_error() -> int:
    return int(lib().sdt_last_hip_error())


def num_tiles() -> int:
    return int(lib().sdt_num_tiles())


def tile_info(tile_id: int) -> dict:
    t = SdtTile()
    rc = lib().sdt_tile_info(int(tile_id), ctypes.byref(t))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_tile_info")
    return t.as_dict()


def plan_tile(tile_id: int, M: int, N: int, K: int, num_cu: int = 256) -> dict:
    """How a launch of rung tile_id on M x N x K is configured (stages, kgroups)."""
    t = SdtTile()
    rc = lib().sdt_plan_tile(int(tile_id), int(M), int(N), int(K), int(num_cu), ctypes.byref(t))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_plan_tile")
    return t.as_dict()


def launch_cfg(tile_id=-1, stages=-1, kgroups=-1, stagger=-1, splits=-1, split_algo=-1,
               persistent=-1, loaders=-1) -> SdtLaunch:
    return SdtLaunch(int(tile_id), int(stages), int(kgroups), int(stagger), int(splits),
                     int(split_algo), int(persistent), int(loaders))


def pick_tile_ws(M: int, N: int, K: int, num_cu: int, workspace_bytes: int) -> dict:
    """The plan gemm_f16_ws makes with a workspace of that many bytes."""
    t = SdtTile()
    rc = lib().sdt_pick_tile_ws(int(M), int(N), int(K), int(num_cu), int(workspace_bytes),
                                ctypes.byref(t))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_pick_tile_ws")
    return t.as_dict()


def gemm_workspace_size(M: int, N: int, K: int, num_cu: int = 0) -> int:
    """Workspace bytes gemm_f16_ws's automatic plan uses (0: no split)."""
    v = int(lib().sdt_gemm_workspace_size(int(M), int(N), int(K), int(num_cu)))
    if v < 0:
        raise SdtError(SDT_ERR_INVALID_ARG, "sdt_gemm_workspace_size")
    return v


def launch_workspace_size(M: int, N: int, K: int, **cfg) -> int:
    """Workspace bytes a forced launch configuration needs (0: no split)."""
    c = launch_cfg(**cfg)
    v = int(lib().sdt_launch_workspace_size(int(M), int(N), int(K), ctypes.byref(c)))
    if v < 0:
        raise SdtError(SDT_ERR_INVALID_ARG, "sdt_launch_workspace_size")
    return v


class Workspace:
    """A device workspace for the k-split entry points: `nbytes` bytes of a
    torch uint8 tensor (16-byte aligned by torch's allocator), its counters
    zeroed once by sdt_workspace_init on the current stream."""

    def __init__(self, nbytes: int, device="cuda", stream=None):
        import torch
        self.nbytes = (int(nbytes) + 15) // 16 * 16
        self.tensor = torch.empty(max(self.nbytes, 16), dtype=torch.uint8, device=device)
        if self.nbytes:
            rc = lib().sdt_workspace_init(self.tensor.data_ptr(), self.nbytes,
                                          _stream_handle(stream))
            if rc != SDT_OK:
                raise SdtError(rc, "sdt_workspace_init")

    def ptr(self):
        return self.tensor.data_ptr() if self.nbytes else None


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    return workspace.ptr(), workspace.nbytes


def pick_tile(M: int, N: int, K: int, num_cu: int) -> dict:
    t = SdtTile()
    rc = lib().sdt_pick_tile(int(M), int(N), int(K), int(num_cu), ctypes.byref(t))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_pick_tile")
    return t.as_dict()


def pick_rung(M: int, N: int, ref_bm: int, ref_bn: int, min_blocks) -> int:
    arr = (_i64 * len(min_blocks))(*[int(v) for v in min_blocks])
    return int(lib().sdt_pick_rung(int(M), int(N), int(ref_bm), int(ref_bn), len(min_blocks), arr))


def stagger_eligible(K: int) -> bool:
    return bool(lib().sdt_stagger_eligible(int(K)))


def stagger_ktile(wg: int, i: int, nkt: int) -> int:
    return int(lib().sdt_stagger_ktile(int(wg), int(i), int(nkt)))


def check_gemm_args(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc) -> int:
    return int(lib().sdt_check_gemm_args(int(M), int(N), int(K), A_ptr, int(lda), B_ptr,
                                         int(ldb), C_ptr, int(ldc)))


def gemv_num_variants() -> int:
    return int(lib().sdt_gemv_num_variants())


def gemv_kn_num_variants() -> int:
    return int(lib().sdt_gemv_kn_num_variants())


def check_gemv_kn_args(N, K, x_ptr, B_ptr, ldb, y_ptr) -> int:
    return int(lib().sdt_check_gemv_kn_args(int(N), int(K), x_ptr, B_ptr, int(ldb), y_ptr))


# ---- compute entry points (torch tensors on a ROCm device) -------------------

def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _rows(t, name, dtype=None):
    import torch
    dtype = torch.float16 if dtype is None else dtype
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit stride along its rows")
    return t.data_ptr(), (t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1]))


def gemm_f16(A, B, C, stream=None) -> None:
    """C[M, N] = A[M, K] . B[N, K]^T (B stored K-major), fp32 accumulate, fp16 out."""
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    pa, lda = _rows(A, "A")
    pb, ldb = _rows(B, "B")
    pc, ldc = _rows(C, "C")
    rc = lib().gemm_f16(M, N, K, pa, lda, pb, ldb, pc, ldc, _stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, "gemm_f16")


def gemm_f16_ex(A, B, C, tile_id: int = -1, stagger: int = -1, stream=None) -> None:
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    pa, lda = _rows(A, "A")
    pb, ldb = _rows(B, "B")
    pc, ldc = _rows(C, "C")
    rc = lib().gemm_f16_ex(M, N, K, pa, lda, pb, ldb, pc, ldc, _stream_handle(stream),
                           int(tile_id), int(stagger))
    if rc != SDT_OK:
        raise SdtError(rc, "gemm_f16_ex")


def gemv_f16_m1(x, B, y, stream=None, variant: int | None = None) -> None:
    """y[N] = x[K] . B[N, K]^T for the M=1 decode shape (B stored K-major)."""
    import torch
    if x.dtype != torch.float16 or y.dtype != torch.float16:
        raise TypeError("x and y must be float16")
    if x.dim() != 1 or y.dim() != 1 or x.stride(0) != 1 or y.stride(0) != 1:
        raise ValueError("x and y must be contiguous vectors")
    N, K = B.shape
    if x.shape[0] != K or y.shape[0] != N:
        raise ValueError(f"shape mismatch x{tuple(x.shape)} B{tuple(B.shape)} y{tuple(y.shape)}")
    pb, ldb = _rows(B, "B")
    h = _stream_handle(stream)
    if variant is None:
        rc = lib().gemv_f16_m1(N, K, x.data_ptr(), pb, ldb, y.data_ptr(), h)
    else:
        rc = lib().gemv_f16_m1_ex(N, K, x.data_ptr(), pb, ldb, y.data_ptr(), h, int(variant))
    if rc != SDT_OK:
        raise SdtError(rc, "gemv_f16_m1")


def stream_read(buf, out, stream=None) -> None:
    """Enqueue the library's read-only streaming kernel over the bytes of the
    contiguous device tensor `buf` (a multiple of 8192 bytes); `out` is a
    contiguous device tensor of at least numel(buf) * itemsize / 8192 int32
    words."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_contiguous() or not out.is_contiguous() or \
            out.numel() * out.element_size() < (nbytes // 8192) * 4:
        raise ValueError("stream_read: contiguous buf, and out of one int32 word per 8 KB")
    rc = lib().sdt_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), _stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_stream_read")


def stream_read_grid(buf, out, workgroups: int, stream=None) -> None:
    """Enqueue the library's grid-stride read-only kernel over the bytes of the
    contiguous device tensor `buf`; `out` holds at least `workgroups` int32
    words."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_contiguous() or not out.is_contiguous() or \
            out.numel() * out.element_size() < 4 * int(workgroups):
        raise ValueError("stream_read_grid: contiguous buf, and out of one int32 word per workgroup")
    rc = lib().sdt_stream_read_grid(buf.data_ptr(), nbytes, out.data_ptr(), int(workgroups),
                                    _stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_stream_read_grid")


MFMA_CEILING_FRAGS = 24          # operand fragments per lane (one k-tile of a 128 x 64 wave tile)
MFMA_CEILING_FLOP_PER_ITER = 8 * 64 * 2 * 16 * 16 * 32   # per workgroup: 8 waves x 64 MFMAs


def mfma_ceiling(frags, iters: int, out, workgroups: int, bf16: bool = False,
                 mfma32: bool = False, stream=None) -> None:
    """Enqueue the library's register-only MFMA loop (16x16x32 MFMAs, or
    32x32x16 with mfma32): `frags` is a contiguous 16-bit device tensor of
    24 x 64 x 8 values (fragment f of lane l at [(f * 64 + l) * 8, +8)),
    `out` a float32 tensor of at least workgroups x 512 values."""
    if frags.element_size() != 2 or frags.numel() < MFMA_CEILING_FRAGS * 64 * 8 or \
            not frags.is_contiguous() or out.element_size() != 4 or \
            out.numel() < 512 * int(workgroups) or not out.is_contiguous():
        raise ValueError("mfma_ceiling: 24 x 64 x 8 16-bit fragments, workgroups x 512 floats out")
    flags = (1 if bf16 else 0) | (2 if mfma32 else 0)
    rc = lib().sdt_mfma_ceiling(frags.data_ptr(), int(iters), out.data_ptr(), int(workgroups),
                                flags, _stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_mfma_ceiling")


def empty_kernel(stream=None) -> None:
    """Enqueue the library's empty kernel (launch-floor measurement)."""
    rc = lib().sdt_empty_kernel(_stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_empty_kernel")


def gemv_f16_m1_kn(x, B, y, stream=None, variant: int | None = None) -> None:
    """y[N] = x[K] . B[K, N] for the M=1 decode shape with the weights stored
    as K rows of N (the N of a row contiguous)."""
    import torch
    if x.dtype != torch.float16 or y.dtype != torch.float16:
        raise TypeError("x and y must be float16")
    if x.dim() != 1 or y.dim() != 1 or x.stride(0) != 1 or y.stride(0) != 1:
        raise ValueError("x and y must be contiguous vectors")
    K, N = B.shape
    if x.shape[0] != K or y.shape[0] != N:
        raise ValueError(f"shape mismatch x{tuple(x.shape)} B{tuple(B.shape)} y{tuple(y.shape)}")
    pb, ldb = _rows(B, "B")
    h = _stream_handle(stream)
    if variant is None:
        rc = lib().gemv_f16_m1_kn(N, K, x.data_ptr(), pb, ldb, y.data_ptr(), h)
    else:
        rc = lib().gemv_f16_m1_kn_ex(N, K, x.data_ptr(), pb, ldb, y.data_ptr(), h, int(variant))
    if rc != SDT_OK:
        raise SdtError(rc, "gemv_f16_m1_kn")


def _gemm_16(entry, A, B, C, stream, dtype, extra=()):
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    pa, lda = _rows(A, "A", dtype)
    pb, ldb = _rows(B, "B", dtype)
    pc, ldc = _rows(C, "C", dtype)
    rc = getattr(lib(), entry)(M, N, K, pa, lda, pb, ldb, pc, ldc, _stream_handle(stream),
                               *extra)
    if rc != SDT_OK:
        raise SdtError(rc, entry)


def _gemm_16_ws(entry, A, B, C, workspace, stream, dtype, extra=()):
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    pa, lda = _rows(A, "A", dtype)
    pb, ldb = _rows(B, "B", dtype)
    pc, ldc = _rows(C, "C", dtype)
    wp, wn = _ws_args(workspace)
    rc = getattr(lib(), entry)(M, N, K, pa, lda, pb, ldb, pc, ldc, wp, wn,
                               _stream_handle(stream), *extra)
    if rc != SDT_OK:
        raise SdtError(rc, entry)


def gemm_f16_noalloc(A, B, C, stream=None) -> None:
    """gemm_f16_ws with the library's own per-device scratch as the workspace
    (no allocation; calls overlapping on one GPU race)."""
    import torch
    _gemm_16("gemm_f16_noalloc", A, B, C, stream, torch.float16)


def gemm_f16_ws(A, B, C, workspace=None, stream=None) -> None:
    """gemm_f16 with a Workspace: the plan may split K across workgroups."""
    import torch
    _gemm_16_ws("gemm_f16_ws", A, B, C, workspace, stream, torch.float16)


def gemm_bf16_ws(A, B, C, workspace=None, stream=None) -> None:
    import torch
    _gemm_16_ws("gemm_bf16_ws", A, B, C, workspace, stream, torch.bfloat16)


def gemm_f16_cfg(A, B, C, tile_id=-1, stages=-1, kgroups=-1, stagger=-1, splits=-1,
                 split_algo=-1, persistent=-1, workspace=None, stream=None, loaders=-1) -> None:
    """gemm_f16_ws with any part of the launch configuration forced (-1 = automatic)."""
    import torch
    cfg = launch_cfg(tile_id, stages, kgroups, stagger, splits, split_algo, persistent, loaders)
    _gemm_16_ws("gemm_f16_cfg", A, B, C, workspace, stream, torch.float16, (ctypes.byref(cfg),))


def gemm_bf16_cfg(A, B, C, tile_id=-1, stages=-1, kgroups=-1, stagger=-1, splits=-1,
                  split_algo=-1, persistent=-1, workspace=None, stream=None, loaders=-1) -> None:
    import torch
    cfg = launch_cfg(tile_id, stages, kgroups, stagger, splits, split_algo, persistent, loaders)
    _gemm_16_ws("gemm_bf16_cfg", A, B, C, workspace, stream, torch.bfloat16, (ctypes.byref(cfg),))


def gemm_bf16(A, B, C, stream=None) -> None:
    """C[M, N] = A[M, K] . B[N, K]^T with torch.bfloat16 tensors, fp32
    accumulate, bf16 out (round to nearest even)."""
    import torch
    _gemm_16("gemm_bf16", A, B, C, stream, torch.bfloat16)


def gemm_bf16_ex(A, B, C, tile_id: int = -1, stagger: int = -1, stream=None) -> None:
    import torch
    _gemm_16("gemm_bf16_ex", A, B, C, stream, torch.bfloat16, (int(tile_id), int(stagger)))


def _gemv_16(entry, x, B, y, stream, dtype, kn):
    if x.dtype != dtype or y.dtype != dtype:
        raise TypeError(f"x and y must be {dtype}")
    if x.dim() != 1 or y.dim() != 1 or x.stride(0) != 1 or y.stride(0) != 1:
        raise ValueError("x and y must be contiguous vectors")
    if kn:
        K, N = B.shape
    else:
        N, K = B.shape
    if x.shape[0] != K or y.shape[0] != N:
        raise ValueError(f"shape mismatch x{tuple(x.shape)} B{tuple(B.shape)} y{tuple(y.shape)}")
    pb, ldb = _rows(B, "B", dtype)
    rc = getattr(lib(), entry)(N, K, x.data_ptr(), pb, ldb, y.data_ptr(), _stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, entry)


def stream_read_runs(buf, rows: int, row_bytes: int, run_bytes: int, rows_per_wg: int, out,
                     stream=None) -> None:
    """Enqueue the run-length read measurement kernel over a device buffer
    (rows x row_bytes bytes); out: an int32 device tensor of at least
    (row_bytes // run_bytes) * (rows // rows_per_wg) elements."""
    rc = lib().sdt_stream_read_runs(buf.data_ptr(), int(rows), int(row_bytes), int(run_bytes),
                                    int(rows_per_wg), out.data_ptr(), _stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, "sdt_stream_read_runs")


def gemv_kn_workspace_size(N: int, K: int) -> int:
    """Bytes of workspace gemv_f16_m1_kn_ws splits with (0: no split)."""
    return int(lib().sdt_gemv_kn_workspace_size(int(N), int(K)))


def _gemv_kn_ws(entry, x, B, y, workspace, stream, dtype):
    if x.dtype != dtype or y.dtype != dtype:
        raise TypeError(f"x and y must be {dtype}")
    if x.dim() != 1 or y.dim() != 1 or x.stride(0) != 1 or y.stride(0) != 1:
        raise ValueError("x and y must be contiguous vectors")
    K, N = B.shape
    if x.shape[0] != K or y.shape[0] != N:
        raise ValueError(f"shape mismatch x{tuple(x.shape)} B{tuple(B.shape)} y{tuple(y.shape)}")
    pb, ldb = _rows(B, "B", dtype)
    wp, wb = _ws_args(workspace)
    rc = getattr(lib(), entry)(N, K, x.data_ptr(), pb, ldb, y.data_ptr(), wp, wb,
                               _stream_handle(stream))
    if rc != SDT_OK:
        raise SdtError(rc, entry)


def gemv_f16_m1_kn_ws(x, B, y, workspace=None, stream=None) -> None:
    """gemv_f16_m1_kn split over K through `workspace` (a Workspace of at least
    gemv_kn_workspace_size(N, K) bytes; smaller or None: the one-launch kernel)."""
    import torch
    _gemv_kn_ws("gemv_f16_m1_kn_ws", x, B, y, workspace, stream, torch.float16)


def gemv_bf16_m1_kn_ws(x, B, y, workspace=None, stream=None) -> None:
    import torch
    _gemv_kn_ws("gemv_bf16_m1_kn_ws", x, B, y, workspace, stream, torch.bfloat16)


def gemv_bf16_m1(x, B, y, stream=None) -> None:
    """y[N] = x[K] . B[N, K]^T with torch.bfloat16 tensors (B stored K-major)."""
    import torch
    _gemv_16("gemv_bf16_m1", x, B, y, stream, torch.bfloat16, kn=False)


def gemv_bf16_m1_kn(x, B, y, stream=None) -> None:
    """y[N] = x[K] . B[K, N] with torch.bfloat16 tensors (B as K rows of N)."""
    import torch
    _gemv_16("gemv_bf16_m1_kn", x, B, y, stream, torch.bfloat16, kn=True)


def gemm_f16_raw(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, stream_ptr=None) -> int:
    """The C call with raw integers/pointers; returns the status."""
    return int(lib().gemm_f16(int(M), int(N), int(K), A_ptr, int(lda), B_ptr, int(ldb),
                              C_ptr, int(ldc), stream_ptr))


def gemv_f16_m1_raw(N, K, x_ptr, B_ptr, ldb, y_ptr, stream_ptr=None) -> int:
    return int(lib().gemv_f16_m1(int(N), int(K), x_ptr, B_ptr, int(ldb), y_ptr, stream_ptr))
