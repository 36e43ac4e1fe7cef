"""ctypes binding over libfkmeans.so: argument marshalling only.

Every function has the name of the C entry point it calls. Tensors are
PyTorch tensors on the current HIP device; work is enqueued on torch's
current stream. Nothing here computes: a missing or broken library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfkmeans.so")

FK_F32, FK_F16, FK_BF16 = 0, 1, 2
FK_OK = 0
STATUS = {0: "FK_OK", 1: "FK_ERR_INVALID", 2: "FK_ERR_UNSUPPORTED", 3: "FK_ERR_WORKSPACE",
          4: "FK_ERR_HIP"}

_lib = None


class FKError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fk_status_string(status)}")


class fk_trace_t(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int32), ("norms_ms", ctypes.c_double),
                ("assign_ms", ctypes.c_double), ("update_ms", ctypes.c_double)]


def load(path: Optional[str] = None):
    """Load libfkmeans.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python -m exact_means_clustering_flashassign_amd.build)")
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "fk_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "fk_version": (I32, []),
        "fk_workspace_size": (SZ, [ctypes.c_int, I64, I64, I64, I64]),
        "fk_norms": (ctypes.c_int, [P, P, P, ctypes.c_int, I64, I64, I64, P]),
        "fk_assign": (ctypes.c_int, [P, P, P, ctypes.c_int, I64, I64, I64, I64, P, P]),
        "fk_update": (ctypes.c_int, [P, P, ctypes.c_int, I64, I64, I64, I64, P, P, P, P, SZ, P]),
        "fk_update_noalloc": (ctypes.c_int, [P, P, ctypes.c_int, I64, I64, I64, I64, P, P, P, P]),
        "fk_update_partial": (ctypes.c_int, [P, P, ctypes.c_int, I64, I64, I64, I64, P, P, P, SZ,
                                             P]),
        "fk_lloyd": (ctypes.c_int, [P, ctypes.c_int, I64, I64, I64, I64, P, I32, ctypes.c_float,
                                    P, P, ctypes.POINTER(I32), P, SZ, P]),
        "fk_workspace_size_host": (SZ, [ctypes.c_int, I64, I64, I64, I64]),
        "fk_lloyd_host": (ctypes.c_int, [P, ctypes.c_int, I64, I64, I64, I64, P, I32,
                                         ctypes.c_float, I64, P, P, ctypes.POINTER(I32), P, SZ,
                                         P]),
        "fk_trace_begin": (ctypes.c_int, [I32]),
        "fk_trace_end": (ctypes.c_int, [ctypes.POINTER(fk_trace_t)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def fk_status_string(status: int) -> str:
    return load().fk_status_string(int(status)).decode()


def fk_version() -> int:
    return int(load().fk_version())


# ---------------------------------------------------------------------------
# tensor helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    torch = _torch()
    codes = {torch.float32: FK_F32, torch.float16: FK_F16, torch.bfloat16: FK_BF16}
    if dtype not in codes:
        raise ValueError(f"unsupported element type {dtype}; use float32, float16 or bfloat16")
    return codes[dtype]


def torch_dtype(code: int):
    torch = _torch()
    return {FK_F32: torch.float32, FK_F16: torch.float16, FK_BF16: torch.bfloat16}[code]


def _dev(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(_torch().cuda.current_stream(t.device).cuda_stream)


def _check(st: int, where: str):
    if st != FK_OK:
        raise FKError(st, where)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def fk_workspace_size(dtype, B: int, N: int, d: int, K: int) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().fk_workspace_size(code, B, N, d, K))


def workspace(dtype, B: int, N: int, d: int, K: int, device):
    """A device workspace tensor of fk_workspace_size bytes (256-byte aligned)."""
    torch = _torch()
    n = fk_workspace_size(dtype, B, N, d, K)
    if n == 0:
        raise ValueError("invalid problem size")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def fk_norms(c, dtype, c_lp=None, cnorm=None) -> Tuple[object, object]:
    """c (B,K,d) fp32 -> (c_lp (B,K,d) dtype, cnorm (B,K) fp32)."""
    torch = _torch()
    code = dtype_code(dtype)
    B, K, d = c.shape
    if c_lp is None:
        c_lp = torch.empty((B, K, d), dtype=dtype, device=c.device)
    if cnorm is None:
        cnorm = torch.empty((B, K), dtype=torch.float32, device=c.device)
    st = load().fk_norms(_dev(c, "c", torch.float32), _dev(c_lp, "c_lp", dtype, (B, K, d)),
                         _dev(cnorm, "cnorm", torch.float32, (B, K)), code, B, K, d, _stream(c))
    _check(st, "fk_norms")
    return c_lp, cnorm


def fk_assign(x, c_lp, cnorm, ids=None):
    """x (B,N,d), c_lp (B,K,d) same dtype, cnorm (B,K) fp32 -> ids (B,N) int32."""
    torch = _torch()
    code = dtype_code(x.dtype)
    B, N, d = x.shape
    K = c_lp.shape[1]
    if ids is None:
        ids = torch.empty((B, N), dtype=torch.int32, device=x.device)
    st = load().fk_assign(_dev(x, "x"), _dev(c_lp, "c_lp", x.dtype, (B, K, d)),
                          _dev(cnorm, "cnorm", torch.float32, (B, K)), code, B, N, d, K,
                          _dev(ids, "ids", torch.int32, (B, N)), _stream(x))
    _check(st, "fk_assign")
    return ids


def fk_update(x, ids, c, counts=None, shift=None, ws=None):
    """In-place centroid update of c (B,K,d) fp32; returns (c, counts, shift)."""
    torch = _torch()
    code = dtype_code(x.dtype)
    B, N, d = x.shape
    K = c.shape[1]
    if counts is None:
        counts = torch.empty((B, K), dtype=torch.int32, device=x.device)
    if shift is None:
        shift = torch.empty((B,), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(x.dtype, B, N, d, K, x.device)
    st = load().fk_update(_dev(x, "x"), _dev(ids, "ids", torch.int32, (B, N)), code, B, N, d, K,
                          _dev(c, "c", torch.float32, (B, K, d)),
                          _dev(counts, "counts", torch.int32, (B, K)),
                          _dev(shift, "shift", torch.float32, (B,)), _dev(ws, "ws", torch.uint8),
                          ws.numel(), _stream(x))
    _check(st, "fk_update")
    return c, counts, shift


FK_NOALLOC_SCRATCH_BYTES = 64 << 20


def fk_update_noalloc(x, ids, c, counts, shift):
    """fk_update with the library's own device scratch (no workspace); the
    caller passes every output. In-place update of c; returns (c, counts, shift)."""
    torch = _torch()
    code = dtype_code(x.dtype)
    B, N, d = x.shape
    K = c.shape[1]
    st = load().fk_update_noalloc(_dev(x, "x"), _dev(ids, "ids", torch.int32, (B, N)), code, B,
                                  N, d, K, _dev(c, "c", torch.float32, (B, K, d)),
                                  _dev(counts, "counts", torch.int32, (B, K)),
                                  _dev(shift, "shift", torch.float32, (B,)), _stream(x))
    _check(st, "fk_update_noalloc")
    return c, counts, shift


def fk_update_partial(x, ids, sums, counts, ws=None):
    """Add this block of points' per-cluster sums (B,K,d) fp32 and counts
    (B,K) int32 into sums and counts (one shard's part of an update)."""
    torch = _torch()
    code = dtype_code(x.dtype)
    B, N, d = x.shape
    K = sums.shape[1]
    if ws is None:
        ws = workspace(x.dtype, B, N, d, K, x.device)
    st = load().fk_update_partial(_dev(x, "x"), _dev(ids, "ids", torch.int32, (B, N)), code, B,
                                  N, d, K, _dev(sums, "sums", torch.float32, (B, K, d)),
                                  _dev(counts, "counts", torch.int32, (B, K)),
                                  _dev(ws, "ws", torch.uint8), ws.numel(), _stream(x))
    _check(st, "fk_update_partial")
    return sums, counts


def fk_lloyd(x, init, max_iter: int, tol: float, ids=None, centers=None, ws=None):
    """Lloyd's loop from init (B,K,d) in x's dtype -> (ids, centers fp32, n_iter).
    init=None resumes from the fp32 centres in `centers` (updated in place)."""
    torch = _torch()
    code = dtype_code(x.dtype)
    B, N, d = x.shape
    if init is None and centers is None:
        raise ValueError("resuming (init=None) needs the fp32 centers to start from")
    K = (init if init is not None else centers).shape[1]
    if ids is None:
        ids = torch.empty((B, N), dtype=torch.int32, device=x.device)
    if centers is None:
        centers = torch.empty((B, K, d), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(x.dtype, B, N, d, K, x.device)
    n_iter = ctypes.c_int32(0)
    ip = None if init is None else _dev(init, "init", x.dtype, (B, K, d))
    st = load().fk_lloyd(_dev(x, "x"), code, B, N, d, K, ip,
                         int(max_iter), float(tol), _dev(ids, "ids", torch.int32, (B, N)),
                         _dev(centers, "centers", torch.float32, (B, K, d)),
                         ctypes.byref(n_iter), _dev(ws, "ws", torch.uint8), ws.numel(),
                         _stream(x))
    _check(st, "fk_lloyd")
    return ids, centers, int(n_iter.value)


def fk_workspace_size_host(dtype, B: int, chunk: int, d: int, K: int) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().fk_workspace_size_host(code, B, chunk, d, K))


def fk_lloyd_host(x_host, init, max_iter: int, tol: float, chunk: int, ids=None, centers=None,
                  ws=None):
    """Lloyd's loop over points in host memory, streamed in chunks of `chunk`
    points per problem -> (ids, centers fp32, n_iter). x_host: a contiguous
    CPU tensor (B,N,d), best page-locked (pin_memory); init (B,K,d) on the GPU,
    or None to resume from the fp32 centres in `centers`."""
    torch = _torch()
    if not isinstance(x_host, torch.Tensor) or x_host.device.type != "cpu":
        raise ValueError("x_host must be a CPU tensor")
    if not x_host.is_contiguous() or x_host.dim() != 3:
        raise ValueError("x_host must be a contiguous (B, N, d) tensor")
    if init is None and centers is None:
        raise ValueError("resuming (init=None) needs the fp32 centers to start from")
    code = dtype_code(x_host.dtype)
    B, N, d = x_host.shape
    start = init if init is not None else centers
    K = start.shape[1]
    dev = start.device
    if ids is None:
        ids = torch.empty((B, N), dtype=torch.int32, device=dev)
    if centers is None:
        centers = torch.empty((B, K, d), dtype=torch.float32, device=dev)
    if ws is None:
        n = fk_workspace_size_host(code, B, chunk, d, K)
        if n == 0:
            raise ValueError("invalid problem size or chunk")
        raw = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        off = (-raw.data_ptr()) % 256
        ws = raw[off:off + n]
    n_iter = ctypes.c_int32(0)
    st = load().fk_lloyd_host(x_host.data_ptr(), code, B, N, d, K,
                              None if init is None else _dev(init, "init", x_host.dtype,
                                                             (B, K, d)), int(max_iter),
                              float(tol), int(chunk), _dev(ids, "ids", torch.int32, (B, N)),
                              _dev(centers, "centers", torch.float32, (B, K, d)),
                              ctypes.byref(n_iter), _dev(ws, "ws", torch.uint8), ws.numel(),
                              _stream(start))
    _check(st, "fk_lloyd_host")
    return ids, centers, int(n_iter.value)


def fk_trace_begin(capacity: int) -> None:
    _check(load().fk_trace_begin(int(capacity)), "fk_trace_begin")


def fk_trace_end() -> dict:
    out = fk_trace_t()
    _check(load().fk_trace_end(ctypes.byref(out)), "fk_trace_end")
    return {"iterations": out.iterations, "norms_ms": out.norms_ms,
            "assign_ms": out.assign_ms, "update_ms": out.update_ms}


# ---------------------------------------------------------------------------
# libfkbaseline: the materialised-distance assign and the scatter-atomic
# update (include/fkmeans_baselines.h), for contrast measurements only.
# ---------------------------------------------------------------------------
BASELINE_LIB_PATH = os.path.join(HERE, "libfkbaseline.so")
_blib = None


def load_baseline(path: Optional[str] = None):
    """Load libfkbaseline.so (once) and declare its signatures."""
    global _blib
    if _blib is not None:
        return _blib
    path = path or BASELINE_LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python -m exact_means_clustering_flashassign_amd.build)")
    lib = ctypes.CDLL(path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.fkb_assign_materialized.restype = ctypes.c_int
    lib.fkb_assign_materialized.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, I64, P, P, P]
    lib.fkb_update_atomic.restype = ctypes.c_int
    lib.fkb_update_atomic.argtypes = [P, P, ctypes.c_int, I64, I64, I64, I64, P, P, P, P]
    lib.fkb_mfma_peak.restype = ctypes.c_int
    lib.fkb_mfma_peak.argtypes = [I64, ctypes.c_int32, ctypes.c_uint32, P, P, P]
    lib.fkb_wall_clock_khz.restype = ctypes.c_int32
    lib.fkb_wall_clock_khz.argtypes = []
    _blib = lib
    return lib


def fkb_assign_materialized(x, c_lp, cnorm, dist=None, ids=None):
    """Standard assign: the (B,N,K) fp32 matrix -2 x.c (rocBLAS), then argmin."""
    torch = _torch()
    code = dtype_code(x.dtype)
    B, N, d = x.shape
    K = c_lp.shape[1]
    if dist is None:
        dist = torch.empty((B, N, K), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty((B, N), dtype=torch.int32, device=x.device)
    st = load_baseline().fkb_assign_materialized(
        _dev(x, "x"), _dev(c_lp, "c_lp", x.dtype, (B, K, d)),
        _dev(cnorm, "cnorm", torch.float32, (B, K)), code, B, N, d, K,
        _dev(dist, "dist", torch.float32, (B, N, K)), _dev(ids, "ids", torch.int32, (B, N)),
        _stream(x))
    _check(st, "fkb_assign_materialized")
    return ids


def fkb_update_atomic(x, ids, c, counts=None, sums=None):
    """Standard update: scatter atomics into sums, then divide; c updated in place."""
    torch = _torch()
    code = dtype_code(x.dtype)
    B, N, d = x.shape
    K = c.shape[1]
    if counts is None:
        counts = torch.empty((B, K), dtype=torch.int32, device=x.device)
    if sums is None:
        sums = torch.empty((B, K, d), dtype=torch.float32, device=x.device)
    st = load_baseline().fkb_update_atomic(
        _dev(x, "x"), _dev(ids, "ids", torch.int32, (B, N)), code, B, N, d, K,
        _dev(c, "c", torch.float32, (B, K, d)), _dev(counts, "counts", torch.int32, (B, K)),
        _dev(sums, "sums", torch.float32, (B, K, d)), _stream(x))
    _check(st, "fkb_update_atomic")
    return c, counts


def fkb_mfma_peak(blocks: int, iters: int, seed: int, out=None, stamps=None, device="cuda"):
    """MFMA peak probe: blocks x 4 waves, each iters x 32 v_mfma_f32_32x32x16_f16.
    Returns (out, stamps); stamps (blocks, 4) int64 = memtime start/end,
    realtime start/end per block."""
    torch = _torch()
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    if stamps is None:
        stamps = torch.empty((blocks, 4), dtype=torch.int64, device=device)
    st = load_baseline().fkb_mfma_peak(int(blocks), int(iters), int(seed) & 0xFFFFFFFF,
                                       _dev(out, "out", torch.float32, (blocks * 256,)),
                                       _dev(stamps, "stamps", torch.int64, (blocks, 4)),
                                       _stream(out))
    _check(st, "fkb_mfma_peak")
    return out, stamps


def fkb_wall_clock_khz() -> int:
    return int(load_baseline().fkb_wall_clock_khz())
