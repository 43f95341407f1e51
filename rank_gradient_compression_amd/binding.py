"""ctypes binding of libpsgd.so: the C ABI of include/psgd.h, same names,
argument marshalling only.  Device pointers are passed as Python ints (for
example `tensor.data_ptr()`), streams as raw `hipStream_t` handles (for example
`torch.cuda.current_stream().cuda_stream`).

Importing this module loads the library; if it has not been built the import
fails loudly -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Callable, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpsgd.so")

PSGD_OK = 0
PSGD_ERR_INVALID_ARG = 1
PSGD_ERR_UNSUPPORTED = 2
PSGD_ERR_WORKSPACE = 3
PSGD_ERR_HIP = 4
PSGD_ERR_HOOK = 5
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP", 5: "HOOK"}

PSGD_MAX_RANK = 64
PSGD_NOALLOC_SCRATCH_BYTES = 64 << 20
PSGD_KIND_VECTOR = 0
PSGD_KIND_PASSTHRU = 1
PSGD_KIND_COMPRESSED = 2
PSGD_FLAG_MOMENTUM = 1
PSGD_FLAG_GRADS_BF16 = 2
PSGD_STEP_NO_ERROR_FEEDBACK = 1
PSGD_STEP_NESTEROV = 2
PSGD_STEP_DEFER_RESIDUAL = 4
PSGD_STEP_RESIDUAL_DEFERRED = 8
PSGD_STEP_PAYLOAD_BF16 = 16
PSGD_STEP_PAYLOAD_FP8 = 32

PSGD_STAGE_EF_P = 0
PSGD_STAGE_GS = 1
PSGD_STAGE_MTP = 2
PSGD_STAGE_QREDUCE = 3
PSGD_STAGE_RESIDUAL = 4
PSGD_STAGE_PASSTHRU = 5
PSGD_STAGE_REFRESH = 6
PSGD_NSTAGES = 7
STAGE_NAMES = ["ef_p", "gs", "mtp", "qreduce", "residual", "passthru", "refresh"]

# Every symbol include/psgd.h declares.
EXPORTED = [
    "psgd_plan_create", "psgd_plan_destroy", "psgd_plan_get_info", "psgd_plan_tensor",
    "psgd_workspace_init", "psgd_compress", "psgd_compress_noalloc", "psgd_decompress", "psgd_refresh", "psgd_init_q",
    "psgd_step_stats", "psgd_subspace_overlap",
    "psgd_timing_enable", "psgd_timing_stages", "psgd_timing_read", "psgd_stream_probe", "psgd_stream_copy", "psgd_last_error",
    "psgd_version",
]


class PsgdError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class psgd_plan_info_t(ctypes.Structure):
    _fields_ = [
        ("ntensors", ctypes.c_int32), ("ncompressed", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("flat_elems", ctypes.c_size_t), ("p_elems", ctypes.c_size_t),
        ("passthru_elems", ctypes.c_size_t), ("p_buffer_elems", ctypes.c_size_t), ("q_elems", ctypes.c_size_t),
        ("payload_elems", ctypes.c_size_t), ("dense_elems", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class psgd_step_opts_t(ctypes.Structure):
    _fields_ = [
        ("power_iters", ctypes.c_int32), ("refresh_iters", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("sgd_lr", ctypes.c_float), ("sgd_momentum", ctypes.c_float), ("params", ctypes.c_void_p),
        ("sgd_buf", ctypes.c_void_p), ("zero_cols", ctypes.c_void_p),
    ]


def step_opts(power_iters: int = 0, refresh_iters: int = 0, flags: int = 0, sgd_lr: float = 0.0,
              sgd_momentum: float = 0.0, params: int = 0, sgd_buf: int = 0, zero_cols: int = 0) -> psgd_step_opts_t:
    return psgd_step_opts_t(power_iters, refresh_iters, flags, sgd_lr, sgd_momentum, params or None, sgd_buf or None,
                            zero_cols or None)


psgd_reduce_fn = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")

# libpsgd.so needs the HIP runtime by soname (libamdhip64.so.7).  PyTorch for
# ROCm ships its own copy; loading PyTorch first makes the soname resolve to
# that copy, so that both share one runtime (and PyTorch's streams are valid
# handles here).
try:
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - plain C ABI use without PyTorch
    pass
lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l and "/" in l})
    except OSError:  # pragma: no cover
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process (" + ", ".join(_hip_runtimes()) + "): import "
                      "rank_gradient_compression_amd before anything that loads another libamdhip64")

_vp = ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)

lib.psgd_plan_create.argtypes = [ctypes.c_int32, _i64p, _i64p, _i64p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float,
                                 ctypes.POINTER(_vp)]
lib.psgd_plan_destroy.argtypes = [_vp]
lib.psgd_plan_destroy.restype = None
lib.psgd_plan_get_info.argtypes = [_vp, ctypes.POINTER(psgd_plan_info_t)]
lib.psgd_plan_tensor.argtypes = [_vp, ctypes.c_int32, _i32p, _i64p, _i64p, _i64p]
lib.psgd_workspace_init.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
lib.psgd_compress.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(psgd_step_opts_t), psgd_reduce_fn,
                              _vp, _vp, ctypes.c_size_t, _vp]
lib.psgd_compress_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(psgd_step_opts_t),
                                      psgd_reduce_fn, _vp, _vp]
lib.psgd_decompress.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.psgd_refresh.argtypes = [_vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
lib.psgd_init_q.argtypes = [_vp, _vp, ctypes.c_uint64, _vp, ctypes.c_size_t, _vp]
lib.psgd_step_stats.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.psgd_subspace_overlap.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.psgd_timing_enable.argtypes = [_vp, ctypes.c_int32]
lib.psgd_timing_stages.argtypes = [_vp, ctypes.c_uint32]
lib.psgd_timing_read.argtypes = [_vp, ctypes.POINTER(ctypes.c_double), _i64p]
lib.psgd_stream_copy.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
lib.psgd_stream_probe.argtypes = [_vp, ctypes.c_int32, _vp, ctypes.c_int32, ctypes.c_size_t, _vp, _vp]
lib.psgd_last_error.restype = ctypes.c_char_p
lib.psgd_version.restype = ctypes.c_char_p
for _f in ["psgd_plan_create", "psgd_plan_get_info", "psgd_plan_tensor", "psgd_workspace_init", "psgd_compress",
           "psgd_compress_noalloc",
           "psgd_decompress", "psgd_refresh", "psgd_init_q", "psgd_timing_enable", "psgd_timing_stages", "psgd_timing_read",
           "psgd_stream_copy",
           "psgd_stream_probe", "psgd_step_stats", "psgd_subspace_overlap"]:
    getattr(lib, _f).restype = ctypes.c_int


def _check(fn: str, status: int) -> None:
    if status != PSGD_OK:
        raise PsgdError(fn, status, lib.psgd_last_error().decode(errors="replace"))


def _arr64(xs: Optional[Sequence[int]]):
    if xs is None:
        return None
    return (ctypes.c_int64 * len(xs))(*[int(x) for x in xs])


def psgd_last_error() -> str:
    return lib.psgd_last_error().decode(errors="replace")


def psgd_version() -> str:
    return lib.psgd_version().decode()


def psgd_plan_create(rows: Sequence[int], cols: Sequence[int], rank: int, flags: int = 0, beta: float = 0.0,
                     offsets: Optional[Sequence[int]] = None) -> int:
    if len(rows) != len(cols) or (offsets is not None and len(offsets) != len(rows)):
        raise ValueError("rows, cols and offsets must have the same length")
    out = _vp()
    st = lib.psgd_plan_create(len(rows), _arr64(rows), _arr64(cols), _arr64(offsets), rank, flags, beta,
                              ctypes.byref(out))
    _check("psgd_plan_create", st)
    return out.value


def psgd_plan_destroy(plan: int) -> None:
    lib.psgd_plan_destroy(plan)


def psgd_plan_get_info(plan: int) -> dict:
    info = psgd_plan_info_t()
    _check("psgd_plan_get_info", lib.psgd_plan_get_info(plan, ctypes.byref(info)))
    return info.as_dict()


def psgd_plan_tensor(plan: int, tensor: int):
    kind = ctypes.c_int32()
    off, poff, qoff = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("psgd_plan_tensor", lib.psgd_plan_tensor(plan, tensor, ctypes.byref(kind), ctypes.byref(off),
                                                    ctypes.byref(poff), ctypes.byref(qoff)))
    return kind.value, off.value, poff.value, qoff.value


def psgd_workspace_init(plan: int, workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    _check("psgd_workspace_init", lib.psgd_workspace_init(plan, workspace, workspace_bytes, stream))


def make_hook(fn: Callable[[int, int, int], int]):
    """Wraps fn(buf_ptr, count, stream) -> int as a psgd_reduce_fn.  Keep the
    returned object alive while the library may call it."""
    return psgd_reduce_fn(lambda buf, count, stream, user: int(fn(buf or 0, count, stream or 0)))


def psgd_compress(plan: int, grads: int, err: int, mom: int, q: int, p: int, mhat: int,
                  opts: Optional[psgd_step_opts_t], hook, workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    h = hook if hook is not None else psgd_reduce_fn()
    o = ctypes.byref(opts) if opts is not None else None
    _check("psgd_compress", lib.psgd_compress(plan, grads, err or None, mom or None, q or None, p, mhat or None, o,
                                              h, None, workspace, workspace_bytes, stream))


def psgd_compress_noalloc(plan: int, grads: int, err: int, mom: int, q: int, p: int, mhat: int,
                          opts: Optional[psgd_step_opts_t], hook, stream: int = 0) -> None:
    h = hook if hook is not None else psgd_reduce_fn()
    o = ctypes.byref(opts) if opts is not None else None
    _check("psgd_compress_noalloc", lib.psgd_compress_noalloc(plan, grads, err or None, mom or None, q or None, p,
                                                              mhat or None, o, h, None, stream))


def psgd_decompress(plan: int, p: int, q: int, out: int, workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    _check("psgd_decompress", lib.psgd_decompress(plan, p, q or None, out, workspace, workspace_bytes, stream))


def psgd_refresh(plan: int, tensor: int, m: int, q: int, iters: int, workspace: int, workspace_bytes: int,
                 stream: int = 0) -> None:
    _check("psgd_refresh", lib.psgd_refresh(plan, tensor, m, q, iters, workspace, workspace_bytes, stream))


def psgd_init_q(plan: int, q: int, seed: int, workspace: int, workspace_bytes: int, stream: int = 0) -> None:
    _check("psgd_init_q", lib.psgd_init_q(plan, q or None, seed & ((1 << 64) - 1), workspace, workspace_bytes,
                                          stream))


def psgd_step_stats(plan: int, err: int, mhat: int, out: int, workspace: int, workspace_bytes: int,
                    stream: int = 0) -> None:
    _check("psgd_step_stats", lib.psgd_step_stats(plan, err or None, mhat or None, out or None, workspace,
                                                  workspace_bytes, stream))


def psgd_subspace_overlap(plan: int, q_a: int, q_b: int, scratch: int, out: int, workspace: int,
                          workspace_bytes: int, stream: int = 0) -> None:
    _check("psgd_subspace_overlap", lib.psgd_subspace_overlap(plan, q_a or None, q_b or None, scratch or None,
                                                              out or None, workspace, workspace_bytes, stream))


def psgd_timing_enable(plan: int, enable: bool) -> None:
    _check("psgd_timing_enable", lib.psgd_timing_enable(plan, 1 if enable else 0))


def psgd_timing_stages(plan: int, mask: int) -> None:
    _check("psgd_timing_stages", lib.psgd_timing_stages(plan, mask & 0xFFFFFFFF))


def psgd_timing_read(plan: int):
    ms = (ctypes.c_double * PSGD_NSTAGES)()
    n = (ctypes.c_int64 * PSGD_NSTAGES)()
    _check("psgd_timing_read", lib.psgd_timing_read(plan, ms, n))
    return list(ms), list(n)


def psgd_stream_copy(dst: int, src: int, n: int, stream: int = 0) -> None:
    _check("psgd_stream_copy", lib.psgd_stream_copy(dst, src, n, stream))


PSGD_PROBE_SINK_FLOATS = 16384


def psgd_stream_probe(ins, outs, n: int, sink: int = 0, stream: int = 0) -> None:
    """ins / outs: device pointers (ints) of the arrays read / written."""
    a_in = (ctypes.c_void_p * max(1, len(ins)))(*ins)
    a_out = (ctypes.c_void_p * max(1, len(outs)))(*outs)
    _check("psgd_stream_probe", lib.psgd_stream_probe(a_in if ins else None, len(ins), a_out if outs else None,
                                                      len(outs), n, sink or None, stream))
