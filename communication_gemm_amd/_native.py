"""ctypes binding of libaggemm.so: argument marshalling only.

Every step of the operation runs in the library's HIP kernels; this module
turns torch tensors into device pointers and sizes, passes the current
stream, and raises on a non-zero status.  The library must have been built
(``python communication_gemm_amd/build.py``); importing this module without
it fails loudly, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libaggemm.so")

(AGG_OK, AGG_E_INVALID, AGG_E_UNSUPPORTED, AGG_E_NOMEM, AGG_E_HIP, AGG_E_TIMEOUT,
 AGG_E_TOO_LARGE) = range(7)
NOALLOC_MAX_BYTES = 64 << 20   # AGG_NOALLOC_MAX_BYTES
MODE_PIPELINED, MODE_COMPUTE_ONLY, MODE_SEQUENTIAL, MODE_COPY_ONLY = range(4)
SCHEME_COUNTERS, SCHEME_BARRIER = range(2)
LINKS_PARALLEL, LINKS_SERIAL = range(2)
PRODUCER_KERNEL, PRODUCER_SDMA, PRODUCER_SEPARATE, PRODUCER_FUSED = range(4)
MAX_SHARDS = 64


class AggError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Options(ctypes.Structure):
    """Mirror of ``struct agg_options`` in include/aggemm.h."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("local_shard", ctypes.c_int),
        ("send_order", ctypes.POINTER(ctypes.c_int)),
        ("mode", ctypes.c_int),
        ("link_gbps", ctypes.c_double),
        ("link_model", ctypes.c_int),
        ("producer_wgs", ctypes.c_int),
        ("consumer_wgs", ctypes.c_int),
        ("tile", ctypes.c_int),
        ("acc_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("timeout_ms", ctypes.c_double),
        ("debug_drop_chunk", ctypes.c_int),
        ("consumer_events", ctypes.c_void_p * 2),
        ("workspace_stages", ctypes.c_int),
        ("scheme", ctypes.c_int),
        ("pvalue", ctypes.c_int),
        ("trace", ctypes.c_void_p),
        ("producer_piece_bytes", ctypes.c_int64),
        ("k_splits", ctypes.c_int),
        ("debug_delay_us", ctypes.c_double),
        ("debug_delay_seed", ctypes.c_uint32),
        ("producer", ctypes.c_int),
        ("producer_cus", ctypes.c_int),
        ("k_block", ctypes.c_int64),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of ``struct agg_plan_info``."""

    _fields_ = [
        ("shard_rows", ctypes.c_int64),
        ("chunk_rows", ctypes.c_int),
        ("chunks_per_source", ctypes.c_int),
        ("tile_m", ctypes.c_int),
        ("tile_n", ctypes.c_int),
        ("m_tiles_per_shard", ctypes.c_int),
        ("n_tiles", ctypes.c_int),
        ("total_tiles", ctypes.c_int64),
        ("total_chunks", ctypes.c_int64),
        ("consumer_wgs", ctypes.c_int),
        ("producer_wgs", ctypes.c_int),
        ("tile_id", ctypes.c_int),
        ("trace_words", ctypes.c_int64),
        ("workspace_stages", ctypes.c_int),
        ("workspace_bytes", ctypes.c_int64),
        ("k_splits", ctypes.c_int),
        ("k_blocks", ctypes.c_int),
        ("k_block", ctypes.c_int64),
        ("producer_fused", ctypes.c_int),
    ]


EXPORTS = {
    # name: (restype, argtypes)
    "ag_gemm_options_init": (None, [ctypes.POINTER(Options)]),
    "ag_gemm_f16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]),
    "ag_gemm_f16_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.POINTER(Options)]),
    "ag_gemm_f16_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.POINTER(Options)]),
    "ag_gemm_bf16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]),
    "ag_gemm_bf16_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.POINTER(Options)]),
    "ag_gemm_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]),
    "ag_gemm_fp8_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.POINTER(Options)]),
    "ag_gemm_i8_dequant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_void_p]),
    "ag_gemm_i8_dequant_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_void_p,
                                             ctypes.POINTER(Options)]),
    "ag_gemm_pick_chunk_rows": (ctypes.c_int, [ctypes.c_int64]),
    "ag_gemm_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_int]),
    "ag_gemm_workspace_reset": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t,
                                               ctypes.c_void_p]),
    "ag_gemm_check": (ctypes.c_int, [ctypes.c_void_p]),
    "ag_gemm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ag_gemm_release": (None, []),
    "ag_gemm_plan": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                    ctypes.POINTER(Options), ctypes.c_int,
                                    ctypes.POINTER(PlanInfo), ctypes.c_void_p,
                                    ctypes.c_void_p]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python communication_gemm_amd/build.py` (hipcc, gfx950)")
    # torch first: it brings its own HIP runtime, and the library must bind
    # to that one.  Loaded the other way round, the process ends up with the
    # system runtime under torch, and torch's first device allocation fails.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.ag_gemm_status_string(int(status)).decode()


def _raise(status: int, what: str):
    if status:
        raise AggError(status, what)


class Prepared:
    """One call with its arguments marshalled once: each call of this object
    only crosses the C ABI (tight loops pay no Python-side checks).  It keeps
    the ctypes arguments and the options alive; the caller keeps the tensors
    alive."""

    __slots__ = ("_fn", "_args", "_what", "_keep")

    def __init__(self, fn, args, what, keep):
        self._fn = fn
        self._args = tuple(args)
        self._what = what
        self._keep = keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc:
            raise AggError(rc, self._what)


def _invoke(plain, ex, args, opts, what, prepare):
    """Call (or, with prepare=True, return a Prepared call of) the plain or
    the _ex entry point with marshalled arguments."""
    fn = plain if opts is None else ex
    full = tuple(args) if opts is None else tuple(args) + (ctypes.byref(opts),)
    if prepare:
        return Prepared(fn, full, what, (args, opts))
    _raise(fn(*full), what)


def options(**kw) -> Options:
    """An agg_options with the library's defaults, then ``kw`` applied.

    ``send_order`` may be a sequence of ints; ``consumer_events`` a pair of
    torch.cuda.Event objects; ``acc_out``/``workspace`` torch tensors.
    """
    o = Options()
    lib.ag_gemm_options_init(ctypes.byref(o))
    keep = []
    for k, v in kw.items():
        if v is None:
            continue
        if k == "send_order":
            arr = (ctypes.c_int * len(v))(*[int(x) for x in v])
            keep.append(arr)
            o.send_order = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int))
        elif k == "consumer_events":
            o.consumer_events[0] = ctypes.c_void_p(v[0].cuda_event)
            o.consumer_events[1] = ctypes.c_void_p(v[1].cuda_event)
        elif k in ("acc_out", "workspace", "trace"):
            if hasattr(v, "data_ptr"):
                if not v.is_cuda or not v.is_contiguous():
                    raise ValueError(f"{k} must be a contiguous CUDA tensor")
                _on_current_device(v)
            setattr(o, k, v.data_ptr() if hasattr(v, "data_ptr") else int(v))
            if k == "workspace" and hasattr(v, "numel"):
                o.workspace_bytes = v.numel() * v.element_size()
            if k == "trace" and hasattr(v, "numel"):
                o._trace_words = v.numel() * v.element_size() // 8
        else:
            setattr(o, k, v)
    o._keep = keep   # keep ctypes arrays alive with the struct
    return o


def _check_trace(kind, n_shards, M, K, N, chunk_rows, opts):
    """A trace tensor must hold the call's plan's trace_words: the library
    takes a bare pointer and writes that many words."""
    words = getattr(opts, "_trace_words", None) if opts is not None else None
    if words is None:
        return
    import torch
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    need = plan(kind, n_shards, M, K, N, chunk_rows, opts, num_cus=cus)[0].trace_words
    if words < need:
        raise ValueError(f"trace holds {words} words; this call's plan needs {need}")


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on_current_device(*tensors):
    """Every tensor lives on the current device (the library launches there
    and takes the pointers as that device's)."""
    import torch
    cur = torch.cuda.current_device()
    for t in tensors:
        if t is not None and t.device.index != cur:
            raise ValueError(f"tensor on {t.device}, but the current device is cuda:{cur}")


def _shard_ptrs(shards, dtype, K):
    import torch
    if not shards:
        raise ValueError("need at least one shard")
    if len(shards) > MAX_SHARDS:
        raise ValueError(f"at most {MAX_SHARDS} shards")
    S = shards[0].shape[0]
    for t in shards:
        if t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"shards must be contiguous 2-D {dtype} CUDA tensors")
        if tuple(t.shape) != (S, K):
            raise ValueError("all shards must be S x K")
    _on_current_device(*shards)
    return (ctypes.c_void_p * len(shards))(*[t.data_ptr() for t in shards]), S


def _check_out(C, shape, dtype):
    if C.dtype != dtype or not C.is_cuda or not C.is_contiguous() or tuple(C.shape) != shape:
        raise ValueError(f"output must be a contiguous {dtype} CUDA tensor of shape {shape}")
    _on_current_device(C)


def _check_vec(v, n, dtype, what):
    """A contiguous (n,) vector of `dtype` on the current device: a strided
    view would be read as if it were contiguous."""
    if v.dtype != dtype or tuple(v.shape) != (n,) or not v.is_cuda or not v.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {dtype} CUDA tensor of shape ({n},)")
    _on_current_device(v)


def ag_gemm_f16(shards, B, C, chunk_rows: int = 0, stream=None, opts: Options | None = None,
                prepare: bool = False):
    """C[M, N] (fp32) = concat(shards)[M, K] (fp16) x B[K, N] (fp16).

    With prepare=True nothing runs: the call is returned as a Prepared
    object (arguments checked and marshalled once) to be called later."""
    import torch
    if B.dtype != torch.float16 or not B.is_cuda or not B.is_contiguous() or B.dim() != 2:
        raise ValueError("B must be a contiguous 2-D fp16 CUDA tensor")
    K, N = B.shape
    _on_current_device(B)
    table, S = _shard_ptrs(shards, torch.float16, K)
    M = S * len(shards)
    _check_out(C, (M, N), torch.float32)
    _check_trace("f16", len(shards), M, K, N, int(chunk_rows), opts)
    st = _stream_handle(stream)
    r = _invoke(lib.ag_gemm_f16, lib.ag_gemm_f16_ex,
                (table, len(shards), B.data_ptr(), C.data_ptr(), M, K, N, int(chunk_rows), st),
                opts, "ag_gemm_f16", prepare)
    return r if prepare else C


def ag_gemm_f16_noalloc(shards, B, C, chunk_rows: int = 0, stream=None,
                        opts: Options | None = None, prepare: bool = False):
    """ag_gemm_f16 through the allocation-free entry point: the library's
    fixed per-GPU scratch array is the workspace (opts.workspace must be
    unset); AggError with AGG_E_TOO_LARGE if the call needs more than
    NOALLOC_MAX_BYTES of it."""
    import torch
    if B.dtype != torch.float16 or not B.is_cuda or not B.is_contiguous() or B.dim() != 2:
        raise ValueError("B must be a contiguous 2-D fp16 CUDA tensor")
    K, N = B.shape
    _on_current_device(B)
    table, S = _shard_ptrs(shards, torch.float16, K)
    M = S * len(shards)
    _check_out(C, (M, N), torch.float32)
    _check_trace("f16", len(shards), M, K, N, int(chunk_rows), opts)
    st = _stream_handle(stream)
    args = (table, len(shards), B.data_ptr(), C.data_ptr(), M, K, N, int(chunk_rows), st,
            ctypes.byref(opts) if opts is not None else None)
    if prepare:
        return Prepared(lib.ag_gemm_f16_noalloc, args, "ag_gemm_f16_noalloc", (table, opts))
    _raise(lib.ag_gemm_f16_noalloc(*args), "ag_gemm_f16_noalloc")
    return C


def ag_gemm_bf16(shards, B, C, chunk_rows: int = 0, stream=None, opts: Options | None = None,
                 prepare: bool = False):
    """C[M, N] (fp32) = concat(shards)[M, K] (bf16) x B[K, N] (bf16)."""
    import torch
    if B.dtype != torch.bfloat16 or not B.is_cuda or not B.is_contiguous() or B.dim() != 2:
        raise ValueError("B must be a contiguous 2-D bf16 CUDA tensor")
    K, N = B.shape
    _on_current_device(B)
    table, S = _shard_ptrs(shards, torch.bfloat16, K)
    M = S * len(shards)
    _check_out(C, (M, N), torch.float32)
    _check_trace("bf16", len(shards), M, K, N, int(chunk_rows), opts)
    st = _stream_handle(stream)
    r = _invoke(lib.ag_gemm_bf16, lib.ag_gemm_bf16_ex,
                (table, len(shards), B.data_ptr(), C.data_ptr(), M, K, N, int(chunk_rows), st),
                opts, "ag_gemm_bf16", prepare)
    return r if prepare else C


def _fp8_dtypes():
    import torch
    return (torch.uint8, torch.float8_e4m3fn)


def ag_gemm_fp8(shards, B, C, chunk_rows: int = 0, stream=None, opts: Options | None = None,
                prepare: bool = False):
    """C[M, N] (fp32) = concat(shards)[M, K] (fp8 E4M3) x B[K, N] (fp8 E4M3).

    Shards and B are torch.float8_e4m3fn tensors, or uint8 tensors holding
    E4M3 bit patterns (all of one dtype)."""
    import torch
    dt = B.dtype
    if dt not in _fp8_dtypes() or not B.is_cuda or not B.is_contiguous() or B.dim() != 2:
        raise ValueError("B must be a contiguous 2-D float8_e4m3fn (or uint8) CUDA tensor")
    K, N = B.shape
    _on_current_device(B)
    table, S = _shard_ptrs(shards, dt, K)
    M = S * len(shards)
    _check_out(C, (M, N), torch.float32)
    _check_trace("fp8", len(shards), M, K, N, int(chunk_rows), opts)
    st = _stream_handle(stream)
    r = _invoke(lib.ag_gemm_fp8, lib.ag_gemm_fp8_ex,
                (table, len(shards), B.data_ptr(), C.data_ptr(), M, K, N, int(chunk_rows), st),
                opts, "ag_gemm_fp8", prepare)
    return r if prepare else C


def ag_gemm_i8_dequant(shards, B, bias, scale, C, chunk_rows: int = 0, stream=None,
                       opts: Options | None = None, prepare: bool = False):
    """C[M, N] (fp16) = fp16(fp32(concat(shards) x B + bias) * scale)."""
    import torch
    if B.dtype != torch.int8 or not B.is_cuda or not B.is_contiguous() or B.dim() != 2:
        raise ValueError("B must be a contiguous 2-D int8 CUDA tensor")
    K, N = B.shape
    _on_current_device(B)
    table, S = _shard_ptrs(shards, torch.int8, K)
    M = S * len(shards)
    _check_vec(bias, N, torch.int32, "bias")
    _check_vec(scale, N, torch.float32, "scale")
    _check_out(C, (M, N), torch.float16)
    _check_trace("i8", len(shards), M, K, N, int(chunk_rows), opts)
    st = _stream_handle(stream)
    r = _invoke(lib.ag_gemm_i8_dequant, lib.ag_gemm_i8_dequant_ex,
                (table, len(shards), B.data_ptr(), bias.data_ptr(), scale.data_ptr(),
                 C.data_ptr(), M, K, N, int(chunk_rows), st),
                opts, "ag_gemm_i8_dequant", prepare)
    return r if prepare else C


def pick_chunk_rows(shard_rows: int) -> int:
    return lib.ag_gemm_pick_chunk_rows(int(shard_rows))


def workspace_bytes(n_shards: int, M: int, K: int, elt_bytes: int) -> int:
    return lib.ag_gemm_workspace_bytes(int(n_shards), int(M), int(K), int(elt_bytes))


def workspace_reset(ws, stream=None):
    rc = lib.ag_gemm_workspace_reset(ctypes.c_void_p(ws.data_ptr()),
                                     ws.numel() * ws.element_size(), _stream_handle(stream))
    _raise(rc, "ag_gemm_workspace_reset")


def check(stream=None) -> int:
    """Synchronise and return the status of the calls since the last check."""
    return lib.ag_gemm_check(_stream_handle(stream))


def release():
    lib.ag_gemm_release()


def plan(kind: str, n_shards: int, M: int, K: int, N: int, chunk_rows: int = 0,
         opts: Options | None = None, num_cus: int = 256, orders: bool = False):
    """Host-only schedule query: (PlanInfo, tile_order or None, chunk_order or None)."""
    import numpy as np
    info = PlanInfo()
    k = {"f16": 0, "i8": 1, "bf16": 2, "fp8": 3}[kind]
    o = ctypes.byref(opts) if opts is not None else None
    rc = lib.ag_gemm_plan(k, n_shards, M, K, N, chunk_rows, o, num_cus, ctypes.byref(info),
                          None, None)
    _raise(rc, "ag_gemm_plan")
    if not orders:
        return info, None, None
    tiles = np.zeros((info.total_tiles, 4), np.int32)
    chunks = np.zeros((max(info.total_chunks, 0), 2), np.int32)
    rc = lib.ag_gemm_plan(k, n_shards, M, K, N, chunk_rows, o, num_cus, ctypes.byref(info),
                          tiles.ctypes.data, chunks.ctypes.data if chunks.size else None)
    _raise(rc, "ag_gemm_plan")
    return info, tiles, chunks
