"""CPU oracle for the streamed AllGather + GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never calls it and
it never calls the product library; the two share no code.  The arithmetic
lives in ``oracle.c`` (plain C, compiled with gcc); this module only builds
that file and marshals numpy arrays into it.

Definitions followed (see ``oracle.c`` for the full statement):
  * gather = the shards' row blocks stacked in shard order, then C = A x B
    (PTO-ISA AllGather+GEMM README, "compute function"; Triton-distributed
    AllGather GEMM tutorial, reference function built from all_gather,
    concatenation on dim 0 and matmul);
  * fp16 path: fp64 sum of exact products, rounded once to fp32;
  * bf16 path: the same with bfloat16 inputs;
  * fp8 path: the same with OCP FP8 E4M3 inputs (the float8_e4m3fn inputs
    of the Ascend grouped-GEMM page's FP8 variant);
  * int8 path: exact integer sum + int32 bias, fp32 conversion, fp32 product
    with the per-channel scale, fp16 rounding (catccos AllGatherMatmulDequant
    design doc, section 2.2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA)."""
    if not force and os.path.exists(_LIB) and \
            os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            lib.oracle_ag_gemm_f16_rows.argtypes = [P, ctypes.c_int, P, I64, I64, I64, P, I64, P, P]
            lib.oracle_ag_gemm_f16.argtypes = [P, ctypes.c_int, P, I64, I64, I64, P, P]
            lib.oracle_ag_gemm_bf16_rows.argtypes = [P, ctypes.c_int, P, I64, I64, I64, P, I64, P, P]
            lib.oracle_bf16_to_double_n.argtypes = [P, P, I64]
            lib.oracle_ag_gemm_fp8_rows.argtypes = [P, ctypes.c_int, P, I64, I64, I64, P, I64, P, P]
            lib.oracle_fp8e4m3_to_double_n.argtypes = [P, P, I64]
            lib.oracle_ag_gemm_i8_rows.argtypes = [P, ctypes.c_int, P, P, P, I64, I64, I64, P, I64, P, P]
            lib.oracle_ag_gemm_i8.argtypes = [P, ctypes.c_int, P, P, P, I64, I64, I64, P, P]
            lib.oracle_half_to_double_n.argtypes = [P, P, I64]
            lib.oracle_float_to_half_n.argtypes = [P, P, I64]
            lib.oracle_dequant_n.argtypes = [P, P, P, I64]
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_threads.restype = ctypes.c_int
            lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_half_to_double.restype = ctypes.c_double
            lib.oracle_float_to_half.argtypes = [ctypes.c_float]
            lib.oracle_float_to_half.restype = ctypes.c_uint16
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _shard_table(shards, dtype):
    arrs = [np.ascontiguousarray(s, dtype=dtype) for s in shards]
    table = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    return arrs, table


def _dims(shards, B):
    S, K = shards[0].shape
    for s in shards:
        if s.shape != (S, K):
            raise ValueError("all shards must have the same shape")
    if B.shape[0] != K:
        raise ValueError("B must be K x N")
    return S * len(shards), K, B.shape[1]


def ag_gemm_f16(shards, B, rows=None, with_abs: bool = True):
    """C = gather(shards) x B in fp32 (rows of C if ``rows`` is given).

    Returns (C, abs_sum); abs_sum[i, j] = sum_k |A[i,k] B[k,j]| (or None).
    """
    lib = _load()
    arrs, table = _shard_table(shards, np.float16)
    B = np.ascontiguousarray(B, dtype=np.float16)
    M, K, N = _dims(arrs, B)
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    C = np.empty((len(rows), N), np.float32)
    S_abs = np.empty((len(rows), N), np.float64) if with_abs else None
    rc = lib.oracle_ag_gemm_f16_rows(table, len(arrs), _ptr(B), M, K, N,
                                     _ptr(rows), len(rows), _ptr(C),
                                     _ptr(S_abs) if with_abs else None)
    if rc:
        raise RuntimeError(f"oracle_ag_gemm_f16_rows failed ({rc})")
    return C, S_abs


def ag_gemm_bf16(shards, B, rows=None, with_abs: bool = True):
    """bf16 variant of ag_gemm_f16.  Shards and B are uint16 arrays of
    bfloat16 bit patterns (numpy has no bfloat16 type)."""
    lib = _load()
    arrs, table = _shard_table(shards, np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    M, K, N = _dims(arrs, B)
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    C = np.empty((len(rows), N), np.float32)
    S_abs = np.empty((len(rows), N), np.float64) if with_abs else None
    rc = lib.oracle_ag_gemm_bf16_rows(table, len(arrs), _ptr(B), M, K, N,
                                      _ptr(rows), len(rows), _ptr(C),
                                      _ptr(S_abs) if with_abs else None)
    if rc:
        raise RuntimeError(f"oracle_ag_gemm_bf16_rows failed ({rc})")
    return C, S_abs


def ag_gemm_fp8(shards, B, rows=None, with_abs: bool = True):
    """fp8 (E4M3) variant of ag_gemm_f16.  Shards and B are uint8 arrays of
    E4M3 bit patterns."""
    lib = _load()
    arrs, table = _shard_table(shards, np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K, N = _dims(arrs, B)
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    C = np.empty((len(rows), N), np.float32)
    S_abs = np.empty((len(rows), N), np.float64) if with_abs else None
    rc = lib.oracle_ag_gemm_fp8_rows(table, len(arrs), _ptr(B), M, K, N,
                                     _ptr(rows), len(rows), _ptr(C),
                                     _ptr(S_abs) if with_abs else None)
    if rc:
        raise RuntimeError(f"oracle_ag_gemm_fp8_rows failed ({rc})")
    return C, S_abs


def fp8_to_double(h: np.ndarray) -> np.ndarray:
    lib = _load()
    h = np.ascontiguousarray(h, dtype=np.uint8)
    out = np.empty(h.shape, np.float64)
    lib.oracle_fp8e4m3_to_double_n(_ptr(h), _ptr(out), h.size)
    return out


def bf16_to_double(h: np.ndarray) -> np.ndarray:
    lib = _load()
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float64)
    lib.oracle_bf16_to_double_n(_ptr(h), _ptr(out), h.size)
    return out


def ag_gemm_i8_dequant(shards, B, bias, scale, rows=None):
    """int8 path: returns (acc int32 = A.B + bias, D fp16 = dequantised)."""
    lib = _load()
    arrs, table = _shard_table(shards, np.int8)
    B = np.ascontiguousarray(B, dtype=np.int8)
    bias = np.ascontiguousarray(bias, dtype=np.int32)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    M, K, N = _dims(arrs, B)
    if bias.shape != (N,) or scale.shape != (N,):
        raise ValueError("bias and scale must have N entries")
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    acc = np.empty((len(rows), N), np.int32)
    D = np.empty((len(rows), N), np.uint16)
    rc = lib.oracle_ag_gemm_i8_rows(table, len(arrs), _ptr(B), _ptr(bias),
                                    _ptr(scale), M, K, N, _ptr(rows),
                                    len(rows), _ptr(acc), _ptr(D))
    if rc == 3:
        raise OverflowError("int8 accumulator left the int32 range")
    if rc:
        raise RuntimeError(f"oracle_ag_gemm_i8_rows failed ({rc})")
    return acc, D.view(np.float16)


def half_to_double(h: np.ndarray) -> np.ndarray:
    lib = _load()
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float64)
    lib.oracle_half_to_double_n(_ptr(h), _ptr(out), h.size)
    return out


def float_to_half(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit patterns, round to nearest even."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.oracle_float_to_half_n(_ptr(x), _ptr(out), x.size)
    return out


def dequant(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp16 bits of fp16(fp32(v) * s), elementwise."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.int32)
    s = np.ascontiguousarray(np.broadcast_to(s, v.shape), dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib.oracle_dequant_n(_ptr(v), _ptr(s), _ptr(out), v.size)
    return out


def set_threads(n: int) -> int:
    """Use n threads in the oracle's loops from now on (n <= 0: unchanged);
    returns the previous count.  Results do not depend on it."""
    return int(_load().oracle_set_threads(int(n)))


def threads_used() -> int:
    """OpenMP threads the oracle's parallel loops will use."""
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit():
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
