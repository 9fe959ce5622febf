"""Streamed AllGather + GEMM for AMD Instinct MI355X (gfx950).

C = concat(A_0, ..., A_{n-1}) x B computed while the shards arrive chunk by
chunk: a producer kernel on a side stream moves the remote shards' chunks
into a workspace and releases each on a per-source counter; a persistent
MFMA GEMM starts on the local shard and consumes the remote chunks in send
order.  fp16 -> fp32 (and its bf16 -> fp32 and fp8 E4M3 -> fp32 variants), and
int8 -> int32 + bias -> per-channel dequant -> fp16.

The work runs in libaggemm.so (HIP, C ABI in include/aggemm.h); this package
only binds it.
"""
from ._native import (  # noqa: F401
    AGG_E_HIP, AGG_E_INVALID, AGG_E_NOMEM, AGG_E_TIMEOUT, AGG_E_TOO_LARGE, AGG_E_UNSUPPORTED,
    AGG_OK, LIB_PATH, NOALLOC_MAX_BYTES, LINKS_PARALLEL, LINKS_SERIAL, MAX_SHARDS, MODE_COMPUTE_ONLY, MODE_COPY_ONLY,
    MODE_PIPELINED, MODE_SEQUENTIAL, PRODUCER_KERNEL, PRODUCER_SDMA, PRODUCER_SEPARATE, PRODUCER_FUSED, SCHEME_BARRIER,
    SCHEME_COUNTERS, AggError, Options,
    PlanInfo, Prepared, ag_gemm_bf16, ag_gemm_f16, ag_gemm_f16_noalloc, ag_gemm_fp8,
    ag_gemm_i8_dequant, check,
    options, pick_chunk_rows, plan, release, status_string, workspace_bytes, workspace_reset,
)
