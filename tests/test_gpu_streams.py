"""Stream semantics of the pipelined mode: the producer runs on the
library's own stream with no event on the caller's stream, so it must take
its start from the consumer.  Work queued on the caller's stream before a
call (here a long sleep, then writes of new shard contents) must be seen by
the producer's copies."""
import numpy as np
import pytest

import synth
from gpu_util import dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def agg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_amd as m
    return m


@pytest.mark.parametrize("kind", ["f16", "i8"])
def test_producer_sees_writes_queued_before_the_call(agg, kind):
    n, S, K, N = 4, 256, 512, 256
    if kind == "f16":
        shards, B = synth.make_f16(n * S, K, N, n, "normal", 60000)
    else:
        shards, B, bias, scale = synth.make_i8(n * S, K, N, n, 60000)
        tb, tsc = dev(bias, torch), dev(scale, torch)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    new = [dev(s, torch) for s in shards]
    out_dtype = torch.float32 if kind == "f16" else torch.float16

    def call(C):
        if kind == "f16":
            agg.ag_gemm_f16(ts, tB, C, 16)
        else:
            agg.ag_gemm_i8_dequant(ts, tB, tb, tsc, C, 16)

    ref = torch.empty((n * S, N), dtype=out_dtype, device="cuda")
    call(ref)
    assert agg.check() == 0
    for t in ts:
        t.zero_()
    torch.cuda.synchronize()
    # about 20 ms of stream work ahead of the call, then the real contents
    torch.cuda._sleep(40_000_000)
    for t, v in zip(ts, new):
        t.copy_(v)
    C = torch.full((n * S, N), 7, dtype=out_dtype, device="cuda")
    call(C)
    assert agg.check() == 0
    assert torch.equal(C, ref)


def _case(agg, seed):
    n, S, K, N = 4, 256, 512, 256
    shards, B = synth.make_f16(n * S, K, N, n, "normal", seed)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    ref = torch.empty((n * S, N), device="cuda")
    agg.ag_gemm_f16(ts, tB, ref, 16)
    assert agg.check() == 0
    return shards, ts, tB, ref


def test_reset_orders_the_producer_after_it(agg):
    """A caller-owned workspace whose header holds stale words (here 0x7F
    bytes: a start word and an error word that would pass for a later
    epoch) is reset behind a long stretch of work and new shard contents on
    the caller's stream.  The first pipelined call's producer, on the
    library's own stream, must not run before that reset: otherwise it
    would copy the old shard contents (or have its counters cleared under
    it) and the call would time out or be wrong."""
    shards, ts, tB, ref = _case(agg, 60100)
    new = [dev(s, torch) for s in shards]
    n, S, K = len(ts), ts[0].shape[0], ts[0].shape[1]
    ws = torch.empty(agg.workspace_bytes(n, n * S, K, 2), dtype=torch.uint8, device="cuda")
    for it in range(2):
        ws.fill_(0x7F)
        for t in ts:
            t.zero_()
        torch.cuda.synchronize()
        torch.cuda._sleep(40_000_000)          # about 20 ms ahead of the reset
        for t, v in zip(ts, new):
            t.copy_(v)
        agg.workspace_reset(ws)
        C = torch.full_like(ref, float("nan"))
        agg.ag_gemm_f16(ts, tB, C, 16, opts=agg.options(workspace=ws))
        assert agg.check() == 0, f"call {it}"
        assert torch.equal(C, ref), f"call {it}"


def test_queued_work_longer_than_the_chunk_limit(agg):
    """More work queued ahead of a pipelined call than its chunk time
    limit: the producer's wait for the consumer's start has a bound of its
    own, so the call succeeds."""
    shards, ts, tB, ref = _case(agg, 60200)
    for kind in ("internal", "caller"):
        kw = dict(timeout_ms=20.0)
        if kind == "caller":
            n, S, K = len(ts), ts[0].shape[0], ts[0].shape[1]
            ws = torch.empty(agg.workspace_bytes(n, n * S, K, 2), dtype=torch.uint8,
                             device="cuda")
            agg.workspace_reset(ws)
            kw["workspace"] = ws
        torch.cuda.synchronize()
        torch.cuda._sleep(200_000_000)         # about 100 ms, five times the limit
        C = torch.full_like(ref, float("nan"))
        agg.ag_gemm_f16(ts, tB, C, 16, opts=agg.options(**kw))
        assert agg.check() == 0, kind
        assert torch.equal(C, ref), kind


def test_binding_rejects_strided_vectors(agg):
    """bias and scale are read as contiguous N-vectors: a strided view is
    refused before anything is launched."""
    n, S, K, N = 2, 64, 64, 32
    shards, B, bias, scale = synth.make_i8(n * S, K, N, n, 60300)
    ts = [dev(s, torch) for s in shards]
    tb2 = torch.zeros((N, 2), dtype=torch.int32, device="cuda")
    C = torch.empty((n * S, N), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        agg.ag_gemm_i8_dequant(ts, dev(B, torch), tb2[:, 0], dev(scale, torch), C)
    sc2 = torch.zeros((N, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        agg.ag_gemm_i8_dequant(ts, dev(B, torch), dev(bias, torch), sc2[:, 1], C)


def test_package_imported_before_torch_still_runs(tmp_path):
    """A fresh process that imports the package before torch: the library
    must still share torch's HIP runtime, so torch's allocations and the
    library's calls both work."""
    import subprocess
    import sys
    root = __import__("os").path.dirname(__import__("os").path.dirname(__file__))
    code = ("import communication_gemm_amd as agg\n"
            "import torch\n"
            "ts = [torch.ones((64, 64), dtype=torch.float16, device='cuda') for _ in range(2)]\n"
            "B = torch.ones((64, 32), dtype=torch.float16, device='cuda')\n"
            "C = torch.empty((128, 32), device='cuda')\n"
            "agg.ag_gemm_f16(ts, B, C)\n"
            "assert agg.check() == 0\n"
            "assert (C == 64).all()\n"
            "print('ok')\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0 and "ok" in out.stdout, out.stdout + out.stderr
