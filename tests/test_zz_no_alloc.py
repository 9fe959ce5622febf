"""The allocation-free entry point, ag_gemm_f16_noalloc, against the
existing one, ag_gemm_f16_ex: the same kernels on the same schedule, so
the same bits, on two calls in a row, the second with a smaller input
(the fixed scratch keeps what the first call left in it).  Neither call
changes the device's free memory, sizes past the scratch are refused
before anything runs, and a workspace ring brings a larger shape under
the limit."""
import numpy as np
import pytest

import synth
from gpu_util import check_f16, dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def agg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_amd as m
    return m


def _pair(agg, shards, B, cr, **kw):
    """(C from ag_gemm_f16_ex, C from ag_gemm_f16_noalloc, device tensors)."""
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    M, N = sum(s.shape[0] for s in shards), B.shape[1]
    ref = torch.full((M, N), float("nan"), device="cuda")
    agg.ag_gemm_f16(ts, tB, ref, cr, opts=agg.options(**kw))
    assert agg.check() == 0
    C = torch.full((M, N), float("nan"), device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    agg.ag_gemm_f16_noalloc(ts, tB, C, cr, opts=agg.options(**kw))
    assert agg.check() == 0
    assert torch.cuda.mem_get_info()[0] == free0, "the allocation-free call changed free memory"
    return ref, C, ts, tB


def test_noalloc_matches_ex_on_two_calls(agg, orc):
    # 8 shards of 1024 x 4096: 7 slots of 8 MiB and the header, most of the
    # scratch; then 2 shards of 128 x 256 (chunks of 32 rows)
    big = synth.make_f16(8 * 1024, 4096, 512, 8, "normal", 70000)
    small = synth.make_f16(2 * 128, 256, 128, 2, "normal", 70001)
    for (shards, B), cr in ((big, 0), (small, 32)):
        ref, C, _, _ = _pair(agg, shards, B, cr)
        assert torch.equal(C, ref), f"{len(shards)} shards"
    Co, So = orc.ag_gemm_f16(*small)
    check_f16(C.cpu().numpy(), Co, So, "allocation-free call, small")


def test_noalloc_every_mode(agg):
    shards, B = synth.make_f16(4 * 256, 512, 256, 4, "normal", 70002)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    ref = torch.empty((1024, 256), device="cuda")
    agg.ag_gemm_f16(ts, tB, ref, 16)
    assert agg.check() == 0
    for mode in (agg.MODE_SEQUENTIAL, agg.MODE_COPY_ONLY, agg.MODE_COMPUTE_ONLY,
                 agg.MODE_PIPELINED):
        C = torch.full_like(ref, float("nan"))
        if mode == agg.MODE_COPY_ONLY:
            agg.ag_gemm_f16_noalloc(ts, tB, C, 16, opts=agg.options(mode=mode))
            assert agg.check() == 0
            continue
        agg.ag_gemm_f16_noalloc(ts, tB, C, 16, opts=agg.options(mode=mode, link_gbps=100.0))
        assert agg.check() == 0
        assert torch.equal(C, ref), mode


def test_noalloc_ring_brings_a_larger_shape_under_the_limit(agg):
    # 2 shards of 4096 x 8192: a full slot is 64 MiB, past the scratch; a
    # ring of 2 panels of 256 rows needs 8 MiB
    shards, B = synth.make_f16(2 * 4096, 8192, 256, 2, "uniform", 70003)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    C = torch.full((8192, 256), 5.0, device="cuda")
    with pytest.raises(agg.AggError) as e:
        agg.ag_gemm_f16_noalloc(ts, tB, C, 0)
    assert e.value.status == agg.AGG_E_TOO_LARGE
    torch.cuda.synchronize()
    assert (C == 5.0).all(), "a refused call wrote C"
    ref, C, _, _ = _pair(agg, shards, B, 0, workspace_stages=2)
    assert torch.equal(C, ref)


def test_noalloc_rejects_a_workspace_argument(agg):
    shards, B = synth.make_f16(2 * 64, 64, 64, 2, "normal", 70004)
    ts = [dev(s, torch) for s in shards]
    ws = torch.empty(agg.workspace_bytes(2, 128, 64, 2), dtype=torch.uint8, device="cuda")
    agg.workspace_reset(ws)
    C = torch.empty((128, 64), device="cuda")
    with pytest.raises(agg.AggError) as e:
        agg.ag_gemm_f16_noalloc(ts, dev(B, torch), C, 0, opts=agg.options(workspace=ws))
    assert e.value.status == agg.AGG_E_INVALID
