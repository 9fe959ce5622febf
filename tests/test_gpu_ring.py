"""The bounded workspace ring: each remote shard gets W row panels instead
of a full slot, and the producer overwrites a panel only after the
consumer has finished every tile of it.  Results match the oracle, and
are bitwise those of the full-slot workspace (the ring changes where rows
wait, not the arithmetic).  With W = 1 and many panels per shard every
panel but the first is written over a panel that was just read, so a
missing wait shows up as wrong rows."""
import numpy as np
import pytest

import synth
from gpu_util import check_f16, check_i8, dev, freivalds_i8, stratified_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def agg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_amd as m
    return m


def f16_call(agg, ts, tB, M, N, cr=0, **kw):
    C = torch.full((M, N), float("nan"), device="cuda")
    agg.ag_gemm_f16(ts, tB, C, cr, opts=agg.options(**kw))
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return C


@pytest.mark.parametrize("stages", [1, 2, 3])
@pytest.mark.parametrize("tile", [13, 2])
def test_ring_parity_small_tiles(agg, orc, stages, tile):
    n, S, K, N = 4, 1000, 256, 200        # 16 (or 8) ragged panels per shard
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 61000 + stages)
    ts = [dev(s, torch) for s in shards]
    C = f16_call(agg, ts, dev(B, torch), n * S, N, 0, workspace_stages=stages, tile=tile)
    info, _, _ = agg.plan("f16", n, n * S, K, N, 0, agg.options(workspace_stages=stages, tile=tile))
    assert info.workspace_stages == stages
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C.cpu().numpy(), Co, So, f"ring {stages} tile {tile}")


@pytest.mark.parametrize("stages", [1, 2])
def test_ring_matches_full_slots_bitwise(agg, stages):
    n, S, K, N = 4, 1024, 4096, 4096      # tile 256: 4 panels per shard
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 62000)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    full = f16_call(agg, ts, tB, n * S, N)
    for kw in (dict(), dict(local_shard=2), dict(link_gbps=200.0)):
        ring = f16_call(agg, ts, tB, n * S, N, workspace_stages=stages, **kw)
        assert torch.equal(ring, full), kw


def test_ring_int8_sampled_rows(agg, orc):
    c = synth.CASES[5]
    shards, B, bias, scale = synth.make_case(c)
    ts = [dev(s, torch) for s in shards]
    acc = torch.empty((c.M, c.N), dtype=torch.int32, device="cuda")
    D = torch.empty((c.M, c.N), dtype=torch.float16, device="cuda")
    info, _, _ = agg.plan("i8", 2, c.M, c.K, c.N, 0, agg.options(workspace_stages=2))
    ws = torch.empty(info.workspace_bytes, dtype=torch.uint8, device="cuda")
    agg.workspace_reset(ws)
    agg.ag_gemm_i8_dequant(ts, dev(B, torch), dev(bias, torch), dev(scale, torch), D, 0,
                           opts=agg.options(workspace_stages=2, workspace=ws, acc_out=acc))
    assert agg.check() == 0
    rows = stratified_rows(c.M, c.n_shards, info.chunk_rows, extra=6)
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale, rows=rows)
    acc = acc.cpu().numpy()
    check_i8(acc[rows], D.cpu().numpy()[rows], ao, Do, "int8 ring")
    assert freivalds_i8(acc, shards, B, bias) == c.M


def test_ring_workspace_size_is_checked(agg):
    n, S, K, N = 2, 1024, 512, 256
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 63000)
    ts = [dev(s, torch) for s in shards]
    info, _, _ = agg.plan("f16", n, n * S, K, N, 0, agg.options(workspace_stages=1))
    assert info.workspace_bytes < agg.workspace_bytes(n, n * S, K, 2)
    ws = torch.empty(info.workspace_bytes, dtype=torch.uint8, device="cuda")
    agg.workspace_reset(ws)
    C = torch.empty((n * S, N), device="cuda")
    agg.ag_gemm_f16(ts, dev(B, torch), C, 0, opts=agg.options(workspace_stages=1, workspace=ws))
    assert agg.check() == 0
    with pytest.raises(agg.AggError) as e:     # the same workspace is too small for full slots
        agg.ag_gemm_f16(ts, dev(B, torch), C, 0, opts=agg.options(workspace=ws))
    assert e.value.status == agg.AGG_E_INVALID


def test_ring_copy_only_does_not_wait(agg):
    n, S, K, N = 4, 1024, 1024, 256
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 64000)
    ts = [dev(s, torch) for s in shards]
    C = torch.empty((n * S, N), device="cuda")
    agg.ag_gemm_f16(ts, dev(B, torch), C, 0,
                    opts=agg.options(workspace_stages=1, mode=agg.MODE_COPY_ONLY))
    assert agg.check() == 0
