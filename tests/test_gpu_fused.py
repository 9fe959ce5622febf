"""Producer and consumer in one launch (agg_options.producer = FUSED, and
the automatic choice for pipelined calls whose two grids fit on the CUs
together) on the GPU.

The fused launch runs the same producer and consumer code in one grid, the
producer's workgroups first, so its output must be bitwise the one of the
separate producer kernel: for every tile it is built for, on every element
path, with paced links, random piece delays, 2-D chunks, the barrier scheme
and split-K.  Calls that change how the producer runs share one workspace,
and a withheld chunk must end in a reported time-out, not a hang.
"""
import numpy as np
import pytest

import synth
from gpu_util import check_f16, check_i8, dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SEPARATE, FUSED = 2, 3
FUSED_TILES = [2, 3, 12, 13, 14]


@pytest.fixture(scope="module")
def agg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_amd as m
    return m


@pytest.fixture(scope="module")
def data():
    shards, B = synth.make_f16(4 * 512, 1024, 768, 4, "normal", 52000)
    return [dev(s, torch) for s in shards], dev(B, torch), shards, B


def f16(agg, data, chunk_rows=0, ws=None, **kw):
    ts, B = data[0], data[1]
    C = torch.full((ts[0].shape[0] * len(ts), B.shape[1]), float("nan"), device="cuda")
    agg.ag_gemm_f16(ts, B, C, chunk_rows, opts=agg.options(workspace=ws, **kw))
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return C


@pytest.mark.parametrize("tile", FUSED_TILES)
def test_fused_matches_separate_every_tile(agg, orc, data, tile):
    sep = f16(agg, data, tile=tile, producer=SEPARATE)
    if tile == 13:
        Co, So = orc.ag_gemm_f16(data[2], data[3])
        check_f16(sep.cpu().numpy(), Co, So, "separate producer, tile 13")
    for rep in range(2):
        assert torch.equal(f16(agg, data, tile=tile, producer=FUSED), sep), (tile, rep)


@pytest.mark.parametrize("kw", [
    dict(chunk_rows=1), dict(chunk_rows=100), dict(local_shard=2, send_order=[3, 0, 1]),
    dict(link_model=1), dict(link_gbps=50.0), dict(link_gbps=20.0, link_model=1),
    dict(k_block=512), dict(k_block=512, chunk_rows=7), dict(producer_wgs=3),
    dict(producer_wgs=1), dict(consumer_wgs=7), dict(producer_piece_bytes=8192),
    dict(scheme=1), dict(scheme=1, pvalue=2),
    dict(debug_delay_us=20.0, debug_delay_seed=9, producer_piece_bytes=8192, chunk_rows=64),
])
def test_fused_schedules_give_the_same_bits(agg, data, kw):
    kw = dict(kw)
    cr = kw.pop("chunk_rows", 0)
    want = f16(agg, data, cr, tile=13, producer=SEPARATE, **kw)
    for rep in range(2):
        assert torch.equal(f16(agg, data, cr, tile=13, producer=FUSED, **kw), want), (kw, rep)


def test_fused_through_one_workspace_with_other_forms(agg, data):
    """Calls alternate between the fused launch, the separate kernel on the
    library's stream, the DMA engines, a CU-masked producer and the
    sequential and copy-then-compute modes on one workspace, NaN-filled
    now and then: every call gives the same bits."""
    ts, B = data[0], data[1]
    want = f16(agg, data, tile=13, producer=SEPARATE)
    M, K = ts[0].shape[0] * len(ts), ts[0].shape[1]
    ws = torch.empty(agg.workspace_bytes(len(ts), M, K, 2) // 2, dtype=torch.float16,
                     device="cuda")
    agg.workspace_reset(ws)
    forms = [dict(producer=FUSED), dict(producer=SEPARATE), dict(producer=FUSED),
             dict(producer=1), dict(producer=FUSED), dict(producer_cus=32),
             dict(producer=FUSED, k_block=512), dict(mode=2), dict(producer=FUSED),
             dict(producer=SEPARATE, link_gbps=40.0), dict(producer=FUSED, link_gbps=40.0),
             dict(producer=FUSED)]
    for it, kw in enumerate(forms):
        if it % 4 == 3:
            ws.fill_(float("nan"))
            agg.workspace_reset(ws)
        assert torch.equal(f16(agg, data, ws=ws, tile=13, **kw), want), f"call {it} {kw}"
    # copy-only then compute-only leave the same C too
    C = torch.full_like(want, float("nan"))
    agg.ag_gemm_f16(ts, B, C, 0, opts=agg.options(workspace=ws, tile=13, mode=3))
    agg.ag_gemm_f16(ts, B, C, 0, opts=agg.options(workspace=ws, tile=13, mode=1))
    assert agg.check() == 0
    assert torch.equal(C, want)
    assert torch.equal(f16(agg, data, ws=ws, tile=13, producer=FUSED), want)


def test_fused_withheld_chunk_times_out_then_recovers(agg, data):
    want = f16(agg, data, tile=13, producer=FUSED)
    ts, B = data[0], data[1]
    C = torch.zeros_like(want)
    agg.ag_gemm_f16(ts, B, C, opts=agg.options(tile=13, producer=FUSED, debug_drop_chunk=5,
                                                timeout_ms=50.0))
    assert agg.check() == agg.AGG_E_TIMEOUT
    assert torch.equal(f16(agg, data, tile=13, producer=FUSED), want)


def test_automatic_fusion_small_calls(agg, orc):
    """The 2 x 128-row, K 256, N 128 call fuses by default on every path,
    with the oracle's result and the separate kernel's bits."""
    shape = (2 * 128, 256, 128, 2)
    shards, B = synth.make_f16(*shape, "normal", 52100)
    ts, tB = [dev(s, torch) for s in shards], dev(B, torch)
    assert agg.plan("f16", 2, 256, 256, 128, 0)[0].producer_fused == 1
    out = {}
    for prod in (0, SEPARATE):
        C = torch.full((256, 128), float("nan"), device="cuda")
        agg.ag_gemm_f16(ts, tB, C, 0, opts=agg.options(producer=prod))
        assert agg.check() == 0
        out[prod] = C
    assert torch.equal(out[0], out[SEPARATE])
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(out[0].cpu().numpy(), Co, So, "fused f16 2 x 128")

    bs, bB = synth.make_bf16(*shape, "normal", 52200)
    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    tbs, tbB = [bf16(s) for s in bs], bf16(bB)
    for prod in (0, SEPARATE):
        C = torch.full((256, 128), float("nan"), device="cuda")
        agg.ag_gemm_bf16(tbs, tbB, C, 0, opts=agg.options(producer=prod))
        assert agg.check() == 0
        out[prod] = C
    assert torch.equal(out[0], out[SEPARATE])
    Co, So = orc.ag_gemm_bf16(bs, bB)
    check_f16(out[0].cpu().numpy(), Co, So, "fused bf16 2 x 128")

    fs, fB = synth.make_fp8(*shape, "normal", 52300)
    for prod in (0, SEPARATE):
        C = torch.full((256, 128), float("nan"), device="cuda")
        agg.ag_gemm_fp8([dev(s, torch) for s in fs], dev(fB, torch), C, 0,
                        opts=agg.options(producer=prod))
        assert agg.check() == 0
        out[prod] = C
    assert torch.equal(out[0], out[SEPARATE])
    Co, So = orc.ag_gemm_fp8(fs, fB)
    check_f16(out[0].cpu().numpy(), Co, So, "fused fp8 2 x 128")

    ishards, iB, bias, scale = synth.make_i8(2 * 128, 512, 256, 2, 52400)
    res = {}
    for prod in (0, SEPARATE):
        acc = torch.full((256, 256), -1, dtype=torch.int32, device="cuda")
        D = torch.full((256, 256), float("nan"), dtype=torch.float16, device="cuda")
        agg.ag_gemm_i8_dequant([dev(s, torch) for s in ishards], dev(iB, torch),
                               dev(bias, torch), dev(scale, torch), D, 0,
                               opts=agg.options(acc_out=acc, producer=prod))
        assert agg.check() == 0
        res[prod] = (acc.cpu().numpy(), D.cpu().numpy())
    assert np.array_equal(res[0][0], res[SEPARATE][0])
    assert np.array_equal(res[0][1].view(np.uint16), res[SEPARATE][1].view(np.uint16))
    ao, Do = orc.ag_gemm_i8_dequant(ishards, iB, bias, scale)
    check_i8(res[0][0], res[0][1], ao, Do, "fused int8 2 x 128")


@pytest.mark.parametrize("kind", ["f16", "i8"])
def test_fused_split_k(agg, kind):
    """Split-K parts (tile 14) in the fused launch: the same bits as with the
    separate producer, the int8 accumulators exactly."""
    if kind == "f16":
        shards, B = synth.make_f16(2 * 32, 4096, 1024, 2, "normal", 52500)
        ts, tB = [dev(s, torch) for s in shards], dev(B, torch)
        outs = []
        for prod in (SEPARATE, FUSED):
            C = torch.full((64, 1024), float("nan"), device="cuda")
            agg.ag_gemm_f16(ts, tB, C, 0, opts=agg.options(tile=14, k_splits=4, producer=prod))
            assert agg.check() == 0
            outs.append(C)
        assert torch.equal(outs[0], outs[1])
    else:
        shards, B, bias, scale = synth.make_i8(2 * 32, 8192, 1024, 2, 52600)
        outs = []
        for prod in (SEPARATE, FUSED):
            acc = torch.full((64, 1024), -1, dtype=torch.int32, device="cuda")
            D = torch.empty((64, 1024), dtype=torch.float16, device="cuda")
            agg.ag_gemm_i8_dequant([dev(s, torch) for s in shards], dev(B, torch),
                                   dev(bias, torch), dev(scale, torch), D, 0,
                                   opts=agg.options(acc_out=acc, tile=14, k_splits=4,
                                                    producer=prod))
            assert agg.check() == 0
            outs.append(acc)
        assert torch.equal(outs[0], outs[1])
