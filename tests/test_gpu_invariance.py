"""Schedule invariance, ordering and failure handling on the GPU.

Chunking cuts A along M only and never changes the order of the K sum, so
the HIP output must be bit-identical whatever the chunk size, local shard,
send order, link pacing, link model, producer width, producer piece size
or mode (the gathered result is the same C: PTO-ISA AllGather+GEMM README,
"compute function").
A consumer that read a chunk before its release would see the NaN planted
in the workspace.  A withheld release must end in a reported time-out, not
a hang.
"""
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


@pytest.fixture(scope="module")
def data():
    shards, B = synth.make_f16(4 * 512, 1024, 768, 4, "normal", 50000)
    return [dev(s, torch) for s in shards], dev(B, torch), shards, B


def call(agg, data, chunk_rows=0, **kw):
    ts, B = data[0], data[1]
    C = torch.full((ts[0].shape[0] * len(ts), B.shape[1]), float("nan"), device="cuda")
    agg.ag_gemm_f16(ts, B, C, chunk_rows, opts=agg.options(**kw))
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return C


@pytest.fixture(scope="module")
def ref(agg, data, orc):
    C = call(agg, data)
    Co, So = orc.ag_gemm_f16(data[2], data[3])
    check_f16(C.cpu().numpy(), Co, So, "reference call")
    return C


@pytest.mark.parametrize("kw", [
    dict(chunk_rows=1), dict(chunk_rows=16), dict(chunk_rows=100), dict(chunk_rows=512),
    dict(local_shard=2), dict(local_shard=3, send_order=[1, 0, 2]),
    dict(send_order=[3, 2, 1]),
    dict(link_model=1), dict(link_model=1, send_order=[2, 3, 1]),
    dict(link_gbps=50.0), dict(link_gbps=20.0, link_model=1),
    dict(producer_wgs=1), dict(producer_wgs=3), dict(consumer_wgs=7),
    dict(mode=2),
    # producer pieces: one sweep; one sweep with 100-row chunks (25 pieces a
    # chunk, the short last chunk mostly empty pieces); a piece larger than
    # every chunk; one sweep on a single producer workgroup
    dict(producer_piece_bytes=8192), dict(producer_piece_bytes=8192, chunk_rows=100),
    dict(producer_piece_bytes=1 << 20), dict(producer_piece_bytes=8192, producer_wgs=1),
    # chunks of rows x one K-block (K = 1024: two blocks of 512)
    dict(k_block=512), dict(k_block=512, chunk_rows=1), dict(k_block=512, chunk_rows=100),
    dict(k_block=512, local_shard=3, send_order=[1, 0, 2]), dict(k_block=512, link_model=1),
    dict(k_block=512, link_gbps=30.0), dict(k_block=512, link_gbps=20.0, link_model=1),
    dict(k_block=512, producer_wgs=1), dict(k_block=512, mode=2),
    dict(k_block=512, producer_piece_bytes=8192, chunk_rows=7),
])
def test_bitwise_invariant(agg, data, ref, kw):
    kw = dict(kw)
    cr = kw.pop("chunk_rows", 0)
    C = call(agg, data, cr, **kw)
    assert torch.equal(C, ref), kw


def test_compute_only_after_copy_only(agg, data, ref):
    ts, B = data[0], data[1]
    C = torch.full_like(ref, float("nan"))
    agg.ag_gemm_f16(ts, B, C, opts=agg.options(mode=3))       # copy only
    agg.ag_gemm_f16(ts, B, C, opts=agg.options(mode=1))       # compute only
    assert agg.check() == 0
    assert torch.equal(C, ref)


def test_repeated_calls_reuse_counters(agg, data, ref):
    # counters are never reset between calls: each call waits for base + n
    for i in range(20):
        C = call(agg, data, [0, 7, 64][i % 3])
        assert torch.equal(C, ref)


def test_nan_poisoned_caller_workspace(agg, data, ref):
    ts, B = data[0], data[1]
    M, K = ts[0].shape[0] * len(ts), ts[0].shape[1]
    nbytes = agg.workspace_bytes(len(ts), M, K, 2)
    ws = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
    for it in range(3):
        ws.fill_(float("nan"))                 # slots hold NaN until released
        agg.workspace_reset(ws)
        C = torch.full_like(ref, float("nan"))
        agg.ag_gemm_f16(ts, B, C, 8, opts=agg.options(workspace=ws, link_gbps=100.0))
        assert agg.check() == 0
        assert torch.equal(C, ref), f"iteration {it}"


def test_unregistered_workspace_rejected(agg, data):
    ts, B = data[0], data[1]
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    C = torch.empty((ts[0].shape[0] * len(ts), B.shape[1]), device="cuda")
    with pytest.raises(agg.AggError) as e:
        agg.ag_gemm_f16(ts, B, C, opts=agg.options(workspace=ws))
    assert e.value.status == agg.AGG_E_INVALID


def test_withheld_chunk_times_out_then_recovers(agg, data, ref):
    ts, B = data[0], data[1]
    C = torch.zeros_like(ref)
    agg.ag_gemm_f16(ts, B, C, opts=agg.options(debug_drop_chunk=5, timeout_ms=50.0))
    assert agg.check() == agg.AGG_E_TIMEOUT
    # the next call starts from re-armed counters and is exact again
    assert torch.equal(call(agg, data), ref)


def test_i8_invariant_across_schedules(agg, orc):
    shards, Bn, bias, scale = synth.make_i8(3 * 256, 512, 256, 3, 51000)
    ts = [dev(s, torch) for s in shards]
    B, tb, tsc = dev(Bn, torch), dev(bias, torch), dev(scale, torch)
    outs = []
    for kw, cr in [(dict(), 0), (dict(local_shard=1, send_order=[0, 2]), 5),
                   (dict(link_model=1, link_gbps=30.0), 64), (dict(mode=2), 3)]:
        C = torch.empty((768, 256), dtype=torch.float16, device="cuda")
        agg.ag_gemm_i8_dequant(ts, B, tb, tsc, C, cr, opts=agg.options(**kw))
        assert agg.check() == 0
        outs.append(C)
    # copy only, then compute only on the rows it left in the workspace
    C = torch.full((768, 256), float("nan"), dtype=torch.float16, device="cuda")
    agg.ag_gemm_i8_dequant(ts, B, tb, tsc, C, 0, opts=agg.options(mode=3))
    agg.ag_gemm_i8_dequant(ts, B, tb, tsc, C, 0, opts=agg.options(mode=1))
    assert agg.check() == 0
    outs.append(C)
    for C in outs[1:]:
        assert torch.equal(C, outs[0])


def test_bf16_invariant_across_schedules(agg):
    """The bf16 path shares the schedule machinery: its output is also
    bitwise independent of chunking, local shard, link pacing and mode."""
    shards, Bn = synth.make_bf16(4 * 256, 512, 384, 4, "normal", 52000)

    def bdev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    ts = [bdev(s) for s in shards]
    B = bdev(Bn)
    outs = []
    for kw, cr in [(dict(), 0), (dict(local_shard=2, send_order=[0, 3, 1]), 5),
                   (dict(link_model=1, link_gbps=40.0), 64), (dict(mode=2), 3)]:
        C = torch.full((1024, 384), float("nan"), device="cuda")
        agg.ag_gemm_bf16(ts, B, C, cr, opts=agg.options(**kw))
        assert agg.check() == 0
        outs.append(C)
    for C in outs[1:]:
        assert torch.equal(C, outs[0])


def test_fp8_invariant_across_schedules(agg):
    """The fp8 path: bitwise the same output whatever the chunking, local
    shard, link pacing and mode."""
    shards, Bn = synth.make_fp8(4 * 256, 512, 384, 4, "normal", 53000)
    ts = [torch.from_numpy(s).cuda() for s in shards]
    B = torch.from_numpy(Bn).cuda()
    outs = []
    for kw, cr in [(dict(), 0), (dict(local_shard=3, send_order=[2, 0, 1]), 5),
                   (dict(link_model=1, link_gbps=40.0), 64), (dict(mode=2), 3)]:
        C = torch.full((1024, 384), float("nan"), device="cuda")
        agg.ag_gemm_fp8(ts, B, C, cr, opts=agg.options(**kw))
        assert agg.check() == 0
        outs.append(C)
    for C in outs[1:]:
        assert torch.equal(C, outs[0])


@pytest.mark.parametrize("kw", [dict(scheme=1), dict(scheme=1, pvalue=2),
                                dict(scheme=1, pvalue=2, workspace_stages=2),
                                dict(scheme=1, link_gbps=150.0)])
def test_barrier_scheme_gives_the_same_bits(agg, kw):
    """The barrier scheme changes only when tiles wait and in what order
    they run, so its output is bitwise that of the counter scheme."""
    shards, Bn = synth.make_f16(4 * 1024, 1024, 512, 4, "normal", 54000)
    ts = [dev(s, torch) for s in shards]
    B = dev(Bn, torch)
    ref = torch.full((4096, 512), float("nan"), device="cuda")
    agg.ag_gemm_f16(ts, B, ref, 0)
    assert agg.check() == 0
    C = torch.full((4096, 512), float("nan"), device="cuda")
    agg.ag_gemm_f16(ts, B, C, 0, opts=agg.options(**kw))
    assert agg.check() == 0
    assert torch.equal(C, ref)


def test_k_blocks_nan_poisoned_workspace(agg, data, ref):
    """K-blocks on a paced link over a workspace whose slots hold NaN until
    each chunk is released: a tile that read a K-block early would carry
    a NaN into C."""
    ts, B = data[0], data[1]
    M, K = ts[0].shape[0] * len(ts), ts[0].shape[1]
    ws = torch.empty(agg.workspace_bytes(len(ts), M, K, 2) // 2, dtype=torch.float16,
                     device="cuda")
    for it, cr in enumerate((8, 64, 1)):
        ws.fill_(float("nan"))
        agg.workspace_reset(ws)
        C = torch.full_like(ref, float("nan"))
        agg.ag_gemm_f16(ts, B, C, cr, opts=agg.options(workspace=ws, link_gbps=60.0,
                                                       k_block=512))
        assert agg.check() == 0
        assert torch.equal(C, ref), f"iteration {it}"


def test_k_blocks_withheld_chunk_times_out_inside_a_tile(agg, data, ref):
    """A chunk of K-block 1 is never released: tiles pass their first wait
    (K-block 0 is in) and time out inside their K loop; the call reports
    the time-out and the next call is exact again."""
    ts, B = data[0], data[1]
    info, _, chunks = agg.plan("f16", len(ts), ts[0].shape[0] * len(ts), ts[0].shape[1],
                               B.shape[1], 8, agg.options(k_block=512), orders=True)
    R = info.chunks_per_source // info.k_blocks
    drop = 3 * R + 5                     # K-block 1 (positions 3R.. on 3 sources)
    assert chunks[drop, 1] // R == 1
    C = torch.zeros_like(ref)
    agg.ag_gemm_f16(ts, B, C, 8, opts=agg.options(k_block=512, debug_drop_chunk=drop,
                                                  timeout_ms=50.0))
    assert agg.check() == agg.AGG_E_TIMEOUT
    assert torch.equal(call(agg, data, 8, k_block=512), ref)
    assert torch.equal(call(agg, data), ref)


@pytest.mark.parametrize("kw", [dict(), dict(link_gbps=40.0), dict(k_block=512),
                                dict(k_block=512, link_gbps=40.0),
                                dict(k_block=512, chunk_rows=1), dict(mode=2)])
def test_alternating_contents_on_one_workspace(agg, orc, data, ref, kw):
    """Two different sets of shards, in turn, through one caller-owned
    workspace: each call must give its own data's result.  The rows of
    consecutive calls sit at the same workspace addresses, so a cache line
    left over from the previous call would show here (with the same data in
    every call it could not)."""
    ts, B = data[0], data[1]
    shards2, _ = synth.make_f16(4 * 512, 1024, 768, 4, "normal", 50500)
    ts2 = [dev(s, torch) for s in shards2]
    C2 = torch.full_like(ref, float("nan"))
    agg.ag_gemm_f16(ts2, B, C2, 0)
    assert agg.check() == 0
    Co, So = orc.ag_gemm_f16(shards2, data[3])
    check_f16(C2.cpu().numpy(), Co, So, "second data set")
    M, K = ts[0].shape[0] * len(ts), ts[0].shape[1]
    ws = torch.empty(agg.workspace_bytes(len(ts), M, K, 2), dtype=torch.uint8, device="cuda")
    agg.workspace_reset(ws)
    kw = dict(kw)
    cr = kw.pop("chunk_rows", 0)
    for it in range(10):
        src, want = (ts, ref) if it % 2 == 0 else (ts2, C2)
        C = torch.full_like(ref, float("nan"))
        agg.ag_gemm_f16(src, B, C, cr, opts=agg.options(workspace=ws, **kw))
        assert agg.check() == 0
        assert torch.equal(C, want), f"call {it} {kw}"


@pytest.mark.parametrize("kw", [
    dict(debug_delay_us=30.0, debug_delay_seed=1),
    dict(debug_delay_us=30.0, debug_delay_seed=2, chunk_rows=1),
    dict(debug_delay_us=20.0, debug_delay_seed=3, producer_piece_bytes=8192, chunk_rows=64),
    dict(debug_delay_us=30.0, debug_delay_seed=4, k_block=512, chunk_rows=8),
    dict(debug_delay_us=30.0, debug_delay_seed=5, k_block=512, link_gbps=40.0),
    dict(debug_delay_us=30.0, debug_delay_seed=6, link_model=1, chunk_rows=16),
    dict(debug_delay_us=10.0, debug_delay_seed=7, workspace_stages=2, chunk_rows=8),
])
def test_random_completion_order(agg, data, ref, kw):
    """Seeded random delays before every producer piece: pieces and chunks
    complete in an order unrelated to the send order (the flag walk and the
    counter must still release exactly the chunks whose pieces are all in).
    The output stays bitwise the same."""
    kw = dict(kw)
    cr = kw.pop("chunk_rows", 0)
    for rep in range(2):
        C = call(agg, data, cr, **dict(kw, debug_delay_seed=kw["debug_delay_seed"] + 100 * rep))
        assert torch.equal(C, ref), (kw, rep)


def test_random_completion_order_nan_poisoned(agg, data, ref):
    ts, B = data[0], data[1]
    M, K = ts[0].shape[0] * len(ts), ts[0].shape[1]
    ws = torch.empty(agg.workspace_bytes(len(ts), M, K, 2) // 2, dtype=torch.float16,
                     device="cuda")
    for it in range(4):
        ws.fill_(float("nan"))
        agg.workspace_reset(ws)
        C = torch.full_like(ref, float("nan"))
        agg.ag_gemm_f16(ts, B, C, [1, 8, 0, 8][it], opts=agg.options(
            workspace=ws, debug_delay_us=25.0, debug_delay_seed=40 + it,
            k_block=[0, 512, 0, 512][it]))
        assert agg.check() == 0
        assert torch.equal(C, ref), f"iteration {it}"


# ---- producer options --------------------------------------------------

@pytest.mark.parametrize("kw", [
    dict(producer=1), dict(producer=1, chunk_rows=1), dict(producer=1, chunk_rows=100),
    dict(producer=1, local_shard=2, send_order=[3, 0, 1]), dict(producer=1, link_model=1),
    dict(producer=1, mode=2), dict(producer=1, scheme=1), dict(producer=1, scheme=1, pvalue=2),
    dict(producer_cus=32), dict(producer_cus=64),
    dict(producer_cus=32, k_block=512), dict(producer_cus=64, link_gbps=40.0),
    dict(producer_cus=32, workspace_stages=2, chunk_rows=8),
    dict(producer_cus=64, workspace_stages=2, chunk_rows=8),
    dict(producer_cus=32, mode=2),
])
def test_producer_options_give_the_same_bits(agg, data, ref, kw):
    """The DMA producer and a CU-masked producer change only what moves the
    rows and where the kernels run: the output is bitwise the same."""
    kw = dict(kw)
    cr = kw.pop("chunk_rows", 0)
    for rep in range(2):
        C = call(agg, data, cr, **kw)
        assert torch.equal(C, ref), (kw, rep)


def test_sdma_copy_then_compute(agg, data, ref):
    ts, B = data[0], data[1]
    C = torch.full_like(ref, float("nan"))
    agg.ag_gemm_f16(ts, B, C, opts=agg.options(mode=3, producer=1))
    agg.ag_gemm_f16(ts, B, C, opts=agg.options(mode=1))
    assert agg.check() == 0
    assert torch.equal(C, ref)


@pytest.mark.parametrize("kw", [dict(producer=1), dict(producer_cus=32),
                                dict(producer_cus=64, k_block=512)])
def test_producer_options_alternating_and_poisoned(agg, orc, data, ref, kw):
    """Two data sets in turn through one workspace, NaN-filled before every
    other call: each call gives its own data's result."""
    ts, B = data[0], data[1]
    shards2, _ = synth.make_f16(4 * 512, 1024, 768, 4, "normal", 50600)
    ts2 = [dev(s, torch) for s in shards2]
    C2 = torch.full_like(ref, float("nan"))
    agg.ag_gemm_f16(ts2, B, C2, 0)
    assert agg.check() == 0
    M, K = ts[0].shape[0] * len(ts), ts[0].shape[1]
    ws = torch.empty(agg.workspace_bytes(len(ts), M, K, 2) // 2, dtype=torch.float16,
                     device="cuda")
    for it in range(8):
        if it % 2 == 0:
            ws.fill_(float("nan"))
            agg.workspace_reset(ws)
        src, want = (ts, ref) if it % 2 == 0 else (ts2, C2)
        C = torch.full_like(ref, float("nan"))
        agg.ag_gemm_f16(src, B, C, 0, opts=agg.options(workspace=ws, **kw))
        assert agg.check() == 0
        assert torch.equal(C, want), f"call {it} {kw}"
