"""The optional device trace: chunk releases and consumer tile phases, in
100 MHz device ticks.  Besides the bookkeeping, it checks the release
protocol itself on a paced run (PTO-ISA AllGather+GEMM README, two-stream
pipeline: the compute side starts a remote tile only after the counter
covers its rows): every remote tile starts computing after the release of
the last chunk it needs, and the pacing really spreads the releases."""
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


def test_trace_orders_releases_before_dependent_tiles(agg):
    n, S, K, N, cr, gbps = 4, 1024, 1024, 512, 32, 20.0
    M = n * S
    shards, B = synth.make_f16(M, K, N, n, "normal", 60000)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    opts = dict(link_gbps=gbps)
    info, tiles, chunks = agg.plan("f16", n, M, K, N, cr, agg.options(**opts), orders=True)
    assert info.trace_words == 1 + info.total_chunks + 3 * info.total_tiles
    trace = torch.zeros(info.trace_words, dtype=torch.int64, device="cuda")
    C = torch.empty((M, N), device="cuda")
    agg.ag_gemm_f16(ts, tB, C, cr, opts=agg.options(trace=trace, **opts))
    assert agg.check() == 0
    ref = torch.empty_like(C)
    agg.ag_gemm_f16(ts, tB, ref, cr, opts=agg.options(**opts))
    assert agg.check() == 0
    assert torch.equal(C, ref)                 # tracing changes nothing computed

    tr = trace.cpu().numpy().view(np.uint64).astype(np.float64)
    nc = info.total_chunks
    start, rel, cons = tr[0], tr[1:1 + nc], tr[1 + nc:].reshape(-1, 3)
    assert start > 0 and (rel > 0).all() and (cons > 0).all()
    assert (cons[:, 0] <= cons[:, 1]).all() and (cons[:, 1] <= cons[:, 2]).all()
    pos = {(int(s), int(j)): i for i, (s, j) in enumerate(chunks)}
    waited = 0
    for p, (shard, m, nn, need) in enumerate(tiles):
        if need > 0:
            r = rel[pos[(int(shard), int(need) - 1)]]
            assert cons[p, 1] >= r, (p, shard, m, need)
            waited += cons[p, 1] > cons[p, 0]
    assert waited > 0
    # a source's S x K fp16 rows cannot cross a 20 GB/s link in less than
    # this; the consumer starts before the producer
    pace_ticks = S * K * 2 / (gbps * 1e9) * 1e8
    assert rel.max() - start >= 0.9 * pace_ticks


def test_trace_k_blocks_gate_every_block(agg):
    """Chunks of rows x one K-block (k_block): a remote tile starts after
    its rows of the first K-block are released and cannot end before its
    rows of the last K-block are; on a paced link the tile waits inside
    its K loop.  The output is bitwise that of whole-K chunks."""
    n, S, K, N, cr, gbps, kbk = 4, 512, 2048, 512, 32, 20.0, 512
    M = n * S
    shards, B = synth.make_f16(M, K, N, n, "normal", 60010)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    opts = dict(link_gbps=gbps, k_block=kbk)
    info, tiles, chunks = agg.plan("f16", n, M, K, N, cr, agg.options(**opts), orders=True)
    R, nkb = S // cr, K // kbk
    assert info.k_blocks == nkb and info.chunks_per_source == R * nkb
    trace = torch.zeros(info.trace_words, dtype=torch.int64, device="cuda")
    C = torch.empty((M, N), device="cuda")
    agg.ag_gemm_f16(ts, tB, C, cr, opts=agg.options(trace=trace, **opts))
    assert agg.check() == 0
    ref = torch.empty_like(C)
    agg.ag_gemm_f16(ts, tB, ref, cr)
    assert agg.check() == 0
    assert torch.equal(C, ref)

    tr = trace.cpu().numpy().view(np.uint64).astype(np.float64)
    nc = info.total_chunks
    start, rel, cons = tr[0], tr[1:1 + nc], tr[1 + nc:].reshape(-1, 3)
    assert (rel > 0).all() and (cons > 0).all()
    pos = {(int(s), int(j)): i for i, (s, j) in enumerate(chunks)}
    # a source's releases come K-block after K-block
    for sh in range(1, n):
        order = [int(j) for s_, j in chunks if s_ == sh]
        assert order == sorted(order, key=lambda j: (j // R, j % R))
    late = 0
    for p, (shard, m, nn, need) in enumerate(tiles):
        if need > 0:
            assert need <= R
            first = rel[pos[(int(shard), int(need) - 1)]]
            last = rel[pos[(int(shard), (nkb - 1) * R + int(need) - 1)]]
            assert cons[p, 1] >= first, (p, shard, m)
            assert cons[p, 2] >= last, (p, shard, m)
            # the tile began computing before its last K-block was there
            late += cons[p, 1] < last
    assert late > 0


def test_trace_buffer_must_hold_the_calls_plan(agg):
    """The library writes the plan's trace_words through a bare pointer, so
    the binding refuses a trace tensor that is too small for the call it is
    given to -- here one sized for whole-K chunks while the call's automatic
    plan cuts K into eight blocks -- before anything runs; with the call's
    own plan's size the trace is whole."""
    n, S, K, N = 4, 1024, 4096, 512
    M = n * S
    shards, B = synth.make_f16(M, K, N, n, "normal", 60020)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    auto = agg.plan("f16", n, M, K, N, 0, agg.options(link_gbps=153.0))[0]
    whole = agg.plan("f16", n, M, K, N, 64, agg.options(link_gbps=153.0))[0]
    assert auto.k_blocks == 8 and whole.k_blocks == 1
    assert auto.trace_words > whole.trace_words
    C = torch.full((M, N), float("nan"), device="cuda")
    for words in (whole.trace_words, auto.trace_words - 1):
        small = torch.zeros(words, dtype=torch.int64, device="cuda")
        with pytest.raises(ValueError):
            agg.ag_gemm_f16(ts, tB, C, 0, opts=agg.options(trace=small, link_gbps=153.0))
    assert torch.isnan(C).all()                  # nothing ran
    trace = torch.zeros(auto.trace_words + 1, dtype=torch.int64, device="cuda")
    agg.ag_gemm_f16(ts, tB, C, 0, opts=agg.options(trace=trace, link_gbps=153.0))
    assert agg.check() == 0
    tr = trace.cpu().numpy()
    assert (tr[:auto.trace_words] > 0).all() and tr[auto.trace_words] == 0


def test_paced_piece_flags_keep_the_pace(agg):
    """A paced call on 256 x 256 tiles, whose waits take piece-flagged
    chunks: no remote tile gets past its first wait before the emulated
    link could have carried the rows it needs (the source's bytes up to
    and including its K-block 0 chunk of the panel's last row group),
    counted from the consumer's start -- the pacing origin is the first
    producer workgroup's start, no earlier -- and the result is exact."""
    n, S, K, N, gbps = 4, 1024, 4096, 512, 20.0
    M = n * S
    shards, B = synth.make_f16(M, K, N, n, "normal", 60030)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    opts = dict(link_gbps=gbps, tile=15)
    info, tiles, chunks = agg.plan("f16", n, M, K, N, 0, agg.options(**opts), orders=True)
    assert info.k_blocks == 8 and info.tile_id == 15
    trace = torch.zeros(info.trace_words, dtype=torch.int64, device="cuda")
    C = torch.empty((M, N), device="cuda")
    agg.ag_gemm_f16(ts, tB, C, 0, opts=agg.options(trace=trace, **opts))
    assert agg.check() == 0
    ref = torch.empty_like(C)
    agg.ag_gemm_f16(ts, tB, ref, 64)           # whole-K chunks, no piece flags
    assert agg.check() == 0
    assert torch.equal(C, ref)
    tr = trace.cpu().numpy().view(np.uint64).astype(np.float64)
    start, cons = tr[0], tr[1 + info.total_chunks:].reshape(-1, 3)
    cr, kbk = info.chunk_rows, info.k_block
    remote = 0
    for p, (shard, m, nn, need) in enumerate(tiles):
        if need <= 0:
            continue
        remote += 1
        row_end = min(int(need) * cr, S)       # the panel's last row group, K-block 0
        paced_s = row_end * kbk * 2 / (gbps * 1e9)
        assert (cons[p, 1] - start) / 1e8 >= paced_s, (p, shard, m, paced_s)
    assert remote > 0
