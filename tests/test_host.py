"""Host-side checks of the C-ABI library: it loads, exports what the header
declares, plans the shared schedule correctly and rejects bad arguments
before touching the GPU.  No kernel runs here.

Schedule properties follow the PTO-ISA AllGather+GEMM README ("optimisation
notes"): the local row-group first with no wait, remote chunks sent in the
order they are consumed, 64-128 chunks per source, per-source monotonic
counters.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import communication_gemm_amd as agg
from communication_gemm_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "aggemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ag_gemm_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(_native.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_native.EXPORTS), "binding and header disagree"


def test_options_struct_matches_header_defaults():
    o = agg.options()
    assert o.struct_size == ctypes.sizeof(_native.Options)
    assert o.local_shard == 0 and o.mode == agg.MODE_PIPELINED
    assert o.debug_drop_chunk == -1 and o.link_gbps == 0.0


def test_status_strings():
    for s in range(6):
        assert agg.status_string(s)
    assert "timed out" in agg.status_string(agg.AGG_E_TIMEOUT)


def test_pick_chunk_rows_exhaustive():
    S = np.arange(1, 65537)
    cr = np.array([agg.pick_chunk_rows(int(s)) for s in S])
    assert (cr >= 1).all()
    nchunks = -(-S // cr)
    assert ((nchunks >= 64) & (nchunks <= 128))[S >= 64].all()
    assert (cr[S < 64] == 1).all()
    # chunks tile the shard exactly: the last one is non-empty
    last = S - (nchunks - 1) * cr
    assert ((last >= 1) & (last <= cr)).all()
    assert agg.pick_chunk_rows(0) == 0


def test_workspace_bytes():
    header = agg.workspace_bytes(1, 100, 64, 2)           # one shard: no slots
    assert header >= 16384 + 64 * 1024 * 4                 # counters + chunk flags
    assert agg.workspace_bytes(8, 8192, 4096, 2) == header + 7 * 1024 * 4096 * 2
    assert agg.workspace_bytes(3, 100, 64, 2) == 0        # M % n != 0
    assert agg.workspace_bytes(2, 2, 8, 1) == header + 256  # slots rounded to 256 B


def test_too_many_chunks_per_source_rejected():
    # the chunk flag matrix holds 1024 chunks per source
    agg.plan("f16", 2, 2 * 1024, 64, 64, 1)
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 2, 2 * 1025, 64, 64, 1)
    assert e.value.status == agg.AGG_E_UNSUPPORTED


def _check_schedule(n, M, K, N, cr=0, **kw):
    opts = agg.options(**kw)
    info, tiles, chunks = agg.plan("f16", n, M, K, N, cr, opts, orders=True)
    S = M // n
    local = kw.get("local_shard", 0)
    order = kw.get("send_order") or [(local + q) % n for q in range(1, n)]
    L = info.m_tiles_per_shard * info.n_tiles
    # every output tile exactly once
    keys = {tuple(t[:3]) for t in tiles}
    assert len(keys) == len(tiles) == n * L
    # local tiles first, never waited on
    assert (tiles[:L, 0] == local).all() and (tiles[:L, 3] == 0).all()
    assert (tiles[L:, 0] != local).all() and (tiles[L:, 3] > 0).all()
    # a remote tile waits for the chunk holding its last row
    for sh, m, _, need in tiles[L:]:
        last_row = min((m + 1) * info.tile_m, S)
        assert need == -(-last_row // info.chunk_rows)
    # every remote chunk sent exactly once, in chunk order within a source
    assert len({tuple(c) for c in chunks}) == len(chunks) == (n - 1) * info.chunks_per_source
    for s in order:
        js = chunks[chunks[:, 0] == s, 1]
        assert (np.diff(js) == 1).all() and js[0] == 0
    # send order = consumption order: the producer position by which a
    # remote tile's data is complete never decreases along the tile list
    pos = {tuple(c): i for i, c in enumerate(chunks)}
    ready = [pos[(sh, need - 1)] for sh, _, _, need in tiles[L:]]
    assert all(a <= b for a, b in zip(ready, ready[1:]))
    return info, tiles, chunks


@pytest.mark.parametrize("n,M,K,N,cr", [
    (2, 256, 256, 128, 32), (2, 2048, 2048, 1024, 0), (4, 4096, 4096, 4096, 0),
    (8, 8192, 4096, 4096, 0), (3, 300, 296, 168, 7), (5, 5 * 1000, 64, 8, 0),
    (1, 64, 64, 64, 0)])
def test_schedule_parallel_links(n, M, K, N, cr):
    if n == 1:
        info, tiles, chunks = agg.plan("f16", n, M, K, N, cr, orders=True)
        assert info.total_chunks == 0 and (tiles[:, 3] == 0).all()
        return
    _check_schedule(n, M, K, N, cr)


def test_schedule_serial_link_is_source_major():
    info, tiles, chunks = _check_schedule(4, 4096, 4096, 4096, 0,
                                          link_model=agg.LINKS_SERIAL, send_order=[3, 1, 2])
    L = info.m_tiles_per_shard * info.n_tiles
    srcs = tiles[L:, 0]
    assert list(dict.fromkeys(srcs.tolist())) == [3, 1, 2]
    assert list(dict.fromkeys(chunks[:, 0].tolist())) == [3, 1, 2]
    assert (np.diff(srcs) != 0).sum() == 2


def test_schedule_parallel_links_go_m_tile_by_m_tile():
    info, tiles, _ = _check_schedule(4, 4096, 4096, 4096, 0, local_shard=2)
    L = info.m_tiles_per_shard * info.n_tiles
    assert (np.diff(tiles[L:, 1]) >= 0).all()          # m-tiles never go back
    first = tiles[L:L + 3 * info.n_tiles]
    assert list(dict.fromkeys(first[:, 0].tolist())) == [3, 0, 1]


def test_schedule_chunk_larger_than_tile():
    # chunks of 100 rows, tiles of 64 rows: several tiles per chunk
    _check_schedule(2, 800, 64, 64, 100, tile=3)


@pytest.mark.parametrize("kw,status", [
    (dict(local_shard=4), agg.AGG_E_INVALID),
    (dict(local_shard=-1), agg.AGG_E_INVALID),
    (dict(send_order=[1, 1, 2]), agg.AGG_E_INVALID),
    (dict(send_order=[0, 1, 2]), agg.AGG_E_INVALID),     # contains the local shard
    (dict(send_order=[1, 2, 7]), agg.AGG_E_INVALID),
    (dict(mode=9), agg.AGG_E_INVALID),
    (dict(link_model=3), agg.AGG_E_INVALID),
    (dict(link_gbps=-1.0), agg.AGG_E_INVALID),
    (dict(tile=99), agg.AGG_E_INVALID),
    (dict(producer_piece_bytes=-8192), agg.AGG_E_INVALID),
    (dict(producer_piece_bytes=1000), agg.AGG_E_INVALID),      # not whole sweeps
    (dict(producer_piece_bytes=8192 + 16), agg.AGG_E_INVALID),
])
def test_plan_rejects_bad_options(kw, status):
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 4, 1024, 64, 64, 0, agg.options(**kw))
    assert e.value.status == status


@pytest.mark.parametrize("kind,n,M,K,N,cr,status", [
    ("f16", 0, 64, 64, 64, 0, agg.AGG_E_INVALID),
    ("f16", 65, 65, 64, 64, 0, agg.AGG_E_UNSUPPORTED),
    ("f16", 3, 100, 64, 64, 0, agg.AGG_E_INVALID),        # M % n
    ("f16", 2, 64, 60, 64, 0, agg.AGG_E_UNSUPPORTED),     # K % 8
    ("f16", 2, 64, 64, 60, 0, agg.AGG_E_UNSUPPORTED),     # N % 8
    ("i8", 2, 64, 72, 64, 0, agg.AGG_E_UNSUPPORTED),      # K % 16
    ("f16", 2, 64, 64, 64, 33, agg.AGG_E_INVALID),        # chunk > S
    ("f16", 2, 64, 64, 64, -1, agg.AGG_E_INVALID),
    ("f16", 2, -64, 64, 64, 0, agg.AGG_E_INVALID),
    ("f16", 2, 64, (1 << 21) + 8, 64, 0, agg.AGG_E_UNSUPPORTED),   # K limit
    ("f16", 2, 64, 64, (1 << 20) + 8, 0, agg.AGG_E_UNSUPPORTED),   # N limit
    ("i8", 2, 64, 64, (1 << 20) + 8, 0, agg.AGG_E_UNSUPPORTED),
    ("fp8", 2, 64, 72, 64, 0, agg.AGG_E_UNSUPPORTED),     # K % 16
    ("fp8", 2, 64, 64, 60, 0, agg.AGG_E_UNSUPPORTED),     # N % 8
])
def test_plan_rejects_bad_sizes(kind, n, M, K, N, cr, status):
    with pytest.raises(agg.AggError) as e:
        agg.plan(kind, n, M, K, N, cr)
    assert e.value.status == status


# ---- the real entry points return argument errors before any HIP call ----

FAKE = 0x10000   # a 16-byte aligned address that is never dereferenced


def _f16(table, n, B, C, M, K, N, cr=0, opts=None):
    t = (ctypes.c_void_p * max(n, 1))(*table) if table is not None else None
    if opts is None:
        return _native.lib.ag_gemm_f16(t, n, B, C, M, K, N, cr, None)
    return _native.lib.ag_gemm_f16_ex(t, n, B, C, M, K, N, cr, None, ctypes.byref(opts))


def test_entry_point_argument_errors():
    lib = _native.lib
    assert _f16(None, 2, FAKE, FAKE, 64, 64, 64) == agg.AGG_E_INVALID
    assert _f16([FAKE, 0], 2, FAKE, FAKE, 64, 64, 64) == agg.AGG_E_INVALID
    assert _f16([FAKE, FAKE + 8], 2, FAKE, FAKE, 64, 64, 64) == agg.AGG_E_UNSUPPORTED
    assert _f16([FAKE, FAKE], 2, FAKE + 2, FAKE, 64, 64, 64) == agg.AGG_E_UNSUPPORTED
    assert _f16([FAKE, FAKE], 2, FAKE, 0, 64, 64, 64) == agg.AGG_E_INVALID
    assert _f16([FAKE, FAKE], 2, FAKE, FAKE, 63, 64, 64) == agg.AGG_E_INVALID
    assert _f16([FAKE, FAKE], 2, FAKE, FAKE, 64, 12, 64) == agg.AGG_E_UNSUPPORTED
    assert _f16([FAKE, FAKE], 2, FAKE, FAKE, 64, 64, 64, 40) == agg.AGG_E_INVALID
    bad = agg.options(send_order=[0])
    assert _f16([FAKE, FAKE], 2, FAKE, FAKE, 64, 64, 64, 0, bad) == agg.AGG_E_INVALID
    short = agg.options()
    short.struct_size = 8
    assert _f16([FAKE, FAKE], 2, FAKE, FAKE, 64, 64, 64, 0, short) == agg.AGG_E_INVALID
    t = (ctypes.c_void_p * 2)(FAKE, FAKE)
    # int8: bias and scale are required
    assert lib.ag_gemm_i8_dequant(t, 2, FAKE, None, FAKE, FAKE, 64, 64, 64, 0, None) == agg.AGG_E_INVALID
    assert lib.ag_gemm_i8_dequant(t, 2, FAKE, FAKE, FAKE + 2, FAKE, 64, 64, 64, 0, None) == agg.AGG_E_UNSUPPORTED
    # fp8: 16 elements per 16-byte load
    assert lib.ag_gemm_fp8(t, 2, FAKE, FAKE, 64, 72, 64, 0, None) == agg.AGG_E_UNSUPPORTED
    assert lib.ag_gemm_fp8(None, 2, FAKE, FAKE, 64, 64, 64, 0, None) == agg.AGG_E_INVALID
    assert lib.ag_gemm_workspace_reset(None, 1 << 20, None) == agg.AGG_E_INVALID


def test_empty_problems_are_no_ops():
    # M = 0 or N = 0: nothing to move or compute, nothing enqueued
    assert _f16([0, 0], 2, 0, 0, 0, 64, 64) == agg.AGG_OK
    assert _f16([FAKE, FAKE], 2, FAKE, 0, 64, 64, 0) == agg.AGG_OK


@pytest.mark.parametrize("kind,n,S,K,N,tile", [
    ("f16", 8, 1024, 4096, 4096, 15),    # 512 tiles of 256 x 256 (16 x 16 blocks)
    ("f16", 4, 1024, 4096, 4096, 15),    # 256 of them: one per CU
    ("bf16", 8, 1024, 4096, 4096, 15),
    ("f16", 2, 1024, 4096, 4096, 11),    # 128 x 256, eight waves
    ("bf16", 2, 1024, 4096, 4096, 11),
    ("f16", 2, 1024, 2048, 1024, 13),    # 2 x 1024 rows, N = 1024: 64 x 64
    ("i8", 2, 8192, 27392, 4096, 8),
    ("i8", 2, 32, 16384, 7168, 13),    # decode-like: 64 x 64, no split
])
def test_automatic_tile(kind, n, S, K, N, tile):
    """The automatic tile: the first of the planner's list (largest first,
    eight-wave before four-wave at equal size) that gives every one of the
    256 CUs a tile."""
    info, _, _ = agg.plan(kind, n, n * S, K, N)
    assert info.tile_id == tile


def test_split_k_plan():
    """Split-K on request: K parts of a multiple of 256, every (shard,
    m-tile, n-tile) once per part, part after part; the workspace grows by
    the partial sums.  The automatic choice does not split."""
    auto, _, _ = agg.plan("i8", 2, 64, 16384, 7168)
    assert auto.k_splits == 1
    info, tiles, _ = agg.plan("i8", 2, 64, 16384, 7168, 0, agg.options(tile=14, k_splits=4),
                              orders=True)
    assert (info.tile_id, info.tile_m, info.tile_n, info.k_splits) == (14, 32, 256, 4)
    base = 2 * 1 * 28
    assert info.total_tiles == base * 4
    plain, _, _ = agg.plan("i8", 2, 64, 16384, 7168, 0, agg.options(k_splits=1))
    assert plain.k_splits == 1 and plain.tile_id == 13
    assert info.workspace_bytes == plain.workspace_bytes + base * 4 * 32 * 256 * 4
    # every (shard, m-tile, n-tile) once per part
    keys, counts = np.unique(tiles[:, :3], axis=0, return_counts=True)
    assert len(keys) == base and (counts == 4).all()
    # part after part; inside a part, the local shard first, with no wait
    assert (tiles[:28, 0] == 0).all() and (tiles[:28, 3] == 0).all()
    assert (tiles[28:56, 0] == 1).all() and (tiles[28:56, 3] > 0).all()
    assert (tiles[56:84, 0] == 0).all()
    # parts hold multiples of 256 of K: 5000 in 3 parts -> 1792, 1792, 1416
    info, _, _ = agg.plan("f16", 2, 40, 5000, 1000, 0, agg.options(k_splits=3, tile=13))
    assert info.k_splits == 3
    info, _, _ = agg.plan("f16", 2, 40, 600, 1000, 0, agg.options(k_splits=8, tile=13))
    assert info.k_splits == 3          # ceil(600 / 256) parts of 256


@pytest.mark.parametrize("kw,status", [
    (dict(k_splits=-1), agg.AGG_E_INVALID),
    (dict(k_splits=2, tile=8), agg.AGG_E_UNSUPPORTED),      # big tiles are built without it
    (dict(k_splits=2, tile=13, scheme=agg.SCHEME_BARRIER), agg.AGG_E_UNSUPPORTED),
    (dict(k_splits=2, tile=13, workspace_stages=1), agg.AGG_E_UNSUPPORTED),
    (dict(k_splits=65, tile=13), agg.AGG_E_UNSUPPORTED),
])
def test_split_k_rejected(kw, status):
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 2, 2048, 4096, 512, 0, agg.options(**kw))
    assert e.value.status == status


def test_fp8_plans_only_tiles_built_for_it():
    """The fp8 path runs the configurations whose slices hold pairs of
    64-byte MFMA steps; the automatic choice stays among them."""
    for tile in (1, 4, 5, 7, 8, 9):
        with pytest.raises(agg.AggError) as e:
            agg.plan("fp8", 8, 8192, 4096, 4096, 0, agg.options(tile=tile))
        assert e.value.status == agg.AGG_E_INVALID
    for tile in (2, 3, 6, 10, 11, 12, 13, 15):
        info, _, _ = agg.plan("fp8", 8, 8192, 4096, 4096, 0, agg.options(tile=tile))
        assert info.tile_id == tile
    info, _, _ = agg.plan("fp8", 8, 8192, 4096, 4096)
    assert (info.tile_m, info.tile_n, info.tile_id) == (256, 256, 15)


def test_workspace_ring_plan():
    """A ring of W row panels per remote shard: the workspace shrinks to
    W x tile-height rows per remote shard; W panels covering the shard
    fall back to full slots."""
    header = agg.workspace_bytes(1, 100, 64, 2)
    full, _, _ = agg.plan("f16", 8, 8192, 4096, 4096)
    assert full.workspace_stages == 0
    assert full.workspace_bytes == agg.workspace_bytes(8, 8192, 4096, 2)
    for w in (1, 2, 3):
        info, _, _ = agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(workspace_stages=w))
        assert info.workspace_stages == w
        assert info.workspace_bytes == header + 7 * w * info.tile_m * 4096 * 2
    info, _, _ = agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(workspace_stages=4))
    assert info.workspace_stages == 0 and info.workspace_bytes == full.workspace_bytes
    c5, _, _ = agg.plan("i8", 2, 16384, 27392, 4096, 0, agg.options(workspace_stages=2))
    assert c5.workspace_bytes == header + 2 * 256 * 27392


def test_workspace_ring_chunks_stay_inside_panels():
    # automatic chunk: the largest divisor of the tile height not above S/64
    info, _, _ = agg.plan("f16", 4, 4 * 1000, 256, 200, 0,
                          agg.options(workspace_stages=2, tile=13))
    assert info.tile_m == 64 and info.chunk_rows == 8       # S/64 = 15 -> 8
    ok, _, _ = agg.plan("f16", 4, 4 * 1000, 256, 200, 16, agg.options(workspace_stages=2, tile=13))
    assert ok.chunk_rows == 16
    for cr in (24, 128):                                    # 64 % cr != 0
        with pytest.raises(agg.AggError) as e:
            agg.plan("f16", 4, 4 * 1000, 256, 200, cr, agg.options(workspace_stages=2, tile=13))
        assert e.value.status == agg.AGG_E_UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(workspace_stages=9), agg.AGG_E_INVALID),
    (dict(workspace_stages=-1), agg.AGG_E_INVALID),
    (dict(workspace_stages=2, mode=agg.MODE_SEQUENTIAL), agg.AGG_E_UNSUPPORTED),
])
def test_workspace_ring_rejects(kw, status):
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(**kw))
    assert e.value.status == status


@pytest.mark.parametrize("n,M,pv,cr", [(4, 4096, 1, 0), (4, 4096, 3, 0), (3, 300, 2, 7),
                                       (8, 8192, 2, 0), (2, 256, 1, 32)])
def test_schedule_barrier_scheme(n, M, pv, cr):
    """Iterations of pv m-tiles over every shard in shard order; every tile
    of an iteration, the local one's too, waits for the chunk holding the
    iteration's last row (on every source)."""
    K, N = 256, 512
    info, tiles, chunks = agg.plan("f16", n, M, K, N, cr, agg.options(
        scheme=agg.SCHEME_BARRIER, pvalue=pv, tile=2), orders=True)
    S = M // n
    mt, nt = info.m_tiles_per_shard, info.n_tiles
    assert len({tuple(t[:3]) for t in tiles}) == len(tiles) == n * mt * nt
    p = 0
    for i in range(-(-mt // pv)):
        ms = list(range(i * pv, min((i + 1) * pv, mt)))
        last_row = min((ms[-1] + 1) * info.tile_m, S)
        need = -(-last_row // info.chunk_rows)
        for sh in range(n):
            for m in ms:
                for nn in range(nt):
                    assert tuple(tiles[p]) == (sh, m, nn, need)
                    p += 1
    assert p == len(tiles)


def test_barrier_scheme_ring_must_hold_an_iteration():
    kw = dict(scheme=agg.SCHEME_BARRIER, pvalue=2)
    info, _, _ = agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(workspace_stages=2, **kw))
    assert info.workspace_stages == 2
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(workspace_stages=1, **kw))
    assert e.value.status == agg.AGG_E_UNSUPPORTED
    with pytest.raises(agg.AggError) as e:       # found by the liveness simulation
        agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(workspace_stages=2,
                                                            link_model=agg.LINKS_SERIAL, **kw))
    assert e.value.status == agg.AGG_E_UNSUPPORTED
    for bad in (dict(scheme=2), dict(scheme=agg.SCHEME_BARRIER, pvalue=-1)):
        with pytest.raises(agg.AggError) as e:
            agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(**bad))
        assert e.value.status == agg.AGG_E_INVALID


# ---- K-blocks (2-D chunks: row chunk x K-block) ------------------------

def test_k_block_plan():
    info, tiles, chunks = agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(k_block=512),
                                   orders=True)
    assert info.k_blocks == 8 and info.k_block == 512
    assert info.chunks_per_source == 64 * 8
    assert info.total_chunks == 7 * 512
    # K-block major: the first 7 * 64 positions are K-block 0 of every source
    R = 64
    assert (chunks[:7 * R, 1] < R).all() and (chunks[7 * R:14 * R, 1] // R == 1).all()
    # inside a K-block, m-tile group by group across sources, as without
    # K-blocks: the first 16 row chunks of each of the 7 sources, then the next
    one, _, c1 = agg.plan("f16", 8, 8192, 4096, 4096, 16, None, orders=True)
    assert one.k_blocks == 1 and one.chunk_rows == 16
    assert (chunks[:7 * R] == c1).all()
    # the tile order (and each tile's first wait) is unchanged
    _, t1, _ = agg.plan("f16", 8, 8192, 4096, 4096, 16, None, orders=True)
    assert (tiles == t1).all()


def test_k_block_last_block_takes_the_remainder():
    info, _, _ = agg.plan("f16", 2, 256, 2560, 128, 32, agg.options(k_block=1024))
    assert info.k_blocks == 2 and info.k_block == 1024
    info, _, _ = agg.plan("fp8", 2, 256, 3072, 128, 32, agg.options(k_block=1024))
    assert info.k_blocks == 3
    # a K-block of all of K (or more) is a chunk of all of K
    for kb in (4096, 8192, 0):
        info, _, _ = agg.plan("f16", 2, 256, 4096, 128, 32, agg.options(k_block=kb))
        assert info.k_blocks == 1 and info.k_block == 4096


@pytest.mark.parametrize("kind,K,kw,status", [
    ("f16", 4096, dict(k_block=-512), agg.AGG_E_INVALID),
    ("f16", 4096, dict(k_block=256), agg.AGG_E_UNSUPPORTED),       # not whole KiB
    ("f16", 4096, dict(k_block=768), agg.AGG_E_UNSUPPORTED),
    ("f16", 4104, dict(k_block=512), agg.AGG_E_UNSUPPORTED),       # K not whole KiB
    ("i8", 27392, dict(k_block=2048), agg.AGG_E_UNSUPPORTED),      # C5's K
    ("i8", 4096, dict(k_block=512), agg.AGG_E_UNSUPPORTED),        # int8: KiB = 1024
    ("f16", 4096, dict(k_block=512, workspace_stages=2), agg.AGG_E_UNSUPPORTED),
    ("f16", 4096, dict(k_block=512, scheme=1), agg.AGG_E_UNSUPPORTED),
])
def test_k_block_rejected(kind, K, kw, status):
    with pytest.raises(agg.AggError) as e:
        agg.plan(kind, 2, 2048, K, 256, 0, agg.options(**kw))
    assert e.value.status == status


def test_k_block_chunk_cap_and_split_k():
    # 1024 row chunks x 2 K-blocks: past the 1024 chunks a source may have
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 2, 2048, 1024, 256, 1, agg.options(k_block=512))
    assert e.value.status == agg.AGG_E_UNSUPPORTED
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 2, 128, 4096, 7168, 0, agg.options(k_block=512, k_splits=2, tile=13))
    assert e.value.status == agg.AGG_E_UNSUPPORTED


@pytest.mark.parametrize("kind,n,M,K,N,opts,cr,nkb", [
    ("f16", 8, 8192, 4096, 4096, {}, 64, 8),          # 3+ remote sources: S/16 rows x K/8
    ("f16", 4, 4096, 4096, 4096, {}, 64, 8),
    ("f16", 2, 2048, 2048, 1024, {}, 64, 4),          # S/16 rows x K/4
    ("f16", 8, 8192, 4096, 4096, {"mode": 2}, 64, 4),  # sequential: K/4
    ("bf16", 8, 8192, 4096, 4096, {}, 64, 8),
    ("fp8", 8, 8192, 4096, 4096, {}, 64, 4),          # int8/fp8: K/8 not whole KiB
    ("i8", 2, 16384, 27392, 4096, {}, 128, 1),        # K not a multiple of 4 KiB
    ("f16", 2, 256, 256, 128, {}, 2, 1),              # K too small: S/64 rows
    ("f16", 8, 8192, 4096, 4096, {"workspace_stages": 2}, 16, 1),
    ("f16", 8, 8192, 4096, 4096, {"scheme": 1}, 16, 1),
    ("f16", 8, 8192, 4096, 4096, {"k_block": 4096}, 16, 1),   # explicitly whole K
    ("f16", 4, 4096, 4096, 4096, {"link_gbps": 153.0}, 64, 8),  # paced: K/8
    ("f16", 4, 4096, 4096, 4096, {"link_gbps": 153.0, "link_model": 1}, 64, 8),
    ("f16", 2, 2048, 4096, 4096, {"link_gbps": 153.0}, 64, 4),  # one remote source
    ("f16", 4, 4096, 2048, 1024, {"link_gbps": 153.0}, 64, 4),  # K/8 not whole KiB
    ("f16", 4, 4096, 6144, 4096, {"link_gbps": 153.0}, 64, 4),
    ("f16", 4, 4096, 4096, 4096, {"link_gbps": 153.0, "mode": 2}, 64, 4),  # sequential
])
def test_automatic_chunks(kind, n, M, K, N, opts, cr, nkb):
    info, _, _ = agg.plan(kind, n, M, K, N, 0, agg.options(**opts))
    assert (info.chunk_rows, info.k_blocks) == (cr, nkb)
    if nkb > 1:
        assert info.chunks_per_source == 16 * nkb and info.k_block == K // nkb
    # an explicit chunk size keeps whole-K chunks
    info, _, _ = agg.plan(kind, n, M, K, N, 8, agg.options(**{k: v for k, v in opts.items()
                                                               if k != "k_block"}))
    assert info.k_blocks == 1


# ---- producer options: DMA engines, CU-masked producer ---------------

@pytest.mark.parametrize("kw,status", [
    (dict(producer=4), agg.AGG_E_INVALID),
    (dict(producer=-1), agg.AGG_E_INVALID),
    (dict(producer=3), agg.AGG_E_UNSUPPORTED),               # 8-wave automatic tile
    (dict(producer=3, tile=13, workspace_stages=2), agg.AGG_E_UNSUPPORTED),
    (dict(producer=3, tile=13, producer_cus=32), agg.AGG_E_UNSUPPORTED),
    (dict(producer=3, tile=6), agg.AGG_E_UNSUPPORTED),       # 256 x 256
    (dict(producer_cus=-8), agg.AGG_E_INVALID),
    (dict(producer_cus=12), agg.AGG_E_UNSUPPORTED),
    (dict(producer_cus=16), agg.AGG_E_UNSUPPORTED),
    (dict(producer_cus=40), agg.AGG_E_UNSUPPORTED),
    (dict(producer=1, producer_cus=32), agg.AGG_E_UNSUPPORTED),
    (dict(producer=1, link_gbps=100.0), agg.AGG_E_UNSUPPORTED),
    (dict(producer=1, workspace_stages=2), agg.AGG_E_UNSUPPORTED),
    (dict(producer=1, k_block=1024), agg.AGG_E_UNSUPPORTED),
    (dict(producer=1, debug_drop_chunk=3), agg.AGG_E_UNSUPPORTED),
    (dict(producer=1, debug_delay_us=5.0), agg.AGG_E_UNSUPPORTED),
])
def test_producer_options_rejected(kw, status):
    with pytest.raises(agg.AggError) as e:
        agg.plan("f16", 4, 4096, 4096, 4096, 0, agg.options(**kw))
    assert e.value.status == status


def test_producer_options_plans():
    # the DMA producer moves whole-K chunks (automatic S/64 rows)
    info, _, _ = agg.plan("f16", 4, 4096, 4096, 4096, 0, agg.options(producer=1))
    assert info.k_blocks == 1 and info.chunk_rows == 16
    # a CU-masked producer: the consumer grid covers the other CUs, the
    # producer grid its own; outside the pipelined mode nothing is masked
    info, _, _ = agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(producer_cus=32))
    assert info.consumer_wgs == 224 and info.producer_wgs == 32
    info, _, _ = agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(producer_cus=64))
    assert info.consumer_wgs == 192 and info.producer_wgs == 64
    info, _, _ = agg.plan("f16", 8, 8192, 4096, 4096, 0,
                          agg.options(producer_cus=32, mode=agg.MODE_SEQUENTIAL))
    assert info.consumer_wgs == 256 and info.producer_wgs == 256


def test_fused_launch_choice():
    # pipelined calls whose two grids fit on the CUs together, on a tile the
    # fused kernel is built for, run in one launch; the automatic producer
    # grid is then whole multiples of 8 workgroups
    small = ("f16", 2, 256, 256, 128, 0)
    info = agg.plan(*small, agg.options())[0]
    assert info.producer_fused == 1 and info.tile_id == 13
    assert info.producer_wgs % 8 == 0 and info.producer_wgs + info.consumer_wgs <= 256
    for kind in ("bf16", "fp8", "i8"):
        assert agg.plan(kind, 2, 256, 256, 128, 0, agg.options())[0].producer_fused == 1
    assert agg.plan(*small, agg.options(link_gbps=153.0))[0].producer_fused == 1
    # an explicit producer grid is kept as asked
    info = agg.plan(*small, agg.options(producer_wgs=3))[0]
    assert info.producer_fused == 1 and info.producer_wgs == 3
    # not fused: the separate kernel asked for, other modes, the DMA engines,
    # a CU-masked producer, a workspace ring, grids that fill the device,
    # the 8-wave tiles
    for kw in (dict(producer=2), dict(mode=agg.MODE_SEQUENTIAL), dict(mode=agg.MODE_COPY_ONLY),
               dict(producer=1), dict(producer_cus=32), dict(tile=8)):
        assert agg.plan(*small, agg.options(**kw))[0].producer_fused == 0, kw
    ringed = ("f16", 2, 1024, 256, 128, 0)
    assert agg.plan(*ringed, agg.options())[0].producer_fused == 1
    info = agg.plan(*ringed, agg.options(workspace_stages=2))[0]
    assert info.workspace_stages == 2 and info.producer_fused == 0
    assert agg.plan("f16", 2, 2048, 2048, 1024, 0, agg.options())[0].producer_fused == 0
    assert agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options())[0].producer_fused == 0
    assert agg.plan("i8", 2, 64, 16384, 7168, 0, agg.options())[0].producer_fused == 0
    # asked for: fused whatever the grids (producer workgroups come first in
    # the launch, so a grid larger than the device still cannot starve);
    # outside the pipelined mode the producer runs as a kernel of its own
    info = agg.plan("f16", 8, 8192, 4096, 4096, 0, agg.options(producer=3, tile=13))[0]
    assert info.producer_fused == 1 and info.consumer_wgs == 256
    for tile in (2, 3, 12, 13, 14):
        assert agg.plan(*small, agg.options(producer=3, tile=tile))[0].producer_fused == 1
    assert agg.plan(*small, agg.options(producer=3, mode=agg.MODE_SEQUENTIAL))[0].producer_fused == 0


def test_automatic_producer_grid():
    # unpaced pipelined calls: half the CUs; paced, copy-only and
    # sequential calls, and an explicit grid: as asked or every CU
    shape = ("f16", 8, 8192, 4096, 4096, 0)
    assert agg.plan(*shape, agg.options())[0].producer_wgs == 128
    # paced with the automatic eight K-blocks: a quarter of the CUs; paced
    # with other chunks: every CU
    assert agg.plan(*shape, agg.options(link_gbps=153.0))[0].producer_wgs == 64
    assert agg.plan(*shape[:5], 64, agg.options(link_gbps=153.0))[0].producer_wgs == 256
    assert agg.plan(*shape, agg.options(link_gbps=153.0, k_block=512))[0].producer_wgs == 256
    assert agg.plan(*shape, agg.options(mode=agg.MODE_COPY_ONLY))[0].producer_wgs == 256
    assert agg.plan(*shape, agg.options(mode=agg.MODE_SEQUENTIAL))[0].producer_wgs == 256
    assert agg.plan(*shape, agg.options(producer_wgs=200))[0].producer_wgs == 200
    assert agg.plan(*shape, agg.options(), num_cus=80)[0].producer_wgs == 40
    # never more workgroups than pieces: 2 x 128 rows, K 256 has 8
    assert agg.plan("f16", 2, 256, 256, 128, 32, agg.options())[0].producer_wgs == 8


def test_producer_grid_leaves_room_for_the_consumer():
    """A pipelined call whose separate producer kernel shares every CU with
    the consumer takes at most one producer workgroup per CU: more could
    fill the CUs before any consumer workgroup starts, and the producer
    waits for the consumer's start.  Copy-only and sequential calls, the
    fused launch and a producer on CUs of its own have no such limit."""
    shape = ("f16", 8, 8192, 4096, 4096, 0)
    for kw in (dict(producer_wgs=257), dict(producer_wgs=512, link_gbps=153.0)):
        with pytest.raises(agg.AggError) as e:
            agg.plan(*shape, agg.options(**kw))
        assert e.value.status == agg.AGG_E_UNSUPPORTED, kw
    with pytest.raises(agg.AggError):
        agg.plan(*shape, agg.options(producer_wgs=81), num_cus=80)
    assert agg.plan(*shape, agg.options(producer_wgs=256))[0].producer_wgs == 256
    for kw in (dict(mode=agg.MODE_COPY_ONLY), dict(mode=agg.MODE_SEQUENTIAL),
               dict(producer_cus=32)):
        assert agg.plan(*shape, agg.options(producer_wgs=512, **kw))[0].producer_wgs == 512
    small = ("f16", 2, 256, 256, 128, 32)
    info = agg.plan(*small, agg.options(producer=3, producer_wgs=8, tile=13))[0]
    assert info.producer_fused == 1
