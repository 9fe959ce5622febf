"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bar (fp16 path): |C_gpu - C_oracle| <= 5e-4 * sum_k |a_ik b_kj| per element.
Bar (int8 path): int32 accumulators bit-exact; fp16 output within 1 ulp.
Every fp16, bf16 and fp8 workload is compared element by element in full,
the full-size ones included.  The int8 workloads whose full oracle would
take minutes (C5, C6) are compared on stratified rows (every 256-row tile
of every shard, every row position within a tile, every column), and their
whole int32 accumulator matrix is checked exactly by random projections.
"""
import numpy as np
import pytest

import synth
from gpu_util import (REL, check_f16, check_i8, dev, freivalds_i8, sample_rows,
                      stratified_rows)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def agg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_amd as m
    return m


def run_f16(agg, shards, B, chunk_rows=0, opts=None):
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    M = sum(s.shape[0] for s in shards)
    C = torch.full((M, B.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    agg.ag_gemm_f16(ts, tB, C, chunk_rows, opts=opts)
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return C.cpu().numpy()


def run_i8(agg, shards, B, bias, scale, chunk_rows=0, opts_kw=None):
    ts = [dev(s, torch) for s in shards]
    M = sum(s.shape[0] for s in shards)
    N = B.shape[1]
    acc = torch.full((M, N), -1, dtype=torch.int32, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    opts = agg.options(acc_out=acc, **(opts_kw or {}))
    agg.ag_gemm_i8_dequant(ts, dev(B, torch), dev(bias, torch), dev(scale, torch), C,
                           chunk_rows, opts=opts)
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return acc.cpu().numpy(), C.cpu().numpy()


# ---------------------------------------------------------------- fp16 path

def test_case1_full(agg, orc):
    c = synth.CASES[1]
    shards, B = synth.make_case(c)
    C = run_f16(agg, shards, B, c.chunk_rows)
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C, Co, So, c.name)


def test_case2_full(agg, orc):
    c = synth.CASES[2]
    shards, B = synth.make_case(c)
    C = run_f16(agg, shards, B, c.chunk_rows)
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C, Co, So, c.name)


@pytest.mark.parametrize("cid", [3, 4])
def test_large_cases_full(agg, orc, cid):
    """C3 (paced producer) and C4 at their full sizes, every element of C,
    in the launch configuration the benchmark times."""
    c = synth.CASES[cid]
    shards, B = synth.make_case(c)
    opts = agg.options(link_gbps=c.link_gbps) if c.link_gbps else None
    C = run_f16(agg, shards, B, c.chunk_rows, opts)
    Co, So = orc.ag_gemm_f16(shards, B)
    print(c.name, "max err/S", check_f16(C, Co, So, c.name))


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 15])
@pytest.mark.parametrize("n,S,K,N,cr", [
    (3, 100, 296, 168, 7),     # ragged rows, k tail, n tail, ragged last chunk
    (2, 300, 520, 264, 0),
    (4, 33, 8, 8, 5),          # K and N of a single vector
])
def test_ragged_shapes(agg, orc, tile, n, S, K, N, cr):
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 31000 + S)
    C = run_f16(agg, shards, B, cr, agg.options(tile=tile))
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C, Co, So, f"tile {tile} n={n} S={S} K={K} N={N}")


@pytest.mark.parametrize("pv,stages", [(1, 0), (2, 0), (3, 3)])
def test_barrier_scheme_ragged(agg, orc, pv, stages):
    shards, B = synth.make_f16(3 * 300, 296, 168, 3, "normal", 37000 + pv)
    # 8-row chunks: a ring needs chunks inside the 64-row panels
    C = run_f16(agg, shards, B, 8 if stages else 7,
                agg.options(scheme=agg.SCHEME_BARRIER, pvalue=pv, workspace_stages=stages, tile=3))
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C, Co, So, f"barrier pvalue {pv} stages {stages}")


@pytest.mark.parametrize("kind,tile", [("f16", 6), ("f16", 3), ("f16", 8), ("i8", 6), ("i8", 2), ("i8", 9)])
def test_no_store_outside_c(agg, kind, tile):
    """Rows past the last shard's end and columns past N are dropped by
    the epilogue: memory right after C (and after acc_out) keeps its
    contents."""
    n, S, K, N = 2, 300, 64, 200          # ragged m- and n-tiles
    M = n * S
    pad = 1 << 16
    if kind == "f16":
        shards, B = synth.make_f16(M, K, N, n, "normal", 33000 + tile)
        ts = [dev(s, torch) for s in shards]
        buf = torch.full((M * N + pad,), 12345.0, device="cuda")
        agg.ag_gemm_f16(ts, dev(B, torch), buf[:M * N].view(M, N), 0,
                        opts=agg.options(tile=tile))
        assert agg.check() == 0
        assert (buf[M * N:] == 12345.0).all()
        assert torch.isfinite(buf[:M * N]).all()
    else:
        shards, B, bias, scale = synth.make_i8(M, K, N, n, 33100 + tile)
        ts = [dev(s, torch) for s in shards]
        buf = torch.full((M * N + pad,), 7.0, dtype=torch.float16, device="cuda")
        acc = torch.full((M * N + pad,), -5, dtype=torch.int32, device="cuda")
        agg.ag_gemm_i8_dequant(ts, dev(B, torch), dev(bias, torch), dev(scale, torch),
                               buf[:M * N].view(M, N), 0,
                               opts=agg.options(tile=tile, acc_out=acc[:M * N]))
        assert agg.check() == 0
        assert (buf[M * N:] == 7.0).all() and (acc[M * N:] == -5).all()


def test_chunks_in_several_pieces(agg, orc):
    """Chunks of 2 MiB are copied as four 512 KiB pieces by different
    producer workgroups; the last chunk of each shard is short, so some of
    its pieces are empty.  Repeated calls on one workspace reuse the
    epoch-tagged piece counters."""
    n, S, K, N, cr = 3, 70, 1 << 16, 64, 16          # 16 rows x 128 KiB per chunk
    info, _, _ = agg.plan("f16", n, n * S, K, N, cr)
    assert info.chunks_per_source == 5
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 34000)
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    ws = torch.empty(agg.workspace_bytes(n, n * S, K, 2), dtype=torch.uint8, device="cuda")
    agg.workspace_reset(ws)
    Co, So = orc.ag_gemm_f16(shards, B)
    for it, kw in enumerate([dict(), dict(producer_wgs=3), dict(mode=agg.MODE_SEQUENTIAL),
                             dict(link_gbps=200.0), dict()]):
        C = torch.full((n * S, N), float("nan"), device="cuda")
        agg.ag_gemm_f16(ts, tB, C, cr, opts=agg.options(workspace=ws, **kw))
        assert agg.check() == 0
        check_f16(C.cpu().numpy(), Co, So, f"pieces, call {it} {kw}")


def test_single_shard_and_many_shards(agg, orc):
    shards, B = synth.make_f16(96, 64, 32, 1, "normal", 32000)
    C = run_f16(agg, shards, B)
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C, Co, So, "one shard")
    shards, B = synth.make_f16(64 * 3, 32, 16, 64, "normal", 32001)
    C = run_f16(agg, shards, B, 1)
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C, Co, So, "64 shards")


def test_k_zero_gives_zeros(agg):
    ts = [torch.empty((16, 0), dtype=torch.float16, device="cuda") for _ in range(2)]
    B = torch.empty((0, 24), dtype=torch.float16, device="cuda")
    C = torch.full((32, 24), 7.0, device="cuda")
    agg.ag_gemm_f16(ts, B, C)
    assert agg.check() == 0
    assert (C == 0).all()


def test_closed_form_all_ones(agg):
    K = 4096
    ts = [torch.ones((256, K), dtype=torch.float16, device="cuda") for _ in range(4)]
    B = torch.ones((K, 512), dtype=torch.float16, device="cuda")
    C = torch.empty((1024, 512), device="cuda")
    agg.ag_gemm_f16(ts, B, C)
    assert agg.check() == 0
    assert (C == K).all()


# ---------------------------------------------------------------- int8 path

def test_i8_small_full(agg, orc):
    shards, B, bias, scale = synth.make_i8(2 * 192, 27392 // 8, 264, 2, 40000)
    acc, D = run_i8(agg, shards, B, bias, scale)
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    check_i8(acc, D, ao, Do, "int8 small")


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 15])
def test_i8_ragged(agg, orc, tile):
    shards, B, bias, scale = synth.make_i8(3 * 77, 16 * 37, 8 * 19, 3, 41000 + tile)
    acc, D = run_i8(agg, shards, B, bias, scale, 9, dict(tile=tile))
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    check_i8(acc, D, ao, Do, f"int8 ragged tile {tile}")


def test_i8_debug_mode_all_ones(agg):
    K, N = 27392, 256
    ts = [torch.ones((128, K), dtype=torch.int8, device="cuda") for _ in range(2)]
    B = torch.ones((K, N), dtype=torch.int8, device="cuda")
    bias = torch.arange(N, dtype=torch.int32, device="cuda") - 128
    scale = torch.full((N,), 5e-4, dtype=torch.float32, device="cuda")
    C = torch.empty((256, N), dtype=torch.float16, device="cuda")
    acc = torch.empty((256, N), dtype=torch.int32, device="cuda")
    agg.ag_gemm_i8_dequant(ts, B, bias, scale, C, opts=agg.options(acc_out=acc))
    assert agg.check() == 0
    want = (K + bias).cpu().numpy()
    assert (acc.cpu().numpy() == want[None, :]).all()
    wantD = (want.astype(np.float32) * np.float32(5e-4)).astype(np.float16)
    assert np.array_equal(C.cpu().numpy().view(np.uint16),
                          np.broadcast_to(wantD.view(np.uint16), (256, N)))


@pytest.mark.parametrize("cid", [5, 6])
def test_i8_cases_stratified_rows(agg, orc, cid):
    """C5 and C6 at full size: fp16 output and int32 accumulators on rows
    that meet every m-tile of every shard and every row position of a
    tile, all columns; and every accumulator exactly, by projection."""
    c = synth.CASES[cid]
    shards, B, bias, scale = synth.make_case(c)
    acc, D = run_i8(agg, shards, B, bias, scale)
    rows = stratified_rows(c.M, c.n_shards, agg.pick_chunk_rows(c.shard_rows), extra=6)
    S = c.shard_rows
    assert {(r // S, (r % S) // 256) for r in rows} == \
        {(s, t) for s in range(c.n_shards) for t in range(-(-S // 256))}
    assert {r % S % 256 for r in rows} == set(range(256))
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale, rows=rows)
    check_i8(acc[rows], D[rows], ao, Do, c.name)
    assert freivalds_i8(acc, shards, B, bias) == c.M


def test_block16_full_sizes(agg, orc):
    """The 16 x 16-block form of the 256 x 256 tile (id 15) at full size:
    C4 fp16, every element of C; C5 int8 on stratified rows, every
    accumulator by projection."""
    c = synth.CASES[4]
    shards, B = synth.make_case(c)
    C = run_f16(agg, shards, B, c.chunk_rows, agg.options(tile=15))
    Co, So = orc.ag_gemm_f16(shards, B)
    print(c.name, "tile 15 max err/S", check_f16(C, Co, So, c.name + " tile 15"))
    c = synth.CASES[5]
    shards, B, bias, scale = synth.make_case(c)
    acc, D = run_i8(agg, shards, B, bias, scale, 0, dict(tile=15))
    rows = stratified_rows(c.M, c.n_shards, agg.pick_chunk_rows(c.shard_rows), extra=6)
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale, rows=rows)
    check_i8(acc[rows], D[rows], ao, Do, c.name + " tile 15")
    assert freivalds_i8(acc, shards, B, bias) == c.M


def test_i8_small_m_full(agg, orc):
    """The decode-like shape: 64 gathered rows, so every shard is a
    single, partial m-tile and the grid is set by the n-tiles."""
    c = synth.CASES[7]
    shards, B, bias, scale = synth.make_case(c)
    acc, D = run_i8(agg, shards, B, bias, scale)
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    check_i8(acc, D, ao, Do, c.name)


# ---------------------------------------------------------------- bf16 path

def bf16_dev(a):
    """uint16 bfloat16 bit patterns -> a bfloat16 CUDA tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def run_bf16(agg, shards, B, chunk_rows=0, opts=None):
    ts = [bf16_dev(s) for s in shards]
    M = sum(s.shape[0] for s in shards)
    C = torch.full((M, B.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    agg.ag_gemm_bf16(ts, bf16_dev(B), C, chunk_rows, opts=opts)
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return C.cpu().numpy()


def test_bf16_small_full(agg, orc):
    shards, B = synth.make_bf16(256, 256, 128, 2, "normal", 35000)
    C = run_bf16(agg, shards, B, 32)
    Co, So = orc.ag_gemm_bf16(shards, B)
    check_f16(C, Co, So, "bf16 small")


@pytest.mark.parametrize("tile", [3, 8, 6, 11, 15])
def test_bf16_ragged(agg, orc, tile):
    shards, B = synth.make_bf16(3 * 100, 296, 168, 3, "uniform", 35100 + tile)
    C = run_bf16(agg, shards, B, 7, agg.options(tile=tile))
    Co, So = orc.ag_gemm_bf16(shards, B)
    check_f16(C, Co, So, f"bf16 ragged tile {tile}")


def test_bf16_large_full(agg, orc):
    n, S, K, N = 8, 1024, 4096, 4096
    shards, B = synth.make_bf16(n * S, K, N, n, "normal", 35200)
    C = run_bf16(agg, shards, B)
    Co, So = orc.ag_gemm_bf16(shards, B)
    print("bf16 8x1024x4096x4096: max err/S", check_f16(C, Co, So, "bf16 8x1024x4096x4096"))


# ---------------------------------------------------------------- fp8 path
# Same bar as the fp16 path.  The fp8 matrix-core instruction does not sum
# its 64 products in full fp32 precision; its error stays a small multiple
# of 2^-24 sum|ab| per instruction, far inside the bound (the largest
# ratio err / sum|ab| is printed).

FP8_TILES = [2, 3, 6, 10, 11, 12, 13, 15]


def run_fp8(agg, shards, B, chunk_rows=0, opts=None, as_float8=False):
    ts = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in shards]
    tB = torch.from_numpy(np.ascontiguousarray(B)).cuda()
    if as_float8:
        ts = [t.view(torch.float8_e4m3fn) for t in ts]
        tB = tB.view(torch.float8_e4m3fn)
    M = sum(s.shape[0] for s in shards)
    C = torch.full((M, B.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    agg.ag_gemm_fp8(ts, tB, C, chunk_rows, opts=opts)
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return C.cpu().numpy()


def test_fp8_small_full(agg, orc):
    shards, B = synth.make_fp8(256, 256, 128, 2, "normal", 36000)
    C = run_fp8(agg, shards, B, 32, as_float8=True)
    Co, So = orc.ag_gemm_fp8(shards, B)
    print("fp8 small: max err/S", check_f16(C, Co, So, "fp8 small"))


@pytest.mark.parametrize("tile", FP8_TILES)
def test_fp8_ragged(agg, orc, tile):
    shards, B = synth.make_fp8(3 * 100, 16 * 37, 8 * 21, 3, "uniform", 36100 + tile)
    C = run_fp8(agg, shards, B, 7, agg.options(tile=tile))
    Co, So = orc.ag_gemm_fp8(shards, B)
    check_f16(C, Co, So, f"fp8 ragged tile {tile}")


def test_fp8_rejects_unbuilt_tile(agg):
    shards, B = synth.make_fp8(256, 256, 128, 2, "normal", 36050)
    with pytest.raises(agg.AggError):
        run_fp8(agg, shards, B, 0, agg.options(tile=8))


@pytest.mark.parametrize("tile", [0, 6, 15])
def test_fp8_large_full(agg, orc, tile):
    """The 8 x 1024-row, K = N = 4096 fp8 call in full, with the automatic
    tile and with both 256 x 256 tiles (four waves, and eight waves on one
    rolling operand set)."""
    n, S, K, N = 8, 1024, 4096, 4096
    shards, B = synth.make_fp8(n * S, K, N, n, "normal", 36200)
    C = run_fp8(agg, shards, B, 0, agg.options(tile=tile))
    Co, So = orc.ag_gemm_fp8(shards, B)
    print(f"fp8 8x1024x4096x4096 tile {tile}: max err/S",
          check_f16(C, Co, So, f"fp8 large tile {tile}"))


# ---------------------------------------------------------------- K-blocks
# Chunks of rows x one K-block: the same sums in the same order, so the
# output is bitwise that of whole-K chunks, and within the bar of the oracle.

@pytest.mark.parametrize("kind,tile,n,S,K,N,cr,kb", [
    ("f16", 8, 3, 300, 2048, 264, 7, 512),     # ragged rows and columns, 4 K-blocks
    ("f16", 13, 3, 100, 2560, 168, 7, 1024),   # the last K-block takes the remainder
    ("f16", 11, 4, 256, 1536, 512, 16, 512),
    ("f16", 9, 2, 300, 2048, 256, 0, 512),     # four-stage ring: three slices ahead
    ("f16", 12, 3, 64, 1024, 64, 1, 512),      # eight-stage ring, one-row chunks
    ("f16", 3, 2, 128, 4096, 64, 32, 4096),    # one K-block: whole-K chunks
    ("bf16", 8, 3, 300, 2048, 264, 7, 512),
    ("fp8", 6, 3, 100, 3072, 168, 7, 1024),
    ("fp8", 13, 2, 130, 2048, 256, 5, 1024),
    ("i8", 8, 3, 77, 3072, 152, 9, 1024),
    ("i8", 13, 2, 130, 2048, 256, 5, 1024),
])
def test_k_blocks_full(agg, orc, kind, tile, n, S, K, N, cr, kb):
    M = n * S
    seed = 38000 + S + K
    if kind == "i8":
        shards, B, bias, scale = synth.make_i8(M, K, N, n, seed)
        acc, D = run_i8(agg, shards, B, bias, scale, cr, dict(tile=tile, k_block=kb))
        ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
        check_i8(acc, D, ao, Do, f"int8 k_block {kb} tile {tile}")
        acc1, D1 = run_i8(agg, shards, B, bias, scale, cr, dict(tile=tile))
        assert np.array_equal(D.view(np.uint16), D1.view(np.uint16))
        return
    if kind == "f16":
        shards, B = synth.make_f16(M, K, N, n, "normal", seed)
        run, oracle_fn = run_f16, orc.ag_gemm_f16
    elif kind == "bf16":
        shards, B = synth.make_bf16(M, K, N, n, "normal", seed)
        run, oracle_fn = run_bf16, orc.ag_gemm_bf16
    else:
        shards, B = synth.make_fp8(M, K, N, n, "normal", seed)
        run, oracle_fn = run_fp8, orc.ag_gemm_fp8
    C = run(agg, shards, B, cr, agg.options(tile=tile, k_block=kb))
    Co, So = oracle_fn(shards, B)
    check_f16(C, Co, So, f"{kind} k_block {kb} tile {tile}")
    C1 = run(agg, shards, B, cr, agg.options(tile=tile))
    assert np.array_equal(C.view(np.uint32), C1.view(np.uint32)), "differs from whole-K chunks"


@pytest.mark.parametrize("cid,kb", [(3, 512), (4, 256 * 2)])
def test_k_blocks_full_size(agg, orc, cid, kb):
    """C3 (paced) and C4 with K-blocks of 512: every element of C."""
    c = synth.CASES[cid]
    shards, B = synth.make_case(c)
    C = run_f16(agg, shards, B, c.chunk_rows, agg.options(link_gbps=c.link_gbps, k_block=kb))
    Co, So = orc.ag_gemm_f16(shards, B)
    print(c.name, "k_block", kb, "max err/S", check_f16(C, Co, So, c.name))


# ---------------------------------------------------------------- producers

@pytest.mark.parametrize("kw", [dict(producer=1), dict(producer_cus=32),
                                dict(producer_cus=64, k_block=1024)])
def test_producer_options_full_size(agg, orc, kw):
    """C4 moved by the DMA engines, or by a producer on 32 or 64 CUs of its
    own: every element of C."""
    c = synth.CASES[4]
    shards, B = synth.make_case(c)
    C = run_f16(agg, shards, B, 0, agg.options(**kw))
    Co, So = orc.ag_gemm_f16(shards, B)
    print(kw, "max err/S", check_f16(C, Co, So, f"{c.name} {kw}"))


@pytest.mark.parametrize("kw", [dict(producer=1), dict(producer_cus=32)])
def test_producer_options_i8(agg, orc, kw):
    shards, B, bias, scale = synth.make_i8(3 * 77, 16 * 37, 8 * 19, 3, 41500)
    acc, D = run_i8(agg, shards, B, bias, scale, 9, kw)
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    check_i8(acc, D, ao, Do, f"int8 {kw}")
