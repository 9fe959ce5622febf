"""Split-K on the GPU (agg_options.k_splits; the automatic choice does not
split): the K parts of an output tile summed by the last part to finish,
in part order.

Each case checks the library's plan first (the split is really taken),
then the HIP result against the oracle at the path's bar: fp32 output
within 5e-4 * sum_k |a_ik b_kj|, int32 accumulators bit-exact and the fp16
dequantised output within 1 ulp.  Shapes are ragged in M, N and K (the
last part holds a partial slice).  The parts are summed in a fixed order,
so the result must not depend on the schedule (chunks, local shard,
producer and consumer grids, mode) nor change over repeated calls, whose
tickets carry on from one call to the next."""
import numpy as np
import pytest

import synth
from gpu_util import check_f16, check_i8, dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def agg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_amd as m
    return m


def f16_call(agg, ts, tB, N, chunk_rows=0, **kw):
    M = sum(t.shape[0] for t in ts)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    agg.ag_gemm_f16(ts, tB, C, chunk_rows, opts=agg.options(**kw))
    rc = agg.check()
    assert rc == 0, agg.status_string(rc)
    return C


def splits(agg, kind, shards, K, N, **kw):
    info, _, _ = agg.plan(kind, len(shards), sum(s.shape[0] for s in shards), K, N, 0,
                          agg.options(**kw))
    return info.k_splits


@pytest.mark.parametrize("tile", [3, 12, 13, 14])
@pytest.mark.parametrize("ks", [2, 3, 7])
def test_f16_split_ragged(agg, orc, tile, ks):
    n, S, K, N = 3, 20, 5000, 1000
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 70000 + 10 * tile + ks)
    assert splits(agg, "f16", shards, K, N, tile=tile, k_splits=ks) == ks
    C = f16_call(agg, [dev(s, torch) for s in shards], dev(B, torch), N, 0,
                 tile=tile, k_splits=ks)
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(C.cpu().numpy(), Co, So, f"split-K f16 tile {tile} ks {ks}")


@pytest.mark.parametrize("tile", [3, 13, 14])
@pytest.mark.parametrize("ks", [2, 5])
def test_i8_split_exact(agg, orc, tile, ks):
    n, S, K, N = 2, 24, 4144, 520
    shards, B, bias, scale = synth.make_i8(n * S, K, N, n, 71000 + 10 * tile + ks)
    assert splits(agg, "i8", shards, K, N, tile=tile, k_splits=ks) == ks
    ts = [dev(s, torch) for s in shards]
    acc = torch.full((n * S, N), -1, dtype=torch.int32, device="cuda")
    D = torch.full((n * S, N), float("nan"), dtype=torch.float16, device="cuda")
    agg.ag_gemm_i8_dequant(ts, dev(B, torch), dev(bias, torch), dev(scale, torch), D, 0,
                           opts=agg.options(acc_out=acc, tile=tile, k_splits=ks))
    assert agg.check() == 0
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    check_i8(acc.cpu().numpy(), D.cpu().numpy(), ao, Do, f"split-K int8 tile {tile} ks {ks}")


def test_bf16_and_fp8_split(agg, orc):
    n, S, K, N = 2, 32, 4096, 768
    shards, B = synth.make_bf16(n * S, K, N, n, "normal", 72000)
    assert splits(agg, "bf16", shards, K, N, tile=14, k_splits=4) == 4
    ts = [torch.from_numpy(np.ascontiguousarray(s).view(np.int16)).cuda().view(torch.bfloat16)
          for s in shards]
    tB = torch.from_numpy(np.ascontiguousarray(B).view(np.int16)).cuda().view(torch.bfloat16)
    C = torch.full((n * S, N), float("nan"), dtype=torch.float32, device="cuda")
    agg.ag_gemm_bf16(ts, tB, C, 0, opts=agg.options(tile=14, k_splits=4))
    assert agg.check() == 0
    Co, So = orc.ag_gemm_bf16(shards, B)
    check_f16(C.cpu().numpy(), Co, So, "split-K bf16")

    shards, B = synth.make_fp8(n * S, K, N, n, "normal", 72100)
    assert splits(agg, "fp8", shards, K, N, tile=14, k_splits=4) == 4
    ts = [dev(s, torch) for s in shards]
    C = torch.full((n * S, N), float("nan"), dtype=torch.float32, device="cuda")
    agg.ag_gemm_fp8(ts, dev(B, torch), C, 0, opts=agg.options(tile=14, k_splits=4))
    assert agg.check() == 0
    Co, So = orc.ag_gemm_fp8(shards, B)
    check_f16(C.cpu().numpy(), Co, So, "split-K fp8")


def test_split_result_independent_of_schedule(agg, orc):
    n, S, K, N = 4, 32, 8192, 2048
    shards, B = synth.make_f16(n * S, K, N, n, "normal", 73000)
    split = dict(tile=14, k_splits=8)
    assert splits(agg, "f16", shards, K, N, **split) == 8
    ts = [dev(s, torch) for s in shards]
    tB = dev(B, torch)
    ref = f16_call(agg, ts, tB, N, **split)
    Co, So = orc.ag_gemm_f16(shards, B)
    check_f16(ref.cpu().numpy(), Co, So, "split-K, 8 parts")
    for cr, kw in ((1, {}), (7, {}), (0, dict(local_shard=2)), (0, dict(producer_wgs=3)),
                   (0, dict(consumer_wgs=7)), (0, dict(consumer_wgs=1)),
                   (0, dict(mode=agg.MODE_SEQUENTIAL)), (0, dict(link_model=agg.LINKS_SERIAL)),
                   (0, {}), (0, {})):
        C = f16_call(agg, ts, tB, N, cr, **split, **kw)
        assert torch.equal(C, ref), (cr, kw)


def test_decode_shape_split_exact(agg, orc):
    """The decode-like int8 workload (2 x 32 rows, K 16384, N 7168) split
    in 4 parts on the 32 x 256 tile, in full against the oracle."""
    c = synth.CASES[7]
    shards, B, bias, scale = synth.make_case(c)
    ts = [dev(s, torch) for s in shards]
    acc = torch.full((c.M, c.N), -1, dtype=torch.int32, device="cuda")
    D = torch.full((c.M, c.N), float("nan"), dtype=torch.float16, device="cuda")
    agg.ag_gemm_i8_dequant(ts, dev(B, torch), dev(bias, torch), dev(scale, torch), D, 0,
                           opts=agg.options(acc_out=acc, tile=14, k_splits=4))
    assert agg.check() == 0
    ao, Do = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    check_i8(acc.cpu().numpy(), D.cpu().numpy(), ao, Do, c.name + " split-K")
