"""A long litmus run of the release protocol through the real kernels.

Thousands of pipelined calls through one caller-owned workspace, the shard
contents changing every call, with B = I so that C must equal the gathered
A exactly (one nonzero term per output element: exact in fp32).  Producer
pieces and consumer tiles are spread over all eight XCDs (workgroup b runs
on XCD b mod 8), so nearly every chunk is written on one XCD and read on
another.  The calls rotate through chunk shapes (one row, odd sizes,
K-blocks), paced and unpaced links and seeded random producer delays.  A
tile that read a chunk before its release, or a cache line left over from
the previous call (its rows sit at the same addresses, with other values),
gives a mismatch.  The run stops at the first one and names the call."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ITERS = 3000


@pytest.fixture(scope="module")
def agg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_amd as m
    return m


@pytest.mark.parametrize("S,tile,iters", [
    (64, 0, ITERS),
    # 256 x 256 tiles: their wait takes a chunk whose pieces are all
    # flagged (unpaced calls, three remote sources)
    (256, 15, ITERS // 2),
])
def test_litmus_changing_contents_across_xcds(agg, S, tile, iters):
    n, K = 4, 1024
    M = n * S
    ts = [torch.empty((S, K), dtype=torch.float16, device="cuda") for _ in range(n)]
    eye = torch.eye(K, dtype=torch.float16, device="cuda")
    C = torch.empty((M, K), device="cuda")
    ws = torch.empty(agg.workspace_bytes(n, M, K, 2), dtype=torch.uint8, device="cuda")
    agg.workspace_reset(ws)
    i = torch.arange(M, device="cuda", dtype=torch.int64)[:, None]
    k = torch.arange(K, device="cuda", dtype=torch.int64)[None, :]
    base = i * 7 + k * 13                       # integers, exact in fp16 below
    bad = torch.zeros(iters, dtype=torch.int64, device="cuda")
    shapes = [dict(cr=1), dict(cr=3), dict(cr=16), dict(cr=8, k_block=512),
              dict(cr=1, k_block=512), dict(cr=0)]
    extras = [dict(), dict(link_gbps=100.0), dict(debug_delay_us=15.0)]
    opts = []
    for it in range(iters):
        sh = dict(shapes[it % len(shapes)])
        ex = dict(extras[(it // len(shapes)) % len(extras)])
        if "debug_delay_us" in ex:
            ex["debug_delay_seed"] = it
        cr = sh.pop("cr")
        opts.append((cr, agg.options(workspace=ws, tile=tile, **sh, **ex), sh, ex))
    checked = 0
    for it in range(iters):
        A = ((base + it * 101) % 2047 - 1023).to(torch.float16)
        for s in range(n):
            ts[s].copy_(A[s * S:(s + 1) * S])
        C.fill_(float("nan"))
        cr, o, sh, ex = opts[it]
        agg.ag_gemm_f16(ts, eye, C, cr, opts=o)
        bad[it] = (C != A.float()).sum()
        if it % 200 == 199 or it == iters - 1:
            rc = agg.check()
            assert rc == 0, f"call {it}: {agg.status_string(rc)}"
            b = bad[:it + 1].nonzero()
            assert b.numel() == 0, (
                f"first mismatch at call {int(b[0])}: {int(bad[int(b[0])])} elements; "
                f"options {opts[int(b[0])][2]} {opts[int(b[0])][3]}")
            checked = it + 1
    assert checked == iters
