"""Helpers for the GPU parity tests: upload seeded inputs, call the library
through its binding, compare with the oracle at the stated tolerances."""
import numpy as np

import synth

# fp32 result: |C_gpu - C_oracle| <= REL * sum_k |a_ik b_kj| elementwise.
# The forward error of any fp32 summation order is at most about
# K * 2^-24 * sum|ab| (2.4e-4 at K = 4096), plus 2^-24 |C| for the final
# rounding, so 5e-4 holds for every shape tested here (K <= 8192).
REL = 5e-4


def dev(x, torch):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def sample_rows(M, n, cr, extra=8, seed=0):
    """Rows covering every shard's first/last rows and chunk edges."""
    S = M // n
    rows = set()
    for s in range(n):
        for r in (0, 1, cr - 1, cr, S // 2, S - 2, S - 1):
            if 0 <= r < S:
                rows.add(s * S + r)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, M, extra).tolist())
    return np.array(sorted(rows), np.int64)


def stratified_rows(M, n, cr, tm=256, extra=8, seed=0):
    """Rows that meet every tm-row tile of every shard, with the tile's row
    positions 0..tm-1 all taken (spread over the tiles: tile i of T gets
    positions i, i + T, i + 2T, ... mod tm), plus every shard's first and
    last rows and chunk edges (sample_rows)."""
    S = M // n
    mt = -(-S // tm)
    T = n * mt
    rows = set(sample_rows(M, n, cr, extra, seed).tolist())
    per = max(1, -(-tm // T))
    for i in range(T):
        s, t = divmod(i, mt)
        for j in range(per):
            r = t * tm + (i + T * j) % tm
            if r < S:
                rows.add(s * S + r)
    return np.array(sorted(rows), np.int64)


def freivalds_i8(acc_gpu, shards, B, bias, trials=2, seed=0, block=2048):
    """Exact check of a whole int32 accumulator matrix without forming A.B:
    acc x == A (B x) + (bias . x) for random integer vectors x, in int64
    (no overflow: |A.B| < 2^31, |x| <= 1000, N, K <= 2^16).  A wrong
    element of acc escapes one trial with probability at most 1/2001.
    Returns the number of rows checked."""
    rng = np.random.default_rng(seed)
    N = B.shape[1]
    B64 = B.astype(np.int64)
    for _ in range(trials):
        x = rng.integers(-1000, 1001, N).astype(np.int64)
        v = B64 @ x
        bx = int(bias.astype(np.int64) @ x)
        r0 = 0
        for sh in shards:
            for b in range(0, sh.shape[0], block):
                a = sh[b:b + block].astype(np.int64)
                want = a @ v + bx
                got = acc_gpu[r0 + b:r0 + b + a.shape[0]].astype(np.int64) @ x
                bad = np.nonzero(got != want)[0]
                assert bad.size == 0, f"acc rows {(r0 + b + bad[:4]).tolist()} differ"
            r0 += sh.shape[0]
    return r0


def check_f16(C_gpu, C_orc, S_abs, what=""):
    C_gpu = np.asarray(C_gpu, np.float64)
    err = np.abs(C_gpu - C_orc.astype(np.float64))
    bound = REL * S_abs
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, (
        f"{what}: {len(bad)} elements out of bound, first {bad[:4].tolist()} "
        f"gpu={C_gpu[tuple(bad[0])]} oracle={C_orc[tuple(bad[0])]} S={S_abs[tuple(bad[0])]}")
    return float((err / np.maximum(S_abs, 1e-300)).max())


def ulp_dist16(a, b):
    """Distance in units in the last place between fp16 arrays (ordered ints)."""
    def ordered(x):
        u = np.asarray(x).view(np.uint16).astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7fff) - 0x8000, u)
    return np.abs(ordered(a) - ordered(b))


def check_i8(acc_gpu, D_gpu, acc_orc, D_orc, what=""):
    assert np.array_equal(acc_gpu, acc_orc), f"{what}: int32 accumulators differ"
    d = ulp_dist16(D_gpu, D_orc)
    assert d.max() <= 1, f"{what}: dequantised output off by {d.max()} ulp"
    return int((d > 0).sum())
