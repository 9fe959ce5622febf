"""Pins for the CPU oracle: checks against things the oracle does not compute
itself (exact rational arithmetic, closed forms, numpy's own routines,
invariants of the definition).

Each test names the passage whose definition it pins:
  * gather-then-GEMM: PTO-ISA AllGather+GEMM README ("compute function":
    rank r owns rows [r*M/n, (r+1)*M/n), C = A x B, fp16 in, fp32 out) and the
    Triton-distributed tutorial's reference function (all_gather, cat on
    dim 0, matmul);
  * int8 + bias + dequant: catccos AllGatherMatmulDequant design doc,
    section 2.2 (int32 sum + bias, times per-channel scale, cast to fp16)
    and section 8.6 (debug mode: all-ones matrices, fixed scale).
"""
import math
import os
import random
import shutil
import subprocess
import ctypes
from fractions import Fraction

import numpy as np
import pytest

import synth


# ----------------------------------------------------------------------------
# helpers written independently of the oracle
# ----------------------------------------------------------------------------

def frac_to_f32(q: Fraction) -> np.float32:
    """Exact rational -> binary32, round to nearest even (no double rounding)."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    q = -q if neg else q
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp_exp = e - 23 if e >= -126 else -149
    scaled = q / (Fraction(2) ** ulp_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * (Fraction(2) ** ulp_exp)
    if val >= Fraction(2) ** 128:
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))  # exact: n has at most 25 bits
    return -out if neg else out


def small_halves(rng, shape):
    """fp16 values m * 2^e with |m| < 64 and e in [-6, 3]: exactly
    representable, and any sum of a few products is exact in double."""
    m = rng.integers(-63, 64, shape)
    e = rng.integers(-6, 4, shape)
    return (m * np.exp2(e)).astype(np.float16)


def f32_bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ----------------------------------------------------------------------------
# fp16 codecs
# ----------------------------------------------------------------------------

def test_half_decode_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint16)
    ours = orc.half_to_double(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_half_encode_matches_numpy_rne(orc):
    rng = np.random.default_rng(7)
    finite = np.arange(65536, dtype=np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)].astype(np.float32)
    # exact halves, midpoints between neighbours (ties) and one fp32 ulp
    # either side of every midpoint
    srt = np.unique(finite.astype(np.float64))
    mids = ((srt[:-1] + srt[1:]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf))])
    rand = rng.standard_normal(200000).astype(np.float32) * \
        np.exp2(rng.integers(-30, 20, 200000)).astype(np.float32)
    special = np.array([65504, 65519.99, 65520, 65536, 1e10, -65520, 2.0**-24,
                        2.0**-25, 2.0**-25 * 1.0000001, 2.0**-26, 1e-30,
                        np.inf, -np.inf, 0.0, -0.0], np.float32)
    x = np.concatenate([finite, mids, near, rand, special])
    ours = orc.float_to_half(x)
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])
    nan = orc.float_to_half(np.array([np.nan], np.float32))
    assert np.isnan(nan.view(np.float16)[0])


# ----------------------------------------------------------------------------
# fp16 x fp16 -> fp32
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_f16_brute_force_exact_rational(orc, seed):
    """C must equal fp32_RNE(exact sum) bit for bit on inputs whose sums
    are exact in double."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(1, 4))
    K = int(rng.integers(1, 9))
    N = int(rng.integers(1, 9))
    M = n * S
    A = small_halves(rng, (M, K))
    B = small_halves(rng, (K, N))
    C, S_abs = orc.ag_gemm_f16(synth.split_rows(A, n), B)
    Af = [[Fraction(float(v)) for v in row] for row in A.astype(np.float64)]
    Bf = [[Fraction(float(v)) for v in row] for row in B.astype(np.float64)]
    for i in range(M):
        for j in range(N):
            exact = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            mag = sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0))
            want = frac_to_f32(exact)
            assert f32_bits(C[i, j]) == f32_bits(want) or \
                (C[i, j] == 0 and want == 0), (i, j, C[i, j], want)
            assert Fraction(float(S_abs[i, j])) == mag


def test_f16_closed_form_identity(orc):
    """B = I_K gives C = A exactly, in shard order."""
    A, _ = synth.make_f16(48, 32, 32, 3, "normal", 5000)
    Afull = np.concatenate(A)
    B = np.eye(32, dtype=np.float16)
    C, _ = orc.ag_gemm_f16(A, B)
    assert np.array_equal(C, Afull.astype(np.float32))


def test_f16_closed_form_all_ones(orc):
    """All-ones A and B give C = K everywhere (and |.| sum = K)."""
    K = 1000
    A = [np.ones((8, K), np.float16) for _ in range(4)]
    B = np.ones((K, 24), np.float16)
    C, S_abs = orc.ag_gemm_f16(A, B)
    assert np.all(C == np.float32(K)) and np.all(S_abs == K)


def test_f16_single_entry_selects_row_of_B(orc):
    """A with one nonzero A[i0, k0] = 1: row i0 of C is row k0 of B, every
    other row is zero.  Pins the index roles of A and B (no transposes)."""
    rng = np.random.default_rng(3)
    M, K, N, n = 12, 7, 9, 3
    B = rng.standard_normal((K, N)).astype(np.float16)
    for i0, k0 in [(0, 0), (5, 6), (11, 3), (4, 1)]:
        A = np.zeros((M, K), np.float16)
        A[i0, k0] = 1
        C, _ = orc.ag_gemm_f16(synth.split_rows(A, n), B)
        want = np.zeros((M, N), np.float32)
        want[i0] = B[k0].astype(np.float32)
        assert np.array_equal(C, want)


def test_f16_matches_numpy_float64(orc):
    """Library special case: float32 of numpy's float64 product."""
    rng = np.random.default_rng(11)
    M, K, N, n = 36, 45, 29, 3
    A = rng.standard_normal((M, K)).astype(np.float16)
    B = rng.standard_normal((K, N)).astype(np.float16)
    C, S_abs = orc.ag_gemm_f16(synth.split_rows(A, n), B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    mag = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(C.astype(np.float64) - ref) <= 1e-12 * mag + 2**-24 * np.abs(ref))
    assert np.allclose(S_abs, mag, rtol=1e-12, atol=0)


def test_f16_shard_permutation_permutes_row_blocks(orc):
    """Reordering the shard list reorders C's row blocks the same way
    (gather is concatenation in shard order), bit for bit."""
    shards, B = synth.make_f16(64, 40, 24, 4, "normal", 6000)
    C, _ = orc.ag_gemm_f16(shards, B)
    perm = [2, 0, 3, 1]
    Cp, _ = orc.ag_gemm_f16([shards[p] for p in perm], B)
    S = 16
    for dst, src in enumerate(perm):
        assert np.array_equal(Cp[dst * S:(dst + 1) * S], C[src * S:(src + 1) * S])


def test_f16_rows_subset_equals_full(orc):
    shards, B = synth.make_f16(96, 64, 40, 2, "uniform", 7000)
    C, S_abs = orc.ag_gemm_f16(shards, B)
    rows = np.array([95, 0, 47, 48, 13])
    Cr, Sr = orc.ag_gemm_f16(shards, B, rows=rows)
    assert np.array_equal(Cr, C[rows]) and np.array_equal(Sr, S_abs[rows])


def test_f16_power_of_two_scaling_is_exact(orc):
    shards, B = synth.make_f16(32, 48, 16, 2, "normal", 8000)
    C, _ = orc.ag_gemm_f16(shards, B)
    C2, _ = orc.ag_gemm_f16([(s.astype(np.float32) * 4).astype(np.float16) for s in shards], B)
    assert np.array_equal(C2, C * 4)


# ----------------------------------------------------------------------------
# int8 x int8 -> int32 (+ bias) -> fp16
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_i8_brute_force_python_ints(orc, seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.choice([1, 2, 3]))
    S, K, N = int(rng.integers(1, 5)), int(rng.integers(1, 20)), int(rng.integers(1, 9))
    M = n * S
    A = rng.integers(-127, 128, (M, K), dtype=np.int8)
    B = rng.integers(-127, 128, (K, N), dtype=np.int8)
    bias = rng.integers(-1000, 1001, N, dtype=np.int32)
    scale = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    acc, D = orc.ag_gemm_i8_dequant(synth.split_rows(A, n), B, bias, scale)
    for i in range(M):
        for j in range(N):
            v = sum(int(A[i, k]) * int(B[k, j]) for k in range(K)) + int(bias[j])
            assert acc[i, j] == v
            # exact product of the two binary32 numbers, then correct
            # rounding to fp16 differs from the two-step rounding by at
            # most one unit in the last place
            exact = Fraction(float(np.float32(v))) * Fraction(float(scale[j]))
            one_step = np.float16(float(exact)).view(np.uint16)
            two_step = D[i, j].view(np.uint16)
            assert abs(int(one_step) - int(two_step)) <= 1


def test_i8_debug_mode_closed_form(orc):
    """All-ones A and B with a fixed scale: acc = K + bias[j] and
    D = fp16(fp32(K + bias[j]) * s), rounded with numpy's own casts."""
    K, N, n, S = 27392, 64, 2, 3
    A = [np.ones((S, K), np.int8) for _ in range(n)]
    B = np.ones((K, N), np.int8)
    bias = np.arange(-32, 32, dtype=np.int32) * 31
    s = np.float32(5e-4)
    acc, D = orc.ag_gemm_i8_dequant(A, B, bias, np.full(N, s, np.float32))
    want_acc = K + bias
    assert np.all(acc == want_acc[None, :])
    want_D = (want_acc.astype(np.float32) * s).astype(np.float16)
    assert np.array_equal(D.view(np.uint16), np.broadcast_to(want_D.view(np.uint16), D.shape))


def test_i8_identity_gives_A_plus_bias(orc):
    rng = np.random.default_rng(9)
    A = rng.integers(-127, 128, (20, 16), dtype=np.int8)
    bias = rng.integers(-1000, 1001, 16, dtype=np.int32)
    acc, _ = orc.ag_gemm_i8_dequant(synth.split_rows(A, 4), np.eye(16, dtype=np.int8),
                                    bias, np.ones(16, np.float32))
    assert np.array_equal(acc, A.astype(np.int32) + bias)


def test_i8_matches_numpy_int64(orc):
    shards, B, bias, scale = synth.make_i8(64, 272, 48, 2, 9000)
    acc, D = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    A = np.concatenate(shards).astype(np.int64)
    ref = A @ B.astype(np.int64) + bias
    assert np.array_equal(acc, ref)
    want = (ref.astype(np.int32).astype(np.float32) * scale).astype(np.float16)
    assert np.array_equal(D.view(np.uint16), want.view(np.uint16))


def test_i8_extreme_values_and_overflow(orc):
    # worst case of the largest workload stays in int32: 127^2 * 27392 + 1000
    K = 27392
    A = [np.full((1, K), 127, np.int8), np.full((1, K), -127, np.int8)]
    B = np.full((K, 2), 127, np.int8)
    acc, D = orc.ag_gemm_i8_dequant(A, B, np.array([1000, -1000], np.int32),
                                    np.array([1e-3, 1e-3], np.float32))
    assert acc[0, 0] == 127 * 127 * K + 1000 and acc[1, 1] == -127 * 127 * K - 1000
    # fp16 overflow of the product rounds to infinity (IEEE, not saturating)
    assert np.isinf(D.astype(np.float32)).all()
    with pytest.raises(OverflowError):
        big = 140000
        orc.ag_gemm_i8_dequant([np.full((1, big), 127, np.int8)],
                               np.full((big, 1), 127, np.int8),
                               np.zeros(1, np.int32), np.ones(1, np.float32))


def test_dequant_matches_numpy(orc):
    rng = np.random.default_rng(12)
    v = rng.integers(-2**31, 2**31, 100000, dtype=np.int64).astype(np.int32)
    v[:1000] = rng.integers(-5000, 5000, 1000)
    s = rng.uniform(1e-4, 1e-3, v.size).astype(np.float32)
    ours = orc.dequant(v, s)
    ref = (v.astype(np.float32) * s).astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_i8_shard_permutation(orc):
    shards, B, bias, scale = synth.make_i8(30, 48, 16, 3, 9100)
    acc, D = orc.ag_gemm_i8_dequant(shards, B, bias, scale)
    acc2, D2 = orc.ag_gemm_i8_dequant(shards[::-1], B, bias, scale)
    S = 10
    for dst, src in enumerate([2, 1, 0]):
        assert np.array_equal(acc2[dst * S:(dst + 1) * S], acc[src * S:(src + 1) * S])
        assert np.array_equal(D2[dst * S:(dst + 1) * S].view(np.uint16),
                              D[src * S:(src + 1) * S].view(np.uint16))


# ----------------------------------------------------------------------------
# the pins have teeth: plant mistakes in a copy of the oracle and check that
# the checks above notice each one
# ----------------------------------------------------------------------------

MUTATIONS = [
    ("acc[j] += p;", "acc[j] -= p;"),                        # wrong sign
    ("for (int64_t k = 0; k < K; k++) {\n                double aik",
     "for (int64_t k = 1; k < K; k++) {\n                double aik"),  # dropped term
    ("const double *b = Bd + k * N;", "const double *b = Bd + (k % (K > 1 ? K - 1 : 1)) * N;"),
    ("int64_t s = i / S;", "int64_t s = 0;"),                 # gather ignores the shard
    ("int64_t v = acc[j] + (int64_t)bias[j];", "int64_t v = acc[j] - (int64_t)bias[j];"),
    ("volatile float p = f * s;", "volatile float p = f * s * 1.0001f;"),
    ("if (rem > halfway || (rem == halfway && (q & 1)))", "if (rem >= halfway)"),
    ("v = ldexp((double)(128 + f), e - 134);", "v = ldexp((double)(128 + f), e - 133);"),  # bf16 bias
    ("v = ldexp((double)(8 + f), e - 10);", "v = ldexp((double)(8 + f), e - 9);"),  # fp8 bias
    ("v = ldexp((double)f, -9);", "v = ldexp((double)f, -10);"),  # fp8 subnormal scale
    ("return oracle_fp8e4m3_to_double(((const uint8_t *)p)[i]);",
     "return oracle_fp8e4m3_to_double(((const uint8_t *)p)[i] & 0x7f);"),  # fp8 sign dropped
]


def _mutant(tmp_path, old, new):
    src = open(os.path.join(os.path.dirname(__file__), "..", "oracle", "oracle.c")).read()
    assert old in src, old
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new, 1))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", str(path), "-o", str(so), "-lm"], check=True)
    return str(so)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed")
@pytest.mark.parametrize("idx", range(len(MUTATIONS)))
def test_planted_mistake_is_caught(orc, tmp_path, idx, monkeypatch):
    import oracle as oracle_mod
    so = _mutant(tmp_path, *MUTATIONS[idx])
    lib = ctypes.CDLL(so)
    saved = oracle_mod._lib
    # rebind the wrapper to the mutant, reusing its argtypes setup
    monkeypatch.setattr(oracle_mod, "_lib", None)
    monkeypatch.setattr(oracle_mod, "build", lambda force=False: so)
    checks = [
        lambda: test_f16_brute_force_exact_rational(oracle_mod, 0),
        lambda: test_f16_brute_force_exact_rational(oracle_mod, 5),
        lambda: test_f16_closed_form_identity(oracle_mod),
        lambda: test_f16_single_entry_selects_row_of_B(oracle_mod),
        lambda: test_f16_shard_permutation_permutes_row_blocks(oracle_mod),
        lambda: test_i8_brute_force_python_ints(oracle_mod, 1),
        lambda: test_i8_debug_mode_closed_form(oracle_mod),
        lambda: test_dequant_matches_numpy(oracle_mod),
        lambda: test_half_encode_matches_numpy_rne(oracle_mod),
        lambda: test_bf16_decode_exhaustive(oracle_mod),
        lambda: test_bf16_brute_force_exact_rational(oracle_mod, 0),
        lambda: test_fp8_decode_exhaustive(oracle_mod),
        lambda: test_fp8_brute_force_exact_rational(oracle_mod, 0),
        lambda: test_fp8_brute_force_exact_rational(oracle_mod, 3),
    ]
    caught = 0
    for chk in checks:
        try:
            chk()
        except AssertionError:
            caught += 1
    del lib
    monkeypatch.setattr(oracle_mod, "_lib", saved)
    assert caught > 0, f"mutation {idx} went unnoticed"


# ----------------------------------------------------------------------------
# hand-worked fixtures (tests/golden)
# ----------------------------------------------------------------------------

def test_golden_f16_hand(orc):
    from golden_io import load
    g = load("f16_hand.txt")
    shards = [g["shard0"].astype(np.float16), g["shard1"].astype(np.float16)]
    C, _ = orc.ag_gemm_f16(shards, g["B"].astype(np.float16))
    assert np.array_equal(C, g["C"].astype(np.float32))


def test_golden_i8_hand(orc):
    from golden_io import load
    g = load("i8_hand.txt")
    # the last shard holds -128, outside the workloads' draw range but a
    # valid int8 value; it exercises the most negative input
    shards = [g[f"shard{s}"].astype(np.int8) for s in range(3)]
    acc, D = orc.ag_gemm_i8_dequant(shards, g["B"].astype(np.int8),
                                    g["bias"][0].astype(np.int32),
                                    g["scale"][0].astype(np.float32))
    assert np.array_equal(acc, g["acc"].astype(np.int32))
    assert np.array_equal(D.astype(np.float64), g["D"])


# ----------------------------------------------------------------------------
# bf16 x bf16 -> fp32 (the fp16 definition with bfloat16 inputs)
# ----------------------------------------------------------------------------

def bf16_ref(h):
    """bfloat16 bits -> float64 through numpy's own binary32 decoding: a
    bfloat16 is the upper half of a binary32."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def small_bf16(rng, shape):
    """bfloat16 values m * 2^e, |m| < 128, e in [-6, 3]: exactly
    representable (8 significant bits), sums of a few products exact."""
    m = rng.integers(-127, 128, shape)
    e = rng.integers(-6, 4, shape)
    return synth.to_bf16_bits((m * np.exp2(e)).astype(np.float32))


def test_bf16_decode_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint16)
    ours = orc.bf16_to_double(h)
    ref = bf16_ref(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_bf16_input_rounding_is_rne():
    """The generator's float32 -> bfloat16 rounding, against exact
    rational rounding of random values and of every tie pattern."""
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        ((np.arange(4096, dtype=np.uint32) << 16) | 0x8000).view(np.float32)])
    x = x[np.isfinite(x)]
    got = bf16_ref(synth.to_bf16_bits(x))
    for v, g in zip(x[::37], got[::37]):
        q = Fraction(float(v))
        lo = bf16_ref(np.array([(np.float32(v).view(np.uint32) >> 16)], np.uint16))[0]
        hi = bf16_ref(np.array([(np.float32(v).view(np.uint32) >> 16) + 1], np.uint16))[0]
        d_lo, d_hi = abs(q - Fraction(lo)), abs(Fraction(hi) - q)
        if d_lo < d_hi:
            want = lo
        elif d_hi < d_lo:
            want = hi
        else:   # tie: the even bit pattern
            want = lo if (int(np.float32(v).view(np.uint32) >> 16) % 2 == 0) else hi
        assert g == want, (v, g, want)


@pytest.mark.parametrize("seed", range(8))
def test_bf16_brute_force_exact_rational(orc, seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(1, 4))
    K = int(rng.integers(1, 9))
    N = int(rng.integers(1, 9))
    M = n * S
    A = small_bf16(rng, (M, K))
    B = small_bf16(rng, (K, N))
    C, S_abs = orc.ag_gemm_bf16(synth.split_rows(A, n), B)
    Af = [[Fraction(float(v)) for v in row] for row in bf16_ref(A)]
    Bf = [[Fraction(float(v)) for v in row] for row in bf16_ref(B)]
    for i in range(M):
        for j in range(N):
            exact = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            mag = sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0))
            want = frac_to_f32(exact)
            assert f32_bits(C[i, j]) == f32_bits(want) or \
                (C[i, j] == 0 and want == 0), (i, j, C[i, j], want)
            assert Fraction(float(S_abs[i, j])) == mag


def test_bf16_closed_forms(orc):
    """B = I gives C = A; all-ones gives K."""
    A, _ = synth.make_bf16(48, 32, 32, 3, "normal", 5100)
    B = synth.to_bf16_bits(np.eye(32, dtype=np.float32))
    C, _ = orc.ag_gemm_bf16(A, B)
    assert np.array_equal(C.astype(np.float64), bf16_ref(np.concatenate(A)))
    K = 1000
    ones = synth.to_bf16_bits(np.ones((8, K), np.float32))
    C1, S1 = orc.ag_gemm_bf16([ones] * 4, synth.to_bf16_bits(np.ones((K, 24), np.float32)))
    assert np.all(C1 == np.float32(K)) and np.all(S1 == K)


def test_bf16_matches_numpy_float64_and_permutation(orc):
    shards, B = synth.make_bf16(36 * 3, 45, 29, 3, "normal", 5200)
    C, S_abs = orc.ag_gemm_bf16(shards, B)
    A64 = bf16_ref(np.concatenate(shards))
    B64 = bf16_ref(B)
    ref = A64 @ B64
    mag = np.abs(A64) @ np.abs(B64)
    assert np.all(np.abs(C.astype(np.float64) - ref) <= 1e-12 * mag + 2**-24 * np.abs(ref))
    perm = [2, 0, 1]
    Cp, _ = orc.ag_gemm_bf16([shards[p] for p in perm], B)
    S = 36
    for dst, src in enumerate(perm):
        assert np.array_equal(Cp[dst * S:(dst + 1) * S], C[src * S:(src + 1) * S])


# ----------------------------------------------------------------------------
# fp8 (OCP E4M3) x fp8 -> fp32 (the fp16 definition with E4M3 inputs)
# ----------------------------------------------------------------------------

def fp8_ref(h):
    """E4M3 bits -> float64 through torch's own float8_e4m3fn decoding."""
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(np.ascontiguousarray(h, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def random_fp8(rng, shape):
    """Random E4M3 codes, NaN codes excluded."""
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)


def test_fp8_decode_exhaustive(orc):
    h = np.arange(256, dtype=np.uint8)
    ours = orc.fp8_to_double(h)
    ref = fp8_ref(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed forms of the format: 1.0, the largest value, the smallest
    # normal and subnormal, negative zero
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_fp8_input_rounding_matches_torch():
    """The generator's float32 -> E4M3 rounding, against torch's
    float8_e4m3fn cast on random values and on every tie."""
    torch = pytest.importorskip("torch")
    v = synth._e4m3_values()
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    x = np.concatenate([np.random.default_rng(6).standard_normal(50000).astype(np.float32) * 8,
                        mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.to_fp8e4m3_bits(x), ref)


@pytest.mark.parametrize("seed", range(8))
def test_fp8_brute_force_exact_rational(orc, seed):
    rng = np.random.default_rng(400 + seed)
    n = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(1, 4))
    K = int(rng.integers(1, 9))
    N = int(rng.integers(1, 9))
    M = n * S
    A = random_fp8(rng, (M, K))
    B = random_fp8(rng, (K, N))
    C, S_abs = orc.ag_gemm_fp8(synth.split_rows(A, n), B)
    Af = [[Fraction(float(v)) for v in row] for row in fp8_ref(A)]
    Bf = [[Fraction(float(v)) for v in row] for row in fp8_ref(B)]
    for i in range(M):
        for j in range(N):
            exact = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            mag = sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0))
            want = frac_to_f32(exact)
            assert f32_bits(C[i, j]) == f32_bits(want) or \
                (C[i, j] == 0 and want == 0), (i, j, C[i, j], want)
            assert Fraction(float(S_abs[i, j])) == mag


def test_fp8_closed_forms(orc):
    """B = I gives C = A; all-ones gives K."""
    A, _ = synth.make_fp8(48, 32, 32, 3, "normal", 5300)
    B = synth.to_fp8e4m3_bits(np.eye(32, dtype=np.float32))
    C, _ = orc.ag_gemm_fp8(A, B)
    assert np.array_equal(C.astype(np.float64), fp8_ref(np.concatenate(A)))
    K = 1000
    ones = synth.to_fp8e4m3_bits(np.ones((8, K), np.float32))
    C1, S1 = orc.ag_gemm_fp8([ones] * 4, synth.to_fp8e4m3_bits(np.ones((K, 24), np.float32)))
    assert np.all(C1 == np.float32(K)) and np.all(S1 == K)


def test_fp8_matches_numpy_float64_and_permutation(orc):
    shards, B = synth.make_fp8(36 * 3, 45, 29, 3, "normal", 5400)
    C, S_abs = orc.ag_gemm_fp8(shards, B)
    A64 = fp8_ref(np.concatenate(shards))
    B64 = fp8_ref(B)
    ref = A64 @ B64
    mag = np.abs(A64) @ np.abs(B64)
    assert np.all(np.abs(C.astype(np.float64) - ref) <= 1e-12 * mag + 2**-24 * np.abs(ref))
    perm = [1, 2, 0]
    Cp, _ = orc.ag_gemm_fp8([shards[p] for p in perm], B)
    S = 36
    for dst, src in enumerate(perm):
        assert np.array_equal(Cp[dst * S:(dst + 1) * S], C[src * S:(src + 1) * S])
