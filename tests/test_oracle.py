"""Pins for the CPU oracle, each against something other than the oracle itself:
independent conversions (numpy, torch), exact rational arithmetic, closed forms
and exact integer products.  CPU only."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth_inputs import draw, to_storage

DTYPES = ["f32", "bf16", "f16"]


def exact_widen(dtype, x):
    """Independent widening: numpy (f32, f16) and torch (bf16)."""
    if dtype == "f32":
        return x.astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float64)
    t = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- widening

def test_widen_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    got = oracle.widen("f16", x)
    ref = x.astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # spot values from the binary16 definition
    assert oracle.widen("f16", np.array([0x3C00], np.uint16).view(np.float16))[0] == 1.0
    assert oracle.widen("f16", np.array([0x0001], np.uint16).view(np.float16))[0] == 2.0 ** -24
    assert oracle.widen("f16", np.array([0x7BFF], np.uint16).view(np.float16))[0] == 65504.0
    assert oracle.widen("f16", np.array([0xC000], np.uint16).view(np.float16))[0] == -2.0


def test_widen_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen("bf16", bits)
    ref = exact_widen("bf16", bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.widen("bf16", np.array([0x3F80], np.uint16))[0] == 1.0
    assert oracle.widen("bf16", np.array([0x0001], np.uint16))[0] == 2.0 ** -133


def test_widen_f32_random():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(10000).astype(np.float32) * np.float32(1e-30)
    x = np.concatenate([x, np.array([0, -0.0, 1e-45, 3.4e38], np.float32)])
    assert np.array_equal(oracle.widen("f32", x), x.astype(np.float64))


# ---------------------------------------------------------------- rounding

def _spread_values(rng, n):
    mags = np.exp2(rng.uniform(-160, 130, size=n))
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return sign * mags


def test_round_f16_matches_numpy_direct_conversion():
    rng = np.random.default_rng(12)
    x = np.concatenate([_spread_values(rng, 20000), rng.uniform(-70000, 70000, 5000),
                        rng.uniform(-1e-4, 1e-4, 5000)])
    # exact ties: odd multiples of half an fp16 ulp at several binades
    ties = (2 * rng.integers(0, 1024, 2000) + 1).astype(np.float64) * 2.0 ** -11 + 1.0
    x = np.concatenate([x, ties, ties * 2.0 ** -20, [65519.99, 65520.0, 65504.0, 2.0 ** -25,
                                                     3 * 2.0 ** -26, 2.0 ** -26]])
    got = oracle.round_to("f16", x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)      # numpy rounds float64 -> float16 directly
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def _bf16_nearest_ok(x, r_bits):
    """Brute force: r is a nearest bf16 to x, ties to an even significand."""
    if np.isinf(oracle.widen("bf16", np.array([r_bits], np.uint16))[0]):
        # overflow: x must be at least max + half an ulp
        return abs(x) >= (2 - 2.0 ** -8) * 2.0 ** 127
    cands = np.array([(int(r_bits) + d) & 0xFFFF for d in (-1, 0, 1)], np.uint16)
    vals = oracle.widen("bf16", cands)
    r = vals[1]
    for v in (vals[0], vals[2]):
        if np.isnan(v) or np.isinf(v) or np.sign(v) != np.sign(r) and r != 0:
            continue
        if abs(x - v) < abs(x - r):
            return False
        if abs(x - v) == abs(x - r) and (int(r_bits) & 1):
            return False
    return True


def test_round_bf16_nearest_even_brute_force():
    rng = np.random.default_rng(13)
    x = np.concatenate([_spread_values(rng, 3000), rng.standard_normal(2000)])
    got = oracle.round_to("bf16", x)
    for xi, gi in zip(x, got):
        assert _bf16_nearest_ok(float(xi), gi), (xi, hex(gi))


@pytest.mark.parametrize("x,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                   # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),               # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),      # above the tie: via fp32 this would double-round to 1.0
    (-1.0 - 2.0 ** -8 - 2.0 ** -30, 0xBF81),
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),      # halfway above the largest finite -> inf
    ((2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -40), 0x7F7F),
    (2.0 ** -133, 0x0001),                       # smallest subnormal
    (2.0 ** -134, 0x0000),                       # half of it: tie to even zero
    (0.0, 0x0000),
])
def test_round_bf16_fixed_cases(x, bits):
    assert int(oracle.round_to("bf16", np.array([x]))[0]) == bits


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(14)
    x = np.concatenate([_spread_values(rng, 20000), rng.standard_normal(5000)])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32)
    assert np.array_equal(oracle.round_to("f32", x).view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- the product

def _fraction_matmul(Aw, Bw):
    M, K = Aw.shape
    N = Bw.shape[1]
    Af = [[Fraction(float(v)) for v in row] for row in Aw]
    Bf = [[Fraction(float(v)) for v in row] for row in Bw]
    C = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    S = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    return C, S


SIZES = [1, 2, 3, 5, 8, 13, 17]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_brute_force_exact_rationals_16bit(dtype):
    """Every shape in SIZES^3.  bf16/fp16 values from N(0,1) have 8/11-bit
    significands in a narrow binade range, so every fp64 partial sum is exact and
    C64 must EQUAL the rational sum."""
    rng = np.random.default_rng(20 if dtype == "bf16" else 21)
    for M in SIZES:
        for N in SIZES:
            for K in SIZES:
                A = draw(rng, (M, K), "normal", dtype)
                B = draw(rng, (K, N), "normal", dtype)
                C64, S = oracle.gemm(dtype, A, B, nthreads=2)
                Cf, Sf = _fraction_matmul(exact_widen(dtype, A), exact_widen(dtype, B))
                for i in range(M):
                    for j in range(N):
                        assert Fraction(C64[i, j]) == Cf[i][j], (M, N, K, i, j)
                        assert Fraction(S[i, j]) == Sf[i][j], (M, N, K, i, j)


def test_brute_force_rationals_f32():
    """fp32 inputs: fp64 sums may round, by at most K * 2^-53 * S per element."""
    rng = np.random.default_rng(22)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 13, 8), (2, 17, 13), (31, 33, 65)]:
        A = draw(rng, (M, K), "uniform", "f32")
        B = draw(rng, (K, N), "uniform", "f32")
        C64, S = oracle.gemm("f32", A, B, nthreads=3)
        Cf, Sf = _fraction_matmul(exact_widen("f32", A), exact_widen("f32", B))
        for i in range(M):
            for j in range(N):
                tolf = Fraction(K) * Fraction(2) ** -53 * Sf[i][j]
                assert abs(Fraction(C64[i, j]) - Cf[i][j]) <= tolf
                assert abs(Fraction(S[i, j]) - Sf[i][j]) <= tolf


@pytest.mark.parametrize("dtype", DTYPES)
def test_identity(dtype):
    rng = np.random.default_rng(23)
    K, N = 37, 29
    B = draw(rng, (K, N), "normal", dtype)
    eye = to_storage(np.eye(K), dtype)
    C64, S = oracle.gemm(dtype, eye, B)
    assert np.array_equal(C64, exact_widen(dtype, B))
    assert np.array_equal(S, np.abs(exact_widen(dtype, B)))
    A = draw(rng, (N, K), "normal", dtype)
    C64, _ = oracle.gemm(dtype, A, eye)
    assert np.array_equal(C64, exact_widen(dtype, A))


@pytest.mark.parametrize("dtype", DTYPES)
def test_all_ones_gives_column_sums(dtype):
    rng = np.random.default_rng(24)
    M, K, N = 5, 300, 41
    B = draw(rng, (K, N), "ints", dtype)
    ones = to_storage(np.ones((M, K)), dtype)
    C64, _ = oracle.gemm(dtype, ones, B)
    colsum = np.array([math.fsum(col) for col in exact_widen(dtype, B).T])
    assert np.array_equal(C64, np.broadcast_to(colsum, (M, N)))
    C64, S = oracle.gemm(dtype, ones, to_storage(np.ones((K, N)), dtype))
    assert np.all(C64 == K) and np.all(S == K)


@pytest.mark.parametrize("dtype", DTYPES)
def test_rank_one_powers_of_two(dtype):
    rng = np.random.default_rng(25)
    M, K, N = 9, 77, 11
    x = np.exp2(rng.integers(-6, 6, M)) * np.where(rng.random(M) < 0.5, -1, 1)
    y = np.exp2(rng.integers(-6, 6, N)) * np.where(rng.random(N) < 0.5, -1, 1)
    A = to_storage(np.repeat(x[:, None], K, axis=1), dtype)
    B = to_storage(np.repeat(y[None, :], K, axis=0), dtype)
    C64, S = oracle.gemm(dtype, A, B)
    assert np.array_equal(C64, K * np.outer(x, y))
    assert np.array_equal(S, K * np.abs(np.outer(x, y)))


@pytest.mark.parametrize("dtype", DTYPES)
def test_integer_inputs_match_integer_matmul(dtype):
    rng = np.random.default_rng(26)
    M, K, N = 33, 257, 65
    A = draw(rng, (M, K), "ints", dtype)
    B = draw(rng, (K, N), "ints", dtype)
    Ai = exact_widen(dtype, A).astype(np.int64)
    Bi = exact_widen(dtype, B).astype(np.int64)
    C64, S = oracle.gemm(dtype, A, B)
    assert np.array_equal(C64, (Ai @ Bi).astype(np.float64))
    assert np.array_equal(S, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(27)
    A = draw(rng, (61, 203), "normal", "f32")
    B = draw(rng, (203, 47), "normal", "f32")
    ref = oracle.gemm("f32", A, B, nthreads=1)
    for t in (2, 3, 8, 64):
        got = oracle.gemm("f32", A, B, nthreads=t)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_row_subset_and_strided_views():
    rng = np.random.default_rng(28)
    A = draw(rng, (40, 70), "normal", "bf16")
    B = draw(rng, (70, 50), "normal", "bf16")
    full = oracle.gemm("bf16", A, B)
    rows = [39, 0, 17, 17]
    sub = oracle.gemm("bf16", A, B, rows=rows)
    assert np.array_equal(sub[0], full[0][rows])
    # same matrices embedded in wider buffers (row pitch > row length)
    Aw = np.zeros((40, 96), np.uint16); Aw[:, :70] = A
    Bw = np.full((70, 64), 0x7FC0, np.uint16); Bw[:, :50] = B   # NaN padding must be ignored
    view = oracle.gemm("bf16", Aw[:, :70], Bw[:, :50])
    assert np.array_equal(view[0], full[0]) and np.array_equal(view[1], full[1])


def test_zero_k_is_empty_sum():
    A = np.zeros((3, 0), np.float32)
    B = np.zeros((0, 4), np.float32)
    C64, S = oracle.gemm("f32", A, B)
    assert C64.shape == (3, 4) and np.all(C64 == 0) and np.all(S == 0)


# ---------------------------------------------------------------- pins catch planted mistakes

def test_pins_catch_planted_mistakes():
    """Emulate three plausible oracle mistakes on the CPU and confirm the exact
    checks above would fail them: a dropped k term, a transposed operand, a sign
    error in one product."""
    rng = np.random.default_rng(29)
    M, K, N = 3, 5, 7
    A = draw(rng, (M, K), "ints", "f32")
    B = draw(rng, (K, N), "ints", "f32")
    ref = exact_widen("f32", A).astype(np.int64) @ exact_widen("f32", B).astype(np.int64)
    dropped, _ = oracle.gemm("f32", np.ascontiguousarray(A[:, :-1]), np.ascontiguousarray(B[:-1]))
    assert not np.array_equal(dropped, ref)
    Bt = np.ascontiguousarray(draw(rng, (K, K), "ints", "f32"))
    sq, _ = oracle.gemm("f32", np.ascontiguousarray(A[:, :K]), Bt)
    tr, _ = oracle.gemm("f32", np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(Bt.T))
    assert not np.array_equal(sq, tr)
    flipped = A.copy(); flipped[0, 0] = -flipped[0, 0] if flipped[0, 0] != 0 else 1
    fl, _ = oracle.gemm("f32", flipped, B)
    assert not np.array_equal(fl, ref)


# ---------------------------------------------------------------- the parity rule

def test_parity_rule_accepts_correct_rounding_and_rejects_errors():
    rng = np.random.default_rng(30)
    A = draw(rng, (16, 512), "normal", "bf16")
    B = draw(rng, (512, 24), "normal", "bf16")
    C64, S = oracle.gemm("bf16", A, B)
    for out in ("f32", "bf16", "f16"):
        good = oracle.widen(out, oracle.round_to(out, C64))
        assert parity.check(good, C64, S, parity.TOL_MFMA, out)["ok"]
    # an fp32-accumulated sum in a different order passes
    fp32 = (exact_widen("bf16", A).astype(np.float32) @ exact_widen("bf16", B).astype(np.float32))
    assert parity.check(fp32.astype(np.float64), C64, S, parity.TOL_MFMA, "f32")["ok"]
    bad = C64.copy(); bad[3, 5] += 3 * parity.bound(C64, S, parity.TOL_MFMA, "f32")[3, 5]
    r = parity.check(bad, C64, S, parity.TOL_MFMA, "f32")
    assert not r["ok"] and r["first_bad"] == (3, 5) and r["n_bad"] == 1
    nan = C64.copy(); nan[0, 0] = np.nan
    assert not parity.check(nan, C64, S, parity.TOL_MFMA, "f32")["ok"]
    # dropping the last k term is far outside the bound for random data
    dropped, _ = oracle.gemm("bf16", np.ascontiguousarray(A[:, :-1]), np.ascontiguousarray(B[:-1]))
    assert not parity.check(dropped, C64, S, parity.TOL_MFMA, "f32")["ok"]
