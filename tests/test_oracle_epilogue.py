"""Pins of the fused-epilogue oracle (oracle/epilogue.py) and its parity bound.

The epilogue's definition, act(alpha * sum_k a_ik b_kj + beta * c_ij + bias_j),
is recomputed here with exact rational arithmetic on small dyadic inputs, so a
dropped term, a wrong sign, a bias applied per row instead of per column, or a
ReLU on the wrong side of zero fails.  The bound is checked against an fp32
emulation of the GPU's arithmetic (it must accept it) and against planted
errors (it must reject them)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.parity import TOL_MFMA, bound_epilogue, check

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def dyadic(rng, shape, lo=-8, hi=8, den=4):
    return rng.integers(lo * den, hi * den + 1, size=shape).astype(np.float64) / den


def brute(A, B, alpha, beta, Cold, bias, relu):
    M, K = A.shape
    N = B.shape[1]
    out = np.empty((M, N), dtype=np.float64)
    for i in range(M):
        for j in range(N):
            s = sum(Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K))
            v = Fraction(alpha) * s
            if beta != 0.0:
                v += Fraction(beta) * Fraction(float(Cold[i, j]))
            if bias is not None:
                v += Fraction(float(bias[j]))
            if relu and v < 0:
                v = Fraction(0)
            out[i, j] = float(v)
    return out


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 2), (5, 3, 7), (4, 4, 4), (2, 9, 13)])
@pytest.mark.parametrize("alpha,beta,use_bias,relu", [
    (1.0, 0.0, False, False), (-1.5, 0.0, False, False), (1.0, 0.75, False, False),
    (0.5, -2.0, True, False), (1.0, 0.0, True, True), (-0.25, 1.0, True, True),
])
def test_epilogue_matches_rational_brute_force(M, N, K, alpha, beta, use_bias, relu):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = dyadic(rng, (M, K)).astype(np.float32)
    B = dyadic(rng, (K, N)).astype(np.float32)
    Cold = dyadic(rng, (M, N))
    bias = dyadic(rng, (N,)) if use_bias else None
    C64, _ = oracle.gemm("f32", A, B)
    E, T = oracle.epilogue(C64, alpha, beta, Cold, bias, relu)
    want = brute(A, B, alpha, beta, Cold, bias, relu)
    assert np.array_equal(E, want)
    assert np.all(T >= np.abs(E) - 1e-300) or relu


def test_identity_parameters_give_the_plain_product():
    rng = np.random.default_rng(7)
    C64 = rng.standard_normal((6, 5))
    E, T = oracle.epilogue(C64, 1.0)
    assert np.array_equal(E, C64)
    assert np.array_equal(T, np.abs(C64))


def test_bias_is_per_column():
    C64 = np.zeros((2, 3))
    E, _ = oracle.epilogue(C64, 1.0, bias64=np.array([1.0, 2.0, 3.0]))
    assert np.array_equal(E, [[1.0, 2.0, 3.0], [1.0, 2.0, 3.0]])
    with pytest.raises(ValueError):
        oracle.epilogue(C64, 1.0, bias64=np.array([1.0, 2.0]))


def test_relu_clamps_negatives_and_keeps_nan():
    C64 = np.array([[-2.0, -0.5, 0.0, 0.5, np.nan]])
    E, _ = oracle.epilogue(C64, 1.0, relu=True)
    assert np.array_equal(E[0, :4], [0.0, 0.0, 0.0, 0.5])
    assert np.isnan(E[0, 4])


def test_zero_beta_never_reads_old_c():
    C64 = np.ones((2, 2))
    E, _ = oracle.epilogue(C64, 2.0, 0.0, np.full((2, 2), np.nan))
    assert np.array_equal(E, np.full((2, 2), 2.0))
    with pytest.raises(ValueError):
        oracle.epilogue(C64, 1.0, 0.5, None)


def gpu_like(C64, S, alpha, beta, Cold, bias, relu, out, rng, drop_bias=False):
    """fp32 emulation of the GPU's epilogue on an fp32 sum off by up to tol*S."""
    s = (C64 + rng.uniform(-1, 1, C64.shape) * TOL_MFMA * S * 0.999).astype(np.float32)
    v = np.float32(alpha) * s
    if beta != 0.0:
        v = v + np.float32(beta) * Cold.astype(np.float32)
    if bias is not None and not drop_bias:
        v = v + bias.astype(np.float32).reshape(1, -1)
    if relu:
        v = np.where(v < 0, np.float32(0), v)
    return oracle.widen(out, oracle.round_to(out, v.astype(np.float64)))


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_bound_accepts_gpu_arithmetic_and_rejects_planted_errors(out):
    rng = np.random.default_rng({"f32": 1, "bf16": 2, "f16": 3}[out])
    M, N, K = 48, 40, 64
    A = oracle.round_to("bf16", rng.standard_normal((M, K)))
    B = oracle.round_to("bf16", rng.standard_normal((K, N)))
    C64, S = oracle.gemm("bf16", A, B)
    Cold = oracle.widen(out, oracle.round_to(out, rng.standard_normal((M, N)) * 4))
    bias = rng.standard_normal(N) * 3
    alpha, beta = -1.75, 0.5
    E, T = oracle.epilogue(C64, alpha, beta, Cold, bias, True)
    b = bound_epilogue(E, T, S, alpha, TOL_MFMA, out)
    good = gpu_like(C64, S, alpha, beta, Cold, bias, True, out, rng)
    assert check(good, E, S, TOL_MFMA, out, b=b)["ok"]
    # planted: the bias left out, or the error pushed just past the bound
    bad = gpu_like(C64, S, alpha, beta, Cold, bias, True, out, rng, drop_bias=True)
    assert not check(bad, E, S, TOL_MFMA, out, b=b)["ok"]
    pushed = E.copy()
    pushed[3, 4] += 1.01 * b[3, 4] * (1 if E[3, 4] >= 0 else -1)
    assert not check(pushed, E, S, TOL_MFMA, out, b=b)["ok"]


# ---------------------------------------------------------------- the 3 x bf16 split's error

def _bf16_rne(x64):
    return oracle.widen("bf16", oracle.round_to("bf16", x64))


def test_three_product_bf16_split_error_bound():
    """The fp32-via-3xbf16 path takes x = hi + lo with hi = bf16(x), lo =
    bf16(x - hi) (nearest even; x - hi is exact in fp32) and a*b as
    ah*bh + ah*bl + al*bh.  Each term is exact in fp32 (8 x 8 significant bits),
    so per product the error is the dropped al*bl plus the two lo truncations:
    at most about 3 * 2^-16 |a b|.  The parity tolerance of that path (1e-4 S)
    rests on this; checked here on random fp32 values and on values built to
    make lo as large as possible."""
    rng = np.random.default_rng(8000)
    a = rng.standard_normal(200000).astype(np.float32).astype(np.float64)
    b = (rng.standard_normal(200000) * 1e3).astype(np.float32).astype(np.float64)
    # worst cases: mantissas whose low 16 bits sit just below a bf16 rounding tie
    worst = np.array([1.0 + 2.0 ** -8 - 2.0 ** -23, 1.0 + 2.0 ** -9 - 2.0 ** -23, 1.99609363079071])
    a = np.concatenate([a, worst, -worst])
    b = np.concatenate([b, worst[::-1], worst])
    ah, bh = _bf16_rne(a), _bf16_rne(b)
    al, bl = _bf16_rne(a - ah), _bf16_rne(b - bh)
    approx = ah * bh + ah * bl + al * bh
    rel = np.abs(approx - a * b) / np.abs(a * b)
    assert rel.max() <= 3 * 2.0 ** -16
    # and the split is not exact, so the bound is not vacuous
    assert rel.max() > 2.0 ** -20
