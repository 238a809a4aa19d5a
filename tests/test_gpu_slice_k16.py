"""The bf16 / fp16 slice-K kernel through the C ABI, against the oracle.

The 16-bit slice-K kernel (slicek16.hip) splits K across the waves of one
workgroup in 64-k blocks, moves each wave's B block through its own LDS region
and reads it back with the LDS transpose read, and sums the waves' partial
tiles in LDS in wave order.  Each instantiation (32 x 32 tiles with 4 or 8
waves, 64 x 64 tiles with 4), for both input formats and both C formats, is
forced through the plan override on shapes with ragged tiles in M and N, a
ragged last 64-k block (and K shorter than one block), fewer blocks than waves
(idle waves), and more workgroups than CUs.  Integer inputs keep every partial
sum exact, so C must equal the oracle's (rounded, for 16-bit C) bit for bit
whatever order the waves' sums take; NaN in the operands' row padding must not
reach C.  Also: normal-distribution parity within the tolerance, the fused
epilogue and K = 0."""
import numpy as np
import pytest
import torch

import dense_gemm_matrix_amd as dg
import oracle
from oracle.parity import TOL_MFMA, bound_epilogue
from synth_inputs import draw, pair
from synth_inputs import to_torch as to_torch_cpu
from tests.gpu_util import dev_matrix, gap_untouched, round_pitch, sentinel_c, to64

pytestmark = pytest.mark.gpu

TILES = [(32, 4), (32, 8), (64, 4)]
FORMATS = [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")]
VARIANTS = [(fmt, out, t, w) for fmt, out in FORMATS for t, w in TILES]
SHAPES = [(1, 1, 1), (33, 65, 7), (300, 264, 200), (257, 130, 1000), (100, 37, 4104),
          (64, 64, 63), (2000, 1500, 300)]


@pytest.fixture(autouse=True)
def clear_override():
    yield
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)


def force(fmt, out, tile, waves):
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, tile, tile, waves)
    p = dg.gemm_ex_plan(fmt, 64, 64, 64, 0, out_same=(out != "f32"))
    assert (p["tile_rows"], p["splits"], p["workspace_bytes"]) == (tile, 1, 0), p


def run(fmt, out, A, B, *, alpha=1.0, beta=0.0, Cold=None, bias=None, relu=False):
    M, K = A.shape
    N = B.shape[1]
    Ad = dev_matrix(A, fmt, round_pitch(K, fmt, 8))
    Bd = dev_matrix(B, fmt, round_pitch(N, fmt, 8))
    Cd = sentinel_c(M, N, out)
    if Cold is not None:
        Cd[:] = to_torch_cpu(Cold, out).to("cuda")
    bd = torch.from_numpy(bias).to("cuda") if bias is not None else None
    torch.cuda.synchronize()
    dg.gemm_ex(Ad, Bd, Cd, alpha=alpha, beta=beta, bias=bd, relu=relu)
    torch.cuda.synchronize()
    return Cd


def expect_exact(out, C64):
    return C64 if out == "f32" else oracle.widen(out, oracle.round_to(out, C64))


@pytest.mark.parametrize("fmt,out,tile,waves", VARIANTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_exact_integers_bitwise(fmt, out, tile, waves, M, N, K):
    force(fmt, out, tile, waves)
    print(f"case slicek16 {fmt}->{out} {tile}/{waves} int {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "ints", fmt, seed=7600 + M + N + K)
    C = run(fmt, out, A, B)
    C64, _ = oracle.gemm(fmt, A, B)
    assert np.array_equal(to64(C), expect_exact(out, C64))
    assert gap_untouched(C)
    C2 = run(fmt, out, A, B)
    assert torch.equal(C, C2)


@pytest.mark.parametrize("fmt,out,tile,waves", VARIANTS)
@pytest.mark.parametrize("M,N,K", [(300, 264, 200), (100, 37, 4104), (512, 512, 512)])
def test_normal_inputs_within_the_tolerance(fmt, out, tile, waves, M, N, K):
    force(fmt, out, tile, waves)
    print(f"case slicek16 {fmt}->{out} {tile}/{waves} normal {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "normal", fmt, seed=7700 + M + K)
    C = run(fmt, out, A, B)
    C64, S = oracle.gemm(fmt, A, B)
    res = oracle.check(to64(C), C64, S, TOL_MFMA, out)
    assert res["ok"], res


@pytest.mark.parametrize("fmt,out,tile,waves", VARIANTS)
@pytest.mark.parametrize("alpha,beta,use_bias,relu", [(0.75, -1.0, True, True),
                                                      (-1.5, 0.5, False, False)])
def test_fused_epilogue(fmt, out, tile, waves, alpha, beta, use_bias, relu):
    force(fmt, out, tile, waves)
    M, N, K = 257, 130, 1000
    print(f"case slicek16 {fmt}->{out} {tile}/{waves} epilogue a={alpha} b={beta} "
          f"bias={use_bias} relu={relu}", flush=True)
    rng = np.random.default_rng(7800 + tile + waves + (10 if relu else 0))
    A = draw(rng, (M, K), "normal", fmt)
    B = draw(rng, (K, N), "normal", fmt)
    Cold = draw(rng, (M, N), "normal", out) if beta != 0.0 else None
    bias = rng.standard_normal(N).astype(np.float32) if use_bias else None
    C = run(fmt, out, A, B, alpha=alpha, beta=beta, Cold=Cold, bias=bias, relu=relu)
    C64, S = oracle.gemm(fmt, A, B)
    E, T = oracle.epilogue(C64, alpha, beta, None if Cold is None else oracle.widen(out, Cold),
                           None if bias is None else bias.astype(np.float64), relu)
    b = bound_epilogue(E, T, S, alpha, TOL_MFMA, out)
    res = oracle.check(to64(C), E, S, TOL_MFMA, out, b=b)
    assert res["ok"], res
    assert gap_untouched(C)


@pytest.mark.parametrize("fmt,out,tile,waves", VARIANTS)
def test_k_zero_applies_the_epilogue_to_the_empty_sum(fmt, out, tile, waves):
    force(fmt, out, tile, waves)
    rng = np.random.default_rng(7900)
    M, N = 70, 90
    dtype = {"bf16": np.uint16, "f16": np.float16}[fmt]
    A = np.zeros((M, 0), dtype=dtype)
    B = np.zeros((0, N), dtype=dtype)
    Cold = draw(rng, (M, N), "normal", out)
    bias = rng.standard_normal(N).astype(np.float32)
    C = run(fmt, out, A, B, alpha=3.0, beta=-0.5, Cold=Cold, bias=bias, relu=True)
    E, T = oracle.epilogue(np.zeros((M, N)), 3.0, -0.5, oracle.widen(out, Cold),
                           bias.astype(np.float64), True)
    b = bound_epilogue(E, T, np.zeros((M, N)), 3.0, TOL_MFMA, out)
    assert oracle.check(to64(C), E, np.zeros((M, N)), TOL_MFMA, out, b=b)["ok"]


@pytest.mark.parametrize("fmt,out", FORMATS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (33, 65, 7), (300, 264, 200), (257, 130, 1000),
                                   (1000, 700, 1100)])
def test_128_tile_ragged_edges_when_forced(fmt, out, M, N, K):
    """16-bit outputs this small now plan slice-K; forced onto the 128 x 128
    grid kernel (4-stage ring: at most 256 workgroups) they keep its ragged-edge
    handling covered for both C formats (integer inputs, bit for bit, NaN row
    padding)."""
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 128, 128, 1)
    assert dg.gemm_ex_plan(fmt, M, N, K, 0, out_same=(out != "f32"))["tile_rows"] == 128
    print(f"case grid128 forced {fmt}->{out} int {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "ints", fmt, seed=8000 + M + N + K)
    C = run(fmt, out, A, B)
    C64, _ = oracle.gemm(fmt, A, B)
    assert np.array_equal(to64(C), expect_exact(out, C64))
    assert gap_untouched(C)


@pytest.mark.parametrize("fmt,out,tile,waves", VARIANTS)
def test_very_deep_k_all_ones(fmt, out, tile, waves):
    """K = 2^20 + 37 (16385 blocks of 64 k, the last one ragged, shared among the
    waves; NaN in A's row padding past K): with all-ones inputs every element of
    C is exactly K (rounded once to 16-bit C), a closed form the oracle's
    definition gives at any size."""
    force(fmt, out, tile, waves)
    M, N, K = 96, 72, (1 << 20) + 37
    print(f"case slicek16 {fmt}->{out} {tile}/{waves} all-ones K={K}", flush=True)
    dtype = {"bf16": torch.bfloat16, "f16": torch.float16}[fmt]
    A = torch.full((M, round_pitch(K, fmt)), float("nan"), dtype=dtype, device="cuda")[:, :K]
    A.fill_(1.0)  # NaN stays in the row padding past K
    B = torch.ones((K, N), dtype=dtype, device="cuda")
    C = sentinel_c(M, N, out)
    dg.gemm_ex(A, B, C)
    torch.cuda.synchronize()
    expect = expect_exact(out, np.full((M, N), float(K)))
    assert np.array_equal(to64(C), expect)
    assert gap_untouched(C)
