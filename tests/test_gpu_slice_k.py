"""The slice-K kernel through the C ABI, against the oracle.

Slice-K splits K across the waves of one workgroup (each wave an equal run of
32-k blocks over the whole tile) and sums the waves' partial tiles in LDS, in
wave order.  It runs fp32 inputs on the fp32 matrix instruction and, for the
3 x bf16 path, on three bf16 products per term.  Each instantiation (32 x 32
tiles with 4 or 8 waves, 64 x 64 tiles with 4, for both formats) is forced
through the plan override on shapes with ragged tiles in M and N, a ragged
last 32-k block, fewer blocks than waves (idle waves), and more workgroups
than CUs.  Integer inputs keep every partial sum exact (and their bf16 lo
parts zero), so C must equal the oracle's rounding bit for bit whatever order
the waves' sums take; NaN in the operands' row padding must not reach C (A's
columns past K are zeroed, B's rows past K read as zeros).  Also: the fused
epilogue, normal-distribution parity within the tolerance, the planner's own
slice-K plans, and the 128 x 128 grid kernels' ragged edges, which small
shapes no longer reach without the override."""
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

VARIANTS = [(fmt, tile, waves) for fmt in ("f32", "f32x3")
            for tile, waves in ((32, 4), (32, 8), (64, 4))]
SHAPES = [(1, 1, 1), (33, 65, 7), (300, 264, 200), (257, 130, 1000), (100, 37, 4104),
          (64, 64, 31), (2000, 1500, 300)]


@pytest.fixture(autouse=True)
def clear_override():
    yield
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)


def force(fmt, tile, waves):
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, tile, tile, waves)
    p = dg.gemm_ex_plan(fmt, 64, 64, 64, 0)
    assert (p["tile_rows"], p["splits"], p["workspace_bytes"]) == (tile, 1, 0), p


def run(A, B, *, alpha=1.0, beta=0.0, Cold=None, bias=None, relu=False, ws=False, fmt="f32"):
    M, K = A.shape
    N = B.shape[1]
    Ad = dev_matrix(A, "f32", round_pitch(K, "f32", 8))
    Bd = dev_matrix(B, "f32", round_pitch(N, "f32", 8))
    Cd = sentinel_c(M, N, "f32")
    if Cold is not None:
        Cd[:] = to_torch_cpu(Cold, "f32").to("cuda")
    bd = torch.from_numpy(bias).to("cuda") if bias is not None else None
    w = torch.empty(1 << 20, dtype=torch.uint8, device="cuda") if ws else None
    torch.cuda.synchronize()
    dg.gemm_ex(Ad, Bd, Cd, alpha=alpha, beta=beta, bias=bd, relu=relu, workspace=w, in_fmt=fmt)
    torch.cuda.synchronize()
    return Cd


@pytest.mark.parametrize("fmt,tile,waves", VARIANTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_exact_integers_bitwise(fmt, tile, waves, M, N, K):
    force(fmt, tile, waves)
    print(f"case slicek {fmt} {tile}/{waves} int {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "ints", "f32", seed=7000 + M + N + K)
    C = run(A, B, fmt=fmt)
    C64, _ = oracle.gemm("f32", A, B)
    assert np.array_equal(to64(C), C64)
    assert gap_untouched(C)
    C2 = run(A, B, fmt=fmt)
    assert torch.equal(C, C2)


@pytest.mark.parametrize("fmt,tile,waves", VARIANTS)
@pytest.mark.parametrize("M,N,K", [(300, 264, 200), (100, 37, 4104), (512, 512, 512)])
def test_normal_inputs_within_the_tolerance(fmt, tile, waves, M, N, K):
    force(fmt, tile, waves)
    print(f"case slicek {fmt} {tile}/{waves} normal {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "normal", "f32", seed=7100 + M + K)
    C = run(A, B, fmt=fmt)
    C64, S = oracle.gemm("f32", A, B)
    res = oracle.check(to64(C), C64, S, TOL_MFMA, "f32")
    assert res["ok"], res


@pytest.mark.parametrize("fmt,tile,waves", VARIANTS)
@pytest.mark.parametrize("alpha,beta,use_bias,relu", [(0.75, -1.0, True, True),
                                                      (-1.5, 0.5, False, False),
                                                      (1.0, 0.0, True, False)])
def test_fused_epilogue(fmt, tile, waves, alpha, beta, use_bias, relu):
    force(fmt, tile, waves)
    M, N, K = 257, 130, 1000
    print(f"case slicek {fmt} {tile}/{waves} epilogue a={alpha} b={beta} bias={use_bias} "
          f"relu={relu}", flush=True)
    rng = np.random.default_rng(7200 + tile + waves + (10 if relu else 0))
    A = draw(rng, (M, K), "normal", "f32")
    B = draw(rng, (K, N), "normal", "f32")
    Cold = draw(rng, (M, N), "normal", "f32") if beta != 0.0 else None
    bias = rng.standard_normal(N).astype(np.float32) if use_bias else None
    C = run(A, B, alpha=alpha, beta=beta, Cold=Cold, bias=bias, relu=relu, fmt=fmt)
    C64, S = oracle.gemm("f32", A, B)
    E, T = oracle.epilogue(C64, alpha, beta, None if Cold is None else oracle.widen("f32", Cold),
                           None if bias is None else bias.astype(np.float64), relu)
    b = bound_epilogue(E, T, S, alpha, TOL_MFMA, "f32")
    res = oracle.check(to64(C), E, S, TOL_MFMA, "f32", b=b)
    assert res["ok"], res
    assert gap_untouched(C)


@pytest.mark.parametrize("fmt,tile,waves", VARIANTS)
def test_k_zero_applies_the_epilogue_to_the_empty_sum(fmt, tile, waves):
    force(fmt, tile, waves)
    rng = np.random.default_rng(7300)
    M, N = 70, 90
    A = np.zeros((M, 0), dtype=np.float32)
    B = np.zeros((0, N), dtype=np.float32)
    Cold = draw(rng, (M, N), "normal", "f32")
    bias = rng.standard_normal(N).astype(np.float32)
    C = run(A, B, alpha=3.0, beta=-0.5, Cold=Cold, bias=bias, relu=True, fmt=fmt)
    E, T = oracle.epilogue(np.zeros((M, N)), 3.0, -0.5, oracle.widen("f32", Cold),
                           bias.astype(np.float64), True)
    b = bound_epilogue(E, T, np.zeros((M, N)), 3.0, TOL_MFMA, "f32")
    assert oracle.check(to64(C), E, np.zeros((M, N)), TOL_MFMA, "f32", b=b)["ok"]


@pytest.mark.parametrize("fmt,M,N,K,tile", [
    ("f32", 512, 512, 512, 32), ("f32", 256, 256, 4096, 32), ("f32", 1024, 1024, 1024, 64),
    ("f32", 96, 64, 2048, 32), ("f32", 1536, 1536, 300, 32),
    ("f32x3", 512, 512, 512, 32), ("f32x3", 256, 256, 2048, 32), ("f32x3", 1024, 1024, 1024, 64),
    ("f32x3", 2048, 512, 512, 64), ("f32x3", 768, 640, 520, 32)])
def test_planner_plans(fmt, M, N, K, tile):
    """The planner's own slice-K plans (no override), offered a workspace they
    do not take: every element of C against the oracle."""
    p = dg.gemm_ex_plan(fmt, M, N, K, 1 << 20)
    assert (p["tile_rows"], p["splits"], p["workspace_bytes"]) == (tile, 1, 0), p
    print(f"case slicek planner {fmt} {M}x{N}x{K} plan {p}", flush=True)
    A, B = pair(M, N, K, "uniform", "f32", seed=7400 + M + K)
    C = run(A, B, ws=True, fmt=fmt)
    C64, S = oracle.gemm("f32", A, B)
    res = oracle.check(to64(C), C64, S, TOL_MFMA, "f32")
    assert res["ok"], res
    assert gap_untouched(C)


@pytest.mark.parametrize("fmt", ["f32", "f32x3"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (33, 65, 7), (300, 264, 200), (257, 130, 1000),
                                   (1000, 700, 1100)])
def test_128_tile_ragged_edges_when_forced(fmt, M, N, K):
    """Shapes this small now plan slice-K; forced onto the 128 x 128 grid
    kernels they keep those kernels' ragged-edge handling covered (integer
    inputs, bit for bit, NaN row padding)."""
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 128, 128, 1)
    assert dg.gemm_ex_plan(fmt, M, N, K, 0)["tile_rows"] == 128
    print(f"case grid128 forced {fmt} int {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "ints", "f32", seed=7500 + M + N + K)
    C = run(A, B, fmt=fmt)
    C64, _ = oracle.gemm("f32", A, B)
    assert np.array_equal(to64(C), C64)
    assert gap_untouched(C)


@pytest.mark.parametrize("fmt,tile,waves", VARIANTS)
def test_very_deep_k_all_ones(fmt, tile, waves):
    """K = 2^20 + 37 (32769 blocks of 32 k, the last one ragged, shared among the
    waves; NaN in A's row padding past K): with all-ones inputs every element of
    C is exactly K (< 2^24, so exact in fp32; the bf16 lo parts are zero), a
    closed form the oracle's definition gives at any size."""
    force(fmt, tile, waves)
    M, N, K = 96, 72, (1 << 20) + 37
    print(f"case slicek {fmt} {tile}/{waves} all-ones K={K}", flush=True)
    A = torch.full((M, round_pitch(K, "f32")), float("nan"), device="cuda")[:, :K]
    A.fill_(1.0)  # NaN stays in the row padding past K
    B = torch.ones((K, N), dtype=torch.float32, device="cuda")
    C = sentinel_c(M, N, "f32")
    dg.gemm_ex(A, B, C, in_fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(to64(C), np.full((M, N), float(K)))
    assert gap_untouched(C)
