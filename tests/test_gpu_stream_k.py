"""Stream-K plans on the GPU (the nine-levels tutorial, section 2.9), through
the C ABI, against the oracle.

The plan is forced with dgemm_set_plan_override, so every case runs the
persistent Stream-K kernel whatever the cost model would pick.  Checks: every
element of C against the oracle (random data); bit for bit against the
oracle's rounding and the one-tile-per-workgroup plan (integer data, where
every partial sum is exact in fp32); the no-wait path (each reducer computes
every piece it does not find) bit for bit equal to the waiting path; the
fused epilogue; repeated and interleaved launches on one workspace (flags of
earlier launches are never taken); graph capture (Stream-K is not used there).
C is prefilled with NaN and its row-pitch gap must stay NaN; the workspace
bytes past what the plan uses must stay untouched."""
import numpy as np
import pytest
import torch

import dense_gemm_matrix_amd as dg
import oracle
from oracle.parity import TOL_MFMA, bound_epilogue
from synth_inputs import draw, pair, workload
from tests.gpu_util import dev_matrix, gap_untouched, round_pitch, sentinel_c, to64
from synth_inputs import to_torch as to_torch_cpu

pytestmark = pytest.mark.gpu

SK_WS = 2 * 256 * 256 * 256 * 4 + 256 * 8


@pytest.fixture
def stream_k():
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_STREAM_K)
    dg.dgemm_set_stream_k_wait_us(-1)
    yield
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
    dg.dgemm_set_stream_k_wait_us(-1)


def sk_plan(dtype, out, M, N, K):
    p = dg.gemm_ex_plan(dtype, M, N, K, SK_WS, out_same=(out != "f32"))
    assert p["stream_k"] and p["workspace_bytes"] == SK_WS, p
    return p


class Run:
    """Device copies of A and B (padded pitches, NaN gaps) and a workspace with
    a NaN-filled spare tail, for repeated gemm_ex calls."""

    def __init__(self, dtype, A, B, spare=4096):
        self.dtype = dtype
        self.M, self.K = A.shape
        self.N = B.shape[1]
        self.Ad = dev_matrix(A, dtype, round_pitch(self.K, dtype, 8))
        self.Bd = dev_matrix(B, dtype, round_pitch(self.N, dtype, 8))
        self.ws = torch.full(((SK_WS + spare) // 4,), float("nan"), dtype=torch.float32,
                             device="cuda")

    def __call__(self, out, *, alpha=1.0, beta=0.0, Cold=None, bias=None, relu=False):
        C = sentinel_c(self.M, self.N, out)
        if Cold is not None:
            C[:] = to_torch_cpu(Cold, out).to("cuda")
        bd = torch.from_numpy(np.asarray(bias, dtype=np.float32)).to("cuda") \
            if bias is not None else None
        torch.cuda.synchronize()
        dg.gemm_ex(self.Ad, self.Bd, C, alpha=alpha, beta=beta, bias=bd, relu=relu,
                   workspace=self.ws[: SK_WS // 4])
        torch.cuda.synchronize()
        return C

    def spare_untouched(self):
        return bool(torch.isnan(self.ws[SK_WS // 4:]).all().item())


# (dtype, C, M, N, K): ragged shapes; few tiles (XCDs without work); one tile
# over 32 workgroups (32 contributors); the one-GPU row share of 4096^3 (8
# workgroups per tile); 225 tiles (XCDs with 28 and 29); one whole tile per
# workgroup (256 tiles).
CASES = [("bf16", "f32", 300, 520, 8000), ("f16", "f16", 1000, 700, 2100),
         ("bf16", "f32", 256, 256, 2048), ("bf16", "bf16", 512, 4096, 4096),
         ("f16", "f32", 2304, 2560, 1024), ("bf16", "bf16", 3840, 3840, 1280),
         ("f16", "f32", 4096, 4096, 4096)]


@pytest.mark.parametrize("dtype,out,M,N,K", CASES)
def test_parity_every_element(stream_k, dtype, out, M, N, K):
    sk_plan(dtype, out, M, N, K)
    print(f"case sk-parity {dtype}->{out} {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "normal", dtype, seed=7000 + M + N + K)
    run = Run(dtype, A, B)
    C = run(out)
    C64, S = oracle.gemm(dtype, A, B)
    res = oracle.check(to64(C), C64, S, TOL_MFMA, out)
    assert res["ok"], res
    assert gap_untouched(C) and run.spare_untouched()


def test_ragged_workload_every_element(stream_k):
    """The 4000 x 3000 x 4104 bf16 workload (normal(0, 0.02), bf16 C) on the
    Stream-K plan: 192 tiles over 256 workgroups, every element against the
    oracle."""
    A, B, meta = workload("bf16_4000x3000x4104")
    M, N, K = meta["M"], meta["N"], meta["K"]
    sk_plan("bf16", "bf16", M, N, K)
    print(f"case sk-workload {M}x{N}x{K}", flush=True)
    run = Run("bf16", A, B)
    C = run("bf16")
    C64, S = oracle.gemm("bf16", A, B)
    res = oracle.check(to64(C), C64, S, TOL_MFMA, "bf16")
    assert res["ok"], res
    assert gap_untouched(C) and run.spare_untouched()


INT_CASES = [("f16", "f16", 4000, 3000, 4104), ("bf16", "f32", 256, 256, 2048),
             ("bf16", "f32", 3840, 3840, 1280), ("bf16", "bf16", 512, 4096, 4096)]


@pytest.mark.parametrize("dtype,out,M,N,K", INT_CASES)
def test_exact_integers_bitwise_against_the_oracle_and_the_grid_plan(stream_k, dtype, out, M, N,
                                                                      K):
    sk_plan(dtype, out, M, N, K)
    print(f"case sk-ints {dtype}->{out} {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "ints", dtype, seed=7100 + M + K)
    run = Run(dtype, A, B)
    C = run(out)
    C64, _ = oracle.gemm(dtype, A, B)
    assert np.max(np.abs(C64)) < 2 ** 24
    assert np.array_equal(to64(C), oracle.widen(out, oracle.round_to(out, C64)))
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 256, 256, 1)
    Cg = run(out)
    assert torch.equal(C, Cg)


@pytest.mark.parametrize("dtype,out,M,N,K", [("bf16", "bf16", 4000, 3000, 4104),
                                             ("bf16", "f32", 256, 256, 2048),
                                             ("f16", "f32", 512, 4096, 4096),
                                             ("bf16", "f32", 3840, 3840, 1280)])
def test_no_wait_path_is_bitwise_the_waiting_path(stream_k, dtype, out, M, N, K):
    """With a zero wait every reducer computes each piece of its tile it does
    not find already published; the results must not depend on which path
    ran."""
    sk_plan(dtype, out, M, N, K)
    print(f"case sk-nowait {dtype}->{out} {M}x{N}x{K}", flush=True)
    A, B = pair(M, N, K, "normal", dtype, seed=7200 + M + K)
    run = Run(dtype, A, B)
    C1 = run(out)
    dg.dgemm_set_stream_k_wait_us(0)
    C2 = run(out)
    C3 = run(out)
    dg.dgemm_set_stream_k_wait_us(-1)
    assert torch.equal(C1, C2) and torch.equal(C1, C3)
    assert run.spare_untouched()


@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"),
                                       ("f16", "f32")])
def test_fused_epilogue(stream_k, dtype, out):
    M, N, K = 1000, 700, 2100
    sk_plan(dtype, out, M, N, K)
    rng = np.random.default_rng(7300 + len(dtype + out))
    A = draw(rng, (M, K), "normal", dtype)
    B = draw(rng, (K, N), "normal", dtype)
    C64, S = oracle.gemm(dtype, A, B)
    run = Run(dtype, A, B)
    for alpha, beta, use_bias, relu in [(0.75, -1.0, True, True), (-1.5, 0.5, False, False),
                                        (1.0, 0.0, True, False)]:
        print(f"case sk-epilogue {dtype}->{out} a={alpha} b={beta} bias={use_bias} relu={relu}",
              flush=True)
        Cold = draw(rng, (M, N), "normal", out) if beta != 0.0 else None
        bias = rng.standard_normal(N).astype(np.float32) if use_bias else None
        C = run(out, alpha=alpha, beta=beta, Cold=Cold, bias=bias, relu=relu)
        E, T = oracle.epilogue(C64, alpha, beta, None if Cold is None else oracle.widen(out, Cold),
                               None if bias is None else bias.astype(np.float64), relu)
        b = bound_epilogue(E, T, S, alpha, TOL_MFMA, out)
        res = oracle.check(to64(C), E, S, TOL_MFMA, out, b=b)
        assert res["ok"], res
        assert gap_untouched(C)


@pytest.mark.parametrize("dtype,out,M,N,K", [("bf16", "bf16", 1000, 701, 2100),
                                             ("f16", "f16", 777, 1023, 4100),
                                             ("bf16", "f32", 513, 255, 3000)])
def test_odd_and_ragged_shapes_with_epilogue(stream_k, dtype, out, M, N, K):
    """Odd N (the per-element store path of 16-bit C), row and column counts
    one past or short of a tile, K ragged in its last piece; alpha, beta, bias
    and ReLU; every element against the oracle."""
    sk_plan(dtype, out, M, N, K)
    print(f"case sk-odd {dtype}->{out} {M}x{N}x{K}", flush=True)
    rng = np.random.default_rng(7600 + M + N)
    A = draw(rng, (M, K), "normal", dtype)
    B = draw(rng, (K, N), "normal", dtype)
    Cold = draw(rng, (M, N), "normal", out)
    bias = rng.standard_normal(N).astype(np.float32)
    run = Run(dtype, A, B)
    C = run(out, alpha=-0.5, beta=1.5, Cold=Cold, bias=bias, relu=True)
    C64, S = oracle.gemm(dtype, A, B)
    E, T = oracle.epilogue(C64, -0.5, 1.5, oracle.widen(out, Cold), bias.astype(np.float64), True)
    b = bound_epilogue(E, T, S, -0.5, TOL_MFMA, out)
    res = oracle.check(to64(C), E, S, TOL_MFMA, out, b=b)
    assert res["ok"], res
    assert gap_untouched(C) and run.spare_untouched()


def test_launches_sharing_one_workspace(stream_k):
    """Launches of two shapes interleaved on one workspace: each repeats its
    own first result bit for bit (a flag or partial left by another launch is
    never taken for this launch's)."""
    A1, B1 = pair(1000, 700, 2100, "normal", "bf16", seed=7400)
    A2, B2 = pair(300, 520, 8000, "normal", "bf16", seed=7401)
    r1 = Run("bf16", A1, B1)
    r2 = Run("bf16", A2, B2)
    r2.ws = r1.ws
    print("case sk-shared-workspace", flush=True)
    ref1, ref2 = r1("f32"), r2("bf16")
    for _ in range(3):
        assert torch.equal(r1("f32"), ref1)
        assert torch.equal(r2("bf16"), ref2)
    C64, S = oracle.gemm("bf16", A2, B2)
    assert oracle.check(to64(ref2), C64, S, TOL_MFMA, "bf16")["ok"]
    # back to back on the stream, no host synchronisation between them
    C = sentinel_c(1000, 700, "f32")
    torch.cuda.synchronize()
    for _ in range(4):
        dg.gemm_ex(r1.Ad, r1.Bd, C, workspace=r1.ws[: SK_WS // 4])
    torch.cuda.synchronize()
    assert torch.equal(C, ref1)


def test_graph_capture_takes_a_grid_plan(stream_k):
    """Under graph capture the Stream-K plan is not taken (a replay would reuse
    the launch's flag value); the captured plan replays the eager grid plan's
    result bit for bit, with eager work between the replays."""
    M, N, K = 1000, 700, 2100
    A, B = pair(M, N, K, "normal", "f16", seed=7500)
    run = Run("f16", A, B)
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
    assert not dg.gemm_ex_plan("f16", M, N, K, SK_WS, out_same=True)["stream_k"]
    print("case sk-graph eager", flush=True)
    ref = run("f16")
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_STREAM_K)
    C = sentinel_c(M, N, "f16")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dg.gemm_ex(run.Ad, run.Bd, C, workspace=run.ws[: SK_WS // 4])  # warm-up outside capture
        torch.cuda.synchronize()
        C.fill_(float("nan"))
        with torch.cuda.graph(g, stream=s):
            dg.gemm_ex(run.Ad, run.Bd, C, workspace=run.ws[: SK_WS // 4])
    torch.cuda.synchronize()
    print("case sk-graph replays", flush=True)
    for _ in range(3):
        C.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, ref)
        run("f16")  # eager work between replays
