"""gemm_ex on the GPU: the fused epilogue (alpha, beta, bias, ReLU) and split-K
plans, through the C ABI, against the oracle.

Epilogue results are compared with oracle.epilogue (fp64) within
oracle.parity.bound_epilogue; split-K results with the plain GEMM bound (the
split only changes the fp32 summation order), bit for bit where the inputs are
integers.  C is prefilled with NaN (so beta = 0 must never read it) and its row
pitch gap must stay NaN; the workspace bytes past what the plan uses must stay
untouched."""
import numpy as np
import pytest
import torch

import dense_gemm_matrix_amd as dg
import oracle
from oracle.parity import TOL_MFMA, bound_epilogue
from synth_inputs import draw, pair
from tests.gpu_util import TORCH, dev_matrix, gap_untouched, round_pitch, sentinel_c, to64
from synth_inputs import to_torch as to_torch_cpu

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("no_stream_k")]

PATHS = [("f32", "f32"), ("f32x3", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"),
         ("f16", "f16")]
PLAIN = {"f32": dg.gemm_f32, "f32x3": dg.gemm_f32_3xbf16, "bf16": dg.gemm_bf16,
         "f16": dg.gemm_f16}


def store(path):
    return "f32" if path == "f32x3" else path


def run_ex(path, out, A, B, *, alpha=1.0, beta=0.0, Cold=None, bias=None, relu=False,
           ws_bytes=0, spare=4096):
    """gemm_ex on seeded storage arrays; returns (C, workspace tensor or None)."""
    M, K = A.shape
    N = B.shape[1]
    dtype = store(path)
    Ad = dev_matrix(A, dtype, round_pitch(K, dtype, 8))
    Bd = dev_matrix(B, dtype, round_pitch(N, dtype, 8))
    Cd = sentinel_c(M, N, out)
    if Cold is not None:
        Cd[:] = to_torch_cpu(Cold, out).to("cuda")
    bd = torch.from_numpy(np.asarray(bias, dtype=np.float32)).to("cuda") if bias is not None \
        else None
    ws = None
    if ws_bytes:
        ws = torch.full(((ws_bytes + spare) // 4,), float("nan"), dtype=torch.float32,
                        device="cuda")
    torch.cuda.synchronize()
    dg.gemm_ex(Ad, Bd, Cd, alpha=alpha, beta=beta, bias=bd, relu=relu,
               workspace=None if ws is None else ws[: ws_bytes // 4],
               in_fmt="f32x3" if path == "f32x3" else None)
    torch.cuda.synchronize()
    return Cd, ws


def spare_untouched(ws, used_bytes):
    return ws is None or bool(torch.isnan(ws[used_bytes // 4:]).all().item())


@pytest.mark.parametrize("path,out", PATHS)
def test_identity_epilogue_equals_the_plain_entry_point(path, out):
    A, B = pair(300, 264, 200, "normal", store(path), seed=5000)
    C, _ = run_ex(path, out, A, B)
    dtype = store(path)
    Ad, Bd = dev_matrix(A, dtype), dev_matrix(B, dtype)
    Cp = sentinel_c(300, 264, out)
    PLAIN[path](Ad, Bd, Cp)
    torch.cuda.synchronize()
    assert torch.equal(C, Cp)


EPIS = [(-1.5, 0.0, True, False), (1.0, 0.5, False, True), (0.75, -1.0, True, True)]


@pytest.mark.parametrize("path,out", PATHS)
@pytest.mark.parametrize("M,N,K", [(257, 300, 65), (33, 7, 257), (256, 256, 64)])
def test_epilogue_parity(path, out, M, N, K):
    rng = np.random.default_rng(5100 + M + N + K + PATHS.index((path, out)))
    dtype = store(path)
    A = draw(rng, (M, K), "normal", dtype)
    B = draw(rng, (K, N), "normal", dtype)
    C64, S = oracle.gemm(dtype, A, B)
    for alpha, beta, use_bias, relu in EPIS:
        print(f"case epilogue {path}->{out} {M}x{N}x{K} a={alpha} b={beta} bias={use_bias} "
              f"relu={relu}", flush=True)
        Cold = draw(rng, (M, N), "normal", out) if beta != 0.0 else None
        bias = rng.standard_normal(N).astype(np.float32) if use_bias else None
        C, _ = run_ex(path, out, A, B, alpha=alpha, beta=beta, Cold=Cold, bias=bias, relu=relu)
        E, T = oracle.epilogue(C64, alpha, beta, None if Cold is None else oracle.widen(out, Cold),
                               None if bias is None else bias.astype(np.float64), relu)
        b = bound_epilogue(E, T, S, alpha, TOL_MFMA, out)
        res = oracle.check(to64(C), E, S, TOL_MFMA, out, b=b)
        assert res["ok"], res
        assert gap_untouched(C)


@pytest.mark.parametrize("path,out", PATHS)
def test_k_zero_applies_the_epilogue_to_the_empty_sum(path, out):
    rng = np.random.default_rng(5200)
    M, N = 70, 90
    dtype = store(path)
    A = np.zeros((M, 0), dtype=draw(rng, (1, 1), "normal", dtype).dtype)
    B = np.zeros((0, N), dtype=A.dtype)
    Cold = draw(rng, (M, N), "normal", out)
    bias = rng.standard_normal(N).astype(np.float32)
    C, _ = run_ex(path, out, A, B, alpha=3.0, beta=-0.5, Cold=Cold, bias=bias, relu=True)
    E, T = oracle.epilogue(np.zeros((M, N)), 3.0, -0.5, oracle.widen(out, Cold),
                           bias.astype(np.float64), True)
    b = bound_epilogue(E, T, np.zeros((M, N)), 3.0, TOL_MFMA, out)
    assert oracle.check(to64(C), E, np.zeros((M, N)), TOL_MFMA, out, b=b)["ok"]


# Shapes whose best plan splits K, with the workspace it asks for.  fp32 and
# 3 x bf16 outputs this small take the slice-K kernel instead, so those cases
# force the split plan (128 x 128 tiles, 8 splits) through the plan override,
# which the module's fixture clears after each test.
SPLIT_CASES = [("f32", "f32", 512, 512, 512), ("f32x3", "f32", 512, 512, 512),
               ("bf16", "f32", 64, 64, 4096), ("bf16", "bf16", 200, 136, 3000),
               ("f16", "f16", 64, 72, 4104), ("f16", "f32", 256, 256, 16384)]
FORCED_SPLITS = {("f32", 512, 512, 512): (128, 128, 8), ("f32x3", 512, 512, 512): (128, 128, 8)}


def split_plan(path, out, M, N, K):
    force = FORCED_SPLITS.get((path, M, N, K))
    if force:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, *force)
    p = dg.gemm_ex_plan(path, M, N, K, 1 << 40, out_same=(out != "f32"))
    assert p["splits"] > 1, p
    return p


@pytest.mark.parametrize("path,out,M,N,K", SPLIT_CASES)
def test_split_k_parity(path, out, M, N, K):
    p = split_plan(path, out, M, N, K)
    print(f"case splitk {path}->{out} {M}x{N}x{K} plan {p}", flush=True)
    dtype = store(path)
    A, B = pair(M, N, K, "normal", dtype, seed=5300 + M + K)
    C, ws = run_ex(path, out, A, B, ws_bytes=p["workspace_bytes"])
    C64, S = oracle.gemm(dtype, A, B)
    res = oracle.check(to64(C), C64, S, TOL_MFMA, out)
    assert res["ok"], res
    assert gap_untouched(C) and spare_untouched(ws, p["workspace_bytes"])


@pytest.mark.parametrize("path,out,M,N,K", SPLIT_CASES)
def test_split_k_with_epilogue(path, out, M, N, K):
    p = split_plan(path, out, M, N, K)
    rng = np.random.default_rng(5400 + M + K)
    dtype = store(path)
    A = draw(rng, (M, K), "normal", dtype)
    B = draw(rng, (K, N), "normal", dtype)
    Cold = draw(rng, (M, N), "normal", out)
    bias = rng.standard_normal(N).astype(np.float32)
    C, ws = run_ex(path, out, A, B, alpha=0.5, beta=2.0, Cold=Cold, bias=bias, relu=True,
                   ws_bytes=p["workspace_bytes"])
    C64, S = oracle.gemm(dtype, A, B)
    E, T = oracle.epilogue(C64, 0.5, 2.0, oracle.widen(out, Cold), bias.astype(np.float64), True)
    b = bound_epilogue(E, T, S, 0.5, TOL_MFMA, out)
    res = oracle.check(to64(C), E, S, TOL_MFMA, out, b=b)
    assert res["ok"], res
    assert gap_untouched(C) and spare_untouched(ws, p["workspace_bytes"])


@pytest.mark.parametrize("path,out,M,N,K", SPLIT_CASES)
def test_split_k_exact_integers_bitwise_and_repeatable(path, out, M, N, K):
    """Integer inputs keep every partial sum exact in fp32, so the split result
    must equal the oracle's rounding bit for bit; a second run must repeat it."""
    p = split_plan(path, out, M, N, K)
    dtype = store(path)
    A, B = pair(M, N, K, "ints", dtype, seed=5500 + M + K)
    C1, _ = run_ex(path, out, A, B, ws_bytes=p["workspace_bytes"])
    C2, _ = run_ex(path, out, A, B, ws_bytes=p["workspace_bytes"])
    C64, _ = oracle.gemm(dtype, A, B)
    assert np.max(np.abs(C64)) < 2 ** 24   # |a b| <= 64 and K <= 16384
    assert np.array_equal(to64(C1), oracle.widen(out, oracle.round_to(out, C64)))
    assert torch.equal(C1, C2)


# Split plans on the larger tiles: the smallest shapes (found by scanning the
# planner) whose plan splits K on a 256 x 256 or 192 x 256 macro-tile.
BIG_TILE_SPLITS = [("f32x3", "f32", 512, 6144, 2048, 256), ("bf16", "f32", 768, 6144, 8192, 256),
                   ("f16", "f16", 768, 6144, 8192, 256), ("bf16", "bf16", 768, 4096, 12288, 192),
                   ("f16", "f32", 768, 4096, 12288, 192)]


@pytest.mark.parametrize("path,out,M,N,K,tile", BIG_TILE_SPLITS)
def test_split_k_on_the_larger_tiles(path, out, M, N, K, tile):
    """Integer inputs (every partial sum exact in fp32): every element of C is
    written, sampled rows equal the oracle's rounding bit for bit, and an fp32 C
    satisfies Freivalds' identity exactly."""
    p = split_plan(path, out, M, N, K)
    assert p["tile_rows"] == tile, p
    print(f"case bigtile-split {path}->{out} {M}x{N}x{K} plan {p}", flush=True)
    dtype = store(path)
    A, B = pair(M, N, K, "ints", dtype, seed=5600 + M + K)
    C, ws = run_ex(path, out, A, B, ws_bytes=p["workspace_bytes"])
    Cn = to64(C)
    assert not np.isnan(Cn).any(), "unwritten elements"
    rng = np.random.default_rng(5601 + K)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, M - 1],
                                     rng.integers(0, M, 12)]))
    C64, _ = oracle.gemm(dtype, A, B, rows=rows)
    assert np.array_equal(Cn[rows], oracle.widen(out, oracle.round_to(out, C64)))
    if out == "f32":
        Aw, Bw = oracle.widen(dtype, A), oracle.widen(dtype, B)
        x = rng.integers(-4, 5, N).astype(np.float64)
        assert np.array_equal(Cn @ x, Aw @ (Bw @ x))
        y = rng.integers(-4, 5, M).astype(np.float64)
        assert np.array_equal(y @ Cn, (y @ Aw) @ Bw)
    assert gap_untouched(C) and spare_untouched(ws, p["workspace_bytes"])


def test_one_gpu_row_share_of_4096_cubed():
    """512 x 4096 x 4096 bf16 (one GPU's share of 4096^3 split by rows over 8):
    the split plan through matmul, sampled rows against the oracle, and every
    element written."""
    M, N, K = 512, 4096, 4096
    p = split_plan("bf16", "bf16", M, N, K)
    A, B = pair(M, N, K, "normal002", "bf16", seed=5600)
    Ad, Bd = dev_matrix(A, "bf16", K), dev_matrix(B, "bf16", N)
    C = dg.matmul(Ad, Bd)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(C.float()).any().item())
    rows = np.array([0, 1, 31, 127, 128, 255, 256, 300, 383, 384, 510, 511])
    C64, S = oracle.gemm("bf16", A, B, rows=rows)
    res = oracle.check(to64(C[torch.from_numpy(rows).to("cuda")]), C64, S, TOL_MFMA, "bf16")
    assert res["ok"], (p, res)


def test_split_k_on_a_non_default_stream_matches_the_default_stream():
    """The split plan's two kernels are ordered on the caller's stream."""
    M, N, K = 64, 64, 4096
    p = split_plan("bf16", "bf16", M, N, K)
    A, B = pair(M, N, K, "normal", "bf16", seed=5700)
    Ad, Bd = dev_matrix(A, "bf16", K), dev_matrix(B, "bf16", N)
    ws = torch.empty(p["workspace_bytes"], dtype=torch.uint8, device="cuda")
    ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dg.gemm_ex(Ad, Bd, ref, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    got = torch.empty_like(ref)
    ws2 = torch.empty_like(ws)
    with torch.cuda.stream(s):
        for _ in range(3):
            dg.gemm_ex(Ad, Bd, got, workspace=ws2, stream=s)
    s.synchronize()
    assert torch.equal(ref, got)


def test_workspace_smaller_than_the_best_plan_still_gives_the_product():
    """With less workspace than the preferred plan needs, gemm_ex picks a plan
    that fits (here: unsplit) and the result still matches the oracle."""
    M, N, K = 64, 64, 4096
    best = split_plan("f16", "f16", M, N, K)
    small = best["workspace_bytes"] // 4
    fit = dg.gemm_ex_plan("f16", M, N, K, small, out_same=True)
    assert fit["workspace_bytes"] <= small
    A, B = pair(M, N, K, "normal", "f16", seed=5800)
    C, ws = run_ex("f16", "f16", A, B, ws_bytes=small)
    C64, S = oracle.gemm("f16", A, B)
    assert oracle.check(to64(C), C64, S, TOL_MFMA, "f16")["ok"]
    assert gap_untouched(C) and spare_untouched(ws, fit["workspace_bytes"])


def test_full_size_ragged_workload_with_fused_epilogue():
    """4000 x 3000 x 4104 (192 x 256 tiles, ragged in every dimension) with
    alpha, beta, bias and ReLU, bf16 C: every element against the oracle."""
    from synth_inputs import workload
    A, B, meta = workload("bf16_4000x3000x4104")
    M, N, K = meta["M"], meta["N"], meta["K"]
    assert dg.gemm_ex_plan("bf16", M, N, K, 0, out_same=True)["tile_rows"] == 192
    rng = np.random.default_rng(5900)
    Cold = draw(rng, (M, N), "normal", "bf16")
    bias = rng.standard_normal(N).astype(np.float32) * 0.1
    Ad, Bd = dev_matrix(A, "bf16", K), dev_matrix(B, "bf16", N)
    C = to_torch_cpu(Cold, "bf16").to("cuda")
    dg.gemm_ex(Ad, Bd, C, alpha=2.0, beta=-0.5, bias=torch.from_numpy(bias).to("cuda"),
               relu=True)
    torch.cuda.synchronize()
    C64, S = oracle.gemm("bf16", A, B)
    E, T = oracle.epilogue(C64, 2.0, -0.5, oracle.widen("bf16", Cold),
                           bias.astype(np.float64), True)
    b = bound_epilogue(E, T, S, 2.0, TOL_MFMA, "bf16")
    res = oracle.check(to64(C), E, S, TOL_MFMA, "bf16", b=b)
    assert res["ok"], res


@pytest.mark.parametrize("path,out", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"),
                                      ("f16", "f32"), ("f32x3", "f32")])
@pytest.mark.parametrize("alpha,beta,use_bias,relu", [(0.75, -1.0, True, True),
                                                      (-1.5, 0.5, False, False)])
def test_fused_epilogue_on_the_256_tile(path, out, alpha, beta, use_bias, relu):
    """4096 x 4096 outputs with no workspace run the 256 x 256 instantiations
    that apply the epilogue in the GEMM kernel itself (split plans apply it in
    the reduction instead).  K = 200 keeps the oracle quick while giving four K
    steps with a ragged last one.  Every element of C against the oracle."""
    M = N = 4096
    K = 200
    plan = dg.gemm_ex_plan(path, M, N, K, 0, out_same=(out != "f32"))
    assert (plan["tile_rows"], plan["tile_cols"], plan["splits"]) == (256, 256, 1), plan
    print(f"case epi256 {path}->{out} a={alpha} b={beta} bias={use_bias} relu={relu}", flush=True)
    rng = np.random.default_rng(5950 + PATHS.index((path, out)) + (10 if relu else 0))
    dtype = store(path)
    A = draw(rng, (M, K), "normal", dtype)
    B = draw(rng, (K, N), "normal", dtype)
    Cold = draw(rng, (M, N), "normal", out) if beta != 0.0 else None
    bias = rng.standard_normal(N).astype(np.float32) if use_bias else None
    C, _ = run_ex(path, out, A, B, alpha=alpha, beta=beta, Cold=Cold, bias=bias, relu=relu)
    C64, S = oracle.gemm(dtype, A, B)
    E, T = oracle.epilogue(C64, alpha, beta, None if Cold is None else oracle.widen(out, Cold),
                           None if bias is None else bias.astype(np.float64), relu)
    b = bound_epilogue(E, T, S, alpha, TOL_MFMA, out)
    res = oracle.check(to64(C), E, S, TOL_MFMA, out, b=b)
    assert res["ok"], res
    assert gap_untouched(C)


def random_cases(n=96, seed=6100):
    rng = np.random.default_rng(seed)
    for i in range(n):
        path, out = PATHS[int(rng.integers(len(PATHS)))]
        M = int(rng.integers(1, 700))
        N = int(rng.integers(1, 700))
        K = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 6000))]))
        alpha = float(rng.choice([1.0, -0.5, 1.25]))
        beta = float(rng.choice([0.0, 0.0, 1.0, -2.0]))
        use_bias = bool(rng.integers(2))
        relu = bool(rng.integers(2))
        yield i, path, out, M, N, K, alpha, beta, use_bias, relu


@pytest.mark.parametrize("case", list(random_cases()), ids=lambda c: f"r{c[0]}")
def test_random_shapes_epilogues_and_plans(case):
    """Seeded random shapes, formats, epilogues; the workspace the best plan asks
    for, so deep-K cases split and the rest do not."""
    i, path, out, M, N, K, alpha, beta, use_bias, relu = case
    p = dg.gemm_ex_plan(path, M, N, K, 1 << 40, out_same=(out != "f32"))
    print(f"case r{i} {path}->{out} {M}x{N}x{K} a={alpha} b={beta} bias={use_bias} relu={relu} "
          f"plan {p}", flush=True)
    rng = np.random.default_rng(6200 + i)
    dtype = store(path)
    A = draw(rng, (M, K), "normal", dtype)
    B = draw(rng, (K, N), "normal", dtype)
    Cold = draw(rng, (M, N), "normal", out) if beta != 0.0 else None
    bias = rng.standard_normal(N).astype(np.float32) if use_bias else None
    C, ws = run_ex(path, out, A, B, alpha=alpha, beta=beta, Cold=Cold, bias=bias, relu=relu,
                   ws_bytes=p["workspace_bytes"])
    C64, S = oracle.gemm(dtype, A, B)
    E, T = oracle.epilogue(C64, alpha, beta, None if Cold is None else oracle.widen(out, Cold),
                           None if bias is None else bias.astype(np.float64), relu)
    b = bound_epilogue(E, T, S, alpha, TOL_MFMA, out)
    res = oracle.check(to64(C), E, S, TOL_MFMA, out, b=b)
    assert res["ok"], res
    assert gap_untouched(C) and spare_untouched(ws, p["workspace_bytes"])


@pytest.mark.parametrize("path,out,M,N,K", [("bf16", "bf16", 64, 72, 4104), ("f16", "f32", 300, 264, 200),
                                            ("f32", "f32", 512, 512, 512),
                                            ("f32x3", "f32", 1024, 1024, 1024),
                                            ("bf16", "f32", 1024, 1024, 1024)])
def test_hip_graph_capture_replays_match_eager(path, out, M, N, K):
    """gemm_ex captured into a HIP graph, on the planner's plans: a split plan
    (bf16 64 x 72 x 4104) and slice-K on 32 x 32 and 64 x 64 tiles (the others;
    the 64 x 64 tiles move B through LDS with direct-to-LDS loads): every
    replay, with eager work on the same stream between replays, reproduces the
    eager result bit for bit.  The library enqueues only kernel launches (no
    memset, no allocation), which is what capture requires."""
    p = dg.gemm_ex_plan(path, M, N, K, 1 << 40, out_same=(out != "f32"))
    print(f"case graph {path}->{out} {M}x{N}x{K} plan {p}", flush=True)
    rng = np.random.default_rng(6300 + M)
    dtype = store(path)
    A = draw(rng, (M, K), "normal", dtype)
    B = draw(rng, (K, N), "normal", dtype)
    Ad, Bd = dev_matrix(A, dtype), dev_matrix(B, dtype)
    bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).to("cuda")
    ws = torch.empty(max(p["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
    fmt = "f32x3" if path == "f32x3" else None
    ref = torch.empty((M, N), dtype=TORCH[out], device="cuda")
    dg.gemm_ex(Ad, Bd, ref, bias=bias, relu=True, workspace=ws, in_fmt=fmt)
    torch.cuda.synchronize()
    C = torch.empty_like(ref)
    other = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dg.gemm_ex(Ad, Bd, C, bias=bias, relu=True, workspace=ws, in_fmt=fmt)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dg.gemm_ex(Ad, Bd, C, bias=bias, relu=True, workspace=ws, in_fmt=fmt)
    for rep in range(4):
        C.fill_(float("nan"))
        g.replay()
        dg.gemm_ex(Ad, Bd, other, workspace=ws, in_fmt=fmt)       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(C, ref), rep
