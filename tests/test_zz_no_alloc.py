"""gemm_ex_static, the allocation-free gemm_ex, through the C ABI on the GPU.

Its split-K partials go to the library's static device scratch instead of a
caller workspace.  With the same byte budget it must choose the same plan as
gemm_ex and give the same C, bit for bit, and C must match the oracle.  Two
calls in a row, the second with a smaller input (the scratch then still holds
the first call's partials), check that nothing depends on what the scratch
held before."""
import ctypes

import numpy as np
import pytest
import torch

import dense_gemm_matrix_amd as dg
import oracle
from oracle.parity import TOL_MFMA, bound_epilogue
from synth_inputs import draw
from tests.gpu_util import TORCH, dev_matrix, gap_untouched, sentinel_c, to64

pytestmark = pytest.mark.gpu

IN = {"f32": 0, "bf16": 1, "f16": 2, "f32x3": 3}


def store(path):
    return "f32" if path == "f32x3" else path


def static_raw(path, out, Ad, Bd, Cd, alpha, beta, bias, relu, scratch_bytes):
    """gemm_ex_static called through ctypes with the tensors' pointers and pitches."""
    M, K = Ad.shape
    N = Bd.shape[1]
    lib = dg.raw()
    return lib.gemm_ex_static(
        IN[path], 0 if out == "f32" else 1, M, N, K,
        ctypes.c_void_p(Ad.data_ptr()), Ad.stride(0), ctypes.c_void_p(Bd.data_ptr()), Bd.stride(0),
        ctypes.c_void_p(Cd.data_ptr()), Cd.stride(0), ctypes.c_float(alpha), ctypes.c_float(beta),
        ctypes.c_void_p(bias.data_ptr()) if bias is not None else None, 1 if relu else 0,
        ctypes.c_size_t(scratch_bytes),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (path, out, M, N, K, alpha, beta, bias, relu): each pair's second call is smaller.
SEQUENCES = [
    [("bf16", "bf16", 512, 4096, 4096, 1.0, 0.0, True, False),
     ("bf16", "bf16", 64, 72, 4104, 0.5, 1.0, True, True)],
    [("f32", "f32", 512, 512, 512, 1.0, 0.0, False, False),
     ("f16", "f32", 200, 136, 3000, -1.0, 0.0, True, True)],
    [("f32x3", "f32", 512, 512, 512, 2.0, -0.5, False, True),
     ("f16", "f16", 64, 64, 4096, 1.0, 0.0, False, False)],
]


# fp32 and 3 x bf16 outputs this small take the slice-K kernel (no scratch):
# those calls force the split plan through the plan override.
FORCED_SPLITS = {("f32", 512, 512, 512): (128, 128, 8), ("f32x3", 512, 512, 512): (128, 128, 8)}


@pytest.fixture
def clear_override():
    yield
    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_static_scratch_matches_gemm_ex_on_two_calls_in_a_row(seq, clear_override):
    for i, (path, out, M, N, K, alpha, beta, use_bias, relu) in enumerate(SEQUENCES[seq]):
        budget = dg.DGEMM_STATIC_SCRATCH_BYTES
        force = FORCED_SPLITS.get((path, M, N, K))
        dg.dgemm_set_plan_override(*((dg.DGEMM_PLAN_GRID,) + force if force else (dg.DGEMM_PLAN_AUTO,)))
        plan = dg.gemm_ex_plan(path, M, N, K, budget, out_same=(out != "f32"))
        assert plan["splits"] > 1 and plan["workspace_bytes"] <= budget, plan
        print(f"case static seq{seq} call{i} {path}->{out} {M}x{N}x{K} plan {plan}", flush=True)
        rng = np.random.default_rng(9000 + 10 * seq + i)
        dtype = store(path)
        A = draw(rng, (M, K), "normal", dtype)
        B = draw(rng, (K, N), "normal", dtype)
        Cold = draw(rng, (M, N), "normal", out) if beta != 0.0 else None
        bias_np = rng.standard_normal(N).astype(np.float32) if use_bias else None
        Ad, Bd = dev_matrix(A, dtype), dev_matrix(B, dtype)
        bias = torch.from_numpy(bias_np).to("cuda") if use_bias else None

        C_static = sentinel_c(M, N, out)
        C_ref = sentinel_c(M, N, out)
        if Cold is not None:
            from synth_inputs import to_torch
            C_static[:] = to_torch(Cold, out).to("cuda")
            C_ref[:] = to_torch(Cold, out).to("cuda")
        torch.cuda.synchronize()
        st = static_raw(path, out, Ad, Bd, C_static, alpha, beta, bias, relu, budget)
        assert st == dg.DGEMM_OK, dg.dgemm_status_string(st)
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
        dg.gemm_ex(Ad, Bd, C_ref, alpha=alpha, beta=beta, bias=bias, relu=relu, workspace=ws,
                   in_fmt="f32x3" if path == "f32x3" else None)
        torch.cuda.synchronize()
        assert torch.equal(C_static, C_ref)
        assert gap_untouched(C_static)
        C64, S = oracle.gemm(dtype, A, B)
        E, T = oracle.epilogue(C64, alpha, beta, None if Cold is None else oracle.widen(out, Cold),
                               None if bias_np is None else bias_np.astype(np.float64), relu)
        b = bound_epilogue(E, T, S, alpha, TOL_MFMA, out)
        res = oracle.check(to64(C_static), E, S, TOL_MFMA, out, b=b)
        assert res["ok"], res


def test_no_scratch_budget_is_the_unsplit_product():
    M, N, K = 64, 64, 4096
    rng = np.random.default_rng(9100)
    A = draw(rng, (M, K), "normal", "bf16")
    B = draw(rng, (K, N), "normal", "bf16")
    Ad, Bd = dev_matrix(A, "bf16"), dev_matrix(B, "bf16")
    C_static = sentinel_c(M, N, "f32")
    C_plain = sentinel_c(M, N, "f32")
    assert static_raw("bf16", "f32", Ad, Bd, C_static, 1.0, 0.0, None, False, 0) == dg.DGEMM_OK
    dg.gemm_bf16(Ad, Bd, C_plain)
    torch.cuda.synchronize()
    assert torch.equal(C_static, C_plain)


def test_scratch_budget_beyond_the_array_is_rejected():
    Ad = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    Bd = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    C = torch.full((64, 64), 7.0, dtype=TORCH["f32"], device="cuda")
    st = static_raw("bf16", "f32", Ad, Bd, C, 1.0, 0.0, None, False,
                    dg.DGEMM_STATIC_SCRATCH_BYTES + 1)
    assert st == dg.DGEMM_ERR_SCRATCH_SIZE
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
