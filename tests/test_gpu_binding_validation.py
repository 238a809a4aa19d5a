"""The Python binding rejects malformed calls before anything reaches the
library, with ValueError (shape, layout, device) or TypeError (dtype), and leaves
C untouched."""
import pytest
import torch

import dense_gemm_matrix_amd as dg

pytestmark = pytest.mark.gpu


def dev(*shape, dtype=torch.bfloat16):
    return torch.ones(*shape, dtype=dtype, device="cuda")


def sentinel(M, N, dtype=torch.float32):
    return torch.full((M, N), 7.0, dtype=dtype, device="cuda")


@pytest.mark.parametrize("fn,dt", [(dg.gemm_bf16, torch.bfloat16), (dg.gemm_f16, torch.float16),
                                   (dg.gemm_f32, torch.float32), (dg.gemm_f32_3xbf16, torch.float32)])
def test_plain_entries_reject_bad_operands(fn, dt):
    A, B = dev(64, 32, dtype=dt), dev(32, 48, dtype=dt)
    C = sentinel(64, 48)
    cases = [
        (ValueError, (A[0], B, C)),                                    # 1-D A
        (ValueError, (A, dev(33, 48, dtype=dt), C)),                   # inner sizes differ
        (ValueError, (A, B, sentinel(64, 47))),                        # wrong C shape
        (ValueError, (A.cpu(), B, C)),                                 # host tensor
        (ValueError, (dev(32, 64, dtype=dt).t(), B, C)),               # column-major A
        (TypeError, (A.to(torch.float64), B.to(torch.float64), C)),    # unsupported dtype
    ]
    for exc, args in cases:
        print("case", fn.__name__, exc.__name__, [tuple(a.shape) for a in args], flush=True)
        with pytest.raises(exc):
            fn(*args)
    torch.cuda.synchronize()
    assert bool((C == 7.0).all()), "a rejected call wrote C"


def test_matmul_rejects_before_allocating():
    A, B = dev(64, 32), dev(32, 48)
    with pytest.raises(TypeError):
        dg.matmul(A.to(torch.int32), B.to(torch.int32))
    with pytest.raises(TypeError):
        dg.matmul(A, B.to(torch.float16))
    with pytest.raises(TypeError):
        dg.matmul(A, B, out_dtype=torch.float16)
    with pytest.raises(ValueError):
        dg.matmul(A[0], B)
    with pytest.raises(ValueError):
        dg.matmul(A, dev(31, 48))


def test_gemm_ex_rejects_bad_bias_and_workspace():
    A, B, C = dev(64, 32), dev(32, 48), sentinel(64, 48)
    with pytest.raises(ValueError):
        dg.gemm_ex(A, B, C, bias=torch.zeros(47, device="cuda"))
    with pytest.raises(ValueError):
        dg.gemm_ex(A, B, C, bias=torch.zeros(48, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        dg.gemm_ex(A, B, C, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()
    assert bool((C == 7.0).all()), "a rejected call wrote C"
