"""Host threads calling the library at the same time, each on its own stream.

The C ABI keeps no state between calls except a per-device flag that records
whether the device is a gfx950 (an atomic), and every plan is a function of the
arguments alone, so calls made from several threads on several streams must
give the same bytes as the same calls made one at a time.  ctypes releases the
interpreter lock for the duration of each foreign call, so the threads do enter
the library together.  The cases include split-K plans, whose workspace the
binding takes from torch's allocator on the calling thread's stream, and fp32
slice-K plans (K split across the waves of a workgroup)."""
import threading

import pytest
import torch

import dense_gemm_matrix_amd as dg
from synth_inputs import pair, to_torch

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("no_stream_k")]

# (path, M, N, K, C dtype); "f32x3" is fp32 data through the 3 x bf16 split.
CASES = [
    ("bf16", 300, 264, 520, torch.float32),
    ("f16", 64, 72, 4104, torch.float16),      # a split-K plan
    ("f32", 257, 132, 300, torch.float32),     # slice-K, 4 waves per workgroup
    ("f32x3", 200, 136, 300, torch.float32),
    ("bf16", 512, 512, 1024, torch.bfloat16),
    ("f32", 96, 64, 2048, torch.float32),      # slice-K, 8 waves per workgroup (deep K)
]
ITERS = 25


def launch(path, A, B, out):
    """One product on the current stream; C and any workspace come from it."""
    if path == "f32x3":
        C = torch.empty((A.shape[0], B.shape[1]), dtype=out, device="cuda")
        dg.gemm_f32_3xbf16(A, B, C)
        return C
    return dg.matmul(A, B, out_dtype=out)


def as_bits(C):
    return C.view(torch.int32 if C.dtype == torch.float32 else torch.int16)


def test_threads_on_their_own_streams_match_one_at_a_time():
    inputs = []
    for i, (path, M, N, K, _) in enumerate(CASES):
        dt = "f32" if path == "f32x3" else path
        A, B = pair(M, N, K, "uniform", dt, seed=8100 + i)
        inputs.append((to_torch(A, dt).cuda(), to_torch(B, dt).cuda()))
    assert dg.gemm_ex_plan("f16", 64, 72, 4104, 1 << 40, out_same=True)["splits"] > 1
    for M, N, K in [(257, 132, 300), (96, 64, 2048)]:
        p = dg.gemm_ex_plan("f32", M, N, K, 1 << 40)
        assert (p["tile_rows"], p["splits"]) == (32, 1), p
    refs = [as_bits(launch(c[0], *inputs[i], c[4])).clone() for i, c in enumerate(CASES)]
    torch.cuda.synchronize()

    results = [[] for _ in CASES]
    errors = []
    start = threading.Barrier(len(CASES))

    def worker(t):
        try:
            path, _, _, _, out = CASES[t]
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(ITERS):
                    results[t].append(launch(path, *inputs[t], out))
            s.synchronize()
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(len(CASES))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    print(f"concurrency: {len(CASES)} threads x {ITERS} calls", flush=True)
    for t, (path, M, N, K, out) in enumerate(CASES):
        assert len(results[t]) == ITERS
        for i, C in enumerate(results[t]):
            assert torch.equal(as_bits(C), refs[t]), f"{path} {M}x{N}x{K} call {i} differs"


def test_matmul_on_a_side_stream_keeps_its_workspace_on_that_stream(monkeypatch):
    """matmul(..., stream=s) with a split-K plan while the current stream is
    another one: the workspace must come from s's pool, so that once matmul has
    returned, an allocation of the same size on the current stream does not get
    the block that s's kernels (held back here behind a long product) have yet
    to use."""
    import dense_gemm_matrix_amd._binding as binding
    M, N, K = 64, 72, 4104
    plan = dg.gemm_ex_plan("bf16", M, N, K, 1 << 40, out_same=True)
    assert plan["splits"] > 1
    A, B = pair(M, N, K, "uniform", "bf16", seed=8200)
    Ad, Bd = to_torch(A, "bf16").cuda(), to_torch(B, "bf16").cuda()
    ref = as_bits(dg.matmul(Ad, Bd)).clone()
    Xa = torch.randn(4096, 4096, device="cuda").to(torch.bfloat16)
    Xc = torch.empty(4096, 4096, device="cuda")
    torch.cuda.synchronize()

    seen = []
    real = binding.gemm_ex

    def spy(*args, **kw):
        seen.append(kw["workspace"].data_ptr() if kw.get("workspace") is not None else None)
        return real(*args, **kw)

    monkeypatch.setattr(binding, "gemm_ex", spy)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s):
            for _ in range(10):          # ~1 ms of work ahead of the product on s
                dg.gemm_bf16(Xa, Xa, Xc)
        outs.append(dg.matmul(Ad, Bd, stream=s))
        assert seen[-1] is not None
        # The current stream asks for a block of the workspace's size and fills it.
        other = torch.full((plan["workspace_bytes"],), 0x7f, dtype=torch.uint8, device="cuda")
        assert other.data_ptr() != seen[-1], "the workspace went back to the current stream's pool"
    s.synchronize()
    torch.cuda.synchronize()
    for i, C in enumerate(outs):
        assert torch.equal(as_bits(C), ref), f"call {i} differs"
