"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every case draws seeded inputs, runs the library on cuda:0 and compares with
the oracle on the same storage bytes: element by element within
|C - C64| <= tol*S*(1+u) + u*|C64| (+ subnormal slack), bit for bit where the
inputs make the answer exact.  C is prefilled with NaN and its row pitch gap
must stay NaN, so missed and stray stores both show."""
import functools

import numpy as np
import pytest
import torch

import dense_gemm_matrix_amd as dg
import oracle
from oracle.parity import TOL_MFMA
from synth_inputs import draw, pair, workload
from synth_inputs import to_torch as TORCH_FROM
from tests.gpu_util import TORCH, dev_matrix, gap_untouched, round_pitch, sentinel_c, to64

pytestmark = pytest.mark.gpu

# path -> entry point; "f32x3" is fp32 data through the 3 x bf16 split entry.
ENTRY = {"f32": dg.gemm_f32, "f32x3": dg.gemm_f32_3xbf16, "bf16": dg.gemm_bf16, "f16": dg.gemm_f16}
COMBOS = [("f32", "f32"), ("f32x3", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"),
          ("f16", "f16")]


def store(path):
    """Storage dtype of a path's inputs."""
    return "f32" if path == "f32x3" else path


def run(path, out, A, B, a_extra=0, b_extra=0, c_extra=4, stream=None):
    M, K = A.shape
    N = B.shape[1]
    dtype = store(path)
    Ad = dev_matrix(A, dtype, round_pitch(K, dtype, a_extra))
    Bd = dev_matrix(B, dtype, round_pitch(N, dtype, b_extra))
    Cd = sentinel_c(M, N, out, round_pitch(N, out, c_extra))
    ENTRY[path](Ad, Bd, Cd, stream=stream)
    if stream is not None:
        stream.synchronize()
    torch.cuda.synchronize()
    return Cd


def assert_exact(C, dtype, out, A, B):
    """Every element of C equals the oracle's exact sum rounded once to C's
    format (integer inputs: every fp32 partial sum is exact)."""
    C64, _ = oracle.gemm(dtype, A, B)
    want = oracle.widen(out, oracle.round_to(out, C64))
    got = to64(C)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} of {got.size} elements differ, first {tuple(bad[0])}"


DIMS_MN = [1, 7, 33, 255, 256, 257]
DIMS_K = [1, 7, 64, 65, 255, 257]


@pytest.mark.parametrize("path,out", COMBOS)
def test_small_and_ragged_shapes(path, out):
    rng = np.random.default_rng(1000 + COMBOS.index((path, out)))
    dtype = store(path)
    for M in DIMS_MN:
        for N in DIMS_MN:
            for K in DIMS_K:
                print(f"case {path}->{out} {M}x{N}x{K}", flush=True)
                A = draw(rng, (M, K), "normal", dtype)
                B = draw(rng, (K, N), "normal", dtype)
                C = run(path, out, A, B, a_extra=8, b_extra=8)
                C64, S = oracle.gemm(dtype, A, B)
                res = oracle.check(to64(C), C64, S, TOL_MFMA, out)
                assert res["ok"], (M, N, K, res)
                assert gap_untouched(C), (M, N, K)


@pytest.mark.parametrize("path,out", COMBOS)
@pytest.mark.parametrize("M,N,K", [(1000, 700, 1100), (512, 768, 4104), (300, 264, 200)])
def test_exact_integer_inputs_bitwise(path, out, M, N, K):
    """Integers in [-8, 8]: every partial sum is an integer below 2^24, so the fp32
    accumulator is exact in any order; C must equal the oracle's C64 rounded once
    to C's format, bit for bit.  This pins tiling, staging, the LDS layout, the
    operand layouts, masking, the tile map and the epilogue."""
    print(f"case int {path}->{out} {M}x{N}x{K}", flush=True)
    dtype = store(path)
    A, B = pair(M, N, K, "ints", dtype, seed=2000 + M + N + K)
    C = run(path, out, A, B, a_extra=8, b_extra=16)
    C64, _ = oracle.gemm(dtype, A, B)
    want = oracle.widen(out, oracle.round_to(out, C64))
    assert np.array_equal(to64(C), want)
    assert gap_untouched(C)


# (workload, path, the macro-tile its plain launch uses).  Parametrizations of
# one workload are adjacent so that the oracle's result is computed once.
WORKLOAD_RUNS = [("f32_512", "f32", 32), ("f32_512", "f32x3", 32),
                 ("f32_4096", "f32", 128), ("f32_4096", "f32x3", 256),
                 ("bf16_4096", "bf16", 256), ("f16_4096", "f16", 256),
                 ("bf16_16384x4096x4096", "bf16", 256), ("bf16_4000x3000x4104", "bf16", 192)]


@functools.lru_cache(maxsize=1)
def workload_oracle(name):
    """Inputs and the oracle's (C64, S) over all of C for a named workload."""
    A, B, meta = workload(name)
    C64, S = oracle.gemm(meta["dtype"], A, B)
    return A, B, meta, C64, S


@pytest.mark.parametrize("name,path,tile", WORKLOAD_RUNS)
def test_workloads(name, path, tile):
    """The six workloads at full size (fp32 ones through both fp32 entry
    points), in the launch configuration the benchmark times (packed pitches,
    the planner's tile): every element of C against the oracle, and the
    fraction equal to the oracle's own rounding reported."""
    A, B, meta, C64, S = workload_oracle(name)
    dtype, out, M, N = meta["dtype"], meta["out"], meta["M"], meta["N"]
    assert dg.dgemm_tile_map(M, N, path)["tile_rows"] == tile
    print(f"case workload {name} via {path} (tile {tile})", flush=True)
    Ad = dev_matrix(A, dtype, A.shape[1])
    Bd = dev_matrix(B, dtype, B.shape[1])
    Cd = torch.full((M, N), float("nan"), dtype=TORCH[out], device="cuda")
    ENTRY[path](Ad, Bd, Cd)
    torch.cuda.synchronize()
    got = to64(Cd)
    del Ad, Bd, Cd
    res = oracle.check(got, C64, S, TOL_MFMA, out, C_round=oracle.widen(out, oracle.round_to(out, C64)))
    print(f"{name}: max err/bound {res['max_ratio']:.3g} over {got.size} elements, equal to the "
          f"oracle's rounding {res['exact_frac']:.3f}", flush=True)
    assert res["ok"], res


@pytest.mark.parametrize("path,out,M,N,K,tile", [
    ("f16", "f16", 4096, 4096, 4096, 256),          # the fp16 workload's shape, fp16 C
    ("bf16", "bf16", 16384, 4096, 4096, 256),       # the tall bf16 workload's shape
    ("bf16", "bf16", 4000, 3000, 4104, 192),        # the ragged bf16 workload's shape
    ("bf16", "f32", 4000, 3000, 4104, 192),
])
def test_16bit_c_full_size_integer_inputs_bitwise(path, out, M, N, K, tile):
    """The kernels that run the 16-bit-C workloads, at those shapes and packed
    pitches, with integers in [-8, 8]: every fp32 partial sum is exact, so the
    one rounding to C's format must give the oracle's direct rounding of its
    exact sum in every element of C."""
    assert dg.dgemm_tile_map(M, N, path)["tile_rows"] == tile
    print(f"case int full {path}->{out} {M}x{N}x{K} tile {tile}", flush=True)
    A, B = pair(M, N, K, "ints", path, seed=3700 + M + K)
    Ad = dev_matrix(A, path, K)
    Bd = dev_matrix(B, path, N)
    Cd = torch.full((M, N), float("nan"), dtype=TORCH[out], device="cuda")
    ENTRY[path](Ad, Bd, Cd)
    torch.cuda.synchronize()
    del Ad, Bd
    assert_exact(Cd, path, out, A, B)


@pytest.mark.parametrize("path", ["f32", "f32x3", "bf16", "f16"])
def test_exact_integer_full_size_bitwise(path):
    """4096^3 with integer inputs and fp32 C: C is exact and must equal the
    oracle's sum in every element."""
    M = N = K = 4096
    print(f"case int 4096 {path}", flush=True)
    dtype = store(path)
    A, B = pair(M, N, K, "ints", dtype, seed=3000)
    C = run(path, "f32", A, B)
    assert_exact(C, dtype, "f32", A, B)
    assert gap_untouched(C)


@pytest.mark.parametrize("path", ["f32", "f32x3", "bf16", "f16"])
@pytest.mark.parametrize("K", [1, 33, 65, 100])
def test_largest_tile_with_few_ragged_k_steps(path, K):
    """4096 x 4096 selects each path's largest tile (256 x 256 for the 16-bit
    and 3 x bf16 kernels, 128 x 128 for fp32); K = 1, 33, 65, 100 gives one to
    four K steps with a ragged last one, so the tail handling of the first step
    and of a later step both run, with NaN in A's row padding.  Integer inputs:
    C is exact and must equal the oracle in every element."""
    M = N = 4096
    largest = {"f32": 128, "f32x3": 256, "bf16": 256, "f16": 256}[path]
    assert dg.dgemm_tile_map(M, N, path)["tile_rows"] == largest
    print(f"case largest-tile {path} K={K}", flush=True)
    dtype = store(path)
    A, B = pair(M, N, K, "ints", dtype, seed=3200 + K)
    C = run(path, "f32", A, B, a_extra=8, b_extra=8)
    assert_exact(C, dtype, "f32", A, B)
    assert gap_untouched(C)


@pytest.mark.parametrize("path", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [
    (2048, 4096, 1), (2048, 4096, 130), (2000, 4000, 4104),               # > 256 workgroups
    (1000, 2000, 1), (1000, 2000, 65), (1000, 2000, 200), (2048, 2048, 4104),  # <= 256
])
def test_128_tile_with_either_ring_depth(path, M, N, K):
    """The 16-bit 128 x 128 tile keeps a 2-stage LDS ring when the grid has more
    workgroups than the chip's 256 CUs and a 4-stage one otherwise.  K = 1, 65,
    130 and 200 give fewer K steps than the deeper ring has stages, or exactly as
    many, with a ragged last step; 4104 gives 65 steps with a ragged one.
    Integer inputs, fp32 C: exact, equal to the oracle in every element."""
    tm = dg.dgemm_tile_map(M, N, path)
    assert tm["tile_rows"] == 128 and tm["tile_cols"] == 128
    ring = 4 if tm["num_wg"] <= 256 else 2
    assert ring == (4 if M * N <= 2048 * 2048 else 2)
    print(f"case tile128 {path} {M}x{N}x{K} ring {ring}", flush=True)
    A, B = pair(M, N, K, "ints", path, seed=3400 + K + M)
    C = run(path, "f32", A, B, a_extra=8, b_extra=8)
    assert_exact(C, path, "f32", A, B)
    assert gap_untouched(C)


@pytest.mark.parametrize("K", [1, 31, 32, 33, 64, 95, 96, 97, 150, 160, 191, 200])
def test_3xbf16_128_tile_step_counts(K):
    """The 3 x bf16 kernel's 128 x 128 tile stages through two register sets,
    alternating by step, with each step loading three steps ahead and the K loop
    unrolled by two.  K from 1 to 200 gives 1 to 7 steps of 32, even and odd
    counts, with the ragged last step in either set.  Integer inputs (lo parts
    zero): C is exact and must equal the oracle bit for bit.  1100 x 1000 is 72
    tiles of 128 x 128, past the outputs that take slice-K."""
    M, N = 1100, 1000
    tm = dg.dgemm_tile_map(M, N, "f32x3")
    assert tm["tile_rows"] == 128
    print(f"case x3-128 K={K}", flush=True)
    A, B = pair(M, N, K, "ints", "f32", seed=3600 + K)
    C = run("f32x3", "f32", A, B, a_extra=8, b_extra=8)
    C64, _ = oracle.gemm("f32", A, B)
    assert np.array_equal(to64(C), C64)
    assert gap_untouched(C)


@pytest.mark.parametrize("path", ["bf16", "f16"])
@pytest.mark.parametrize("out", ["f32", "same"])
def test_exact_integer_192_tile_padded_pitches(path, out):
    """4000 x 3000 x 4104 selects the 192 x 256 macro-tile; here with padded
    row pitches (the workload itself uses packed ones).  Integer inputs: equal
    to the oracle in every element, for fp32 C and for C in the input format."""
    M, N, K = 4000, 3000, 4104
    out = path if out == "same" else out
    assert dg.dgemm_tile_map(M, N, path)["tile_rows"] == 192
    print(f"case int192 {path}->{out}", flush=True)
    A, B = pair(M, N, K, "ints", path, seed=3100)
    C = run(path, out, A, B, a_extra=8, b_extra=8)
    assert_exact(C, path, out, A, B)
    assert gap_untouched(C)


@pytest.mark.parametrize("path", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K,tile", [
    (4608, 4608, 100, (192, 256)),    # 432 tiles: one round, then 176 (69 % of the CUs)
    (1536, 12288, 65, (192, 256)),    # 384 tiles: one round, then 128
    (8192, 5120, 72, (256, 256)),     # 640 tiles: two rounds, then 128
])
def test_exact_integer_multi_round_grids(path, M, N, K, tile):
    """Outputs of more than one round of 192 x 256 or 256 x 256 tiles with a
    partly filled last round (the planner's tiles for these shapes): every
    workgroup index past the CU count maps to its own tile.  Integer inputs,
    fp32 C and C in the input format alternately; equal to the oracle in every
    element."""
    tm = dg.dgemm_tile_map(M, N, path)
    assert (tm["tile_rows"], tm["tile_cols"]) == tile
    out = "f32" if (M + K) % 2 == 0 else path
    print(f"case multi-round {path}->{out} {M}x{N}x{K} tile {tile}", flush=True)
    A, B = pair(M, N, K, "ints", path, seed=3150 + K)
    C = run(path, out, A, B, a_extra=8, b_extra=8)
    assert_exact(C, path, out, A, B)
    assert gap_untouched(C)


def test_repeat_runs_are_bitwise_identical():
    A, B = pair(1024, 1024, 2048, "normal", "bf16", seed=4000)
    C1 = run("bf16", "f32", A, B)
    C2 = run("bf16", "f32", A, B)
    assert torch.equal(C1, C2)


def test_non_default_stream():
    A, B = pair(520, 260, 300, "normal", "f16", seed=4100)
    ref = run("f16", "f16", A, B)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = run("f16", "f16", A, B, stream=s)
    assert torch.equal(ref, got)


@pytest.mark.parametrize("path,out", COMBOS)
def test_leading_dimensions_larger_than_rows(path, out):
    dtype = store(path)
    A, B = pair(333, 290, 515, "normal", dtype, seed=4200)
    C = run(path, out, A, B, a_extra=136, b_extra=264, c_extra=72)
    C64, S = oracle.gemm(dtype, A, B)
    assert oracle.check(to64(C), C64, S, TOL_MFMA, out)["ok"]
    assert gap_untouched(C)


@pytest.mark.parametrize("path,out", COMBOS)
def test_k_zero_writes_zeros_and_empty_outputs(path, out):
    dtype = store(path)
    A = np.zeros((300, 0), dtype=np.float32)
    Ad = torch.zeros((300, 8), dtype=TORCH[dtype], device="cuda")[:, :0]
    Bd = torch.zeros((1, 264), dtype=TORCH[dtype], device="cuda")[:0]
    C = sentinel_c(300, 264, out)
    ENTRY[path](Ad, Bd, C)
    torch.cuda.synchronize()
    assert bool((C.float() == 0).all().item()) and gap_untouched(C)
    assert A.shape[1] == 0
    C0 = torch.empty((0, 5), dtype=TORCH[out], device="cuda")
    ENTRY[path](torch.zeros((0, 3), dtype=TORCH[dtype], device="cuda"),
                 torch.zeros((3, 5), dtype=TORCH[dtype], device="cuda"), C0)


def test_invalid_arguments_leave_c_untouched():
    A, B = pair(64, 64, 64, "normal", "bf16", seed=4300)
    Ad = dev_matrix(A, "bf16")
    Bd = dev_matrix(B, "bf16")
    C = sentinel_c(64, 64, "f32")
    raw = torch.full((64 * 72 + 8,), 0, dtype=torch.bfloat16, device="cuda")
    mis = raw[1:1 + 64 * 72].view(64, 72)[:, :64]   # base misaligned by 2 bytes
    with pytest.raises(dg.DgemmError) as e:
        dg.gemm_bf16(mis, Bd, C)
    assert e.value.status == dg.DGEMM_ERR_MISALIGNED
    Cal = torch.full((64, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dg.DgemmError) as e:
        dg.gemm_bf16(Cal, Bd, Cal)
    assert e.value.status == dg.DGEMM_ERR_ALIAS
    torch.cuda.synchronize()
    assert bool(torch.isnan(C).all().item())
    assert bool(torch.isnan(Cal.float()).all().item())
    dg.gemm_bf16(Ad, Bd, C)
    torch.cuda.synchronize()
    C64, S = oracle.gemm("bf16", A, B)
    assert oracle.check(to64(C), C64, S, TOL_MFMA, "f32")["ok"]


def test_column_windows_of_one_buffer_are_not_an_alias():
    """A = X[:, :K] and C = X[:, K:] of one buffer share a row pitch and no
    byte: accepted, and A's window is left as it was."""
    M, K, N = 300, 264, 136
    A, B = pair(M, N, K, "ints", "bf16", seed=4400)
    X = torch.full((M, K + N), float("nan"), dtype=torch.bfloat16, device="cuda")
    X[:, :K] = TORCH_FROM(A, "bf16").to("cuda")
    Bd = dev_matrix(B, "bf16")
    dg.gemm_bf16(X[:, :K], Bd, X[:, K:])
    torch.cuda.synchronize()
    assert_exact(X[:, K:], "bf16", "bf16", A, B)
    assert torch.equal(X[:, :K].cpu(), TORCH_FROM(A, "bf16"))


def test_leading_dimensions_at_the_32_bit_descriptor_limit():
    """A's row pitch just under the largest a 256-row panel allows (256 lda 2 B
    < 2 GiB) and B's just under the largest a 64-row K step allows (128 ldb B
    < 2 GiB): the kernel's 32-bit buffer offsets reach ~2.14e9 bytes.  Each
    operand then spans about 2.1 GB of device memory."""
    M, N, K = 256, 64, 64
    lda = (1 << 31) // (256 * 2) - 8
    ldb = (1 << 31) // 128 - 8
    A, B = pair(M, N, K, "normal", "bf16", seed=7000)
    Abuf = torch.empty(((M - 1) * lda + K,), dtype=torch.bfloat16, device="cuda")
    Bbuf = torch.empty(((K - 1) * ldb + N,), dtype=torch.bfloat16, device="cuda")
    Ad = torch.as_strided(Abuf, (M, K), (lda, 1))
    Bd = torch.as_strided(Bbuf, (K, N), (ldb, 1))
    Ad.copy_(TORCH_FROM(A, "bf16"))
    Bd.copy_(TORCH_FROM(B, "bf16"))
    C = sentinel_c(M, N, "f32")
    dg.gemm_bf16(Ad, Bd, C)
    torch.cuda.synchronize()
    C64, S = oracle.gemm("bf16", A, B)
    assert oracle.check(to64(C), C64, S, TOL_MFMA, "f32")["ok"]
    assert gap_untouched(C)
    del Abuf, Bbuf


def test_output_beyond_2_31_elements():
    """C with 70000 x 32768 > 2^31 elements (4.6 GB of bf16): the epilogue's
    64-bit element offsets; rows at both ends checked against the oracle."""
    M, N, K = 70000, 32768, 64
    A, B = pair(M, N, K, "ints", "bf16", seed=7100)
    Ad, Bd = dev_matrix(A, "bf16", K), dev_matrix(B, "bf16", N)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dg.gemm_bf16(Ad, Bd, C)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 65535, 65536, 65537, M - 257, M - 256, M - 2, M - 1])
    C64, _ = oracle.gemm("bf16", A, B, rows=rows)
    got = to64(C[torch.from_numpy(rows).to("cuda")])
    assert np.array_equal(got, oracle.widen("bf16", oracle.round_to("bf16", C64)))
    del C
