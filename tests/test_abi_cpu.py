"""The C ABI on the CPU: the library loads, exports every function the header
declares, rejects invalid arguments before touching a device, and its
workgroup -> tile map is a bijection.  No kernel is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import dense_gemm_matrix_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|char|void)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("gemm_f32", "gemm_f32_3xbf16", "gemm_bf16", "gemm_f16", "gemm_ex",
                 "gemm_ex_static", "gemm_ex_plan", "dgemm_status_string", "dgemm_tile_map"):
        assert want in names


def test_library_exports_every_declared_function():
    lib = dg.raw()
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings():
    seen = set()
    for s in range(9):
        msg = dg.dgemm_status_string(s)
        assert msg.startswith("DGEMM_") and msg not in seen
        seen.add(msg)
    assert "unknown" in dg.dgemm_status_string(99)


# Fake, never-dereferenced addresses: validation happens before any device call.
PA, PB, PC = 0x10000000, 0x20000000, 0x30000000
V = ctypes.c_void_p


def call(fn, M, N, K, A, lda, B, ldb, C, ldc, out=0):
    lib = dg.raw()
    if fn in ("gemm_f32", "gemm_f32_3xbf16"):
        return getattr(lib, fn)(M, N, K, V(A), lda, V(B), ldb, V(C), ldc, None)
    return getattr(lib, fn)(M, N, K, V(A), lda, V(B), ldb, V(C), ldc, out, None)


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_f32_3xbf16", "gemm_bf16", "gemm_f16"])
def test_validation_errors(fn):
    es = 4 if fn.startswith("gemm_f32") else 2
    ok_ld = 64
    assert call(fn, -1, 8, 8, PA, ok_ld, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_INVALID_VALUE
    assert call(fn, 8, -1, 8, PA, ok_ld, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_INVALID_VALUE
    assert call(fn, 8, 8, -1, PA, ok_ld, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_INVALID_VALUE
    assert call(fn, 8, 8, 8, 0, ok_ld, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_INVALID_VALUE
    assert call(fn, 8, 8, 8, PA, ok_ld, 0, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_INVALID_VALUE
    assert call(fn, 8, 8, 8, PA, ok_ld, PB, ok_ld, 0, ok_ld) == dg.DGEMM_ERR_INVALID_VALUE
    if not fn.startswith("gemm_f32"):
        assert call(fn, 8, 8, 8, PA, ok_ld, PB, ok_ld, PC, ok_ld, out=2) == dg.DGEMM_ERR_INVALID_VALUE
    assert call(fn, 8, 8, 72, PA, 64, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_LEADING_DIM
    assert call(fn, 8, 72, 8, PA, ok_ld, PB, 64, PC, 80) == dg.DGEMM_ERR_LEADING_DIM
    assert call(fn, 8, 72, 8, PA, ok_ld, PB, 80, PC, 64) == dg.DGEMM_ERR_LEADING_DIM
    assert call(fn, 8, 8, 8, PA + 2, ok_ld, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_MISALIGNED
    assert call(fn, 8, 8, 8, PA, ok_ld, PB + 8, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_MISALIGNED
    assert call(fn, 8, 8, 8, PA, ok_ld, PB, ok_ld, PC + 4, ok_ld) == dg.DGEMM_ERR_MISALIGNED
    odd = 16 // es + 1  # a row pitch that is not a multiple of 16 bytes
    assert call(fn, 8, 2, 2, PA, odd, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_MISALIGNED
    assert call(fn, 8, 2, 2, PA, ok_ld, PB, odd, PC, ok_ld) == dg.DGEMM_ERR_MISALIGNED
    # C overlapping A or B
    assert call(fn, 8, 8, 8, PA, ok_ld, PB, ok_ld, PA + 64 * es, ok_ld) == dg.DGEMM_ERR_ALIAS
    assert call(fn, 8, 8, 8, PA, ok_ld, PB, ok_ld, PB, ok_ld) == dg.DGEMM_ERR_ALIAS
    # 32-bit descriptor range
    huge = (1 << 31) // (256 * es)
    assert call(fn, 8, 8, 8, PA, huge, PB, ok_ld, PC, ok_ld) == dg.DGEMM_ERR_TOO_LARGE
    # one K step of B spans 128 * ldb bytes (64 rows of 16-bit data, 32 of fp32)
    far = 0x7000000000
    assert call(fn, 8, 8, 8, PA, ok_ld, PB, (1 << 31) // 128, far, ok_ld) == dg.DGEMM_ERR_TOO_LARGE
    # a 256-row panel of C spans 256 * ldc * esize_out bytes (fp32 C here)
    big_c = (1 << 31) // (256 * 4)
    assert call(fn, 8, 8, 8, PA, ok_ld, PB, ok_ld, far, big_c) == dg.DGEMM_ERR_TOO_LARGE



def byte_overlap(base_x, rows_x, row_bytes_x, pitch_x, base_y, rows_y, row_bytes_y, pitch_y):
    """Brute force: whether two row-strided byte sets share a byte."""
    xs = set()
    for i in range(rows_x):
        xs.update(range(base_x + i * pitch_x, base_x + i * pitch_x + row_bytes_x))
    for j in range(rows_y):
        r = range(base_y + j * pitch_y, base_y + j * pitch_y + row_bytes_y)
        if not xs.isdisjoint(r):
            return True
    return False


def test_alias_rule_against_brute_force():
    """C against A (gemm_bf16, bf16 C): with equal row pitches the library
    decides overlap exactly, row by row, so column windows of one buffer are
    accepted; with different pitches it compares first-to-last-byte spans.
    B's pitch is made too large for the 32-bit descriptor range, a check that
    comes after the alias check: every call returns before any launch, with
    ALIAS or TOO_LARGE telling the alias decision."""
    import random
    rnd = random.Random(77)
    far_b = 0x6000000000
    ldb_huge = (1 << 31) // 128 + 8
    n_exact = 0
    for trial in range(400):
        M = rnd.randint(1, 6)
        K = 8 * rnd.randint(1, 4)
        N = 8 * rnd.randint(1, 4)
        lda = max(K, N) + 8 * rnd.randint(0, 5)
        ldc = lda if trial % 3 else N + 8 * rnd.randint(0, 5)
        a0 = 0x10000000
        c0 = a0 + 16 * rnd.randint(-4 * lda // 8, 4 * lda // 8 + 4)
        st = call("gemm_bf16", M, N, K, a0, lda, far_b, ldb_huge, c0, ldc, out=1)
        assert st in (dg.DGEMM_ERR_ALIAS, dg.DGEMM_ERR_TOO_LARGE), st
        exact = byte_overlap(a0, M, 2 * K, 2 * lda, c0, M, 2 * N, 2 * ldc)
        if lda == ldc or M == 1:
            want = exact
            n_exact += 1
        else:
            want = a0 < c0 + 2 * ((M - 1) * ldc + N) and c0 < a0 + 2 * ((M - 1) * lda + K)
        assert (st == dg.DGEMM_ERR_ALIAS) == want, (M, N, K, lda, ldc, c0 - a0)
    assert n_exact > 200
    # Two column windows of one buffer X[M, K + N]: A = X[:, :K], C = X[:, K:].
    M, K, N = 64, 64, 32
    st = call("gemm_bf16", M, N, K, PA, K + N, far_b, ldb_huge, PA + 2 * K, K + N, out=1)
    assert st == dg.DGEMM_ERR_TOO_LARGE
    st = call("gemm_bf16", M, N, K, PA, K + N, far_b, ldb_huge, PA + 2 * K - 16, K + N, out=1)
    assert st == dg.DGEMM_ERR_ALIAS


def test_static_scratch_size_and_its_limit():
    """The binding's constant is the header's, and a budget beyond the static
    array is rejected before anything else (no device needed)."""
    text = open(HEADER).read()
    m = re.search(r"#define DGEMM_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == dg.DGEMM_STATIC_SCRATCH_BYTES
    lib = dg.raw()
    st = lib.gemm_ex_static(1, 0, 8, 8, 8, V(PA), 64, V(PB), 64, V(PC), 64, ctypes.c_float(1.0),
                            ctypes.c_float(0.0), None, 0, dg.DGEMM_STATIC_SCRATCH_BYTES + 1, None)
    assert st == dg.DGEMM_ERR_SCRATCH_SIZE
    assert "DGEMM_STATIC_SCRATCH_BYTES" in dg.dgemm_status_string(st)
    # otherwise the same validation as gemm_ex, before any device call
    st = lib.gemm_ex_static(1, 0, 8, 8, 72, V(PA), 64, V(PB), 64, V(PC), 64, ctypes.c_float(1.0),
                            ctypes.c_float(0.0), None, 0, 0, None)
    assert st == dg.DGEMM_ERR_LEADING_DIM
    st = lib.gemm_ex_static(1, 0, 8, 8, 8, V(PA), 64, V(PB), 64, V(PA), 64, ctypes.c_float(1.0),
                            ctypes.c_float(0.0), None, 0, 1 << 20, None)
    assert st == dg.DGEMM_ERR_ALIAS


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_f32_3xbf16", "gemm_bf16", "gemm_f16"])
def test_empty_output_is_a_no_op_without_device(fn):
    # M == 0 or N == 0: nothing to write, no device needed, even with NULL pointers.
    assert call(fn, 0, 8, 8, 0, 8, 0, 8, 0, 8) == dg.DGEMM_OK
    assert call(fn, 8, 0, 8, 0, 8, 0, 1, 0, 1) == dg.DGEMM_OK


@pytest.mark.parametrize("M,N", [(1, 1), (256, 256), (4096, 4096), (16384, 4096), (4000, 3000),
                                 (257, 4097), (2560, 256), (256, 9000), (7777, 3333), (512, 512)])
@pytest.mark.parametrize("fmt", ["f32", "bf16", "f32x3"])
def test_tile_map_is_a_bijection(M, N, fmt):
    info = dg.dgemm_tile_map(M, N, fmt)
    tm_n = -(-M // info["tile_rows"])
    tn_n = -(-N // info["tile_cols"])
    assert info["num_wg"] == tm_n * tn_n
    seen = set()
    for wg in range(info["num_wg"]):
        t = dg.dgemm_tile_map(M, N, fmt, wg)
        assert 0 <= t["tile_m"] < tm_n and 0 <= t["tile_n"] < tn_n
        seen.add((t["tile_m"], t["tile_n"]))
    assert len(seen) == info["num_wg"]


def test_tile_map_gives_each_xcd_a_compact_block():
    """At 4096 x 4096 (16 x 16 tiles) the workgroups of one XCD (wg % 8) cover a
    4 x 8 block of tiles: 4 A panels and 8 B panels instead of up to 32 each."""
    for x in range(8):
        tiles = [dg.dgemm_tile_map(4096, 4096, "bf16", wg) for wg in range(x, 256, 8)]
        rows = {t["tile_m"] for t in tiles}
        cols = {t["tile_n"] for t in tiles}
        assert len(tiles) == 32 and len(rows) == 4 and len(cols) == 8


def test_tile_map_rejects_bad_arguments():
    lib = dg.raw()
    z = ctypes.c_int()
    assert lib.dgemm_tile_map(-1, 4, 1, 0, *[ctypes.byref(z)] * 5) == dg.DGEMM_ERR_INVALID_VALUE
    assert lib.dgemm_tile_map(4, 4, 7, 0, *[ctypes.byref(z)] * 5) == dg.DGEMM_ERR_INVALID_VALUE


@pytest.mark.parametrize("M,N,fmt,tile", [
    (4096, 4096, "bf16", (256, 256)),     # 256 tiles: one per CU
    (16384, 4096, "bf16", (256, 256)),    # four full waves of tiles
    (4000, 3000, "bf16", (192, 256)),     # 252 tiles instead of 192
    (4000, 3000, "f16", (192, 256)),
    # a last round that fills part of the CUs counts less than a full one for the
    # 16-bit 256^2 and 192x256 tiles (a partly filled chip clocks higher)
    (4608, 4608, "bf16", (192, 256)),     # 432 tiles (1.69 rounds) beat 1296 of 128^2
    (4096, 5120, "f16", (192, 256)),      # 440 tiles (1.72 rounds)
    (1536, 12288, "bf16", (192, 256)),    # 384 tiles (1.5 rounds)
    (12288, 5120, "bf16", (256, 256)),    # 960 tiles (3.75 rounds) beat 1280 of 192x256
    (8192, 8192, "bf16", (256, 256)),     # four full rounds
    (6144, 4096, "bf16", (192, 256)),     # two full rounds beat 1536 tiles of 128^2 (three
                                          # rounds of pairs, each 1.35x one workgroup)
    (8192, 5120, "bf16", (256, 256)),     # 2.5 rounds beat 2560 tiles of 128^2
    (2048, 4096, "bf16", (128, 128)),     # 512 tiles of 128^2: one round of pairs (1.26x)
    (512, 512, "bf16", (32, 32)),         # slice-K: 256 tiles of 32^2
    (1024, 1024, "f16", (64, 64)),        # slice-K: 256 tiles of 64^2
    (1024, 1152, "bf16", (128, 128)),     # 72 tiles of 128^2: past the 16-bit slice-K limit of 64
    (2048, 2048, "f16", (128, 128)),      # 256 tiles instead of 64
    (4000, 3000, "f32", (128, 128)),      # 768 tiles (3 waves) beat 192 of 256^2
    (4096, 4096, "f32", (128, 128)),      # fp32 prefers 128^2 (two workgroups per CU)
    (2048, 2048, "f32", (128, 128)),      # 256 tiles of 128^2
    (2048, 1280, "f32", (128, 128)),      # 160 tiles of 128^2: past the fp32 slice-K limit of 144
    (1536, 1536, "f32", (32, 32)),        # 144 tiles of 128^2: slice-K
    (1024, 1152, "f32", (32, 32)),        # 72 tiles of 128^2: slice-K
    (1024, 1024, "f32", (64, 64)),        # 64 tiles of 128^2: slice-K, 256 tiles of 64^2
    (768, 768, "f32", (32, 32)),          # slice-K: 576 tiles of 32^2 share CUs three at a time
    (512, 512, "f32", (32, 32)),          # slice-K: 256 tiles of 32^2
    (1, 1, "f32", (32, 32)),
    (4000, 3000, "f32x3", (256, 256)),
    (4608, 4608, "f32x3", (128, 128)),    # 3 x bf16 keeps whole rounds for its 256^2 tile
    (4096, 5120, "f32x3", (128, 128)),
    (1024, 1152, "f32x3", (128, 128)),    # 72 tiles of 128^2: past the 3 x bf16 slice-K limit of 64
    (1024, 1024, "f32x3", (64, 64)),      # slice-K, 256 tiles of 64^2
    (768, 768, "f32x3", (64, 64)),
    (512, 512, "f32x3", (32, 32)),        # slice-K: 256 tiles of 32^2
])
def test_tile_choice(M, N, fmt, tile):
    info = dg.dgemm_tile_map(M, N, fmt)
    assert (info["tile_rows"], info["tile_cols"]) == tile


# ---------------------------------------------------------------- gemm_ex

def call_ex(in_fmt, out, M, N, K, A, lda, B, ldb, C, ldc, alpha=1.0, beta=0.0, bias=0, act=0,
            ws=0, ws_bytes=0):
    return dg.raw().gemm_ex(in_fmt, out, M, N, K, V(A), lda, V(B), ldb, V(C), ldc, alpha, beta,
                            V(bias) if bias else None, act, V(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("in_fmt", [0, 1, 2, 3])
def test_gemm_ex_validation_errors(in_fmt):
    es = 4 if in_fmt in (0, 3) else 2
    ld = 64
    ok = dict(A=PA, lda=ld, B=PB, ldb=ld, C=PC, ldc=ld)
    INV, MIS, ALI = dg.DGEMM_ERR_INVALID_VALUE, dg.DGEMM_ERR_MISALIGNED, dg.DGEMM_ERR_ALIAS
    assert dg.raw().gemm_ex(7, 0, 8, 8, 8, V(PA), ld, V(PB), ld, V(PC), ld, 1.0, 0.0, None, 0,
                            None, 0, None) == INV
    assert call_ex(in_fmt, 2, 8, 8, 8, **ok) == INV          # bad out
    assert call_ex(in_fmt, 0, 8, 8, 8, **ok, act=2) == INV   # bad act
    assert call_ex(in_fmt, 0, 8, 8, 8, **ok, ws=0, ws_bytes=64) == INV  # bytes without memory
    assert call_ex(in_fmt, 0, -1, 8, 8, **ok) == INV
    assert call_ex(in_fmt, 0, 8, 8, 72, **ok) == dg.DGEMM_ERR_LEADING_DIM
    assert call_ex(in_fmt, 0, 8, 8, 8, **ok, bias=0x40000002) == MIS
    assert call_ex(in_fmt, 0, 8, 8, 8, **ok, ws=0x50000008, ws_bytes=1 << 20) == MIS
    assert call_ex(in_fmt, 0, 8, 8, 8, **ok, bias=PC + 4 * 2) == ALI   # bias inside C's row 0
    assert call_ex(in_fmt, 0, 8, 8, 8, A=PA, lda=ld, B=PB, ldb=ld, C=PA, ldc=ld) == ALI
    # a workspace that a split plan would use, overlapping A (small fp32 outputs
    # take the slice-K kernel, which uses none)
    M, N, K = (1024, 1024, 16384) if in_fmt == 0 else (64, 64, 1 << 14)
    plan = dg.gemm_ex_plan({0: "f32", 1: "bf16", 2: "f16", 3: "f32x3"}[in_fmt], M, N, K, 1 << 30)
    assert plan["splits"] > 1
    assert call_ex(in_fmt, 0, M, N, K, A=PA, lda=K, B=PB, ldb=N, C=PC, ldc=N,
                   ws=PA + 16 * es, ws_bytes=1 << 30) == ALI
    # empty outputs stay a no-op without a device, whatever the epilogue
    assert call_ex(in_fmt, 0, 0, 8, 8, 0, 8, 0, 8, 0, 8, alpha=2.0, beta=1.0, act=1) == dg.DGEMM_OK


def test_gemm_ex_plan_rejects_bad_arguments():
    lib = dg.raw()
    z = ctypes.c_int()
    u = ctypes.c_size_t()
    assert lib.gemm_ex_plan(5, 0, 8, 8, 8, 0, *[ctypes.byref(z)] * 3, ctypes.byref(u)) == \
        dg.DGEMM_ERR_INVALID_VALUE
    assert lib.gemm_ex_plan(1, 3, 8, 8, 8, 0, *[ctypes.byref(z)] * 3, ctypes.byref(u)) == \
        dg.DGEMM_ERR_INVALID_VALUE
    assert lib.gemm_ex_plan(1, 0, 8, -8, 8, 0, *[ctypes.byref(z)] * 3, ctypes.byref(u)) == \
        dg.DGEMM_ERR_INVALID_VALUE


@pytest.mark.parametrize("M,N,K,fmt", [(4096, 4096, 4096, "bf16"), (16384, 4096, 4096, "bf16"),
                                       (4000, 3000, 4104, "bf16"), (4096, 4096, 4096, "f32"),
                                       (512, 4096, 4096, "bf16"), (512, 512, 512, "f32")])
def test_plan_without_workspace_is_the_plain_launch(M, N, K, fmt):
    p = dg.gemm_ex_plan(fmt, M, N, K, 0)
    t = dg.dgemm_tile_map(M, N, fmt)
    assert p["splits"] == 1 and p["workspace_bytes"] == 0
    assert (p["tile_rows"], p["tile_cols"]) == (t["tile_rows"], t["tile_cols"])


@pytest.mark.parametrize("M,N,K,fmt,splits", [
    (4096, 4096, 4096, "bf16", 1),      # 256 tiles already fill the CUs
    (16384, 4096, 4096, "bf16", 1),
    (4000, 3000, 4104, "bf16", 1),
    (512, 4096, 4096, "bf16", None),    # one GPU's row share of the 4096^3 problem
    (1024, 1024, 16384, "f32", None),   # deep K: 8 splits of 128^2 beat slice-K
    (256, 256, 8192, "f32x3", None),    # deep K: 16 splits of 128^2 beat slice-K
    (64, 64, 4096, "f16", None),
    (256, 256, 65536, "bf16", None),
    (1024, 1024, 2048, "bf16", 1),      # slice-K (12.5 us) beats every split (16.8 us best)
    (1024, 1024, 4104, "bf16", 4),      # full 64x64 slice-K grid: its per-block cost grows
    (512, 2048, 4104, "bf16", 4),       # with the fill, and 4 splits measure 10-16 % faster
    (4608, 4096, 16384, "bf16", 2),     # split-K is weighed with whole rounds: two splits
    (12288, 1536, 16384, "bf16", 2),    # of 192x256 measured 4-6 % faster than unsplit
])
@pytest.mark.usefixtures("no_stream_k")
def test_split_plans(M, N, K, fmt, splits):
    p = dg.gemm_ex_plan(fmt, M, N, K, 1 << 40)
    if splits == 1:
        assert p["splits"] == 1 and p["workspace_bytes"] == 0
        return
    if splits is not None:
        assert p["splits"] == splits
    assert p["splits"] > 1
    ldw = -(-N // 4) * 4
    assert p["workspace_bytes"] == p["splits"] * M * ldw * 4
    # less workspace than the best plan wants: a plan that fits, possibly unsplit
    q = dg.gemm_ex_plan(fmt, M, N, K, p["workspace_bytes"] - 1)
    assert q["workspace_bytes"] <= p["workspace_bytes"] - 1
    assert q["splits"] < p["splits"] or (q["tile_rows"], q["tile_cols"]) != \
        (p["tile_rows"], p["tile_cols"])


# ---------------------------------------------------------------- planner properties

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=300, deadline=None)
@given(M=st.integers(0, 20000), N=st.integers(0, 20000), K=st.integers(0, 70000),
       fmt=st.sampled_from(["f32", "bf16", "f16", "f32x3"]),
       ws=st.sampled_from([0, 1, 1 << 16, 1 << 20, 1 << 24, 1 << 28, 1 << 40]))
def test_plan_invariants(M, N, K, fmt, ws):
    p = dg.gemm_ex_plan(fmt, M, N, K, ws)
    slice = {(64, 64), (32, 32)}
    tiles = {"f32": {(128, 128)} | slice, "bf16": {(256, 256), (192, 256), (128, 128)} | slice,
             "f16": {(256, 256), (192, 256), (128, 128)} | slice,
             "f32x3": {(256, 256), (128, 128)} | slice}[fmt]
    assert (p["tile_rows"], p["tile_cols"]) in tiles
    assert p["workspace_bytes"] <= ws
    if p["tile_rows"] < 128:
        # slice-K: outputs of at most 144 tiles of 128^2 (fp32) or 64 (the others), no workspace
        assert -(-M // 128) * -(-N // 128) <= (144 if fmt == "f32" else 64)
        assert p["splits"] == 1 and p["workspace_bytes"] == 0
    if p["stream_k"]:
        # one persistent workgroup per CU; two fp32 tiles and a flag each
        assert fmt in ("bf16", "f16") and M > 0 and N > 0 and K > 0
        assert (p["tile_rows"], p["tile_cols"], p["splits"]) == (256, 256, 0)
        assert p["workspace_bytes"] == 2 * 256 * 256 * 256 * 4 + 256 * 8
        dg.dgemm_stream_k_schedule(fmt, M, N, K, 0)  # a shape the schedule runs
        return
    assert 1 <= p["splits"] <= 16
    if p["splits"] == 1:
        assert p["workspace_bytes"] == 0
        t = dg.dgemm_tile_map(M, N, fmt)
        assert (p["tile_rows"], p["tile_cols"]) == (t["tile_rows"], t["tile_cols"])
    else:
        assert M > 0 and N > 0 and K > 0
        assert p["workspace_bytes"] == p["splits"] * M * (-(-N // 4) * 4) * 4
        bk = 64 if fmt in ("bf16", "f16") else 32
        nk = -(-K // bk)
        steps = -(-nk // p["splits"])
        # every split gets at least one K step, and the splits cover K exactly once
        assert (p["splits"] - 1) * steps < nk <= p["splits"] * steps


def test_header_is_plain_c_and_the_c_client_links():
    """include/dgemm.h compiles as C11 (-Wall -Wextra -Werror) in the C test
    client, and the client built by build() resolves libdgemm.so in-tree."""
    import shutil
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    src = os.path.join(here, "c_client", "gemm_client.c")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    subprocess.run([gcc, "-std=c11", "-fsyntax-only", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include", src],
                   check=True)
    binary = os.path.join(here, "c_client", "gemm_client")
    assert os.path.exists(binary), "run build() first"
    ldd = subprocess.run(["ldd", binary], capture_output=True, text=True, check=True).stdout
    line = [l for l in ldd.splitlines() if "libdgemm.so" in l]
    assert line and os.path.join(root, "dense_gemm_matrix_amd") in os.path.realpath(
        line[0].split("=>")[1].split("(")[0].strip()), ldd


def test_slice_k_plans_and_their_override():
    """Small outputs get the slice-K tiles (K split across the waves of a
    workgroup), in every input format: no workspace, whatever is offered,
    unless a split plan is estimated clearly faster.  The plan override forces
    a slice-K tile with its wave count in place of the split count."""
    for fmt in ("f32", "f32x3", "bf16", "f16"):
        for M, N, K in [(512, 512, 512), (256, 256, 2048), (1024, 1024, 1024), (37, 65, 7),
                        (8, 8, 0)]:
            for ws in (0, 1 << 30):
                p = dg.gemm_ex_plan(fmt, M, N, K, ws)
                t = dg.dgemm_tile_map(M, N, fmt)
                assert p["tile_rows"] in (32, 64) and p["splits"] == 1 and p["workspace_bytes"] == 0
                assert (p["tile_rows"], p["tile_cols"]) == (t["tile_rows"], t["tile_cols"])
    try:
        for fmt in ("f32", "f32x3", "bf16", "f16"):
            for tile, waves in ((32, 4), (32, 8), (64, 4), (32, 1), (64, 1)):
                dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, tile, tile, waves)
                p = dg.gemm_ex_plan(fmt, 2000, 1500, 300, 1 << 30)  # beyond the automatic limit
                assert (p["tile_rows"], p["tile_cols"], p["splits"], p["workspace_bytes"]) == \
                    (tile, tile, 1, 0)
            dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
            auto = dg.gemm_ex_plan(fmt, 2000, 1500, 300, 0)
            assert auto["tile_rows"] in (128, 192, 256)
            for tile, waves in ((64, 8), (32, 3), (32, 2)):    # no such kernel: the planner's plan
                dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, tile, tile, waves)
                assert dg.gemm_ex_plan(fmt, 2000, 1500, 300, 0) == auto
        # the 128 x 128 grid, split or not, stays reachable for small outputs
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 128, 128, 8)
        for fmt in ("f32", "f32x3", "bf16", "f16"):
            p = dg.gemm_ex_plan(fmt, 512, 512, 512, 1 << 30)
            assert (p["tile_rows"], p["splits"]) == (128, 8)
    finally:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
