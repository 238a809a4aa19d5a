"""The Stream-K schedule on the CPU, through the library's host query of it
(dgemm_stream_k_schedule runs the same schedule functions as the kernel).

Stream-K (the nine-levels tutorial, section 2.9) gives each of the 256
persistent workgroups an equal run of 64-k iterations across tile boundaries;
every tile is then reduced by its contributors together.  For every shape
below, over all 256 workgroups: every (tile, k step) is computed exactly once;
every 32 x 32 output block is reduced exactly once, by a contributor of its
tile, from exactly the pieces the tile's contributors computed, in k order; a
missing piece is recomputed with its contributor's own tile, k range and slot;
runs are balanced; and the pieces of one tile never leave one XCD.  No kernel
is launched."""
import collections

import pytest

import dense_gemm_matrix_amd as dg

G, XCD, BK, T, R = 256, 8, 64, 256, 32

SHAPES = [
    (4000, 3000, 4104),    # ragged: 192 tiles; K not a multiple of 64
    (512, 4096, 4096),     # 32 tiles: 8 workgroups per tile, runs on tile boundaries
    (2048, 2048, 2048),    # 64 tiles, 4 per tile
    (4096, 4096, 4096),    # 256 tiles: one whole tile per workgroup
    (256, 256, 2048),      # one tile, 32 workgroups of one XCD, one step each
    (300, 520, 8000),      # ragged in all three; 6 tiles over 6 XCDs
    (1000, 700, 2100),     # 12 tiles, 33 steps: runs of 2.06 and 3.09 steps
    (3840, 3840, 1280),    # 225 tiles, 20 steps: some XCDs with 28 tiles, some with 29
]


def schedule(M, N, K, present=True, fmt="bf16"):
    return {wg: dg.dgemm_stream_k_schedule(fmt, M, N, K, wg, present) for wg in range(G)}


def steps(item):
    return range(item["k_begin"] // BK, (item["k_end"] + BK - 1) // BK)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_every_step_once_every_block_reduced_once(M, N, K):
    tm, tn, nk = -(-M // T), -(-N // T), -(-K // BK)
    sched = schedule(M, N, K)
    cover = collections.Counter()
    blocks = collections.Counter()
    for wg, items in sched.items():
        for it in items:
            assert 0 <= it["tile_m"] < tm and 0 <= it["tile_n"] < tn
            tile = (it["tile_m"], it["tile_n"])
            assert it["role"] != "recompute"  # every piece present
            if it["role"] == "piece":
                assert 0 <= it["k_begin"] < it["k_end"] <= K
                assert it["k_begin"] % BK == 0 and (it["k_end"] % BK == 0 or it["k_end"] == K)
                for s in steps(it):
                    cover[tile + (s,)] += 1
            else:
                assert 0 <= it["lo"] <= it["hi"] <= 64
                for q in range(it["lo"], it["hi"]):
                    blocks[tile + (q,)] += 1
    assert set(cover) == {(i, j, s) for i in range(tm) for j in range(tn) for s in range(nk)}
    assert set(cover.values()) == {1}
    assert set(blocks) == {(i, j, q) for i in range(tm) for j in range(tn) for q in range(64)}
    assert set(blocks.values()) == {1}


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_reducers_add_exactly_the_tiles_pieces_in_k_order(M, N, K):
    sched = schedule(M, N, K)
    pieces = collections.defaultdict(dict)   # tile -> {rank: piece}
    for wg, items in sched.items():
        roles = [it["role"] for it in items]
        n = roles.count("piece")
        assert 1 <= n <= 2 or (n == 0 and not items)
        # pieces first, then one reduction per tile touched, in the same tile order
        assert roles == ["piece"] * n + ["reduce"] * n
        for i in range(n):
            pc, red = items[i], items[n + i]
            assert (pc["tile_m"], pc["tile_n"]) == (red["tile_m"], red["tile_n"])
            assert pc["slot"] == 2 * wg + i
            assert pc["first"] <= wg // XCD <= pc["last"]
            pieces[(pc["tile_m"], pc["tile_n"])][wg // XCD] = pc
        if n == 2:
            assert items[0]["k_end"] == K and items[1]["k_begin"] == 0
    for wg, items in sched.items():
        for red in (it for it in items if it["role"] == "reduce"):
            tile = (red["tile_m"], red["tile_n"])
            assert set(pieces[tile]) == set(range(red["first"], red["last"] + 1))
            # contributor order is k order, pieces end to end
            ps = [pieces[tile][p] for p in range(red["first"], red["last"] + 1)]
            assert ps[0]["k_begin"] == 0 and ps[-1]["k_end"] == K
            for a, b in zip(ps, ps[1:]):
                assert a["k_end"] == b["k_begin"]
            # the share is this rank's equal part of the 64 blocks
            n, i = len(ps), wg // XCD - red["first"]
            assert (red["lo"], red["hi"]) == (64 * i // n, 64 * (i + 1) // n)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_missing_pieces_are_recomputed_as_their_contributor_would(M, N, K):
    present, missing = schedule(M, N, K, True), schedule(M, N, K, False)
    own = {}
    for wg, items in present.items():
        for it in items:
            if it["role"] == "piece":
                own[it["slot"]] = it
    for wg in range(G):
        a, b = present[wg], missing[wg]
        assert [it for it in b if it["role"] != "recompute"] == a
        x = wg % XCD
        i = 0
        for red in (it for it in a if it["role"] == "reduce"):
            # before this reduction: every other contributor's piece of the tile, in rank order
            while b[i] != red:
                i += 1
            others = [p for p in range(red["first"], red["last"] + 1) if p != wg // XCD]
            rec = b[i - len(others): i]
            assert [it["role"] for it in rec] == ["recompute"] * len(others)
            for p, it in zip(others, rec):
                src = own[it["slot"]]
                assert it["slot"] in (2 * (x + XCD * p), 2 * (x + XCD * p) + 1)
                for key in ("tile_m", "tile_n", "k_begin", "k_end", "slot"):
                    assert it[key] == src[key]
            i += 1


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_runs_are_balanced_and_tiles_stay_on_one_xcd(M, N, K):
    nk = -(-K // BK)
    sched = schedule(M, N, K)
    per_xcd = collections.defaultdict(list)
    tile_xcd = {}
    for wg, items in sched.items():
        n = sum(len(steps(it)) for it in items if it["role"] == "piece")
        assert n <= nk
        if items:
            per_xcd[wg % XCD].append(n)
        for it in items:
            tile = (it["tile_m"], it["tile_n"])
            assert tile_xcd.setdefault(tile, wg % XCD) == wg % XCD
    for x, ns in per_xcd.items():
        assert len(ns) == R and min(ns) >= 1 and max(ns) - min(ns) <= 1, (x, ns)
    allns = [n for ns in per_xcd.values() for n in ns]
    assert max(allns) - min(allns) <= -(-nk // R) + 1


def test_shapes_stream_k_does_not_run_are_rejected():
    bad = [("f32", 4096, 4096, 4096),      # 16-bit inputs only
           ("bf16", 256, 256, 1984),       # one tile with fewer 64-k steps than 32 ranks
           ("bf16", 4097, 4096, 4096),     # more tiles than CUs
           ("f16", 4096, 4096, 0), ("f16", 4096, 4096, -1)]
    for fmt, M, N, K in bad:
        with pytest.raises(dg.DgemmError):
            dg.dgemm_stream_k_schedule(fmt, M, N, K, 0)
    with pytest.raises(dg.DgemmError):
        dg.dgemm_stream_k_schedule("bf16", 4096, 4096, 4096, 256)  # outside the grid
    # XCDs without a tile: their workgroups have nothing to do
    assert dg.dgemm_stream_k_schedule("bf16", 300, 520, 8000, 7) == []


def test_plan_override_and_the_plan_query():
    ws = 1 << 30
    sk_ws = 2 * G * T * T * 4 + G * 8
    try:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_STREAM_K)
        p = dg.gemm_ex_plan("bf16", 4000, 3000, 4104, ws, out_same=True)
        assert p["stream_k"] and p["splits"] == 0
        assert (p["tile_rows"], p["tile_cols"]) == (256, 256)
        assert p["workspace_bytes"] == sk_ws
        # too little workspace, fp32 inputs, shapes Stream-K does not run: the cost model's plan
        for args in (("bf16", 4000, 3000, 4104, sk_ws - 1), ("f32", 4000, 3000, 4104, ws),
                     ("bf16", 256, 256, 64, ws), ("f16", 4352, 4096, 4096, ws)):
            q = dg.gemm_ex_plan(*args)
            assert not q["stream_k"] and q["splits"] >= 1
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 192, 256, 3)
        p = dg.gemm_ex_plan("bf16", 4000, 3000, 4104, ws)
        assert (p["tile_rows"], p["tile_cols"], p["splits"]) == (192, 256, 3)
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 128, 128, 1)
        p = dg.gemm_ex_plan("f16", 4000, 3000, 4104, ws)
        assert (p["tile_rows"], p["tile_cols"], p["splits"], p["workspace_bytes"]) == (128, 128, 1, 0)
        # a tile shape the kernel does not have: the cost model's plan
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
        auto = dg.gemm_ex_plan("bf16", 4000, 3000, 4104, ws)
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 96, 96, 1)
        assert dg.gemm_ex_plan("bf16", 4000, 3000, 4104, ws) == auto
        # Stream-K ruled out
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_NO_STREAM_K)
        for M, N, K in [(512, 4096, 4096), (2048, 2048, 2048), (4000, 3000, 4104)]:
            assert not dg.gemm_ex_plan("bf16", M, N, K, ws)["stream_k"]
        with pytest.raises(dg.DgemmError):
            dg.dgemm_set_plan_override(7)
        with pytest.raises(dg.DgemmError):
            dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 128, 128, 0)
    finally:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
    with pytest.raises(dg.DgemmError):
        dg.dgemm_set_stream_k_wait_us(float("nan"))
    dg.dgemm_set_stream_k_wait_us(-1)
