"""Benchmark: GEMM TFLOP/s at M = N = K = 4096 and fraction of the MI355X
matrix-core peak, on one GPU.

A step is one C = A*B call of the library (global -> LDS staging, the LDS ring,
the swizzled layout, the matrix-instruction loop and the epilogue all run inside
that one kernel) on inputs already resident in HBM.  The headline line is the
bf16 4096^3 product with normal(0,1) inputs and fp32 C; the fp16 (fp16 C) and
fp32-input 4096^3 products are measured the same way and reported under
"per_dtype".  Also reported: the register-only matrix-instruction ceiling the
bf16 kernel is held to under the board's power limit ("mfma_ceiling"); the same product from a cold cache (each launch
after a 512 MiB write), with --vendor torch.matmul (hipBLASLt) on the same inputs,
and the graphics clock and socket power amd-smi reads while the product runs.  The
other parity workloads, and one GPU's row share of the 4096^3
product (512 x 4096 x 4096), are timed under "other_shapes", unsplit and, where
the planner splits K, through gemm_ex with a workspace; each both launched call by
call from Python and replayed from a HIP graph (the small shapes are otherwise
bound by the host's launch rate).  "plan_compare" times the cost model's plan
against a forced Stream-K plan on the shapes with fewer tiles than CUs;
"plan_compare_small" the slice-K plans of small outputs against the 128 x 128
grid kernel; "plan_compare_tiles" the cost model's unsplit tile against each
16-bit tile forced, on outputs of one to four rounds of 256 x 256 tiles.

    python bench.py [--steps K] [--warmup W] [--dtype bf16|f16|f32]
                    [--no-cpu-baseline] [--no-per-dtype] [--no-shapes]
                    [--no-power-clock] [--no-cold-cache] [--no-ceiling] [--no-plans]
                    [--vendor] [--settle-s S]
    python bench.py --copy-calibration      # plain copy of known size, for HBM counters

Only one GPU is used; --gpus N with N > 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s at M=N=K=4096 bf16/fp16/fp32 and % of MI355X MFMA peak"
# MI355X published dense matrix peaks, TFLOP/s.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
WORKLOAD_FOR = {"bf16": "bf16_4096", "f16": "f16_4096", "f32": "f32_4096"}
DESCRIPTION = {
    "bf16_4096": "bf16 GEMM M=N=K=4096, row-major A and B, normal(0,1) inputs, fp32 accumulate, fp32 C",
    "f16_4096": "fp16 GEMM M=N=K=4096, row-major A and B, uniform[-1,1] inputs, fp32 accumulate, fp16 C",
    "f32_4096": "fp32 GEMM M=N=K=4096, row-major A and B, uniform[-1,1] inputs, fp32 accumulate, fp32 C",
}
# The files that define the dominant (16-bit) kernel: counters taken on it stay
# valid while these are unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "dense_gemm_matrix_amd", "csrc", f)
                  for f in ("gemm16.hip", "kern_common.h", "dgemm_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def gemm_flops(M: int, N: int, K: int) -> int:
    """Floating-point operations of one product: one multiply and one add per term."""
    return 2 * M * N * K


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    return gemm_flops(M, N, K) / seconds / 1e12


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha():
        return None
    v = fields.get(f"{workload}_hbm_bytes_per_launch")
    return int(v) if v else None


def device_inputs(name):
    import torch
    from synth_inputs import to_torch, torch_dtype, workload
    A, B, meta = workload(name)
    Ad = to_torch(A, meta["dtype"]).to("cuda")
    Bd = to_torch(B, meta["dtype"]).to("cuda")
    Cd = torch.empty((meta["M"], meta["N"]), dtype=torch_dtype(meta["out"]), device="cuda")
    return A, B, Ad, Bd, Cd, meta


def settle_clock(entry, Ad, Bd, Cd, seconds: float) -> int:
    """Launches back to back for `seconds` of wall time, a few launches queued
    ahead at most, and returns how many ran.  The chip's clock and power
    controller take tens of milliseconds to settle after a change of load
    (right after the inputs are uploaded the first launches run 10-25 % slower
    than the steady state), so timing starts from a settled clock."""
    import torch
    if seconds <= 0:
        return 0
    stream = torch.cuda.current_stream()
    end = time.perf_counter() + seconds
    n = 0
    prev = None
    while time.perf_counter() < end:
        for _ in range(8):
            entry(Ad, Bd, Cd, stream=stream)
        n += 8
        ev = torch.cuda.Event()
        ev.record(stream)
        if prev is not None:
            prev.synchronize()
        prev = ev
    torch.cuda.synchronize()
    return n


def time_gemm(entry, Ad, Bd, Cd, steps: int, warmup: int, settle_s: float = 0.0, info=None):
    """Average kernel duration (s) over `steps` back-to-back launches, timed with
    HIP events recorded on the stream the library launches on, after `warmup`
    launches and then `settle_s` seconds of launches.  `info` (a dict), if
    given, receives the number of launches before the timed ones."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        entry(Ad, Bd, Cd, stream=stream)
    torch.cuda.synchronize()
    settled = settle_clock(entry, Ad, Bd, Cd, settle_s)
    if info is not None:
        info["launches_before_timed"] = warmup + settled
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        entry(Ad, Bd, Cd, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) * 1e-3 / steps, wall


def vendor_library(Ad, Bd, steps: int, warmup: int):
    """torch.matmul on the same device inputs (hipBLASLt on ROCm), timed like
    time_gemm, for context only.  Its C has the input format (for 16-bit inputs
    torch's product writes a 16-bit C), so its epilogue writes half the bytes of
    an fp32 C."""
    import torch
    Cv = torch.empty((Ad.shape[0], Bd.shape[1]), dtype=Ad.dtype, device=Ad.device)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        torch.matmul(Ad, Bd, out=Cv)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        torch.matmul(Ad, Bd, out=Cv)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e-3 / steps


def host_cpus() -> dict:
    """The host's CPU count beside the oracle's thread count: one GPU's share of
    the host is 16 CPUs, so the oracle runs at most 16 threads however many CPUs
    the machine shows."""
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        allowed = os.cpu_count() or 1
    return {"host_cpus": os.cpu_count(), "host_cpus_allowed": allowed,
            "cores_rule": "threads = min(16, CPUs this process may use); 16 is one GPU's "
                          "share of the host"}


def cpu_baseline(A, B, meta, target_s: float = 12.0):
    """The oracle, untuned, on a bounded sample of the same product: the first
    r rows of C, r chosen so the timed run takes about target_s seconds; when
    the whole product takes less than that, the whole product, repeated until
    about target_s seconds have been timed (at most 10 times).  Two probes (r
    and 4 r rows) size the sample: time = fixed + per_row * rows, the fixed
    part being mostly the widening of B."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    dt = meta["dtype"]
    M, N, K = meta["M"], meta["N"], meta["K"]
    times = []
    for r in (min(M, max(threads, 8)), min(M, 4 * max(threads, 8))):
        t0 = time.perf_counter()
        oracle.gemm(dt, A, B, rows=np.arange(r), nthreads=threads)
        times.append((r, time.perf_counter() - t0))
    (r1, t1), (r2, t2) = times
    per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-6)
    fixed = max(t1 - per_row * r1, 0.0)
    probe, t_probe = r2, t2
    if fixed + per_row * M <= target_s:
        total, reps = 0.0, 0
        while reps < 10 and total < 0.8 * target_s:
            t0 = time.perf_counter()
            oracle.gemm(dt, A, B, nthreads=threads)
            total += time.perf_counter() - t0
            reps += 1
        return {"value": round(tflops(M * reps, N, K, total), 6), "unit": "TFLOP/s",
                "cores": threads, **host_cpus(), "kind": "oracle",
                "sample": f"the whole {meta['name']} product ({M}x{N} outputs, K={K}), {reps} "
                          f"times, fp64 triple loop incl. exact widening of B, {total:.1f} s"}
    rows = int(min(M, max(probe, (target_s - fixed) / per_row)))
    rows = max(threads, rows // threads * threads)
    t0 = time.perf_counter()
    oracle.gemm(dt, A, B, rows=np.arange(rows), nthreads=threads)
    t = time.perf_counter() - t0
    return {"value": round(tflops(rows, N, K, t), 6), "unit": "TFLOP/s",
            "cores": threads, **host_cpus(), "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of C ({rows}x{N} outputs, K={K}) of the "
                      f"{meta['name']} product, fp64 triple loop incl. exact widening of B, "
                      f"{t:.1f} s"}


def cpu_single_thread(meta_rows: int = 96):
    """The oracle on one thread: the fp32 512^3 workload in full, and the first
    meta_rows rows of the bf16 4096^3 product, extrapolated to all 4096 rows
    (labelled as such) from a second run of meta_rows / 3 rows, which separates
    the fixed cost (widening B) from the cost per row."""
    import numpy as np
    import oracle
    from synth_inputs import workload
    out = {"cores": 1, "kind": "oracle"}
    A, B, m = workload("f32_512")
    t0 = time.perf_counter()
    oracle.gemm(m["dtype"], A, B, nthreads=1)
    t = time.perf_counter() - t0
    out["f32_512_full"] = {"s": round(t, 3), "tflops": round(tflops(m["M"], m["N"], m["K"], t), 6)}
    A, B, m = workload("bf16_4096")
    ts = []
    for r in (meta_rows // 3, meta_rows):
        t0 = time.perf_counter()
        oracle.gemm(m["dtype"], A, B, rows=np.arange(r), nthreads=1)
        ts.append(time.perf_counter() - t0)
    per_row = max((ts[1] - ts[0]) / (meta_rows - meta_rows // 3), 1e-9)
    fixed = max(ts[0] - per_row * (meta_rows // 3), 0.0)
    out["bf16_4096_rows"] = {"rows": meta_rows, "s": round(ts[1], 3),
                             "fixed_s": round(fixed, 3), "per_row_s": round(per_row, 5),
                             "extrapolated_full_s": round(fixed + per_row * m["M"], 1),
                             "tflops": round(tflops(meta_rows, m["N"], m["K"], ts[1]), 6)}
    return out


def _smi_values(node, key):
    """All numeric 'value' fields under dict keys starting with `key`."""
    out = []
    if isinstance(node, dict):
        for k, v in node.items():
            if k.startswith(key) and isinstance(v, dict):
                inner = v.get("clk", v)
                val = inner.get("value") if isinstance(inner, dict) else None
                if isinstance(val, (int, float)):
                    out.append(float(val))
            else:
                out += _smi_values(v, key)
    elif isinstance(node, list):
        for v in node:
            out += _smi_values(v, key)
    return out


def cold_cache(entry, Ad, Bd, Cd, launches: int = 20):
    """Mean time of single launches, each after writing a 512 MiB buffer (which
    evicts A, B and C from L2 and the 256 MB MALL)."""
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    total = 0.0
    for _ in range(launches):
        scratch.fill_(1)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        entry(Ad, Bd, Cd, stream=stream)
        stop.record(stream)
        torch.cuda.synchronize()
        total += start.elapsed_time(stop) * 1e-3
    del scratch
    return total / launches


def power_clock(entry, Ad, Bd, Cd, per_launch_s: float, value_tflops: float, peak: float,
                samples: int = 5):
    """Graphics clock and socket power while the GEMM runs.  This process keeps
    the GPU busy with blocks of ~20 ms of launches, never more than three blocks
    ahead, for 1 s before the first sample and 0.5 s between samples (amd-smi's
    readings trail the load), and while amd-smi (a child process) runs, `samples`
    times in turn.  The readings swing under the power limit, hence the list and
    its mean.  None when amd-smi is missing or fails."""
    import subprocess
    import torch
    stream = torch.cuda.current_stream()
    block = int(min(2000, max(20, 0.02 / max(per_launch_s, 1e-6))))

    def queue_block():
        for _ in range(block):
            entry(Ad, Bd, Cd, stream=stream)
        done = torch.cuda.Event()
        done.record(stream)
        return done

    pending = []

    def keep_busy(until):
        """Queue blocks until `until()` is true, at most three blocks ahead."""
        n = 0
        while not until():
            pending.append(queue_block())
            n += block
            while len(pending) > 3:
                pending.pop(0).synchronize()
        return n

    def for_seconds(sec):
        end = time.perf_counter() + sec
        return lambda: time.perf_counter() >= end

    launches = keep_busy(for_seconds(1.0))
    clks, powers = [], []
    for i in range(samples):
        if i:
            launches += keep_busy(for_seconds(0.5))
        try:
            proc = subprocess.Popen(["amd-smi", "metric", "--clock", "--power", "--json"],
                                    stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError:
            break
        deadline = time.perf_counter() + 60.0
        launches += keep_busy(lambda: proc.poll() is not None or time.perf_counter() >= deadline)
        if proc.poll() is None:
            proc.kill()
        out = proc.communicate()[0]
        # The last block still queued or running: the GPU was busy throughout.
        if proc.returncode != 0 or pending[-1].query():
            break
        try:
            data = json.loads(out)
        except ValueError:
            break
        c = _smi_values(data, "gfx_")
        if not c:
            break
        clks.append(sum(c) / len(c))
        pw = _smi_values(data, "socket_power")
        if pw:
            powers.append(pw[0])
    torch.cuda.synchronize()
    if not clks:
        return None
    sclk = sum(clks) / len(clks)
    adj_peak = peak * sclk / 2400.0
    return {"sclk_mhz_mean": round(sclk, 1), "sclk_mhz_samples": [round(c, 1) for c in clks],
            "socket_power_w_samples": powers,
            "clock_adjusted_peak_tflops": round(adj_peak, 1),
            "frac_of_clock_adjusted_peak": round(value_tflops / adj_peak, 4),
            "how": f"{len(clks)} amd-smi samples (mean over the XCDs each) taken while the GPU "
                   f"ran {launches} launches back to back"}


def mfma_ceiling(gemm_tflops: float, peak: float, steps: int, settle_s: float, with_power: bool):
    """The register-only matrix-instruction ceiling (libmfma_ceiling.so): one
    workgroup per CU running the 256 x 256 GEMM kernel's own sequence of
    v_mfma_f32_32x32x16_bf16 on operands held in registers, drawn from the
    workload's normal(0,1) bf16 distribution.  Timed like the GEMM, with the
    clock and power sampled while it runs.  The GEMM's rate over this one is the
    share of the attainable matrix throughput (at the power limit) that moving
    the operands leaves."""
    import ctypes
    import numpy as np
    import torch
    from synth_inputs import draw, to_torch
    path = os.path.join(ROOT, "dense_gemm_matrix_amd", "libmfma_ceiling.so")
    lib = ctypes.CDLL(path)
    lib.mfma_ceiling_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    lib.mfma_ceiling_run.restype = ctypes.c_int
    grid = int(torch.cuda.get_device_properties(0).multi_processor_count)
    ops = to_torch(draw(np.random.default_rng(7), (4096 * 8,), "normal", "bf16"), "bf16").to("cuda")
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    iters = 80                       # ~0.1 ms per launch, about one 4096^3 GEMM
    flop = grid * 4 * iters * 64 * 32768

    def entry(a, b, c, stream=None):
        st = stream if stream is not None else torch.cuda.current_stream()
        rc = lib.mfma_ceiling_run(ops.data_ptr(), sink.data_ptr(), iters, grid, st.cuda_stream)
        if rc:
            raise RuntimeError(f"mfma_ceiling_run failed ({rc})")

    t, _ = time_gemm(entry, None, None, None, steps, 5, settle_s)
    ceil_tflops = flop / t / 1e12
    out = {"tflops": round(ceil_tflops, 2), "frac_of_peak": round(ceil_tflops / peak, 4),
           "gemm_frac_of_ceiling": round(gemm_tflops / ceil_tflops, 4),
           "us_per_launch": round(t * 1e6, 2), "launches": steps,
           "how": f"{grid} workgroups x 4 waves x {iters} x 64 v_mfma_f32_32x32x16_bf16 on "
                  f"register-resident normal(0,1) bf16 operands, the GEMM kernel's block order"}
    if with_power:
        out["power_clock"] = power_clock(entry, None, None, None, t, ceil_tflops, peak)
    return out


def copy_calibration(gib: float = 1.0, reps: int = 5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "reps": reps}), flush=True)


# (label, workload name or (dtype, M, N, K), path)
SHAPES = [("f32 512^3", "f32_512", "f32"),
          ("bf16 16384x4096x4096, bf16 C", "bf16_16384x4096x4096", "bf16"),
          ("bf16 4000x3000x4104, bf16 C", "bf16_4000x3000x4104", "bf16"),
          ("bf16 512x4096x4096 (row share of 4096^3 over 8 GPUs), bf16 C",
           ("bf16", 512, 4096, 4096), "bf16")]


def time_graph(entry, Ad, Bd, Cd, launches: int):
    """Mean time per call of `launches` calls captured in one HIP graph and
    replayed: the kernels back to back, without the host's per-call launch cost."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            entry(Ad, Bd, Cd)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e-3 / launches


def other_shapes(dg, args):
    """Per shape: the plain entry point, and gemm_ex with the workspace its
    split-K plan asks for when the plan splits."""
    import torch
    from synth_inputs import pair, to_torch, torch_dtype
    out = []
    for label, wl, path in SHAPES:
        if isinstance(wl, str):
            A, B, Ad, Bd, Cd, meta = device_inputs(wl)
            M, N, K = meta["M"], meta["N"], meta["K"]
        else:
            dt, M, N, K = wl
            A, B = pair(M, N, K, "normal002", dt, seed=6000)
            Ad, Bd = to_torch(A, dt).to("cuda"), to_torch(B, dt).to("cuda")
            Cd = torch.empty((M, N), dtype=torch_dtype(dt), device="cuda")
        print(f"bench: shape {label}", file=sys.stderr, flush=True)
        plain = {"f32": dg.gemm_f32, "bf16": dg.gemm_bf16, "f16": dg.gemm_f16}[path]
        flop_s = gemm_flops(M, N, K)
        steps = max(10, min(args.steps, int(2e4 * 1e9 / flop_s)))
        warm = max(3, min(args.warmup, steps))
        t, _ = time_gemm(plain, Ad, Bd, Cd, steps, warm, min(args.settle_s, 0.3))
        tg = time_graph(plain, Ad, Bd, Cd, min(steps, 100))
        rec = {"shape": label, "M": M, "N": N, "K": K, "steps": steps,
               "plain_us": round(t * 1e6, 2), "plain_tflops": round(tflops(M, N, K, t), 2),
               "plain_graph_us": round(tg * 1e6, 2)}
        plan = dg.gemm_ex_plan(path, M, N, K, 1 << 40, out_same=(Cd.dtype == Ad.dtype and
                                                                   path != "f32"))
        rec["plan"] = plan
        if plan["workspace_bytes"] > 0:  # a split-K or Stream-K plan
            ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")

            def split_entry(a, b, c, stream=None, ws=ws):
                dg.gemm_ex(a, b, c, workspace=ws, stream=stream)
            t2, _ = time_gemm(split_entry, Ad, Bd, Cd, steps, warm, min(args.settle_s, 0.3))
            t2g = time_graph(split_entry, Ad, Bd, Cd, min(steps, 100))
            rec["split_us"] = round(t2 * 1e6, 2)
            rec["split_tflops"] = round(tflops(M, N, K, t2), 2)
            rec["split_graph_us"] = round(t2g * 1e6, 2)
            rec["split_graph_tflops"] = round(tflops(M, N, K, t2g), 2)
            del ws
        out.append(rec)
        del Ad, Bd, Cd
    return out


PLAN_SHAPES = [("bf16 512x4096x4096 (row share of 4096^3 over 8 GPUs), bf16 C", 512, 4096, 4096),
               ("bf16 4000x3000x4104, bf16 C", "bf16_4000x3000x4104", 0, 0),
               ("bf16 2048^3, bf16 C", 2048, 2048, 2048),
               ("bf16 3840x3840x8192 (225 tiles, runs not on tile boundaries), bf16 C", 3840, 3840, 8192)]


def plan_compare(dg, args):
    """Per shape: gemm_ex with a workspace Stream-K fits in, once with the cost
    model's plan and once with the Stream-K plan forced (dgemm_set_plan_override),
    each timed like the other shapes: the three shapes with fewer tiles than
    CUs, and a deep-K one whose Stream-K runs do not start on tile boundaries."""
    import torch
    from synth_inputs import pair, to_torch, torch_dtype
    out = []
    ws = torch.empty(2 * 256 * 256 * 256 * 4 + 256 * 8, dtype=torch.uint8, device="cuda")

    def ex_entry(a, b, c, stream=None):
        dg.gemm_ex(a, b, c, workspace=ws, stream=stream)
    try:
        for label, M, N, K in PLAN_SHAPES:
            if isinstance(M, str):
                _, _, Ad, Bd, Cd, meta = device_inputs(M)
                M, N, K = meta["M"], meta["N"], meta["K"]
            else:
                A, B = pair(M, N, K, "normal002", "bf16", seed=6000)
                Ad, Bd = to_torch(A, "bf16").to("cuda"), to_torch(B, "bf16").to("cuda")
                Cd = torch.empty((M, N), dtype=torch_dtype("bf16"), device="cuda")
            print(f"bench: plans {label}", file=sys.stderr, flush=True)
            steps = max(10, min(args.steps, int(2e4 * 1e9 / gemm_flops(M, N, K))))
            rec = {"shape": label, "M": M, "N": N, "K": K, "steps": steps}
            for key, kind in (("cost_model", dg.DGEMM_PLAN_AUTO), ("stream_k", dg.DGEMM_PLAN_STREAM_K)):
                dg.dgemm_set_plan_override(kind)
                plan = dg.gemm_ex_plan("bf16", M, N, K, ws.numel(), out_same=True)
                t, _ = time_gemm(ex_entry, Ad, Bd, Cd, steps, 3, min(args.settle_s, 0.3))
                rec[key] = {"plan": plan, "us": round(t * 1e6, 2),
                            "tflops": round(tflops(M, N, K, t), 2)}
            rec["stream_k_over_cost_model"] = round(rec["stream_k"]["us"] / rec["cost_model"]["us"], 3)
            out.append(rec)
            del Ad, Bd, Cd
    finally:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
    return out


# Small outputs, every input format: the cost model's slice-K plan against the
# 128 x 128 grid kernel forced unsplit and split (the split count the best of
# a sweep of 2-16 splits); fp32 C.  (format, label, M, N, K, splits)
SMALL_PLAN_SHAPES = [("f32", "f32 512^3 (the fp32 512^3 workload's shape)", 512, 512, 512, 8),
                     ("f32", "f32 768^3", 768, 768, 768, 6),
                     ("f32", "f32 1024^3", 1024, 1024, 1024, 4),
                     ("f32", "f32 256x256x4096", 256, 256, 4096, 16),
                     ("f32x3", "f32 via 3xbf16 512^3", 512, 512, 512, 4),
                     ("f32x3", "f32 via 3xbf16 1024^3", 1024, 1024, 1024, 4),
                     ("f32x3", "f32 via 3xbf16 512x512x4096", 512, 512, 4096, 16),
                     ("bf16", "bf16 512^3", 512, 512, 512, 2),
                     ("bf16", "bf16 1024^3", 1024, 1024, 1024, 2),
                     ("bf16", "bf16 512x512x4096", 512, 512, 4096, 8),
                     ("bf16", "bf16 256x256x8192", 256, 256, 8192, 16)]


def plan_compare_small(dg, args):
    """Per shape: gemm_ex timed by graph replay (these kernels take a few
    microseconds, less than the host's per-call cost) with the cost model's
    plan, and with the 128 x 128 grid kernel forced unsplit and split."""
    import torch
    from synth_inputs import pair, to_torch
    out = []
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    try:
        for fmt, label, M, N, K, splits in SMALL_PLAN_SHAPES:
            def ex_entry(a, b, c, stream=None, fmt=fmt):
                dg.gemm_ex(a, b, c, workspace=ws, in_fmt=fmt, stream=stream)
            dt = "f32" if fmt == "f32x3" else fmt
            A, B = pair(M, N, K, "uniform", dt, seed=6100)
            Ad, Bd = to_torch(A, dt).to("cuda"), to_torch(B, dt).to("cuda")
            Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
            print(f"bench: small-output plans {label}", file=sys.stderr, flush=True)
            rec = {"shape": label, "format": fmt, "M": M, "N": N, "K": K}
            for key, force in (("cost_model", None), ("grid_128_unsplit", (128, 128, 1)),
                               ("grid_128_split", (128, 128, splits))):
                if force:
                    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, *force)
                else:
                    dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
                plan = dg.gemm_ex_plan(fmt, M, N, K, ws.numel())
                for _ in range(20):
                    ex_entry(Ad, Bd, Cd)
                torch.cuda.synchronize()
                t = min(time_graph(ex_entry, Ad, Bd, Cd, 100) for _ in range(3))
                rec[key] = {"plan": plan, "graph_us": round(t * 1e6, 2),
                            "tflops": round(tflops(M, N, K, t), 2)}
            out.append(rec)
            del Ad, Bd, Cd
    finally:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
    return out


# Outputs between one and four rounds of 256 x 256 tiles: the cost model's
# unsplit tile against each 16-bit tile forced (bf16 inputs, normal(0, 0.02),
# bf16 C, no workspace).
TILE_PLAN_SHAPES = [("bf16 4608^2 x 4096", 4608, 4608, 4096),
                    ("bf16 1536x12288x4104", 1536, 12288, 4104),
                    ("bf16 12288x5120x2048", 12288, 5120, 2048),
                    ("bf16 6144x4096x4096", 6144, 4096, 4096)]


def plan_compare_tiles(dg, args):
    """Per shape: the plain launch with the cost model's tile, and with each
    16-bit tile (256 x 256, 192 x 256, 128 x 128) forced unsplit, timed by graph
    replay, best of two alternating passes."""
    import torch
    from synth_inputs import pair, to_torch, torch_dtype
    out = []

    def ex_entry(a, b, c, stream=None):
        dg.gemm_ex(a, b, c, stream=stream)
    try:
        for label, M, N, K in TILE_PLAN_SHAPES:
            A, B = pair(M, N, K, "normal002", "bf16", seed=6200)
            Ad, Bd = to_torch(A, "bf16").to("cuda"), to_torch(B, "bf16").to("cuda")
            Cd = torch.empty((M, N), dtype=torch_dtype("bf16"), device="cuda")
            del A, B
            print(f"bench: tile plans {label}", file=sys.stderr, flush=True)
            rec = {"shape": label, "M": M, "N": N, "K": K}
            best = {}
            # two passes over the plans, best of each: the first timing after a
            # change of load trails the power controller
            for _ in range(2):
                for key, force in (("cost_model", None), ("tile_256x256", (256, 256, 1)),
                                   ("tile_192x256", (192, 256, 1)), ("tile_128x128", (128, 128, 1))):
                    if force:
                        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, *force)
                    else:
                        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
                    plan = dg.gemm_ex_plan("bf16", M, N, K, 0, out_same=True)
                    for _ in range(3):
                        ex_entry(Ad, Bd, Cd)
                    torch.cuda.synchronize()
                    t = min(time_graph(ex_entry, Ad, Bd, Cd, 8) for _ in range(3))
                    best[key] = (min(t, best[key][0]) if key in best else t,
                                 [plan["tile_rows"], plan["tile_cols"]])
            for key, (t, tile) in best.items():
                rec[key] = {"tile": tile, "graph_us": round(t * 1e6, 2),
                            "tflops": round(tflops(M, N, K, t), 2)}
            out.append(rec)
            del Ad, Bd, Cd
    finally:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--dtype", choices=["bf16", "f16", "f32"], default="bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-dtype", action="store_true")
    ap.add_argument("--no-shapes", action="store_true")
    ap.add_argument("--no-power-clock", action="store_true")
    ap.add_argument("--no-cold-cache", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the register-only matrix-instruction ceiling run")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on the same inputs, for context")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of launches after the warm-up before each timed block, "
                         "so that timing starts from a settled clock (default 1.0)")
    ap.add_argument("--no-plans", action="store_true",
                    help="skip the cost model's plans against forced Stream-K (bf16) and forced "
                         "128 x 128 grid plans (small outputs)")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this GEMM engine has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import dense_gemm_matrix_amd as dg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return

    entry = {"bf16": dg.gemm_bf16, "f16": dg.gemm_f16, "f32": dg.gemm_f32}
    name = WORKLOAD_FOR[args.dtype]
    print(f"bench: preparing {name}", file=sys.stderr, flush=True)
    A, B, Ad, Bd, Cd, meta = device_inputs(name)
    M, N, K = meta["M"], meta["N"], meta["K"]
    torch.cuda.synchronize()
    print(f"bench: timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    timing_info = {}
    per_launch, wall = time_gemm(entry[args.dtype], Ad, Bd, Cd, args.steps, args.warmup,
                                 args.settle_s, timing_info)
    # Five more timed blocks of the same K steps (no further warm-up), for the
    # spread between trials; `value` stays the first block's.
    trials = [time_gemm(entry[args.dtype], Ad, Bd, Cd, args.steps, 0)[0] for _ in range(5)]
    value = tflops(M, N, K, per_launch)
    peak = PEAK_TFLOPS[args.dtype]
    traffic = measured_traffic(name)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_launch * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": DESCRIPTION[name], "M": M, "N": N, "K": K,
                   "frac_of_peak": round(value / peak, 4), "wall_s_timed_region": round(wall, 4),
                   "settle_s": args.settle_s,
                   "launches_before_timed": timing_info["launches_before_timed"],
                   "trials_ms_per_step": [round(t * 1e3, 5) for t in trials],
                   "trials_median_ms": round(sorted(trials)[2] * 1e3, 5),
                   "trials_min_ms": round(min(trials) * 1e3, 5)},
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(value / peak, 4), "traffic": traffic},
    }
    props = torch.cuda.get_device_properties(0)
    cus = int(props.multi_processor_count)
    # Dense matrix FLOP per clock per CU on CDNA4: 4 SIMDs x 1024 (bf16/fp16) or
    # x 64 (fp32); at the 2.4 GHz peak engine clock.
    per_cu_clk = {"bf16": 4096, "f16": 4096, "f32": 256}[args.dtype]
    line["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                      "compute_units": cus, "hbm_gib": round(props.total_memory / 2**30, 1),
                      "peak_from_cus_tflops": round(cus * per_cu_clk * 2.4e9 / 1e12, 1),
                      "peak_used_tflops": peak}
    if not args.no_cold_cache:
        t_cold = cold_cache(entry[args.dtype], Ad, Bd, Cd)
        line["cold_cache"] = {"us": round(t_cold * 1e6, 2), "tflops": round(tflops(M, N, K, t_cold), 2),
                              "launches": 20, "how": "each launch after writing a 512 MiB buffer"}
    if args.vendor:
        print("bench: timing torch.matmul on the same inputs", file=sys.stderr, flush=True)
        t_v = vendor_library(Ad, Bd, args.steps, min(args.warmup, 50))
        line["vendor_library"] = {
            "what": f"torch.matmul (hipBLASLt) on the same device inputs, C in {args.dtype}",
            "us": round(t_v * 1e6, 2), "tflops": round(tflops(M, N, K, t_v), 2),
            "frac_of_peak": round(tflops(M, N, K, t_v) / peak, 4)}
    if not args.no_power_clock:
        print("bench: sampling clock and power under load", file=sys.stderr, flush=True)
        line["power_clock"] = power_clock(entry[args.dtype], Ad, Bd, Cd, per_launch, value, peak)
    if not args.no_ceiling and args.dtype == "bf16":
        print("bench: matrix-instruction ceiling", file=sys.stderr, flush=True)
        line["mfma_ceiling"] = mfma_ceiling(value, peak, args.steps, min(args.settle_s, 1.0),
                                            not args.no_power_clock)
    if not args.no_per_dtype:
        # The other dtypes of the metric, and fp32 inputs through the 3 x bf16
        # entry (its peak is the bf16 matrix peak: three bf16 products per term).
        per = {}
        runs = [(dt, dt, entry[dt]) for dt in ("bf16", "f16", "f32") if dt != args.dtype]
        runs.append(("f32_3xbf16", "f32", dg.gemm_f32_3xbf16))
        for key, dt, fn in runs:
            wn = WORKLOAD_FOR[dt]
            print(f"bench: per-dtype {key} {wn}", file=sys.stderr, flush=True)
            _, _, a2, b2, c2, m2 = device_inputs(wn)
            steps = max(10, args.steps // (8 if key == "f32" else 1))
            t2, _ = time_gemm(fn, a2, b2, c2, steps, max(3, args.warmup // 4),
                              min(args.settle_s, 0.5))
            v2 = tflops(m2["M"], m2["N"], m2["K"], t2)
            peak = PEAK_TFLOPS["bf16"] / 3 if key == "f32_3xbf16" else PEAK_TFLOPS[dt]
            per[key] = {"workload": DESCRIPTION[wn], "value": round(v2, 2), "unit": "TFLOP/s",
                        "ms_per_launch": round(t2 * 1e3, 5), "steps": steps,
                        "frac_of_peak": round(v2 / peak, 4), "peak": round(peak, 1)}
            del a2, b2, c2
        line["per_dtype"] = per
    if not args.no_shapes:
        line["other_shapes"] = other_shapes(dg, args)
    if not args.no_plans:
        line["plan_compare"] = plan_compare(dg, args)
        line["plan_compare_small"] = plan_compare_small(dg, args)
        line["plan_compare_tiles"] = plan_compare_tiles(dg, args)
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(A, B, meta)
        line["cpu_single_thread"] = cpu_single_thread()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
