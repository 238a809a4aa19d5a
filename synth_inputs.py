"""Seeded synthetic inputs for the GEMM tests and benchmark.

This module only draws numbers and stores them in the dtype the GEMM consumes;
it contains none of the GEMM's arithmetic.  Both the HIP path's tests and the
oracle receive the very arrays made here.

Recipe: numpy's PCG64 generator (numpy.random.default_rng(seed)) draws A, then B,
row-major, in fp64; the draw is rounded to fp32 (round to nearest even), then,
for 16-bit workloads, to bf16 or fp16 (round to nearest even, done by torch /
numpy conversions).  Neither page fixes a distribution for the 4096^3 runs, so
the workloads below follow the distributions named for them.

Storage: "f32" -> float32, "bf16" -> uint16 bit patterns, "f16" -> float16.
"""
import numpy as np

STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64/fp32 array -> storage dtype, via fp32, each step round-to-nearest-even."""
    f32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return f32
    if dtype == "f16":
        return f32.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(f32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def draw(rng: np.random.Generator, shape, dist: str, dtype: str) -> np.ndarray:
    """One matrix.  dist: 'uniform' (U[-1,1]), 'normal' (N(0,1)), 'normal002'
    (N(0,0.02)), 'ints' (integers in [-8, 8], exact in every dtype), 'ones'."""
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.normal(0.0, 1.0, size=shape)
    elif dist == "normal002":
        x = rng.normal(0.0, 0.02, size=shape)
    elif dist == "ints":
        x = rng.integers(-8, 9, size=shape).astype(np.float64)
    elif dist == "ones":
        x = np.ones(shape)
    else:
        raise ValueError(dist)
    return to_storage(x, dtype)


def pair(M: int, N: int, K: int, dist: str, dtype: str, seed: int):
    """A [M, K] then B [K, N] from one generator seeded with `seed`."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (M, K), dist, dtype)
    B = draw(rng, (K, N), dist, dtype)
    return A, B


# The five workloads: (name, dtype, M, N, K, dist, seed, C format).
WORKLOADS = {
    "f32_512": ("f32", 512, 512, 512, "uniform", 0, "f32"),
    "f32_4096": ("f32", 4096, 4096, 4096, "uniform", 1, "f32"),
    "bf16_4096": ("bf16", 4096, 4096, 4096, "normal", 2, "f32"),
    "f16_4096": ("f16", 4096, 4096, 4096, "uniform", 3, "f16"),
    "bf16_16384x4096x4096": ("bf16", 16384, 4096, 4096, "normal002", 4, "bf16"),
    "bf16_4000x3000x4104": ("bf16", 4000, 3000, 4104, "normal002", 5, "bf16"),
}


def workload(name: str):
    """(A, B, meta) for a named workload."""
    dtype, M, N, K, dist, seed, out = WORKLOADS[name]
    A, B = pair(M, N, K, dist, dtype, seed)
    return A, B, {"name": name, "dtype": dtype, "M": M, "N": N, "K": K,
                  "dist": dist, "seed": seed, "out": out}


def to_torch(x: np.ndarray, dtype: str):
    """A storage array as a CPU torch tensor of the matching dtype (no copy of values)."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x))


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
