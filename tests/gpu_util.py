"""Helpers for the GPU tests: move seeded storage arrays to the device (with
padded row pitches and NaN-filled gaps), and bring results back as float64."""
import numpy as np
import torch

from synth_inputs import to_torch as to_torch_cpu

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
PER16 = {"f32": 4, "bf16": 8, "f16": 8}


def round_pitch(cols: int, dtype: str, extra: int = 0) -> int:
    p = PER16[dtype]
    return (max(cols, 1) + extra + p - 1) // p * p


def dev_matrix(x: np.ndarray, dtype: str, pitch: int = None, fill=float("nan")) -> torch.Tensor:
    """x (storage array) on cuda:0 as a [rows, cols] view of a [rows, pitch]
    buffer whose gap columns hold `fill`."""
    rows, cols = x.shape
    if pitch is None:
        pitch = round_pitch(cols, dtype)
    buf = torch.full((rows, pitch), fill, dtype=TORCH[dtype], device="cuda")
    buf[:, :cols] = to_torch_cpu(x, dtype).to("cuda")
    return buf[:, :cols]


def sentinel_c(M: int, N: int, out: str, pitch: int = None) -> torch.Tensor:
    if pitch is None:
        pitch = round_pitch(N, out, extra=4)
    buf = torch.full((M, pitch), float("nan"), dtype=TORCH[out], device="cuda")
    return buf[:, :N]


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def gap_untouched(C: torch.Tensor) -> bool:
    """The columns between N and the row pitch still hold the NaN sentinel."""
    M, N = C.shape
    if M == 0:
        return True
    pitch = C.stride(0)
    full = torch.as_strided(C, (M, pitch), (pitch, 1))
    return bool(torch.isnan(full[:, N:].float()).all().item())
