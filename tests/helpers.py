"""Shared test helpers: moving seeded inputs to the GPU and the parity metric."""
import numpy as np
import torch

import synth


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 tensor on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def f64(bits_or_f32: np.ndarray, bf16: bool) -> np.ndarray:
    return (synth.bf16_bits_to_f32(bits_or_f32) if bf16 else np.asarray(bits_or_f32)).astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """Normwise max relative error: max|out - ref| / max|ref|."""
    return float(np.max(np.abs(out - ref)) / max(np.max(np.abs(ref)), 1e-30))


BF16_TOL = 2e-2     # bf16 inputs, fp32 accumulation
F32_TOL = 1e-4      # fp32 inputs and accumulation
LSE_TOL = 1e-2      # absolute, natural-log units
