"""Helpers for the GPU parity tests: move bf16-bit arrays to and from the
device, and compare results to the oracle's."""
import sys

import numpy as np
import torch

import oracle as O


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits (numpy) -> int16 CUDA tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def dev_i32(x) -> torch.Tensor:
    return torch.tensor(np.asarray(x, dtype=np.int32), dtype=torch.int32, device="cuda")


def host(t: torch.Tensor) -> np.ndarray:
    """CUDA int16/bf16 tensor -> numpy uint16 bits."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place (same-sign values; 0 for equal bits)."""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    # map sign-magnitude to a monotone integer line
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


def attn_errors(o_bits: np.ndarray, ref: np.ndarray):
    """(max-abs, mean-abs, rel-L2) of a bf16 output against an fp64 reference."""
    got = O.bf16_to_f64(o_bits)
    d = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return float(d.max()), float(d.mean()), rel


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# Contract tolerances for bf16 attention outputs, plus the relative-L2 gate
# that keeps them meaningful when |O| is small.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2
