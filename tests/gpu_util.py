"""Helpers shared by the GPU parity tests: moving seeded numpy inputs onto the
GPU and results back.  No method arithmetic lives here."""
import os
import sys

import numpy as np
import pytest
import torch

DEV = "cuda:0"


def gpu_available():
    return torch.cuda.is_available()


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 GPU tensor (bit-preserving)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(DEV)


def to_gpu_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_gpu_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def np_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().view(np.uint32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def announce(msg: str):
    """Print and flush what the next GPU step is, so a fault names its case."""
    print(f"[gpu-case] {msg}", flush=True)
