"""Host <-> device helpers for the GPU parity tests (no method arithmetic)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"

_NP_TO_TORCH = {
    np.dtype(np.float32): torch.float32,
    np.dtype(np.float64): torch.float64,
    np.dtype(np.int32): torch.int32,
    np.dtype(np.int64): torch.int64,
    np.dtype(np.uint8): torch.uint8,
}


def to_dev(x: np.ndarray, bf16: bool = False, f16: bool = False) -> torch.Tensor:
    """Upload a numpy array; uint16 bit patterns become bf16 (or f16) tensors."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        t = torch.from_numpy(x.view(np.int16)).to(DEV)
        return t.view(torch.float16 if f16 else torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Download a tensor; bf16/f16 come back as uint16 bit patterns."""
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def say(*msg):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def random_bits(rng, shape, dtype):
    """Random element bit patterns (never all-zero) for bit-exact movement tests."""
    if dtype == np.uint16:
        return rng.integers(1, 0x7F00, shape, dtype=np.uint16)
    if dtype == np.float32:
        return rng.standard_normal(shape).astype(np.float32)
    if dtype == np.float64:
        return rng.standard_normal(shape)
    if dtype == np.uint8:
        return rng.integers(1, 256, shape, dtype=np.uint8)
    if dtype == np.int32:
        return rng.integers(1, 1 << 30, shape, dtype=np.int32)
    if dtype == np.int64:
        return rng.integers(1, 1 << 62, shape, dtype=np.int64)
    raise TypeError(dtype)
