"""Helpers shared by the GPU parity tests (device transfer, stress inputs)."""

import sys

import numpy as np
import torch


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def dev_bf16(bits):
    """uint16 bf16 patterns (numpy) -> torch.bfloat16 on cuda:0 (same bits)."""
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to("cuda:0").view(torch.bfloat16)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda:0")


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def stress_blocks(seed=0):
    """One 32-element block per positive finite bf16 amax pattern.

    Block p holds the amax p at a seeded position and 31 seeded patterns whose
    magnitudes are at most p, with seeded signs -- every scale byte, denormal
    blocks, zero blocks and a wide spread of element patterns per scale. Returns a
    [n_blocks, 32] uint16 array (n_blocks = 0x7F80 + 2, incl. a +0 and a -0 block).
    """
    rng = np.random.default_rng(seed)
    amax = np.arange(0x7F80, dtype=np.int64)
    n = len(amax)
    mags = (rng.random((n, 32)) * (amax[:, None] + 1)).astype(np.int64)
    mags = np.minimum(mags, amax[:, None])
    pos = rng.integers(0, 32, size=n)
    mags[np.arange(n), pos] = amax
    signs = rng.integers(0, 2, size=(n, 32)).astype(np.int64) << 15
    blocks = (mags | signs).astype(np.uint16)
    extra = np.zeros((2, 32), np.uint16)
    extra[1, :] = 0x8000
    return np.concatenate([blocks, extra])
