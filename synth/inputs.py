"""Seeded random operands.

Values are standard normal (or a stated standard deviation) drawn in float32
and rounded to bfloat16 with round-to-nearest-even.  Large operands are drawn
directly on the GPU with a seeded ``torch.Generator`` so a 14 GB QKVG tensor
takes seconds; small ones are drawn on the CPU.  Either way the oracle is
handed the very same bits (a host copy of the tensor).
"""
from __future__ import annotations

import numpy as np
import torch


def normal_bf16(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """A bf16 tensor of N(0, std^2) values from a generator seeded with ``seed``."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=dev)
    flat = out.view(-1)
    step = 1 << 28   # draw in slices to bound the float32 staging buffer
    for start in range(0, flat.numel(), step):
        stop = min(flat.numel(), start + step)
        tmp = torch.randn(stop - start, generator=gen, dtype=torch.float32, device=dev)
        if std != 1.0:
            tmp.mul_(std)
        flat[start:stop].copy_(tmp)
        del tmp
    return out


def normal_bf16_bits(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """Host bf16 bit patterns (uint16) of :func:`normal_bf16` drawn on the CPU."""
    t = normal_bf16(shape, seed, std, device="cpu")
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def unique_pattern_bits(shape) -> np.ndarray:
    """uint16 array whose entries encode their own position modulo 65536.

    Used where a relayout must be checked by decoding where each element came
    from; for shapes under 65536 elements every entry is distinct.
    """
    n = int(np.prod(shape))
    return (np.arange(n, dtype=np.int64) % 65536).astype(np.uint16).reshape(shape)
