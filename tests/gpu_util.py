"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# The parity bar: relayouts bit for bit; attention and AdaLN outputs (bf16)
# against the unrounded fp64 oracle within these bounds over one call's output.
ATOL = 2e-2
REL_RMS = 5e-3


def say(*parts) -> None:
    """Name the case on stdout before a GPU step, flushed."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def to_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> host uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_device(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare(got_bits: np.ndarray, ref: np.ndarray, what: str, atol: float = ATOL, rel_rms: float = REL_RMS):
    got = bits_to_f64(got_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = got - ref
    max_abs = float(np.abs(err).max()) if err.size else 0.0
    norm = float(np.linalg.norm(ref))
    rr = float(np.linalg.norm(err) / norm) if norm > 0 else float(np.linalg.norm(err))
    say(f"{what}: max_abs={max_abs:.3e} rel_rms={rr:.3e} max|ref|={float(np.abs(ref).max()):.3f}")
    assert max_abs <= atol, f"{what}: max-abs {max_abs:.4e} > {atol}"
    assert rr <= rel_rms, f"{what}: rel-RMS {rr:.4e} > {rel_rms}"
    return max_abs, rr


def sample_rows(cu, seed: int, per_tile: int = 128, boundaries=(), limit: int = None) -> np.ndarray:
    """One seeded row per 128-row tile of every segment, plus each segment's first
    and last row and the rows either side of the given token boundaries."""
    rng = np.random.default_rng(seed)
    rows = set()
    n = int(cu[-1])
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        rows.update((a, b - 1))
        for t0 in range(a, b, per_tile):
            t1 = min(b, t0 + per_tile)
            rows.add(int(rng.integers(t0, t1)))
    for x in boundaries:
        for r in (x - 1, x):
            if 0 <= r < n:
                rows.add(int(r))
    out = np.array(sorted(rows), dtype=np.int64)
    if limit is not None and out.size > limit:
        keep = set(int(cu[s]) for s in range(len(cu) - 1)) | set(int(cu[s + 1]) - 1 for s in range(len(cu) - 1))
        rest = np.array([r for r in out if r not in keep])
        pick = rng.choice(rest, size=max(0, limit - len(keep)), replace=False)
        out = np.array(sorted(keep | set(int(x) for x in pick)), dtype=np.int64)
    return out
