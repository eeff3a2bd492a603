"""The five synthetic workloads and their packed-segment tables.

The pages time the real model on synthetic inputs that carry real H3 packing
("[perf] Harden Ulysses agreement and tune bounded H3 transfers", H3
full-model performance) at 32k, 64k, 128k and 250k packed tokens, with 56 heads
of width 128 ("Distributed H3 Execution", Partition Contract).  The shapes
below follow that: token counts, segment mixes, virtual-rank counts and plane
counts.  Segment cut points are drawn uniformly without repetition from a
seeded generator, so every segment is non-empty.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

N_HEADS = 56
HEAD_DIM = 128


def _random_cuts(n_tokens: int, n_segments: int, seed: int) -> List[int]:
    rng = np.random.Generator(np.random.PCG64(seed))
    cuts = rng.choice(np.arange(1, n_tokens), size=n_segments - 1, replace=False)
    return [0] + sorted(int(c) for c in cuts) + [n_tokens]


@dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    world: int                 # virtual ranks P
    planes: int                # 3 = QKV, 4 = QKVG
    cu: Tuple[int, ...]        # global segment offsets
    seed: int
    attn_rank: Optional[int]   # None: attention for every rank's heads; j: only rank j's share
    relayout_rank: int = -1    # -1: relayout into every rank's buffers; j: only rank j's share
    max_chunk_bytes: int = 0   # 0: one launch per plane; else source-byte cap per launch
    description: str = ""

    @property
    def n_segments(self) -> int:
        return len(self.cu) - 1

    @property
    def segment_lengths(self) -> List[int]:
        return [self.cu[i + 1] - self.cu[i] for i in range(len(self.cu) - 1)]


def segment_offsets(lengths) -> Tuple[int, ...]:
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return tuple(out)


WORKLOADS = {
    "tiny512": Workload(
        name="tiny512", n_tokens=512, world=2, planes=3,
        cu=segment_offsets([96, 160, 256]), seed=1001, attn_rank=None,
        description="512 packed tokens in 3 segments (96,160,256), P=2 (28 heads each), QKV, "
                    "attention on every head, AdaLN per segment"),
    "8k_p6": Workload(
        name="8k_p6", n_tokens=8192, world=6, planes=3,
        cu=tuple(_random_cuts(8192, 12, 1002)), seed=1002, attn_rank=None,
        description="8192 packed tokens, 12 seeded random segments, P=6 ragged "
                    "(heads 10,10,9,9,9,9), full seq2head -> attention on all ranks -> head2seq"),
    "32k_p4": Workload(
        name="32k_p4", n_tokens=32768, world=4, planes=3,
        cu=segment_offsets([8192] * 4), seed=1003, attn_rank=0,
        description="32768 packed tokens, 4 segments of 8192, P=4, full QKV seq2head into 4 "
                    "virtual-rank buffers, attention over one rank's 14 heads, head2seq"),
    "128k_p4_qkvg": Workload(
        name="128k_p4_qkvg", n_tokens=131072, world=4, planes=4,
        cu=segment_offsets([98304, 32768]), seed=1004, attn_rank=0, relayout_rank=0,
        description="131072 packed tokens, QKVG [131072,4,56,128], segments 98304+32768, P=4, "
                    "rank share (14 heads), plane-at-a-time relayout, gated attention, "
                    "head2seq, AdaLN modulation on [131072,7168]"),
    "250k_p8_qkvg": Workload(
        name="250k_p8_qkvg", n_tokens=250000, world=8, planes=4,
        cu=tuple(_random_cuts(250000, 8, 1005)), seed=1005, attn_rank=0, relayout_rank=0,
        max_chunk_bytes=896_000_000,
        description="250000 packed tokens, 8 seeded random segments, P=8 (7 heads), QKVG "
                    "relayout in launches of at most 896,000,000 source bytes, gated attention, "
                    "head2seq"),
}
