"""One pass of the Ulysses H3 hot path on one GPU, as a sequence of C-ABI calls.

``UlyssesStep`` owns the device buffers of one workload and enqueues, on one
stream, the four library calls in the order the Ulysses block runs them
("Distributed H3 Execution", introduction and Partition Contract):

1. ``h3_seq2head``   packed ``[N, K, 56, 128]`` -> virtual-rank buffers
                     ``[N, H_j, 128]`` (every rank, or one rank's share), one
                     plane at a time, in bounded chunks when asked;
2. ``h3_packed_attn`` for the heads of each attended rank (gated for QKVG);
3. ``h3_head2seq``   the attention outputs back to ``[N, 56, 128]``;
4. ``h3_adaln_segment`` per virtual rank's token interval, with the segment
                     table clipped and rebased to it, on ``[N_j, 7168]`` rows.

With ``with_backward=True`` the attention also stores each row's
log-sum-exp, and ``backward()`` enqueues the path's backward in reverse
order: ``h3_head2seq_backward`` of ``grad_out``, ``h3_packed_attn_backward``
for each attended rank, and ``h3_seq2head_backward`` into ``grad_qkv``.

It allocates nothing inside ``run()`` or ``backward()``; buffers are made once
by the constructor.  All arithmetic happens in libh3.so.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import torch

from . import h3 as _h3

H3_HEADS = 56
H3_CHANNELS = H3_HEADS * _h3.HEAD_DIM


@dataclass
class StepTimes:
    """Milliseconds per step of the last timed ``run``."""
    seq2head: float = 0.0
    attention: float = 0.0
    head2seq: float = 0.0
    adaln: float = 0.0

    @property
    def total(self) -> float:
        return self.seq2head + self.attention + self.head2seq + self.adaln


class UlyssesStep:
    def __init__(self, n_tokens: int, cu: Sequence[int], world: int, planes: int,
                 attn_ranks: Optional[Sequence[int]] = None, relayout_rank: int = -1,
                 max_chunk_bytes: int = 0, n_heads: int = H3_HEADS, channels: Optional[int] = None,
                 scale: float = _h3.HEAD_DIM ** -0.5, eps: float = 1e-6, adaln_modes=("modulate",),
                 with_backward: bool = False, device: str = "cuda"):
        self.n_tokens = int(n_tokens)
        self.cu = [int(c) for c in cu]
        self.world = int(world)
        self.planes = int(planes)
        self.n_heads = int(n_heads)
        self.channels = int(channels if channels is not None else n_heads * _h3.HEAD_DIM)
        self.scale = float(scale)
        self.eps = float(eps)
        self.max_chunk_bytes = int(max_chunk_bytes)
        self.relayout_rank = int(relayout_rank)
        self.attn_ranks = list(range(world)) if attn_ranks is None else [int(j) for j in attn_ranks]
        if self.relayout_rank >= 0 and any(j != self.relayout_rank for j in self.attn_ranks):
            raise ValueError("attention can only run on ranks whose buffers the relayout fills")
        self.adaln_modes = tuple(adaln_modes)
        self.gated = self.planes >= 4
        self.heads = _h3.head_split(self.n_heads, self.world)
        self.tokens = [_h3.partition(self.n_tokens, self.world, i) for i in range(self.world)]
        dev = torch.device(device)
        bf = torch.bfloat16
        n, d = self.n_tokens, _h3.HEAD_DIM
        s = len(self.cu) - 1
        # inputs (the caller fills them)
        self.qkv = torch.empty((n, self.planes, self.n_heads, d), dtype=bf, device=dev)
        self.x = torch.empty((n, self.channels), dtype=bf, device=dev)
        self.branch = torch.empty((n, self.channels), dtype=bf, device=dev) if "gate" in self.adaln_modes else None
        self.shift = torch.empty((s, self.channels), dtype=bf, device=dev)
        self.ada_scale = torch.empty((s, self.channels), dtype=bf, device=dev)
        self.gate = torch.empty((s, self.channels), dtype=bf, device=dev)
        # intermediate and output buffers, one allocation each
        relayout_ranks = range(self.world) if self.relayout_rank < 0 else [self.relayout_rank]
        self.rank_bufs: List[Optional[List[torch.Tensor]]] = [None] * self.world
        for j in relayout_ranks:
            self.rank_bufs[j] = [torch.empty((n, self.heads[j][1], d), dtype=bf, device=dev)
                                 for _ in range(self.planes)]
        self.attn_out: List[Optional[torch.Tensor]] = [None] * self.world
        for j in self.attn_ranks:
            self.attn_out[j] = torch.empty((n, self.heads[j][1], d), dtype=bf, device=dev)
        self.out = torch.zeros((n, self.n_heads, d), dtype=bf, device=dev)
        self.y = torch.empty((n, self.channels), dtype=bf, device=dev)
        self.y_gate = torch.empty((n, self.channels), dtype=bf, device=dev) if "gate" in self.adaln_modes else None
        self.head2seq_rank = -1 if len(self.attn_ranks) == self.world else (
            self.attn_ranks[0] if len(self.attn_ranks) == 1 else None)
        if self.head2seq_rank is None:
            raise ValueError("attention must cover one rank or every rank")
        self.last_plans: Dict[str, List[_h3.PlanInfo]] = {}
        # backward buffers: the caller fills grad_out (the gradient of `out`)
        self.with_backward = bool(with_backward)
        self.lse: List[Optional[torch.Tensor]] = [None] * self.world
        if self.with_backward:
            f32 = torch.float32
            self.grad_out = torch.empty((n, self.n_heads, d), dtype=bf, device=dev)
            self.grad_attn: List[Optional[torch.Tensor]] = [None] * self.world
            self.grad_bufs: List[Optional[List[torch.Tensor]]] = [None] * self.world
            self.workspace: List[Optional[torch.Tensor]] = [None] * self.world
            for j in self.attn_ranks:
                hj = self.heads[j][1]
                self.lse[j] = torch.empty((n, hj), dtype=f32, device=dev)
                self.grad_attn[j] = torch.empty((n, hj, d), dtype=bf, device=dev)
                self.grad_bufs[j] = [torch.empty((n, hj, d), dtype=bf, device=dev) for _ in range(self.planes)]
                self.workspace[j] = torch.empty(_h3.packed_attn_backward_workspace(n, hj, self.gated),
                                                dtype=torch.uint8, device=dev)
            # heads outside the attended ranks receive no gradient and stay zero
            self.grad_qkv = torch.zeros((n, self.planes, self.n_heads, d), dtype=bf, device=dev)

    # -- the four steps -------------------------------------------------------------
    def seq2head(self, stream=None) -> _h3.PlanInfo:
        return _h3.seq2head(self.qkv, self.rank_bufs, self.world, rank=self.relayout_rank,
                            max_chunk_bytes=self.max_chunk_bytes, stream=stream)

    def attention(self, stream=None) -> List[_h3.PlanInfo]:
        plans = []
        for j in self.attn_ranks:
            b = self.rank_bufs[j]
            plans.append(_h3.packed_attn(b[0], b[1], b[2], b[3] if self.gated else None, self.attn_out[j],
                                         self.cu, self.scale, stream=stream, lse=self.lse[j]))
        return plans

    def head2seq(self, stream=None) -> _h3.PlanInfo:
        return _h3.head2seq(self.attn_out, self.out, self.world, rank=self.head2seq_rank,
                            max_chunk_bytes=self.max_chunk_bytes, stream=stream)

    def adaln(self, stream=None) -> List[_h3.PlanInfo]:
        plans = []
        for a, cnt in self.tokens:
            if "modulate" in self.adaln_modes:
                plans.append(_h3.adaln_segment(_h3.H3_ADALN_MODULATE, self.x[a:a + cnt], None, self.shift,
                                               self.ada_scale, None, self.y[a:a + cnt], a, a + cnt, self.cu,
                                               self.eps, stream=stream))
            if "gate" in self.adaln_modes:
                plans.append(_h3.adaln_segment(_h3.H3_ADALN_GATE_RESIDUAL, self.x[a:a + cnt],
                                               self.branch[a:a + cnt], None, None, self.gate,
                                               self.y_gate[a:a + cnt], a, a + cnt, self.cu, 0.0, stream=stream))
        return plans

    def run(self, stream=None, events: Optional[Dict[str, List]] = None) -> None:
        """Enqueue one whole pass.  With ``events`` = {name: [start, end]} of
        ``torch.cuda.Event(enable_timing=True)``, each step is bracketed on the stream."""
        steps = (("seq2head", self.seq2head), ("attention", self.attention), ("head2seq", self.head2seq),
                 ("adaln", self.adaln))
        st = stream if stream is not None else torch.cuda.current_stream()
        for name, fn in steps:
            if events is not None:
                events[name][0].record(st)
            plan = fn(stream=st)
            self.last_plans[name] = plan if isinstance(plan, list) else [plan]
            if events is not None:
                events[name][1].record(st)

    # -- the backward of the relayouts and the attention --------------------------------
    def backward(self, stream=None, events: Optional[Dict[str, List]] = None) -> Dict[str, List[_h3.PlanInfo]]:
        """Gradients of the packed operand from ``grad_out`` (after a ``run``):
        head2seq adjoint, attention backward per attended rank, seq2head
        adjoint (of the attended ranks' heads, with the forward's chunking)."""
        if not self.with_backward:
            raise RuntimeError("construct the step with with_backward=True")
        st = stream if stream is not None else torch.cuda.current_stream()
        plans: Dict[str, List[_h3.PlanInfo]] = {}

        def timed(name, fn):
            if events is not None:
                events[name][0].record(st)
            res = fn()
            if events is not None:
                events[name][1].record(st)
            plans[name] = res if isinstance(res, list) else [res]

        timed("head2seq_backward", lambda: _h3.head2seq_backward(
            self.grad_out, self.grad_attn, self.world, rank=self.head2seq_rank,
            max_chunk_bytes=self.max_chunk_bytes, stream=st))

        def attn_bwd():
            out = []
            for j in self.attn_ranks:
                b, gb = self.rank_bufs[j], self.grad_bufs[j]
                out.append(_h3.packed_attn_backward(
                    b[0], b[1], b[2], b[3] if self.gated else None, self.attn_out[j], self.grad_attn[j],
                    self.lse[j], gb[0], gb[1], gb[2], gb[3] if self.gated else None, self.workspace[j], self.cu,
                    self.scale, stream=st))
            return out

        timed("attention_backward", attn_bwd)
        timed("seq2head_backward", lambda: _h3.seq2head_backward(
            self.grad_bufs, self.grad_qkv, self.world, rank=self.head2seq_rank,
            max_chunk_bytes=self.max_chunk_bytes, stream=st))
        return plans

    # -- algorithmic work of one pass ------------------------------------------------
    def attention_flops(self) -> float:
        per_head = sum((self.cu[i + 1] - self.cu[i]) ** 2 for i in range(len(self.cu) - 1))
        heads = sum(self.heads[j][1] for j in self.attn_ranks)
        return 4.0 * _h3.HEAD_DIM * heads * per_head

    def relayout_bytes(self) -> Dict[str, int]:
        d = _h3.HEAD_DIM * 2
        s2h_heads = self.n_heads if self.relayout_rank < 0 else self.heads[self.relayout_rank][1]
        h2s_heads = sum(self.heads[j][1] for j in self.attn_ranks)
        return {"seq2head": 2 * self.n_tokens * self.planes * s2h_heads * d,
                "head2seq": 2 * self.n_tokens * h2s_heads * d}

    def adaln_bytes(self) -> int:
        row = self.channels * 2
        total = 0
        if "modulate" in self.adaln_modes:
            total += 2 * self.n_tokens * row
        if "gate" in self.adaln_modes:
            total += 3 * self.n_tokens * row
        return total
