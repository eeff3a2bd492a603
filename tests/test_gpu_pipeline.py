"""The whole hot path at every workload's real size, in the launch configuration
bench.py times (UlyssesStep), checked stage by stage against the oracle.

Relayout buffers are compared bit for bit; the final [N, 56, 128] output of the
attended heads and the AdaLN rows are compared on sampled rows (every segment
edge and virtual-rank boundary included) within the fp tolerance.  All oracle
inputs are host copies of the seeded synthetic inputs, and the oracle builds its
own rank buffers with its own seq2head.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS
from synth.inputs import normal_bf16
from tests.gpu_util import compare, say, sample_rows, to_bits

pytestmark = pytest.mark.gpu


def _make_step(w):
    from ulysses_layout_amd.pipeline import UlyssesStep
    attn_ranks = None if w.attn_rank is None else [w.attn_rank]
    step = UlyssesStep(w.n_tokens, w.cu, w.world, w.planes, attn_ranks=attn_ranks, relayout_rank=w.relayout_rank,
                       max_chunk_bytes=w.max_chunk_bytes, adaln_modes=("modulate", "gate"))
    step.qkv.copy_(normal_bf16(step.qkv.shape, seed=w.seed, device="cuda"))
    step.x.copy_(normal_bf16(step.x.shape, seed=w.seed + 1, device="cuda"))
    step.branch.copy_(normal_bf16(step.branch.shape, seed=w.seed + 2, device="cuda"))
    for i, t in enumerate((step.shift, step.ada_scale, step.gate)):
        t.copy_(normal_bf16(t.shape, seed=w.seed + 3 + i, std=0.1, device="cuda"))
    return step


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_pipeline_workload(name):
    w = WORKLOADS[name]
    say("pipeline", name)
    step = _make_step(w)
    step.run()
    torch.cuda.synchronize()
    plans = step.last_plans
    if w.max_chunk_bytes:
        assert all(p.max_launch_src_bytes <= w.max_chunk_bytes for p in plans["seq2head"])
        assert plans["seq2head"][0].launches == w.planes * plans["seq2head"][0].chunks

    src = to_bits(step.qkv)
    relayout_ranks = range(w.world) if w.relayout_rank < 0 else [w.relayout_rank]
    ref_bufs = oracle.seq2head(src, w.world, ranks=list(relayout_ranks))
    del src
    for (j, p), ref in ref_bufs.items():
        assert np.array_equal(to_bits(step.rank_bufs[j][p]), ref), (name, j, p)

    # attention through head2seq: attended heads of the final [N, 56, 128] output
    bounds = [a for a, _ in step.tokens]
    full_rows = w.n_tokens <= 8192
    rows = np.arange(w.n_tokens) if full_rows else sample_rows(w.cu, seed=w.seed + 7, per_tile=4096,
                                                                 boundaries=bounds, limit=96)
    out = to_bits(step.out)
    for j in step.attn_ranks:
        hb, hn = step.heads[j]
        g = ref_bufs[(j, 3)] if w.planes >= 4 else None
        ref = oracle.attention_rows(ref_bufs[(j, 0)], ref_bufs[(j, 1)], ref_bufs[(j, 2)], g, w.cu, step.scale,
                                    rows=rows)
        compare(out[rows][:, hb:hb + hn], ref, f"{name} pipeline attention rank {j}")
    # heads of ranks that were not attended stay untouched (zero)
    attended = np.zeros(56, bool)
    for j in step.attn_ranks:
        attended[step.heads[j][0]:step.heads[j][0] + step.heads[j][1]] = True
    if not attended.all():
        assert not out[:, ~attended].any()
    del out

    # AdaLN on every virtual rank's token interval
    xb, bb = to_bits(step.x), to_bits(step.branch)
    prm = [to_bits(t) for t in (step.shift, step.ada_scale, step.gate)]
    y, yg = to_bits(step.y), to_bits(step.y_gate)
    for a, cnt in step.tokens:
        local_cu = [0] + [e for _, _, e in oracle.clip_segments(w.cu, a, a + cnt)]
        r = np.arange(cnt) if full_rows else sample_rows(local_cu, seed=w.seed + a, per_tile=2048, limit=48)
        for mode, got, eps in ((0, y, step.eps), (1, yg, 0.0)):
            ref = oracle.adaln_rows(mode, xb[a:a + cnt], bb[a:a + cnt], prm[0], prm[1], prm[2], a, a + cnt, w.cu,
                                    eps, rows=r)
            compare(got[a:a + cnt][r], ref, f"{name} pipeline adaln mode {mode} @ {a}")
