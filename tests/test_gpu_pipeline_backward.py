"""The path's backward through ``UlyssesStep.backward()`` -- head2seq adjoint,
attention backward per attended rank, seq2head adjoint -- against the oracle's
composition of the same three steps, as fp64 gradients of the packed operand."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS
from synth.inputs import normal_bf16
from tests.gpu_util import bits_to_f64, compare, say, to_bits

pytestmark = pytest.mark.gpu


def _step(w):
    from ulysses_layout_amd.pipeline import UlyssesStep
    attn_ranks = None if w.attn_rank is None else [w.attn_rank]
    step = UlyssesStep(w.n_tokens, w.cu, w.world, w.planes, attn_ranks=attn_ranks, relayout_rank=w.relayout_rank,
                       max_chunk_bytes=w.max_chunk_bytes, with_backward=True)
    step.qkv.copy_(normal_bf16(step.qkv.shape, seed=w.seed + 80, device="cuda"))
    step.x.copy_(normal_bf16(step.x.shape, seed=w.seed + 81, device="cuda"))
    for i, t in enumerate((step.shift, step.ada_scale, step.gate)):
        t.copy_(normal_bf16(t.shape, seed=w.seed + 82 + i, std=0.1, device="cuda"))
    step.grad_out.copy_(normal_bf16(step.grad_out.shape, seed=w.seed + 85, device="cuda"))
    return step


@pytest.mark.parametrize("name,check_ranks", [("tiny512", [0, 1]), ("8k_p6", [5])])
def test_pipeline_backward_against_oracle(name, check_ranks):
    w = WORKLOADS[name]
    say("pipeline backward", name, check_ranks)
    step = _step(w)
    step.run()
    plans = step.backward()
    torch.cuda.synchronize()
    src, go = to_bits(step.qkv), to_bits(step.grad_out)
    bufs = oracle.seq2head(src, w.world, ranks=check_ranks)
    gattn = oracle.head2seq_backward(go, w.world, ranks=check_ranks)
    grads = {}
    for j in check_ranks:
        g = bufs[(j, 3)] if step.gated else None
        r = oracle.attention_backward(bufs[(j, 0)], bufs[(j, 1)], bufs[(j, 2)], g, gattn[j], w.cu, step.scale)
        for p, key in enumerate(("dq", "dk", "dv", "dg")[:step.planes]):
            grads[(j, p)] = r[key]
    ref = oracle.seq2head_backward(grads, w.n_tokens, step.planes, 56, w.world, ranks=check_ranks)
    got = bits_to_f64(to_bits(step.grad_qkv))
    for j in check_ranks:
        hb, hn = step.heads[j]
        for p in range(step.planes):
            r = ref[:, p, hb:hb + hn]
            compare(to_bits(step.grad_qkv[:, p, hb:hb + hn]), r, f"{name} grad plane {p} rank {j}",
                    atol=2e-2 * float(np.abs(r).max()), rel_rms=5e-3)
    # every plan of the backward: one head2seq adjoint, one attention backward per rank, one seq2head adjoint
    assert len(plans["head2seq_backward"]) == 1 and len(plans["seq2head_backward"]) == 1
    assert len(plans["attention_backward"]) == len(step.attn_ranks)
    assert all(p.launches == 3 for p in plans["attention_backward"])
    assert np.isfinite(got).all()


def test_pipeline_backward_rank_share_leaves_other_heads_zero():
    """One attended rank (the 128k layout at 2 segments of 64 tokens, P=4):
    only that rank's heads of the packed gradient are written."""
    from synth.workloads import Workload
    w0 = WORKLOADS["128k_p4_qkvg"]
    cu = [0, 96, 128]
    w = Workload(name="small_share", n_tokens=128, cu=tuple(cu), world=w0.world, planes=w0.planes,
                 attn_rank=w0.attn_rank, relayout_rank=w0.relayout_rank, max_chunk_bytes=0, seed=77)
    step = _step(w)
    step.run()
    step.backward()
    torch.cuda.synchronize()
    hb, hn = step.heads[w.attn_rank]
    got = bits_to_f64(to_bits(step.grad_qkv))
    outside = np.ones(56, bool)
    outside[hb:hb + hn] = False
    assert (got[:, :, outside] == 0).all()
    assert (np.abs(got[:, :, hb:hb + hn]) > 0).mean() > 0.99
