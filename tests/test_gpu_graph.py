"""The whole hot path captured once into a HIP graph and replayed.

libh3.so allocates nothing, clears nothing and never synchronises inside a
call, so one UlyssesStep.run() -- every relayout chunk launch, the attention of
each attended rank and the AdaLN launches of every rank interval -- can be
captured into a single graph.  Each replay must reproduce the eager pass bit
for bit, and a replay after new inputs are written must equal an eager pass
over those inputs (the graph reads the live buffers, it does not hold results).
Between replays the test does eager work of its own (clearing the outputs)
and synchronises, and every replay is checked.
"""
import pytest
import torch

from synth import WORKLOADS
from synth.inputs import normal_bf16
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _step(w):
    from ulysses_layout_amd.pipeline import UlyssesStep
    attn_ranks = None if w.attn_rank is None else [w.attn_rank]
    return UlyssesStep(w.n_tokens, w.cu, w.world, w.planes, attn_ranks=attn_ranks, relayout_rank=w.relayout_rank,
                       max_chunk_bytes=w.max_chunk_bytes, adaln_modes=("modulate", "gate"))


def _fill_inputs(step, seed):
    step.qkv.copy_(normal_bf16(step.qkv.shape, seed=seed, device="cuda"))
    step.x.copy_(normal_bf16(step.x.shape, seed=seed + 1, device="cuda"))
    step.branch.copy_(normal_bf16(step.branch.shape, seed=seed + 2, device="cuda"))
    for i, t in enumerate((step.shift, step.ada_scale, step.gate)):
        t.copy_(normal_bf16(t.shape, seed=seed + 3 + i, std=0.1, device="cuda"))


def _outputs(step):
    outs = [("out", step.out), ("y", step.y), ("y_gate", step.y_gate)]
    for j, bufs in enumerate(step.rank_bufs):
        if bufs is not None:
            outs += [(f"rank{j}.plane{p}", t) for p, t in enumerate(bufs)]
    for j in step.attn_ranks:
        outs.append((f"attn{j}", step.attn_out[j]))
    return outs


def _clear(step):
    for _, t in _outputs(step):
        t.zero_()


def _snapshot(step):
    """Device copies of every output's bit patterns."""
    return {name: t.detach().view(torch.int16).clone() for name, t in _outputs(step)}


def _assert_same(got, ref, what):
    for name in ref:
        assert torch.equal(got[name], ref[name]), f"{what}: {name} differs from the eager pass"


@pytest.mark.parametrize("name", ["tiny512", "8k_p6", "250k_p8_qkvg"])
def test_graph_replays_match_eager(name):
    w = WORKLOADS[name]
    say("graph", name)
    step = _step(w)
    _fill_inputs(step, w.seed)
    step.run()
    torch.cuda.synchronize()
    eager = _snapshot(step)
    eager_plans = {k: [p.launches for p in v] for k, v in step.last_plans.items()}

    _clear(step)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()
    # capture enqueues nothing that runs: the outputs are still clear
    assert not step.out.any().item()
    assert {k: [p.launches for p in v] for k, v in step.last_plans.items()} == eager_plans

    for r in range(3):
        _clear(step)                                   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(_snapshot(step), eager, f"{name} replay {r}")

    # new inputs: the replay computes from the live buffers
    _fill_inputs(step, w.seed + 100)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replayed = _snapshot(step)
    assert not torch.equal(replayed["out"], eager["out"])
    _clear(step)
    step.run()
    torch.cuda.synchronize()
    _assert_same(replayed, _snapshot(step), f"{name} replay on new inputs")
    del graph


def _grads(step):
    outs = [("grad_qkv", step.grad_qkv)]
    for j in step.attn_ranks:
        outs.append((f"grad_attn{j}", step.grad_attn[j]))
        outs += [(f"grad{j}.plane{p}", t) for p, t in enumerate(step.grad_bufs[j])]
    return outs


@pytest.mark.parametrize("name", ["tiny512", "8k_p6", "128k_p4_qkvg"])
def test_graph_replays_backward_match_eager(name):
    """UlyssesStep.backward() -- head2seq adjoint, attention backward with its
    caller-owned workspace, seq2head adjoint -- captured once and replayed."""
    from ulysses_layout_amd.pipeline import UlyssesStep
    w = WORKLOADS[name]
    say("graph backward", name)
    attn_ranks = None if w.attn_rank is None else [w.attn_rank]
    step = UlyssesStep(w.n_tokens, w.cu, w.world, w.planes, attn_ranks=attn_ranks, relayout_rank=w.relayout_rank,
                       max_chunk_bytes=w.max_chunk_bytes, with_backward=True)
    step.qkv.copy_(normal_bf16(step.qkv.shape, seed=w.seed + 200, device="cuda"))
    step.x.copy_(normal_bf16(step.x.shape, seed=w.seed + 201, device="cuda"))
    for i, t in enumerate((step.shift, step.ada_scale, step.gate)):
        t.copy_(normal_bf16(t.shape, seed=w.seed + 202 + i, std=0.1, device="cuda"))
    step.grad_out.copy_(normal_bf16(step.grad_out.shape, seed=w.seed + 205, device="cuda"))
    step.run()
    step.backward()
    torch.cuda.synchronize()
    eager = {name_: t.detach().view(torch.int16).clone() for name_, t in _grads(step)}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.backward()
    torch.cuda.synchronize()
    for r in range(3):
        for _, t in _grads(step):
            t.zero_()                                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {name_: t.detach().view(torch.int16).clone() for name_, t in _grads(step)}
        _assert_same(got, eager, f"{name} backward replay {r}")
    del graph


@pytest.mark.parametrize("name", ["tiny512", "8k_p6"])
def test_graph_replays_token_sharded_ops_match_eager(name):
    """The gated AdaLN chain over every rank interval, the ragged reduce-scatter
    with the bias and the ragged row gather, captured once and replayed."""
    import ulysses_layout_amd as h3
    w = WORKLOADS[name]
    say("graph token-sharded ops", name)
    step = _step(w)
    _fill_inputs(step, w.seed + 300)
    n, c = step.n_tokens, step.channels
    resid, y = torch.empty_like(step.x), torch.empty_like(step.x)
    partials = [normal_bf16((n, c), seed=w.seed + 310 + j, device="cuda") for j in range(w.world)]
    bias = normal_bf16((c,), seed=w.seed + 309, device="cuda")
    shards = [torch.empty((cnt, c), dtype=torch.bfloat16, device="cuda") for _, cnt in step.tokens]
    gathered = torch.empty((n, c), dtype=torch.bfloat16, device="cuda")
    outs = [("resid", resid), ("y", y), ("gathered", gathered)] + [(f"shard{j}", t) for j, t in enumerate(shards)]

    def ops():
        for a, cnt in step.tokens:
            h3.adaln_gate_modulate(step.x[a:a + cnt], step.branch[a:a + cnt], step.gate, step.shift,
                                   step.ada_scale, resid[a:a + cnt], y[a:a + cnt], a, a + cnt, step.cu, step.eps)
        h3.reduce_scatter(partials, bias, shards)
        h3.gather_rows(shards, gathered)

    ops()
    torch.cuda.synchronize()
    eager = {k: t.detach().view(torch.int16).clone() for k, t in outs}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops()
    torch.cuda.synchronize()
    for r in range(3):
        for _, t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same({k: t.detach().view(torch.int16).clone() for k, t in outs}, eager, f"{name} ops replay {r}")
    del graph
