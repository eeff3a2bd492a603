"""GPU edge cases of the backward, the gated chain and the ragged collectives:
the 256-segment table, one row per rank, guard bands around every output and
the workspace, bitwise determinism, and recovery after rejected calls."""
import numpy as np
import pytest
import torch

import oracle
from synth import segment_offsets
from synth.inputs import normal_bf16, normal_bf16_bits
from tests.gpu_util import bits_to_f64, compare, say, to_bits, to_device

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5
CANARY = -12345


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _guarded(shape, dtype=torch.bfloat16, canary_words=4096):
    """A view into a larger allocation whose margins hold a known 16-bit pattern."""
    elem = torch.tensor([], dtype=dtype).element_size()
    n16 = int(np.prod(shape)) * elem // 2
    whole = torch.full((n16 + 2 * canary_words,), CANARY, dtype=torch.int16, device="cuda")
    view = whole[canary_words:canary_words + n16].view(dtype).view(shape)
    return whole, view


def _intact(whole, canary_words=4096):
    h = whole.cpu().numpy()
    return bool((h[:canary_words] == CANARY).all() and (h[-canary_words:] == CANARY).all())


def _grads_close(got, ref, what):
    scale = float(np.abs(ref).max())
    compare(got, ref, what, atol=2e-2 * max(scale, 1e-6), rel_rms=5e-3)


@pytest.mark.parametrize("gated", [False, True])
def test_backward_256_segments_in_guarded_buffers(gated):
    """The longest segment table (256 seeded lengths, 1-token segments among
    them); every output and the workspace sit between canary bands."""
    h3 = _h3()
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 48, size=256)]
    lengths[7] = lengths[100] = 1
    cu = segment_offsets(lengths)
    n, h = cu[-1], 2
    say("backward 256 segments", n, gated)
    bits = [normal_bf16_bits((n, h, 128), seed=3100 + i) for i in range(5)]
    q, k, v, g, do = (to_device(b) for b in bits)
    g = g if gated else None
    o = torch.empty_like(q)
    lse = torch.empty((n, h), dtype=torch.float32, device="cuda")
    h3.packed_attn(q, k, v, g, o, cu, SCALE, lse=lse)
    guards, outs = [], []
    for _ in range(4 if gated else 3):
        wh, view = _guarded((n, h, 128))
        guards.append(wh)
        outs.append(view)
    ws_bytes = h3.packed_attn_backward_workspace(n, h, gated)
    wws, ws = _guarded((ws_bytes,), dtype=torch.uint8)
    h3.packed_attn_backward(q, k, v, g, o, do, lse, outs[0], outs[1], outs[2], outs[3] if gated else None, ws,
                            cu, SCALE)
    torch.cuda.synchronize()
    assert all(_intact(w) for w in guards + [wws])
    ref = oracle.attention_backward(bits[0], bits[1], bits[2], bits[3] if gated else None, bits[4], cu, SCALE)
    for name, t in zip(("dq", "dk", "dv", "dg"), outs):
        _grads_close(to_bits(t), ref[name], f"{name} 256 segments gated={gated}")


def test_backward_is_bitwise_deterministic():
    h3 = _h3()
    cu = segment_offsets([700, 129, 1])
    n, h = cu[-1], 3
    q, k, v, g, do = (normal_bf16((n, h, 128), seed=3200 + i, device="cuda") for i in range(5))
    o = torch.empty_like(q)
    lse = torch.empty((n, h), dtype=torch.float32, device="cuda")
    h3.packed_attn(q, k, v, g, o, cu, SCALE, lse=lse)
    ws = torch.empty(h3.packed_attn_backward_workspace(n, h, True), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(5):
        gr = [torch.empty_like(q) for _ in range(4)]
        h3.packed_attn_backward(q, k, v, g, o, do, lse, gr[0], gr[1], gr[2], gr[3], ws, cu, SCALE)
        runs.append(gr)
    torch.cuda.synchronize()
    for gr in runs[1:]:
        for a, b in zip(gr, runs[0]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n,world", [(7, 7), (64, 64), (65, 64), (3, 1)])
def test_collectives_one_row_per_rank_in_guarded_buffers(n, world):
    h3 = _h3()
    c = 64
    say("collectives", n, world)
    parts = [normal_bf16_bits((n, c), seed=3300 + j) for j in range(world)]
    bias = normal_bf16_bits((c,), seed=3299)
    guards, outs = [], []
    for i in range(world):
        wh, view = _guarded((h3.partition(n, world, i)[1], c))
        guards.append(wh)
        outs.append(view)
    h3.reduce_scatter([to_device(p) for p in parts], to_device(bias), outs)
    wd, dst = _guarded((n, c))
    x = normal_bf16_bits((n, c), seed=3301)
    shards = [to_device(x[a:a + cnt]) for a, cnt in oracle.partition(n, world)]
    h3.gather_rows(shards, dst)
    torch.cuda.synchronize()
    assert all(_intact(w) for w in guards + [wd])
    ref = oracle.reduce_scatter(parts, bias)
    for i in range(world):
        got = bits_to_f64(to_bits(outs[i]))
        assert (np.abs(got - ref[i]) <= 2.0 ** -8 * np.abs(ref[i]) + 1e-4).all(), i
    assert np.array_equal(to_bits(dst), oracle.gather_rows([x[a:a + cnt] for a, cnt in oracle.partition(n, world)]))


def test_chain_256_segments_interval_and_guards():
    h3 = _h3()
    rng = np.random.default_rng(34)
    lengths = [int(x) for x in rng.integers(1, 30, size=256)]
    cu = segment_offsets(lengths)
    n, c = cu[-1], 1024
    a, e = 37, n - 41                        # cuts the first and last segments
    say("chain 256 segments", n)
    x = normal_bf16_bits((n, c), seed=3400)
    b = normal_bf16_bits((n, c), seed=3401)
    gate, shift, scale = (normal_bf16_bits((256, c), seed=3402 + i, std=0.1) for i in range(3))
    wr, resid = _guarded((e - a, c))
    wy, y = _guarded((e - a, c))
    h3.adaln_gate_modulate(to_device(x[a:e]), to_device(b[a:e]), to_device(gate), to_device(shift), to_device(scale),
                           resid, y, a, e, cu, 1e-6)
    torch.cuda.synchronize()
    assert _intact(wr) and _intact(wy)
    r_ref, y_ref = oracle.adaln_gate_modulate(x[a:e], b[a:e], gate, shift, scale, a, e, cu, 1e-6)
    compare(to_bits(resid), r_ref, "chain resid 256 segments")
    compare(to_bits(y), y_ref, "chain y 256 segments")


def test_rejected_calls_then_valid_calls():
    h3 = _h3()
    n, c, world = 100, 64, 3
    parts = [normal_bf16((n, c), seed=3500 + j, device="cuda") for j in range(world)]
    outs = [torch.empty((h3.partition(n, world, i)[1], c), dtype=torch.bfloat16, device="cuda") for i in range(world)]
    with pytest.raises(h3.H3Error) as e:
        h3.reduce_scatter(parts, None, outs, rank=world)                  # no such rank
    assert e.value.status == 1
    big = torch.empty((2 * n, c), dtype=torch.bfloat16, device="cuda")
    shard_views = [big[a:a + cnt] for a, cnt in (h3.partition(n, world, i) for i in range(world))]
    with pytest.raises(h3.H3Error) as e:
        h3.gather_rows(shard_views, big[n - 1:2 * n - 1])                  # dst overlaps the last shard's last row
    assert e.value.status == 5
    h3.reduce_scatter(parts, None, outs)
    dst = torch.empty((n, c), dtype=torch.bfloat16, device="cuda")
    h3.gather_rows(outs, dst)
    torch.cuda.synchronize()
    ref = sum(bits_to_f64(to_bits(p)) for p in parts)
    got = bits_to_f64(to_bits(dst))
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4).all()
