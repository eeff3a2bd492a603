"""GPU edge cases: degenerate partitions and segment tables, size limits, output
guard bands, determinism over repeated calls, and recovery after a rejected call."""
import numpy as np
import pytest
import torch

import oracle
from synth import segment_offsets
from synth.inputs import normal_bf16, normal_bf16_bits
from tests.gpu_util import compare, say, to_bits, to_device

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5


def _h3():
    import ulysses_layout_amd as h3
    return h3


def test_one_head_per_rank_and_single_token():
    h3 = _h3()
    for n, world in ((56, 56), (1, 1), (3, 3), (100, 56)):
        say("relayout edge", n, world)
        src_bits = normal_bf16_bits((n, 2, 56, 128), seed=10 + n)
        src = to_device(src_bits)
        heads = h3.head_split(56, world)
        bufs = [[torch.empty((n, c, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)] for _, c in heads]
        h3.seq2head(src, bufs, world)
        back = torch.empty((n, 56, 128), dtype=torch.bfloat16, device="cuda")
        h3.head2seq([b[1] for b in bufs], back, world)
        torch.cuda.synchronize()
        ref = oracle.seq2head(src_bits, world)
        for j in range(world):
            for p in range(2):
                assert np.array_equal(to_bits(bufs[j][p]), ref[(j, p)])
        assert np.array_equal(to_bits(back), src_bits[:, 1])


def test_empty_partitions_rejected_on_device_path():
    h3 = _h3()
    src = torch.zeros((3, 1, 56, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(h3.H3Error) as e:
        h3.seq2head(src, [[torch.zeros((3, 14, 128), dtype=torch.bfloat16, device="cuda")] for _ in range(4)], 4)
    assert e.value.status == 2
    assert "legal values are 1..3" in e.value.message


@pytest.mark.parametrize("lengths", [[1] * 40, [1, 2, 3, 5, 8, 13, 21, 34, 55, 89], None])
def test_attention_many_tiny_segments(lengths):
    if lengths is None:       # the segment-table limit: 256 seeded segments
        rng = np.random.default_rng(3)
        lengths = [int(x) for x in rng.integers(1, 40, size=256)]
    cu = segment_offsets(lengths)
    n, h = cu[-1], 2
    say("attention tiny segments", len(lengths))
    bits = [normal_bf16_bits((n, h, 128), seed=900 + i) for i in range(4)]
    q, k, v, g = (to_device(b) for b in bits)
    o = torch.empty_like(q)
    _h3().packed_attn(q, k, v, g, o, cu, SCALE)
    torch.cuda.synchronize()
    ref = oracle.attention_rows(bits[0], bits[1], bits[2], bits[3], cu, SCALE)
    compare(to_bits(o), ref, f"attn {len(lengths)} tiny segments")


def test_attention_segment_table_over_limit_rejected():
    h3 = _h3()
    cu = segment_offsets([1] * 257)
    q = torch.zeros((257, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(h3.H3Error) as e:
        h3.packed_attn(q, q.clone(), q.clone(), None, torch.empty_like(q), cu, SCALE)
    assert e.value.status == 3


@pytest.mark.parametrize("c", [8, 520, 16384])
def test_adaln_width_limits(c):
    h3 = _h3()
    cu = segment_offsets([3, 5])
    say("adaln width", c)
    x = normal_bf16_bits((8, c), 71)
    b = normal_bf16_bits((8, c), 72)
    prm = [normal_bf16_bits((2, c), 73 + i, std=0.1) for i in range(3)]
    y = torch.empty((8, c), dtype=torch.bfloat16, device="cuda")
    h3.adaln_segment(0, to_device(x), None, to_device(prm[0]), to_device(prm[1]), None, y, 0, 8, cu, 1e-6)
    yg = torch.empty_like(y)
    h3.adaln_segment(1, to_device(x), to_device(b), None, None, to_device(prm[2]), yg, 0, 8, cu, 0.0)
    torch.cuda.synchronize()
    compare(to_bits(y), oracle.adaln_rows(0, x, None, prm[0], prm[1], None, 0, 8, cu, 1e-6), f"adaln mod c={c}")
    compare(to_bits(yg), oracle.adaln_rows(1, x, b, None, None, prm[2], 0, 8, cu, 0.0), f"adaln gate c={c}")


def _guarded(shape, canary_words=4096):
    """A view into a larger allocation whose margins hold a known pattern."""
    n = int(np.prod(shape))
    whole = torch.full((n + 2 * canary_words,), -12345, dtype=torch.int16, device="cuda")
    view = whole[canary_words:canary_words + n].view(torch.bfloat16).view(shape)
    return whole, view


def _margins_intact(whole, canary_words=4096):
    h = whole.cpu().numpy()
    return (h[:canary_words] == -12345).all() and (h[-canary_words:] == -12345).all()


def test_outputs_stay_inside_their_buffers():
    h3 = _h3()
    n, world = 1000, 6
    say("guard bands")
    src = normal_bf16((n, 3, 56, 128), seed=5, device="cuda")
    heads = h3.head_split(56, world)
    guards, bufs = [], []
    for j, (_, c) in enumerate(heads):
        row = []
        for p in range(3):
            wh, view = _guarded((n, c, 128))
            guards.append(wh)
            row.append(view)
        bufs.append(row)
    h3.seq2head(src, bufs, world, max_chunk_bytes=7 * 56 * 128 * 2)
    wo, out = _guarded((n, 56, 128))
    h3.head2seq([b[0] for b in bufs], out, world)
    cu = segment_offsets([300, 1, 699])
    wa, o = _guarded((n, heads[0][1], 128))
    h3.packed_attn(bufs[0][0], bufs[0][1], bufs[0][2], None, o, cu, SCALE)
    wy, y = _guarded((n, 7168))
    x = normal_bf16((n, 7168), seed=6, device="cuda")
    prm = normal_bf16((3, 7168), seed=7, std=0.1, device="cuda")
    h3.adaln_segment(0, x, None, prm, prm.clone(), None, y, 0, n, cu, 1e-6)
    torch.cuda.synchronize()
    for g in guards + [wo, wa, wy]:
        assert _margins_intact(g)


def test_repeated_calls_are_bitwise_deterministic():
    """100 rounds of seq2head (one rank's share) -> gated attention -> head2seq:
    the relayout buffers, the attention output and the head2seq output are the
    same bits every round (no atomics, no order-dependent reductions)."""
    h3 = _h3()
    n, world, rank = 4097, 4, 1
    cu = segment_offsets([1000, 3097])
    src = normal_bf16((n, 4, 56, 128), seed=8, device="cuda")
    heads = h3.head_split(56, world)
    bufs = [[torch.empty((n, c, 128), dtype=torch.bfloat16, device="cuda") for _ in range(4)] for _, c in heads]
    attn = [torch.empty((n, c, 128), dtype=torch.bfloat16, device="cuda") for _, c in heads]
    out = torch.zeros((n, 56, 128), dtype=torch.bfloat16, device="cuda")
    first = None
    for rnd in range(100):
        h3.seq2head(src, bufs, world, rank=rank)
        b = bufs[rank]
        h3.packed_attn(b[0], b[1], b[2], b[3], attn[rank], cu, SCALE)
        h3.head2seq(attn, out, world, rank=rank)
        snap = [t.view(torch.int16).clone() for t in b + [attn[rank], out]]
        if first is None:
            first = snap
        else:
            assert all(torch.equal(x, y) for x, y in zip(snap, first)), rnd
    torch.cuda.synchronize()


def test_rejected_call_then_valid_call():
    h3 = _h3()
    q = normal_bf16((300, 2, 128), seed=9, device="cuda")
    k, v = q.clone(), normal_bf16((300, 2, 128), seed=10, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(h3.H3Error):
        h3.packed_attn(q, k, v, None, o, [0, 100, 100, 300], SCALE)      # empty segment
    with pytest.raises(h3.H3Error):
        h3.packed_attn(q, k, v, None, q, [0, 300], SCALE)                # output aliases q
    h3.packed_attn(q, k, v, None, o, [0, 100, 300], SCALE)
    torch.cuda.synchronize()
    ref = oracle.attention_rows(to_bits(q), to_bits(k), to_bits(v), None, [0, 100, 300], SCALE)
    compare(to_bits(o), ref, "attention after rejected calls")
