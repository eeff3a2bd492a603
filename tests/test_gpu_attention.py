"""GPU parity of segment-masked packed attention against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, segment_offsets
from synth.inputs import normal_bf16, normal_bf16_bits
from tests.gpu_util import compare, say, sample_rows, to_bits, to_device

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _run(q, k, v, g, cu):
    h3 = _h3()
    o = torch.empty_like(q)
    info = h3.packed_attn(q, k, v, g, o, cu, SCALE)
    torch.cuda.synchronize()
    return o, info


RAGGED = [
    [1],
    [64],
    [1, 63, 64, 65],
    [127, 128, 129],
    [300],
    [5, 250, 1, 77, 130],
    [96, 160, 256],
]


@pytest.mark.parametrize("lengths", RAGGED, ids=lambda x: "-".join(map(str, x)))
@pytest.mark.parametrize("gated", [False, True])
def test_attention_ragged_segments(lengths, gated):
    cu = segment_offsets(lengths)
    n, h = cu[-1], 3
    say("attention ragged", lengths, gated)
    bits = [normal_bf16_bits((n, h, 128), seed=400 + i + n) for i in range(4)]
    q, k, v, g = (to_device(b) for b in bits)
    o, info = _run(q, k, v, g if gated else None, cu)
    ref = oracle.attention_rows(bits[0], bits[1], bits[2], bits[3] if gated else None, cu, SCALE)
    compare(to_bits(o), ref, f"attn {lengths} gated={gated}")
    assert info.launches == 1
    assert info.flops == 4 * 128 * h * sum(L * L for L in lengths)


def _random_tables(count, seed):
    """Seeded segment tables: 1-8 segments of 1-1600 tokens, 1-4 heads, gated or not."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        lengths = [int(x) for x in rng.integers(1, 1601, size=int(rng.integers(1, 9)))]
        out.append((lengths, int(rng.integers(1, 5)), bool(rng.integers(0, 2))))
    return out


RANDOM_TABLES = _random_tables(12, 20261204)


@pytest.mark.parametrize("case", range(len(RANDOM_TABLES)))
def test_attention_random_tables(case):
    """Every output row against the oracle on seeded random segment tables: mixed
    lengths in one launch give partial query tiles, partial last key tiles and
    waves whose rows all lie past their segment's end side by side; the row
    log-sum-exp variant must give the same output bits."""
    lengths, h, gated = RANDOM_TABLES[case]
    cu = segment_offsets(lengths)
    n = cu[-1]
    say("attention random table", case, lengths, h, gated)
    bits = [normal_bf16_bits((n, h, 128), seed=3100 + 10 * case + i) for i in range(4)]
    q, k, v, g = (to_device(b) for b in bits)
    o, info = _run(q, k, v, g if gated else None, cu)
    ref = oracle.attention_rows(bits[0], bits[1], bits[2], bits[3] if gated else None, cu, SCALE)
    compare(to_bits(o), ref, f"attn random table {case}")
    assert info.flops == 4 * 128 * h * sum(L * L for L in lengths)
    o2 = torch.empty_like(q)
    lse = torch.empty((n, h), dtype=torch.float32, device="cuda")
    _h3().packed_attn(q, k, v, g if gated else None, o2, cu, SCALE, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.isfinite(lse).all()


def test_attention_peaky_softmax():
    """Q scaled by 8: large logits exercise the online-softmax rescaling."""
    cu = segment_offsets([700, 333])
    n, h = cu[-1], 2
    say("attention peaky")
    q_bits = normal_bf16_bits((n, h, 128), seed=501, std=8.0)
    k_bits, v_bits = normal_bf16_bits((n, h, 128), seed=502), normal_bf16_bits((n, h, 128), seed=503)
    o, _ = _run(to_device(q_bits), to_device(k_bits), to_device(v_bits), None, cu)
    compare(to_bits(o), oracle.attention_rows(q_bits, k_bits, v_bits, None, cu, SCALE), "attn peaky")


def _ramp_inputs(n, h, total_rise_log2, seed):
    """Q rows all near one direction u and K rows (1 + r*i/n) * u: the logits in
    log2 units move by about ``total_rise_log2`` from the first key to the last."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((h, 128)).astype(np.float32)
    q = u[None] + 0.05 * rng.standard_normal((n, h, 128)).astype(np.float32)
    c = SCALE * np.log2(np.e) * float((u * u).sum(axis=1).mean())
    r = total_rise_log2 / c
    ramp = (1.0 + r * np.arange(n, dtype=np.float32) / n)[:, None, None]
    k = ramp * u[None] + 0.05 * rng.standard_normal((n, h, 128)).astype(np.float32)
    v = rng.standard_normal((n, h, 128)).astype(np.float32)
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits(q), bits(k), bits(v)


@pytest.mark.parametrize("rise", [40.0, -40.0])
def test_attention_drifting_logits(rise):
    """Rising logits: the running max moves every few tiles (rescales) and the tiles in
    between carry probabilities up to 2^8 (the exact-max check without a rescale).
    Falling logits: every later tile underflows against the first one's max."""
    cu = segment_offsets([1000, 130])
    n, h = cu[-1], 2
    say("attention drifting logits", rise)
    qb, kb, vb = _ramp_inputs(n, h, rise, seed=1301 if rise > 0 else 1302)
    o, _ = _run(to_device(qb), to_device(kb), to_device(vb), None, cu)
    compare(to_bits(o), oracle.attention_rows(qb, kb, vb, None, cu, SCALE), f"attn drifting {rise}")


@pytest.mark.parametrize("lengths,qstd", [([1, 63, 64, 65], 1.0), ([300, 5, 700], 1.0), ([900, 130], 8.0)])
def test_attention_lse_output(lengths, qstd):
    """h3_packed_attn_lse: the same output bits as h3_packed_attn, plus the row
    log-sum-exp.  The kernel's row sum adds the bf16-rounded probabilities its
    PV step uses, so lse carries up to ~2^-9 relative error in the sum."""
    cu = segment_offsets(lengths)
    n, h = cu[-1], 3
    say("attention lse", lengths, qstd)
    q_bits = normal_bf16_bits((n, h, 128), seed=1400 + n, std=qstd)
    bits = [q_bits] + [normal_bf16_bits((n, h, 128), seed=1401 + n + i) for i in range(3)]
    q, k, v, g = (to_device(b) for b in bits)
    o = torch.empty_like(q)
    lse = torch.full((n, h), float("nan"), dtype=torch.float32, device="cuda")
    _h3().packed_attn(q, k, v, g, o, cu, SCALE, lse=lse)
    o2, _ = _run(q, k, v, g, cu)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    ref = oracle.attention_backward(bits[0], bits[1], bits[2], bits[3], np.zeros_like(bits[0]), cu, SCALE,
                                    k_rows=[])["lse"]
    got = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    assert (err <= 4e-3 + 1e-6 * np.abs(ref)).all(), float(err.max())


def test_attention_gate_zero_halves_exactly():
    cu = segment_offsets([200, 57])
    n, h = cu[-1], 2
    say("attention G=0")
    q, k, v = (normal_bf16((n, h, 128), seed=600 + i, device="cuda") for i in range(3))
    o, _ = _run(q, k, v, None, cu)
    og, _ = _run(q, k, v, torch.zeros_like(q), cu)
    assert torch.equal(og.float() * 2, o.float())


def test_attention_segments_do_not_mix():
    """Changing one segment's keys and values leaves every other segment's output bits unchanged."""
    cu = segment_offsets([130, 200, 70])
    n, h = cu[-1], 2
    say("attention isolation")
    q, k, v = (normal_bf16((n, h, 128), seed=700 + i, device="cuda") for i in range(3))
    o1, _ = _run(q, k, v, None, cu)
    k2, v2 = k.clone(), v.clone()
    k2[130:330] = normal_bf16((200, h, 128), seed=711, device="cuda")
    v2[130:330] = normal_bf16((200, h, 128), seed=712, device="cuda")
    o2, _ = _run(q, k2, v2, None, cu)
    assert torch.equal(o1[:130].view(torch.int16), o2[:130].view(torch.int16))
    assert torch.equal(o1[330:].view(torch.int16), o2[330:].view(torch.int16))
    assert not torch.equal(o1[130:330].view(torch.int16), o2[130:330].view(torch.int16))


def test_attention_deterministic():
    cu = segment_offsets([1000, 24])
    n, h = cu[-1], 4
    q, k, v, g = (normal_bf16((n, h, 128), seed=800 + i, device="cuda") for i in range(4))
    o1, _ = _run(q, k, v, g, cu)
    o2, _ = _run(q, k, v, g, cu)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny512", "8k_p6"])
def test_attention_workload_every_row(name):
    """Small workloads: every rank's heads, every row, element by element."""
    h3 = _h3()
    w = WORKLOADS[name]
    say("attention workload full", name)
    src = normal_bf16((w.n_tokens, w.planes, 56, 128), seed=w.seed, device="cuda")
    src_bits = to_bits(src)
    heads = h3.head_split(56, w.world)
    for j, (_, c) in enumerate(heads):
        ref_in = oracle.seq2head(src_bits, w.world, ranks=[j])
        q, k, v = (to_device(ref_in[(j, p)]) for p in range(3))
        o, _ = _run(q, k, v, None, w.cu)
        ref = oracle.attention_rows(ref_in[(j, 0)], ref_in[(j, 1)], ref_in[(j, 2)], None, w.cu, SCALE)
        compare(to_bits(o), ref, f"{name} rank {j}")


@pytest.mark.parametrize("name", ["32k_p4", "128k_p4_qkvg", "250k_p8_qkvg"])
def test_attention_workload_sampled_rows(name):
    """Large workloads at full size, in the launch configuration of the bench:
    one rank's heads over the whole packed sequence, checked on sampled rows."""
    h3 = _h3()
    w = WORKLOADS[name]
    j = w.attn_rank
    say("attention workload sampled", name, "rank", j)
    heads = h3.head_split(56, w.world)
    n, c = w.n_tokens, heads[j][1]
    ops = [normal_bf16((n, c, 128), seed=w.seed + 10 + p, device="cuda") for p in range(w.planes)]
    g = ops[3] if w.planes >= 4 else None
    o, info = _run(ops[0], ops[1], ops[2], g, w.cu)
    bounds = [a for a, _ in (h3.partition(n, w.world, i) for i in range(w.world))]
    rows = sample_rows(w.cu, seed=w.seed, per_tile=2048, boundaries=bounds, limit=160)
    bits = [to_bits(t) for t in ops]
    ref = oracle.attention_rows(bits[0], bits[1], bits[2], bits[3] if g is not None else None, w.cu, SCALE,
                                rows=rows)
    got = to_bits(o)[rows]
    compare(got, ref, f"{name} sampled {len(rows)} rows")
    expected_flops = 4 * 128 * c * sum(L * L for L in w.segment_lengths)
    assert info.flops == expected_flops


@pytest.mark.timeout(900)
def test_attention_32k_every_row():
    """The 32k workload (four 8192-token segments, one rank's 14 heads, QKV) in
    the bench's launch configuration, every row of every head against the fp64
    oracle: 1.9e12 oracle FLOPs, about a minute on 16 host cores."""
    h3 = _h3()
    w = WORKLOADS["32k_p4"]
    j = w.attn_rank
    heads = h3.head_split(56, w.world)
    n, c = w.n_tokens, heads[j][1]
    say("attention 32k every row", "rank", j, "heads", c, "oracle threads", oracle.default_threads())
    ops = [normal_bf16((n, c, 128), seed=w.seed + 10 + p, device="cuda") for p in range(3)]
    o, info = _run(ops[0], ops[1], ops[2], None, w.cu)
    assert info.flops == 4 * 128 * c * sum(L * L for L in w.segment_lengths)
    bits = [to_bits(t) for t in ops]
    got = to_bits(o)
    del ops, o
    ref = oracle.attention_rows(bits[0], bits[1], bits[2], None, w.cu, SCALE)
    assert ref.shape == (n, c, 128)
    compare(got, ref, f"32k every row ({n} rows x {c} heads)")
    # the per-segment errors as well, so that no segment hides behind the others
    for s in range(len(w.cu) - 1):
        a, b = w.cu[s], w.cu[s + 1]
        compare(got[a:b], ref[a:b], f"32k segment {s}")
