"""GPU parity of the attention backward (dq, dk, dv, dg) against the fp64
oracle's chain rule, on ragged packed segments and at the workloads' sizes."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, segment_offsets
from synth.inputs import normal_bf16_bits
from tests.gpu_util import bits_to_f64, compare, say, sample_rows, to_bits, to_device

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5
# Gradients are compared against the unrounded fp64 chain rule with the same
# rel-RMS bar as the forward; the max-abs bar is relative to the largest
# reference entry, because gradient magnitudes differ from output magnitudes.
GRAD_REL_RMS = 5e-3
GRAD_MAX_REL = 2e-2


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _run_backward(bits, cu, gated):
    """Forward with lse, then backward, on device copies of the given bit patterns."""
    h3 = _h3()
    q, k, v, g, do = (to_device(b) for b in bits)
    if not gated:
        g = None
    n, h, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((n, h), dtype=torch.float32, device="cuda")
    h3.packed_attn(q, k, v, g, o, cu, SCALE, lse=lse)
    grads = [torch.full_like(q, float("nan")) for _ in range(4 if gated else 3)]
    ws = torch.empty(h3.packed_attn_backward_workspace(n, h, gated), dtype=torch.uint8, device="cuda")
    info = h3.packed_attn_backward(q, k, v, g, o, do, lse, grads[0], grads[1], grads[2],
                                   grads[3] if gated else None, ws, cu, SCALE)
    torch.cuda.synchronize()
    return [to_bits(t) for t in grads], to_bits(o), info


def _check(got_bits, ref, what):
    scale = float(np.abs(ref).max())
    return compare(got_bits, ref, what, atol=GRAD_MAX_REL * max(scale, 1e-6), rel_rms=GRAD_REL_RMS)


RAGGED = [[64], [1, 63, 64, 65], [127, 128, 129], [300], [5, 250, 1, 77, 130], [96, 160, 256], [700, 333]]


@pytest.mark.parametrize("lengths", RAGGED, ids=lambda x: "-".join(map(str, x)))
@pytest.mark.parametrize("gated", [False, True])
def test_attn_backward_ragged(lengths, gated):
    cu = segment_offsets(lengths)
    n, h = cu[-1], 3
    say("attn backward ragged", lengths, gated)
    bits = [normal_bf16_bits((n, h, 128), seed=2000 + 10 * i + n) for i in range(5)]
    grads, _, info = _run_backward(bits, cu, gated)
    ref = oracle.attention_backward(bits[0], bits[1], bits[2], bits[3] if gated else None, bits[4], cu, SCALE)
    for name, got in zip(("dq", "dk", "dv", "dg"), grads):
        _check(got, ref[name], f"{name} {lengths} gated={gated}")
    assert info.launches == 3
    assert info.flops == 10 * 128 * h * sum(L * L for L in lengths)


def _random_tables(count, seed):
    """Seeded segment tables: 1-6 segments of 1-800 tokens, 1-3 heads, gated or not."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        lengths = [int(x) for x in rng.integers(1, 801, size=int(rng.integers(1, 7)))]
        out.append((lengths, int(rng.integers(1, 4)), bool(rng.integers(0, 2))))
    return out


RANDOM_TABLES = _random_tables(12, 20261203)


@pytest.mark.parametrize("case", range(len(RANDOM_TABLES)))
def test_attn_backward_random_tables(case):
    """Every row of every gradient against the oracle on seeded random segment
    tables: mixed segment lengths in one launch reach every exit point of the
    key-block kernel's loop over query tiles (unrolled by three) and every
    partial fill of its 48-key slices and 192-key blocks."""
    lengths, h, gated = RANDOM_TABLES[case]
    cu = segment_offsets(lengths)
    n = cu[-1]
    say("attn backward random table", case, lengths, h, gated)
    bits = [normal_bf16_bits((n, h, 128), seed=2500 + 10 * case + i) for i in range(5)]
    grads, _, info = _run_backward(bits, cu, gated)
    ref = oracle.attention_backward(bits[0], bits[1], bits[2], bits[3] if gated else None, bits[4], cu, SCALE)
    for name, got in zip(("dq", "dk", "dv", "dg"), grads):
        _check(got, ref[name], f"{name} random table {case}")
    assert info.flops == 10 * 128 * h * sum(L * L for L in lengths)


@pytest.mark.parametrize("gated", [False, True])
def test_attn_backward_one_token_segment(gated):
    """A one-token segment has p = 1, so dq = dk = 0 exactly and dv = do * sig(g).
    The kernel forms ds = p (<e, v> - D) from bf16-rounded e = do * sig(g) and
    o, so dq and dk carry rounding noise of order scale * 2^-8 * |do||v||k|
    instead of zeros; they are bounded absolutely, dv and dg compared as usual."""
    cu = [0, 1]
    say("attn backward one token", gated)
    bits = [normal_bf16_bits((1, 4, 128), seed=2100 + i) for i in range(5)]
    grads, _, _ = _run_backward(bits, cu, gated)
    ref = oracle.attention_backward(bits[0], bits[1], bits[2], bits[3] if gated else None, bits[4], cu, SCALE)
    for name in ("dq", "dk"):
        assert np.array_equal(ref[name], np.zeros_like(ref[name]))
        assert np.abs(bits_to_f64(grads[0 if name == "dq" else 1])).max() <= 2e-2, name
    _check(grads[2], ref["dv"], f"dv one token gated={gated}")
    if gated:
        _check(grads[3], ref["dg"], "dg one token")


def _workload_bits(w, heads, seed_off=0):
    n = w.n_tokens
    return [normal_bf16_bits((n, heads, 128), seed=w.seed + 60 + seed_off + i) for i in range(5)]


@pytest.mark.parametrize("name", ["tiny512", "8k_p6"])
def test_attn_backward_workload_every_row(name):
    w = WORKLOADS[name]
    h = _h3().head_split(56, w.world)[0][1]          # rank 0's heads
    gated = w.planes >= 4
    say("attn backward workload", name, h)
    bits = _workload_bits(w, h)
    grads, _, _ = _run_backward(bits, w.cu, gated)
    hs = slice(0, h) if name == "tiny512" else slice(h - 2, h)     # the oracle checks every row of these heads
    one = [np.ascontiguousarray(b[:, hs]) for b in bits]
    ref = oracle.attention_backward(one[0], one[1], one[2], one[3] if gated else None, one[4], w.cu, SCALE)
    for name_, got in zip(("dq", "dk", "dv", "dg"), grads):
        _check(np.ascontiguousarray(got[:, hs]), ref[name_], f"{name_} {name}")


def _key_sample(cu, seed, max_len, per_seg=24):
    """Seeded key rows (first, last and random ones) from the segments no longer than max_len."""
    rng = np.random.default_rng(seed)
    rows = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b - a <= max_len:
            rows += [a, b - 1] + [int(x) for x in rng.integers(a, b, size=per_seg)]
    return np.array(sorted(set(rows)), dtype=np.int64)


@pytest.mark.parametrize("name", ["32k_p4", "128k_p4_qkvg", "250k_p8_qkvg"])
def test_attn_backward_workload_sampled(name):
    """The rank's whole head share on the GPU; one head checked against the oracle
    on sampled query rows, on sampled key rows of the segments the oracle can
    afford, and on every segment through the exact identities
    sum_u dk_u = 0 and sum_u dv_u = sum_t do_t * sig(g_t)."""
    w = WORKLOADS[name]
    h = _h3().head_split(56, w.world)[0][1]
    gated = w.planes >= 4
    say("attn backward workload sampled", name, h)
    bits = _workload_bits(w, h)
    grads, _, _ = _run_backward(bits, w.cu, gated)
    hh = 1                                            # the checked head
    one = [np.ascontiguousarray(b[:, hh:hh + 1]) for b in bits]
    q_rows = sample_rows(w.cu, seed=w.seed + 71, per_tile=4096, limit=48)
    k_rows = _key_sample(w.cu, seed=w.seed + 72, max_len=8192)
    ref = oracle.attention_backward(one[0], one[1], one[2], one[3] if gated else None, one[4], w.cu, SCALE,
                                    q_rows=q_rows, k_rows=k_rows)
    got = {n_: g[:, hh:hh + 1] for n_, g in zip(("dq", "dk", "dv", "dg"), grads)}
    _check(got["dq"][q_rows], ref["dq"], f"dq {name} sampled")
    if gated:
        _check(got["dg"][q_rows], ref["dg"], f"dg {name} sampled")
    if len(k_rows):
        _check(got["dk"][k_rows], ref["dk"], f"dk {name} sampled")
        _check(got["dv"][k_rows], ref["dv"], f"dv {name} sampled")
    # identities on every segment of the checked head
    dk = bits_to_f64(got["dk"])[:, 0]
    dv = bits_to_f64(got["dv"])[:, 0]
    e = bits_to_f64(one[4])[:, 0]
    if gated:
        # the kernel feeds its products with e = do * sig(g) rounded to bf16
        e = torch.from_numpy(e / (1.0 + np.exp(-bits_to_f64(one[3])[:, 0]))).to(torch.bfloat16).double().numpy()
    for s in range(len(w.cu) - 1):
        a, b = int(w.cu[s]), int(w.cu[s + 1])
        # Both sums cancel exactly in exact arithmetic; what is left is the
        # rounding of o (which enters D), of ds and p to bf16 for the MFMA and
        # of the bf16 outputs, summed over L rows like a random walk. Emulating
        # those roundings in fp64 on random inputs puts the largest of the 128
        # columns at 0.7-1.2 x 2^-7 sqrt(L) RMS; the bar is four times that.
        bound_k = 2.0 ** -5 * np.sqrt(b - a) * np.sqrt((dk[a:b] ** 2).mean()) + 1e-4
        ev = e[a:b].sum(axis=0)
        bound_v = 2.0 ** -5 * np.sqrt(b - a) * np.sqrt((dv[a:b] ** 2).mean()) + 1e-4
        say(f"identities {name} segment {s} (L={b - a}): sum dk {np.abs(dk[a:b].sum(axis=0)).max() / bound_k:.3f} "
            f"of the bar, sum dv - sum e {np.abs(dv[a:b].sum(axis=0) - ev).max() / bound_v:.3f} of the bar")
        assert np.abs(dk[a:b].sum(axis=0)).max() <= bound_k, (name, s)
        assert np.abs(dv[a:b].sum(axis=0) - ev).max() <= bound_v, (name, s)
