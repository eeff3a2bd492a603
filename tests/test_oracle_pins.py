"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to something fixed from outside: the tables
the pages print (tests/golden/), closed forms, invariants the pages name, and
library routines that the method reduces to in special cases (torch's
scaled-dot-product attention and layer norm in float64 on the CPU).  They are
chosen so that a dropped term, a wrong sign or index, or a swapped operand in
the oracle fails at least one of them.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS
from synth.inputs import normal_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# partition
# ---------------------------------------------------------------------------

def test_head_partition_matches_printed_table():
    rows = _read_golden("head_partition.txt")
    assert len(rows) == 4
    for ranks, heads in rows:
        expected = [int(h) for h in heads.split(",")]
        got = oracle.partition(56, int(ranks))
        assert [c for _, c in got] == expected
        # ranks own consecutive head ranges starting at 0
        assert [b for b, _ in got] == list(np.cumsum([0] + expected[:-1]))


def test_token_window_identity():
    """One bf16 plane of one rank's token shard at 250k / four ranks is the printed window."""
    g = dict(_read_golden("transfer_window.txt"))
    tokens, ranks = int(g["tokens"]), int(g["ranks"])
    shard = oracle.partition(tokens, ranks)
    assert all(c == 62500 for _, c in shard)
    window = shard[0][1] * int(g["heads"]) * int(g["head_dim"]) * int(g["bytes_per_element"])
    assert window == int(g["window_bytes"])
    assert window < int(g["cap_bytes"])


@pytest.mark.parametrize("total,parts", [(0, 1), (5, 6), (56, 57), (56, 0), (56, -1)])
def test_partition_rejects_empty_parts(total, parts):
    with pytest.raises(oracle.EmptyPartition):
        oracle.partition(total, parts)


def test_partition_properties_brute_force():
    for total in range(1, 70):
        for parts in range(1, total + 1):
            got = oracle.partition(total, parts)
            counts = [c for _, c in got]
            assert sum(counts) == total
            assert max(counts) - min(counts) <= 1
            assert counts == sorted(counts, reverse=True)      # larger parts first
            ends = [b + c for b, c in got]
            assert [b for b, _ in got] == [0] + ends[:-1]       # contiguous, in rank order


def test_token_split_of_8k_over_six():
    got = oracle.partition(8192, 6)
    assert [c for _, c in got] == [1366, 1366, 1365, 1365, 1365, 1365]
    assert [b for b, _ in got] == [0, 1366, 2732, 4097, 5462, 6827]


# ---------------------------------------------------------------------------
# clip and rebase
# ---------------------------------------------------------------------------

def test_clip_worked_examples():
    cu = [0, 96, 256, 512]
    assert oracle.clip_segments(cu, 0, 256) == [(0, 0, 96), (1, 96, 256)]
    assert oracle.clip_segments(cu, 256, 512) == [(2, 0, 256)]
    assert oracle.clip_segments(cu, 50, 300) == [(0, 0, 46), (1, 46, 206), (2, 206, 250)]
    # a segment boundary that equals a rank start gives no empty entry
    cu4 = [0, 98304, 131072]
    assert oracle.clip_segments(cu4, 98304, 131072) == [(1, 0, 32768)]
    assert oracle.clip_segments(cu4, 65536, 98304) == [(0, 0, 32768)]


def test_clip_brute_force_per_token():
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(2, 60))
        s = int(rng.integers(1, n + 1))
        cuts = sorted(rng.choice(np.arange(1, n), size=s - 1, replace=False)) if s > 1 else []
        cu = [0] + [int(c) for c in cuts] + [n]
        a = int(rng.integers(0, n))
        b = int(rng.integers(a + 1, n + 1))
        table = oracle.clip_segments(cu, a, b)
        for t in range(a, b):
            global_seg = max(i for i in range(len(cu) - 1) if cu[i] <= t)
            hits = [sid for sid, lo, hi in table if lo <= t - a < hi]
            assert hits == [global_seg]
        # pieces are disjoint, ordered and tile [0, b - a)
        assert table[0][1] == 0 and table[-1][2] == b - a
        for e0, e1 in zip(table, table[1:]):
            assert e0[2] == e1[1] and e0[0] < e1[0]


def test_clip_union_over_ranks_is_global_segmentation():
    w = WORKLOADS["8k_p6"]
    pieces = []
    for a, cnt in oracle.partition(w.n_tokens, w.world):
        for s, lo, hi in oracle.clip_segments(w.cu, a, a + cnt):
            pieces.append((s, a + lo, a + hi))
    merged = {}
    for s, lo, hi in pieces:
        merged.setdefault(s, []).append((lo, hi))
    for s, spans in merged.items():
        spans.sort()
        assert spans[0][0] == w.cu[s] and spans[-1][1] == w.cu[s + 1]
        for x, y in zip(spans, spans[1:]):
            assert x[1] == y[0]
    assert sorted(merged) == list(range(w.n_segments))


# ---------------------------------------------------------------------------
# relayouts
# ---------------------------------------------------------------------------

def _coded_qkv(n, k, h, d):
    """int64 operand whose entry at (t, p, h, d) is the number of that position."""
    return np.arange(n * k * h * d, dtype=np.int64).reshape(n, k, h, d)


@pytest.mark.parametrize("world", [1, 2, 4, 6, 8])
def test_seq2head_elements_come_from_their_owner_head(world):
    table = {int(r): [int(x) for x in hs.split(",")] for r, hs in _read_golden("head_partition.txt")}
    n, k, h, d = 37, 3, 56, 4        # 37 tokens: a ragged token split for every world size
    src = _coded_qkv(n, k, h, d)
    out = oracle.seq2head(src, world)
    counts = table.get(world, [56])
    starts = np.cumsum([0] + counts[:-1])
    for j in range(world):
        for p in range(k):
            buf = out[(j, p)]
            assert buf.shape == (n, counts[j], d)
            t, hl, dd = np.meshgrid(np.arange(n), np.arange(counts[j]), np.arange(d), indexing="ij")
            decoded_h = (buf // d) % h
            decoded_p = (buf // (d * h)) % k
            decoded_t = buf // (d * h * k)
            assert np.array_equal(decoded_t, t)
            assert np.array_equal(decoded_p, np.full_like(t, p))
            assert np.array_equal(decoded_h, starts[j] + hl)
            assert np.array_equal(buf % d, dd)
            assert not np.shares_memory(buf, src)


@pytest.mark.parametrize("world", [1, 2, 4, 6, 8])
def test_transport_identity_round_trip(world):
    src = normal_bf16_bits((45, 4, 56, 8), seed=11)
    out = oracle.seq2head(src, world)
    for p in range(4):
        back = oracle.head2seq([out[(j, p)] for j in range(world)], 56)
        assert back.dtype == np.uint16
        assert np.array_equal(back, src[:, p])


def test_world_size_one_is_a_copy():
    src = normal_bf16_bits((19, 3, 56, 8), seed=12)
    out = oracle.seq2head(src, 1)
    for p in range(3):
        assert np.array_equal(out[(0, p)], src[:, p])
        assert not np.shares_memory(out[(0, p)], src)


def test_head2seq_elements_land_on_their_global_head():
    n, h, d, world = 23, 56, 4, 6
    heads = oracle.partition(h, world)
    bufs = []
    for hb, hn in heads:
        t, hl, dd = np.meshgrid(np.arange(n), np.arange(hn), np.arange(d), indexing="ij")
        bufs.append((t * h + hb + hl) * d + dd)        # code of the global position
    out = oracle.head2seq(bufs, h)
    assert np.array_equal(out.reshape(-1), np.arange(n * h * d))


# ---- backward of the relayouts ------------------------------------------------

@pytest.mark.parametrize("world", [1, 2, 3, 6, 8])
def test_seq2head_backward_is_the_adjoint(world):
    """<seq2head(x), y> = <x, seq2head_backward(y)> exactly, on integer-valued data."""
    rng = np.random.default_rng(40 + world)
    n, k, h, d = 29, 3, 56, 4
    x = rng.integers(-50, 50, size=(n, k, h, d)).astype(np.float64)
    heads = oracle.partition(h, world)
    y = {(j, p): rng.integers(-50, 50, size=(n, heads[j][1], d)).astype(np.float64)
         for j in range(world) for p in range(k)}
    fx = oracle.seq2head(x, world)
    lhs = sum(float((fx[key] * y[key]).sum()) for key in y)
    rhs = float((x * oracle.seq2head_backward(y, n, k, h, world)).sum())
    assert lhs == rhs


@pytest.mark.parametrize("world", [1, 2, 3, 6, 8])
def test_seq2head_backward_matches_library_autograd(world):
    """Gradient of the relayout written with torch.tensor_split (torch's own
    quotient/remainder split) and taken by autograd."""
    rng = np.random.default_rng(60 + world)
    n, k, h, d = 17, 4, 56, 3
    x = torch.tensor(rng.standard_normal((n, k, h, d)), dtype=torch.float64, requires_grad=True)
    parts = torch.tensor_split(x, world, dim=2)
    w = {(j, p): rng.standard_normal((n, parts[j].shape[2], d)) for j in range(world) for p in range(k)}
    loss = sum((parts[j][:, p] * torch.from_numpy(w[(j, p)])).sum() for j in range(world) for p in range(k))
    loss.backward()
    assert np.array_equal(oracle.seq2head_backward(w, n, k, h, world), x.grad.numpy())


def test_seq2head_backward_rank_share_and_round_trip():
    src = normal_bf16_bits((33, 4, 56, 8), seed=13)
    for world in (1, 4, 6):
        fwd = oracle.seq2head(src, world)
        assert np.array_equal(oracle.seq2head_backward(fwd, 33, 4, 56, world), src)
        # one rank's share: its heads are written, the rest keep the initial values
        j = world - 1
        hb, hn = oracle.partition(56, world)[j]
        init = np.full(src.shape, 7, np.uint16)
        part = oracle.seq2head_backward({(j, p): fwd[(j, p)] for p in range(4)}, 33, 4, 56, world, ranks=[j],
                                        out=init)
        assert np.array_equal(part[:, :, hb:hb + hn], src[:, :, hb:hb + hn])
        mask = np.ones(56, bool)
        mask[hb:hb + hn] = False
        assert (part[:, :, mask] == 7).all()


@pytest.mark.parametrize("world", [1, 2, 5, 8])
def test_head2seq_backward_matches_library_autograd(world):
    """Gradient of head2seq written as torch.cat of the rank buffers along heads."""
    rng = np.random.default_rng(80 + world)
    n, h, d = 21, 56, 3
    sizes = [t.shape[2] for t in torch.tensor_split(torch.empty(1, 1, h), world, dim=2)]
    bufs = [torch.tensor(rng.standard_normal((n, c, d)), dtype=torch.float64, requires_grad=True) for c in sizes]
    w = rng.standard_normal((n, h, d))
    (torch.cat(bufs, dim=1) * torch.from_numpy(w)).sum().backward()
    got = oracle.head2seq_backward(w, world)
    for j in range(world):
        assert np.array_equal(got[j], bufs[j].grad.numpy())


def test_head2seq_backward_is_the_adjoint_and_inverts_head2seq():
    rng = np.random.default_rng(91)
    n, h, d, world = 26, 56, 4, 6
    heads = oracle.partition(h, world)
    bufs = [rng.integers(-9, 9, size=(n, hn, d)).astype(np.float64) for _, hn in heads]
    y = rng.integers(-9, 9, size=(n, h, d)).astype(np.float64)
    gb = oracle.head2seq_backward(y, world)
    assert float((oracle.head2seq(bufs, h) * y).sum()) == sum(float((bufs[j] * gb[j]).sum()) for j in range(world))
    back = oracle.head2seq_backward(oracle.head2seq(bufs, h), world)
    for j in range(world):
        assert np.array_equal(back[j], bufs[j])


def test_head2seq_rejects_wrong_buffer_shape():
    bufs = [np.zeros((8, 28, 4), np.uint16), np.zeros((8, 27, 4), np.uint16)]
    with pytest.raises(ValueError):
        oracle.head2seq(bufs, 56)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _qkvg(n, h, d, seed, qscale=1.0):
    q = normal_bf16_bits((n, h, d), seed, std=qscale)
    k = normal_bf16_bits((n, h, d), seed + 1)
    v = normal_bf16_bits((n, h, d), seed + 2)
    g = normal_bf16_bits((n, h, d), seed + 3)
    return q, k, v, g


def _sdpa_f64(q, k, v, scale):
    """torch's scaled-dot-product attention in float64 on the CPU, [L, H, D] operands."""
    f = lambda a: torch.from_numpy(oracle.bf16_bits_to_f64(a)).permute(1, 0, 2).contiguous()  # noqa: E731
    o = torch.nn.functional.scaled_dot_product_attention(f(q), f(k), f(v), scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("gated", [False, True])
def test_attention_matches_dense_brute_force(gated):
    cu = [0, 1, 17, 64, 65, 130, 200]
    n, h, d = 200, 3, 32
    q, k, v, g = _qkvg(n, h, d, seed=21)
    scale = d ** -0.5
    got = oracle.attention_rows(q, k, v, g if gated else None, cu, scale)
    ref = oracle.attention_dense(q, k, v, g if gated else None, cu, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("qscale", [1.0, 8.0])
def test_attention_segments_match_library_sdpa(qscale):
    cu = [0, 96, 256, 300]
    n, h, d = 300, 4, 128
    q, k, v, g = _qkvg(n, h, d, seed=31, qscale=qscale)
    scale = 128 ** -0.5
    got = oracle.attention_rows(q, k, v, None, cu, scale)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        ref = _sdpa_f64(q[a:b], k[a:b], v[a:b], scale)
        np.testing.assert_allclose(got[a:b], ref, rtol=0, atol=1e-10)


def test_attention_gate_is_sigmoid_of_g():
    cu = [0, 40, 100]
    n, h, d = 100, 2, 64
    q, k, v, g = _qkvg(n, h, d, seed=41)
    scale = 0.125
    got = oracle.attention_rows(q, k, v, g, cu, scale)
    ungated = oracle.attention_rows(q, k, v, None, cu, scale)
    sig = torch.sigmoid(torch.from_numpy(oracle.bf16_bits_to_f64(g))).numpy()
    np.testing.assert_allclose(got, ungated * sig, rtol=1e-13, atol=0)
    # G = 0 halves the output exactly
    half = oracle.attention_rows(q, k, v, np.zeros_like(g), cu, scale)
    assert np.array_equal(half, ungated * 0.5)


def test_attention_closed_forms():
    n, h, d = 48, 2, 16
    q, k, v, g = _qkvg(n, h, d, seed=51)
    cu = [0, 1, 20, 48]
    # a one-token segment returns its own value row exactly
    o = oracle.attention_rows(q, k, v, None, cu, 0.3, rows=[0])
    assert np.array_equal(o[0], oracle.bf16_bits_to_f64(v[0]))
    # a value row that is constant over a segment comes back for every query of it
    v2 = v.copy()
    v2[1:20] = v2[1]
    o = oracle.attention_rows(q, k, v2, None, cu, 0.3)
    np.testing.assert_allclose(o[1:20], np.broadcast_to(oracle.bf16_bits_to_f64(v2[1]), (19, h, d)),
                               rtol=0, atol=1e-12)
    # identical key rows make the weights uniform: the segment mean of V
    k2 = k.copy()
    k2[20:48] = k2[20]
    o = oracle.attention_rows(q, k2, v, None, cu, 0.3)
    mean = oracle.bf16_bits_to_f64(v[20:48]).mean(axis=0)
    np.testing.assert_allclose(o[20:48], np.broadcast_to(mean, (28, h, d)), rtol=0, atol=1e-12)


def test_attention_key_permutation_inside_segment():
    n, h, d = 64, 2, 16
    q, k, v, _ = _qkvg(n, h, d, seed=61)
    cu = [0, 30, 64]
    perm = np.arange(n)
    perm[30:64] = 30 + np.random.default_rng(3).permutation(34)
    o1 = oracle.attention_rows(q, k, v, None, cu, 0.25)
    o2 = oracle.attention_rows(q, k[perm], v[perm], None, cu, 0.25)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    # moving a key across the boundary DOES change the result (segments do not mix)
    swap = np.arange(n)
    swap[29], swap[30] = 30, 29
    o3 = oracle.attention_rows(q, k[swap], v[swap], None, cu, 0.25)
    assert np.abs(o3 - o1).max() > 1e-3


def test_attention_row_subset_equals_full():
    n, h, d = 90, 2, 32
    q, k, v, g = _qkvg(n, h, d, seed=71)
    cu = [0, 33, 90]
    full = oracle.attention_rows(q, k, v, g, cu, 0.2)
    rows = [89, 0, 33, 32, 50]
    sub = oracle.attention_rows(q, k, v, g, cu, 0.2, rows=rows, threads=3)
    assert np.array_equal(sub, full[rows])


# ---- attention backward -----------------------------------------------------

def _autograd_attention(q, k, v, g, dout, cu, scale):
    """Dense N x N masked (gated) attention in float64 through torch autograd;
    returns (lse, dq, dk, dv, dg) for the loss sum(dout * o)."""
    f = lambda a: torch.from_numpy(oracle.bf16_bits_to_f64(a)).requires_grad_(True)  # noqa: E731
    tq, tk, tv = f(q), f(k), f(v)
    tg = None if g is None else f(g)
    n = q.shape[0]
    seg = np.searchsorted(np.asarray(cu), np.arange(n), side="right") - 1
    same = torch.from_numpy(seg[:, None] == seg[None, :])
    logits = torch.einsum("thd,uhd->htu", tq, tk) * scale
    logits = logits.masked_fill(~same, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)                       # [H, N]
    o = torch.einsum("htu,uhd->thd", torch.softmax(logits, dim=-1), tv)
    if tg is not None:
        o = o * torch.sigmoid(tg)
    (o * torch.from_numpy(oracle.bf16_bits_to_f64(dout))).sum().backward()
    return (lse.T.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(),
            None if tg is None else tg.grad.numpy())


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("qscale", [1.0, 8.0])
def test_attention_backward_matches_library_autograd(gated, qscale):
    cu = [0, 1, 37, 90, 130]
    n, h, d = 130, 2, 16
    q, k, v, g = _qkvg(n, h, d, seed=77, qscale=qscale)
    dout = normal_bf16_bits((n, h, d), seed=81)
    scale = 0.25
    got = oracle.attention_backward(q, k, v, g if gated else None, dout, cu, scale)
    lse, dq, dk, dv, dg = _autograd_attention(q, k, v, g if gated else None, dout, cu, scale)
    np.testing.assert_allclose(got["lse"], lse, rtol=1e-12, atol=1e-12)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(got[name], ref, rtol=1e-9, atol=1e-10, err_msg=name)
    if gated:
        np.testing.assert_allclose(got["dg"], dg, rtol=1e-9, atol=1e-10)
    else:
        assert "dg" not in got


def test_attention_backward_closed_forms():
    n, h, d, scale = 40, 2, 8, 0.3
    q, k, v, g = _qkvg(n, h, d, seed=90)
    dout = normal_bf16_bits((n, h, d), seed=91)
    # a one-token segment: p = 1, so ds = 0 -> dq = dk = 0, and dv = do * sig(g)
    cu = [0, 1, 40]
    r = oracle.attention_backward(q, k, v, g, dout, cu, scale, q_rows=[0], k_rows=[0])
    sg = 1 / (1 + np.exp(-oracle.bf16_bits_to_f64(g[0])))
    assert np.array_equal(r["dq"][0], np.zeros((h, d)))
    assert np.array_equal(r["dk"][0], np.zeros((h, d)))
    np.testing.assert_allclose(r["dv"][0], oracle.bf16_bits_to_f64(dout[0]) * sg, rtol=1e-15)
    # identical keys in a segment: the softmax ignores q, so dq = 0
    k2 = k.copy()
    k2[1:40] = k[5]
    r2 = oracle.attention_backward(q, k2, v, None, dout, cu, scale, q_rows=np.arange(1, 40), k_rows=[])
    assert np.abs(r2["dq"]).max() < 1e-12
    # g = 0: dg = do * a / 4 with a the ungated output
    g0 = np.zeros_like(g)
    r3 = oracle.attention_backward(q, k, v, g0, dout, cu, scale, k_rows=[])
    a = oracle.attention_rows(q, k, v, None, cu, scale)
    np.testing.assert_allclose(r3["dg"], oracle.bf16_bits_to_f64(dout) * a / 4, rtol=1e-13, atol=1e-15)


def test_attention_backward_segment_sums():
    """Per segment and head: sum_u dk_u = 0 (the rows of ds sum to zero) and
    sum_u dv_u = sum_t do_t * sig(g_t) (the rows of p sum to one)."""
    cu = [0, 50, 51, 180]
    n, h, d, scale = 180, 3, 8, 0.2
    q, k, v, g = _qkvg(n, h, d, seed=95, qscale=2.0)
    dout = normal_bf16_bits((n, h, d), seed=96)
    r = oracle.attention_backward(q, k, v, g, dout, cu, scale)
    e = oracle.bf16_bits_to_f64(dout) / (1 + np.exp(-oracle.bf16_bits_to_f64(g)))
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        np.testing.assert_allclose(r["dk"][a:b].sum(axis=0), 0.0, atol=1e-11)
        np.testing.assert_allclose(r["dv"][a:b].sum(axis=0), e[a:b].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_attention_backward_row_subsets_equal_full():
    cu = [0, 70, 100]
    n, h, d = 100, 2, 8
    q, k, v, g = _qkvg(n, h, d, seed=97)
    dout = normal_bf16_bits((n, h, d), seed=98)
    full = oracle.attention_backward(q, k, v, g, dout, cu, 0.3)
    rows = [0, 69, 70, 99, 33]
    part = oracle.attention_backward(q, k, v, g, dout, cu, 0.3, q_rows=rows, k_rows=rows[::-1])
    for name in ("lse", "delta", "dq", "dg"):
        assert np.array_equal(part[name], full[name][rows]), name
    for name in ("dk", "dv"):
        assert np.array_equal(part[name], full[name][rows[::-1]]), name


def test_attention_flops_closed_form():
    w = WORKLOADS["128k_p4_qkvg"]
    assert oracle.attention_flops(w.cu, 14, 128) == 4 * 128 * 14 * (98304 ** 2 + 32768 ** 2)


# ---------------------------------------------------------------------------
# AdaLN
# ---------------------------------------------------------------------------

def _adaln_inputs(n, c, s, seed):
    x = normal_bf16_bits((n, c), seed)
    b = normal_bf16_bits((n, c), seed + 1)
    shift = normal_bf16_bits((s, c), seed + 2, std=0.1)
    scale = normal_bf16_bits((s, c), seed + 3, std=0.1)
    gate = normal_bf16_bits((s, c), seed + 4, std=0.1)
    return x, b, shift, scale, gate


def _segment_of_token(cu, t):
    return max(i for i in range(len(cu) - 1) if cu[i] <= t)


def test_adaln_modulate_matches_library_layer_norm():
    cu = [0, 96, 256, 512]
    n, c = 512, 256
    x, b, shift, scale, gate = _adaln_inputs(n, c, 3, seed=81)
    eps = 1e-6
    for a, e in [(0, 512), (0, 256), (256, 512), (100, 300)]:
        got = oracle.adaln_rows(oracle.MODULATE, x[a:e], None, shift, scale, None, a, e, cu, eps)
        xf = torch.from_numpy(oracle.bf16_bits_to_f64(x[a:e]))
        ln = torch.nn.functional.layer_norm(xf, (c,), eps=eps).numpy()
        seg = np.array([_segment_of_token(cu, t) for t in range(a, e)])
        ref = ln * (1.0 + oracle.bf16_bits_to_f64(scale)[seg]) + oracle.bf16_bits_to_f64(shift)[seg]
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_adaln_modulate_closed_forms():
    cu = [0, 5, 12]
    n, c = 12, 64
    x, b, shift, scale, gate = _adaln_inputs(n, c, 2, seed=91)
    zero = np.zeros_like(shift)
    y = oracle.adaln_rows(oracle.MODULATE, x, None, zero, zero, None, 0, n, cu, 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, atol=1e-12)
    # a constant row normalises to zero, leaving exactly the shift of its global segment
    xc = np.broadcast_to(x[:, :1], x.shape).copy()
    y = oracle.adaln_rows(oracle.MODULATE, xc, None, shift, scale, None, 0, n, cu, 1e-6)
    sh = oracle.bf16_bits_to_f64(shift)
    assert np.array_equal(y[:5], np.broadcast_to(sh[0], (5, c)))
    assert np.array_equal(y[5:], np.broadcast_to(sh[1], (7, c)))


def test_adaln_gate_closed_forms():
    cu = [0, 7, 20, 33]
    n, c = 33, 32
    x, b, shift, scale, gate = _adaln_inputs(n, c, 3, seed=101)
    # zero gate: residual passes unchanged
    y = oracle.adaln_rows(oracle.GATE_RESIDUAL, x, b, None, None, np.zeros_like(gate), 0, n, cu, 0.0)
    assert np.array_equal(y, oracle.bf16_bits_to_f64(x))
    # unit branch: y - x is the gate row of the token's global segment
    one = np.full_like(b, 0x3F80)      # bf16 bits of 1.0
    a, e = 5, 30                       # an interval that cuts segments 0 and 2
    y = oracle.adaln_rows(oracle.GATE_RESIDUAL, x[a:e], one[a:e], None, None, gate, a, e, cu, 0.0)
    gf = oracle.bf16_bits_to_f64(gate)
    for t in range(a, e):
        assert np.array_equal(y[t - a] - oracle.bf16_bits_to_f64(x[t]), gf[_segment_of_token(cu, t)])


@pytest.mark.parametrize("mode", [0, 1])
def test_adaln_per_rank_equals_global(mode):
    w = WORKLOADS["8k_p6"]
    n, c = w.n_tokens, 64
    x, b, shift, scale, gate = _adaln_inputs(n, c, w.n_segments, seed=111)
    whole = oracle.adaln_rows(mode, x, b, shift, scale, gate, 0, n, w.cu, 1e-6)
    for a, cnt in oracle.partition(n, w.world):
        part = oracle.adaln_rows(mode, x[a:a + cnt], b[a:a + cnt], shift, scale, gate, a, a + cnt,
                                 w.cu, 1e-6)
        assert np.array_equal(part, whole[a:a + cnt])


def test_adaln_gate_modulate_matches_library_layer_norm():
    """The residual x + gate_s * b, then the next sub-block's modulation of it,
    against torch's fp64 layer_norm of the same residual."""
    cu = [0, 96, 256, 512]
    n, c = 512, 256
    x, b, shift, scale, gate = _adaln_inputs(n, c, 3, seed=121)
    eps = 1e-6
    f = oracle.bf16_bits_to_f64
    for a, e in [(0, 512), (256, 512), (100, 300)]:
        resid, y = oracle.adaln_gate_modulate(x[a:e], b[a:e], gate, shift, scale, a, e, cu, eps)
        seg = np.array([_segment_of_token(cu, t) for t in range(a, e)])
        r_ref = torch.from_numpy(f(x[a:e])) + torch.from_numpy(f(gate)[seg]) * torch.from_numpy(f(b[a:e]))
        np.testing.assert_allclose(resid, r_ref.numpy(), rtol=0, atol=1e-15)
        ln = torch.nn.functional.layer_norm(r_ref, (c,), eps=eps).numpy()
        np.testing.assert_allclose(y, ln * (1.0 + f(scale)[seg]) + f(shift)[seg], rtol=0, atol=1e-12)


def test_adaln_gate_modulate_closed_forms():
    cu = [0, 9, 30]
    n, c = 30, 64
    x, b, shift, scale, gate = _adaln_inputs(n, c, 2, seed=131)
    # zero gate: the residual is x, so the chain is plain modulation of x
    resid, y = oracle.adaln_gate_modulate(x, b, np.zeros_like(gate), shift, scale, 0, n, cu, 1e-6)
    assert np.array_equal(resid, oracle.bf16_bits_to_f64(x))
    assert np.array_equal(y, oracle.adaln_rows(oracle.MODULATE, x, None, shift, scale, None, 0, n, cu, 1e-6))
    # unit gate and b = 5 - x on small integers: a constant residual row, so y is exactly shift_s
    xi = torch.randint(-8, 9, (n, c), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    bi = (5 - xi.float()).to(torch.bfloat16)
    as_bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    one = np.full_like(gate, 0x3F80)
    resid, y = oracle.adaln_gate_modulate(as_bits(xi), as_bits(bi), one, shift, scale, 0, n, cu, 1e-6)
    assert np.array_equal(resid, np.full((n, c), 5.0))
    sh = oracle.bf16_bits_to_f64(shift)
    assert np.array_equal(y[:9], np.broadcast_to(sh[0], (9, c)))
    assert np.array_equal(y[9:], np.broadcast_to(sh[1], (21, c)))


def test_adaln_gate_modulate_per_rank_equals_global():
    w = WORKLOADS["8k_p6"]
    n, c = w.n_tokens, 64
    x, b, shift, scale, gate = _adaln_inputs(n, c, w.n_segments, seed=141)
    r_all, y_all = oracle.adaln_gate_modulate(x, b, gate, shift, scale, 0, n, w.cu, 1e-6)
    for a, cnt in oracle.partition(n, w.world):
        r, y = oracle.adaln_gate_modulate(x[a:a + cnt], b[a:a + cnt], gate, shift, scale, a, a + cnt, w.cu, 1e-6)
        assert np.array_equal(r, r_all[a:a + cnt]) and np.array_equal(y, y_all[a:a + cnt])


# ---------------------------------------------------------------------------
# ragged reduce-scatter and row gather
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("world", [1, 2, 3, 6, 8])
def test_reduce_scatter_is_sum_then_numpy_split(world):
    """Rank i's rows of (sum of the partials + bias), with numpy's array_split
    (first N mod P parts one larger) as the independent row split."""
    n, c = 1003, 24
    parts = [normal_bf16_bits((n, c), seed=150 + j) for j in range(world)]
    bias = normal_bf16_bits((c,), seed=149)
    got = oracle.reduce_scatter(parts, bias)
    total = sum(oracle.bf16_bits_to_f64(p) for p in parts) + oracle.bf16_bits_to_f64(bias)
    for i, ref in enumerate(np.array_split(total, world)):
        np.testing.assert_allclose(got[i], ref, rtol=0, atol=1e-12)


def test_reduce_scatter_adds_bias_once():
    n, c, world = 37, 16, 4
    bias = normal_bf16_bits((c,), seed=160)
    zero = [np.zeros((n, c), np.uint16) for _ in range(world)]
    got = oracle.reduce_scatter(zero, bias)
    assert sum(v.shape[0] for v in got.values()) == n
    for i, v in got.items():
        assert np.array_equal(v, np.broadcast_to(oracle.bf16_bits_to_f64(bias), v.shape))
    same = [normal_bf16_bits((n, c), seed=161)] * world
    got = oracle.reduce_scatter(same, None, ranks=[2])
    a, cnt = oracle.partition(n, world)[2]
    assert np.array_equal(got[2], world * oracle.bf16_bits_to_f64(same[0][a:a + cnt]))
    assert list(got) == [2]


def test_gather_rows_inverts_numpy_split():
    rng = np.random.default_rng(170)
    for world in (1, 2, 3, 5, 8):
        for n in (world, 17, 64, 1001):
            if n < world:
                continue
            x = rng.integers(0, 0x7F00, size=(n, 8), dtype=np.uint16)    # never the 0xFFFF padding rows
            assert np.array_equal(oracle.gather_rows(np.array_split(x, world)), x), (world, n)


def _free_port():
    import socket
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _gloo_worker(rank, world, port, tmp):
    import torch.distributed as dist
    dist.init_process_group("gloo", init_method=f"tcp://127.0.0.1:{port}", rank=rank, world_size=world)
    n, c = 101, 8
    # the reduce-scatter of this rank's fp64 partial, rows split by torch.tensor_split
    part = torch.from_numpy(oracle.bf16_bits_to_f64(normal_bf16_bits((n, c), seed=180 + rank)))
    chunks = list(torch.tensor_split(part, world))
    out = torch.empty_like(chunks[rank])
    dist.reduce_scatter(out, chunks)
    np.save(os.path.join(tmp, f"rs{rank}.npy"), out.numpy())
    # the padded all-gather of this rank's token shard, then the padding stripped
    x = torch.from_numpy(normal_bf16_bits((n, c), seed=190).astype(np.int32))
    shard = torch.tensor_split(x, world)[rank]
    m = -(-n // world)
    padded = torch.cat([shard, torch.full((m - shard.shape[0], c), -1, dtype=torch.int32)])
    blocks = [torch.empty_like(padded) for _ in range(world)]
    dist.all_gather(blocks, padded)
    sizes = [t.shape[0] for t in torch.tensor_split(x, world)]
    np.save(os.path.join(tmp, f"ag{rank}.npy"), torch.cat([b[:s] for b, s in zip(blocks, sizes)]).numpy())
    dist.destroy_process_group()


def test_reduce_scatter_and_gather_match_gloo_collectives(tmp_path):
    """Three gloo processes on the CPU: torch.distributed's ragged
    reduce_scatter and padded all_gather give what the oracle simulates."""
    import torch.multiprocessing as mp
    world, n, c = 3, 101, 8
    mp.spawn(_gloo_worker, args=(world, _free_port(), str(tmp_path)), nprocs=world)
    parts = [normal_bf16_bits((n, c), seed=180 + j) for j in range(world)]
    ref = oracle.reduce_scatter(parts, None)
    x = normal_bf16_bits((n, c), seed=190)
    shards = [x[a:a + cnt] for a, cnt in oracle.partition(n, world)]
    for i in range(world):
        np.testing.assert_allclose(np.load(tmp_path / f"rs{i}.npy"), ref[i], rtol=0, atol=1e-12)
        assert np.array_equal(np.load(tmp_path / f"ag{i}.npy"), oracle.gather_rows(shards).astype(np.int32))
