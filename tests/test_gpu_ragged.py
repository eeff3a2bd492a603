"""GPU parity of the ragged reduce-scatter (bias added once) and of the ragged
row gather against the oracle's message-by-message simulation."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS
from synth.inputs import normal_bf16, normal_bf16_bits
from tests.gpu_util import bits_to_f64, compare, say, to_bits, to_device

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FC1          # a NaN bit pattern no kernel output has


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _check_sum(got_bits, ref, what):
    """A sum of P partials grows like sqrt(P), past the range where a fixed
    max-abs bar means anything for bf16, so each element is held to its
    rounding: the fp32 sum s rounded to nearest bf16 is within half an ulp of
    s, at most 2^-8 |s|, and s is within P 2^-24 sum|terms| (< 2e-5 for these
    inputs) of the exact value; 1e-4 covers that term."""
    got = bits_to_f64(got_bits)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4
    compare(got_bits, ref, what, atol=float(bound.max()))
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"{what}: worst error {worst:.3f} of the rounding bound")
    assert (err <= bound).all(), f"{what}: an element is off by more than its rounding"


def _outputs(n, c, world):
    h3 = _h3()
    return [torch.full((h3.partition(n, world, i)[1], c), SENTINEL, dtype=torch.int16, device="cuda")
            .view(torch.bfloat16) for i in range(world)]


@pytest.mark.parametrize("world,n,c", [(1, 5, 8), (2, 1003, 64), (3, 1003, 8), (6, 4099, 1000), (8, 777, 7168),
                                       (4, 131, 7168), (56, 1000, 16)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_reduce_scatter_ragged(world, n, c, with_bias):
    h3 = _h3()
    say("reduce-scatter", world, n, c, with_bias)
    parts = [normal_bf16_bits((n, c), seed=1300 + j + n) for j in range(world)]
    bias = normal_bf16_bits((c,), seed=1299) if with_bias else None
    out = _outputs(n, c, world)
    info = h3.reduce_scatter([to_device(p) for p in parts], None if bias is None else to_device(bias), out)
    torch.cuda.synchronize()
    ref = oracle.reduce_scatter(parts, bias)
    for i in range(world):
        _check_sum(to_bits(out[i]), ref[i], f"reduce-scatter P={world} N={n} C={c} rank {i}")
    assert info.launches == 1
    assert info.bytes_written == n * c * 2
    assert info.bytes_read == world * n * c * 2 + (c * 2 if with_bias else 0)


def test_reduce_scatter_one_rank_only_writes_its_rows():
    h3 = _h3()
    n, c, world = 1003, 64, 4
    parts = [normal_bf16_bits((n, c), seed=1350 + j) for j in range(world)]
    bias = normal_bf16_bits((c,), seed=1349)
    out = _outputs(n, c, world)
    h3.reduce_scatter([to_device(p) for p in parts], to_device(bias), out, rank=2)
    torch.cuda.synchronize()
    ref = oracle.reduce_scatter(parts, bias, ranks=[2])
    _check_sum(to_bits(out[2]), ref[2], "reduce-scatter rank 2 only")
    for i in (0, 1, 3):
        assert (to_bits(out[i]) == SENTINEL).all(), i


def test_reduce_scatter_exact_cases():
    """Zero partials give exactly the bias (added once, not P times); small
    integers sum exactly, so the result is bit-exact against the oracle."""
    h3 = _h3()
    n, c, world = 517, 7168, 5
    bias = normal_bf16_bits((c,), seed=1360)
    zeros = [torch.zeros((n, c), dtype=torch.bfloat16, device="cuda") for _ in range(world)]
    out = _outputs(n, c, world)
    h3.reduce_scatter(zeros, to_device(bias), out)
    torch.cuda.synchronize()
    for i in range(world):
        assert np.array_equal(to_bits(out[i]), np.broadcast_to(bias, out[i].shape)), i
    g = torch.Generator().manual_seed(1361)
    ints = [torch.randint(-20, 21, (n, c), generator=g).to(torch.bfloat16) for _ in range(world)]
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in ints]
    ib = torch.randint(-20, 21, (c,), generator=g).to(torch.bfloat16)
    out = _outputs(n, c, world)
    h3.reduce_scatter([t.cuda() for t in ints], ib.cuda(), out)
    torch.cuda.synchronize()
    ref = oracle.reduce_scatter(bits, ib.view(torch.int16).numpy().view(np.uint16))
    for i in range(world):
        assert np.array_equal(oracle.bf16_bits_to_f64(to_bits(out[i])), ref[i]), i


@pytest.mark.parametrize("name", ["128k_p4_qkvg", "250k_p8_qkvg"])
def test_reduce_scatter_workload(name):
    """P partials [N, 7168] at the workload's size, every rank: sampled rows
    against the oracle (the concatenation over ranks of a reduce-scatter is the
    full reduction plus bias, whatever the row split, so the oracle runs on the
    sampled rows alone)."""
    h3 = _h3()
    w = WORKLOADS[name]
    n, c = w.n_tokens, 7168
    say("reduce-scatter workload", name)
    parts = [normal_bf16((n, c), seed=w.seed + 40 + j, device="cuda") for j in range(w.world)]
    bias = normal_bf16((c,), seed=w.seed + 39, device="cuda")
    out = _outputs(n, c, w.world)
    info = h3.reduce_scatter(parts, bias, out)
    torch.cuda.synchronize()
    assert info.launches == 1
    rng = np.random.default_rng(w.seed + 41)
    for i in range(w.world):
        a, cnt = h3.partition(n, w.world, i)
        local = np.unique(np.concatenate([[0, cnt - 1], rng.integers(0, cnt, size=62)]))
        idx = torch.from_numpy(local + a).cuda()
        ref_parts = [to_bits(p.index_select(0, idx)) for p in parts]
        ref = oracle.reduce_scatter(ref_parts, to_bits(bias))
        ref_rows = np.concatenate([ref[j] for j in range(w.world)])
        _check_sum(to_bits(out[i].index_select(0, torch.from_numpy(local).cuda())), ref_rows,
                   f"{name} reduce-scatter rank {i}")
    del parts, out


@pytest.mark.parametrize("world,n,c", [(1, 7, 8), (2, 1003, 64), (3, 1003, 8), (6, 4099, 1000), (8, 777, 7168),
                                       (56, 1000, 16)])
def test_gather_rows_strips_padding(world, n, c):
    """Shards as the blocks of a padded [P, M, C] gathered buffer (pad rows
    hold a sentinel) and as separate buffers: both give the oracle's rows bit
    for bit, and no pad row reaches the output."""
    h3 = _h3()
    say("gather rows", world, n, c)
    x = normal_bf16_bits((n, c), seed=1400 + n)
    shards = [x[a:a + cnt] for a, cnt in oracle.partition(n, world)]
    ref = oracle.gather_rows(shards)
    m = max(s.shape[0] for s in shards)
    padded = np.full((world, m, c), SENTINEL, np.uint16)
    for i, s in enumerate(shards):
        padded[i, :s.shape[0]] = s
    pd = to_device(padded)
    dst = torch.empty((n, c), dtype=torch.bfloat16, device="cuda")
    info = h3.gather_rows([pd[i] for i in range(world)], dst)
    torch.cuda.synchronize()
    got = to_bits(dst)
    assert np.array_equal(got, ref)
    assert not (got == SENTINEL).any()
    assert info.launches == 1 and info.bytes_read == n * c * 2
    dst2 = torch.empty_like(dst)
    h3.gather_rows([to_device(s) for s in shards], dst2)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(dst2), ref)


@pytest.mark.parametrize("name", ["128k_p4_qkvg", "250k_p8_qkvg"])
def test_gather_rows_workload(name):
    """Padded blocks of [N_i, 7168] shards at the workload's size: every row equal
    to its shard row (a pure row permutation), sampled rows against the oracle."""
    h3 = _h3()
    w = WORKLOADS[name]
    n, c = w.n_tokens, 7168
    say("gather rows workload", name)
    parts = [h3.partition(n, w.world, i) for i in range(w.world)]
    m = max(cnt for _, cnt in parts)
    padded = torch.full((w.world, m, c), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    for i, (a, cnt) in enumerate(parts):
        padded[i, :cnt] = normal_bf16((cnt, c), seed=w.seed + 50 + i, device="cuda")
    dst = torch.empty((n, c), dtype=torch.bfloat16, device="cuda")
    h3.gather_rows([padded[i] for i in range(w.world)], dst)
    torch.cuda.synchronize()
    for i, (a, cnt) in enumerate(parts):
        assert torch.equal(dst[a:a + cnt].view(torch.int16), padded[i, :cnt].view(torch.int16)), i
    rng = np.random.default_rng(w.seed + 51)
    picks = [np.unique(np.concatenate([[0, cnt - 1], rng.integers(0, cnt, size=30)])) for _, cnt in parts]
    shards = [to_bits(padded[i].index_select(0, torch.from_numpy(p).cuda())) for i, p in enumerate(picks)]
    rows = np.concatenate([p + a for p, (a, _) in zip(picks, parts)])
    assert np.array_equal(to_bits(dst.index_select(0, torch.from_numpy(rows).cuda())), oracle.gather_rows(shards))
