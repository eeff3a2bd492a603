"""GPU parity of the relayouts: bit for bit against the oracle's simulated all-to-all."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS
from synth.inputs import normal_bf16, normal_bf16_bits
from tests.gpu_util import say, to_bits, to_device

pytestmark = pytest.mark.gpu


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _alloc_rank_bufs(n, heads, k, ranks):
    bufs = [None] * len(heads)
    for j in ranks:
        bufs[j] = [torch.empty((n, heads[j][1], 128), dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    return bufs


@pytest.mark.parametrize("n,k,world", [(1, 3, 1), (7, 3, 2), (37, 4, 6), (300, 3, 8), (513, 1, 4), (1000, 4, 7)])
@pytest.mark.parametrize("rank", [-1, "last"])
@pytest.mark.parametrize("chunk_rows", [0, 5])
def test_seq2head_small(n, k, world, rank, chunk_rows):
    h3 = _h3()
    if n < world:
        pytest.skip("empty token partition")
    rank = world - 1 if rank == "last" else rank
    say("seq2head small", n, k, world, rank, chunk_rows)
    src_bits = normal_bf16_bits((n, k, 56, 128), seed=100 + n + k + world)
    src = to_device(src_bits)
    heads = h3.head_split(56, world)
    ranks = range(world) if rank < 0 else [rank]
    bufs = _alloc_rank_bufs(n, heads, k, ranks)
    info = h3.seq2head(src, bufs, world, rank=rank, max_chunk_bytes=chunk_rows * 56 * 128 * 2)
    torch.cuda.synchronize()
    ref = oracle.seq2head(src_bits, world, ranks=list(ranks))
    for j in ranks:
        for p in range(k):
            assert np.array_equal(to_bits(bufs[j][p]), ref[(j, p)]), (j, p)
    # the cap bounds a launch's source bytes: per token it moves the selected ranks' heads
    sel_bytes = sum(heads[j][1] for j in ranks) * 128 * 2
    chunk_tok = n if chunk_rows == 0 else min(n, chunk_rows * 56 * 128 * 2 // sel_bytes)
    chunks = -(-n // chunk_tok)
    assert info.chunks == chunks and info.launches == k * chunks
    assert info.chunk_tokens == chunk_tok
    if chunk_rows:
        assert info.max_launch_src_bytes <= chunk_rows * 56 * 128 * 2
    assert np.array_equal(to_bits(src), src_bits)          # the source is untouched


@pytest.mark.parametrize("n,world", [(1, 1), (9, 2), (37, 6), (300, 8), (1000, 4)])
@pytest.mark.parametrize("rank", [-1, 0])
def test_head2seq_small(n, world, rank):
    h3 = _h3()
    say("head2seq small", n, world, rank)
    heads = h3.head_split(56, world)
    bits = [normal_bf16_bits((n, c, 128), seed=200 + 7 * j + n) for j, (_, c) in enumerate(heads)]
    src = [to_device(b) for b in bits]
    sentinel = normal_bf16_bits((n, 56, 128), seed=299)
    dst = to_device(sentinel)
    h3.head2seq(src, dst, world, rank=rank, max_chunk_bytes=(3 * 56 * 128 * 2 if n > 8 else 0))
    torch.cuda.synchronize()
    got = to_bits(dst)
    if rank < 0:
        assert np.array_equal(got, oracle.head2seq(bits, 56))
    else:
        # only the selected rank's heads change; the rest keep their previous contents
        hb, hn = heads[rank]
        ref = sentinel.copy()
        full = oracle.head2seq([bits[j] if j == rank else sentinel[:, heads[j][0]:heads[j][0] + heads[j][1]]
                                for j in range(world)], 56)
        ref[:, hb:hb + hn] = full[:, hb:hb + hn]
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("world", [1, 2, 4, 6, 8])
def test_round_trip_identity(world):
    """Transport identity: head2seq(seq2head(x)) == x bit for bit, plane by plane."""
    h3 = _h3()
    n, k = 777, 3
    say("round trip", world)
    src = normal_bf16((n, k, 56, 128), seed=300 + world, device="cuda")
    heads = h3.head_split(56, world)
    bufs = _alloc_rank_bufs(n, heads, k, range(world))
    h3.seq2head(src, bufs, world)
    for p in range(k):
        back = torch.empty((n, 56, 128), dtype=torch.bfloat16, device="cuda")
        h3.head2seq([bufs[j][p] for j in range(world)], back, world)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int16), src[:, p].contiguous().view(torch.int16))


def _workload_src(w):
    return normal_bf16((w.n_tokens, w.planes, 56, 128), seed=w.seed, device="cuda")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_seq2head_workload_full(name):
    """Every rank's buffers at the workload's real size, chunked as the workload says."""
    h3 = _h3()
    w = WORKLOADS[name]
    say("seq2head workload", name, "chunk bytes", w.max_chunk_bytes)
    src = _workload_src(w)
    heads = h3.head_split(56, w.world)
    bufs = _alloc_rank_bufs(w.n_tokens, heads, w.planes, range(w.world))
    info = h3.seq2head(src, bufs, w.world, max_chunk_bytes=w.max_chunk_bytes)
    torch.cuda.synchronize()
    if w.max_chunk_bytes:
        assert info.max_launch_src_bytes <= w.max_chunk_bytes
        assert info.launches == w.planes * info.chunks and info.chunks > 1
    src_bits = to_bits(src)
    for p in range(w.planes):
        ref = oracle.seq2head(src_bits, w.world, planes=[p])
        for j in range(w.world):
            assert np.array_equal(to_bits(bufs[j][p]), ref[(j, p)]), (name, j, p)
        del ref


def test_chunked_plan_and_negative_control():
    """The bounded-window plan at 250k: with the 896,000,000-byte cap no launch
    reads more than the window (every rank: 62,500-token chunks of whole
    planes; rank 0's 7-head share: one launch per plane, 448,000,000 bytes),
    and the same assertion fails for the uncapped every-rank plan.  All plans
    give identical bits."""
    h3 = _h3()
    w = WORKLOADS["250k_p8_qkvg"]
    say("chunk control 250k")
    src = _workload_src(w)
    heads = h3.head_split(56, w.world)
    window = 896_000_000
    chunked = _alloc_rank_bufs(w.n_tokens, heads, w.planes, range(w.world))
    info_c = h3.seq2head(src, chunked, w.world, max_chunk_bytes=window)
    torch.cuda.synchronize()
    assert info_c.chunk_tokens == 62500 and info_c.chunks == 4 and info_c.launches == 16
    assert info_c.max_launch_src_bytes == window
    whole = _alloc_rank_bufs(w.n_tokens, heads, w.planes, range(w.world))
    info_w = h3.seq2head(src, whole, w.world, max_chunk_bytes=0)
    torch.cuda.synchronize()
    assert info_w.chunks == 1 and info_w.max_launch_src_bytes > window     # negative control
    for j in range(w.world):
        for p in range(w.planes):
            assert torch.equal(chunked[j][p].view(torch.int16), whole[j][p].view(torch.int16)), (j, p)
    del whole
    share = _alloc_rank_bufs(w.n_tokens, heads, w.planes, [0])
    info_r = h3.seq2head(src, share, w.world, rank=0, max_chunk_bytes=window)
    torch.cuda.synchronize()
    assert info_r.chunks == 1 and info_r.launches == w.planes
    assert info_r.max_launch_src_bytes == w.n_tokens * heads[0][1] * 128 * 2 <= window
    for p in range(w.planes):
        assert torch.equal(share[0][p].view(torch.int16), chunked[0][p].view(torch.int16)), p


def test_rank_share_cap_of_one_token():
    """A cap of exactly one token of the selected rank's heads is legal and gives
    one-token launches with the same bits."""
    h3 = _h3()
    n, world, rank = 37, 6, 4
    say("one-token cap", n, world, rank)
    src_bits = normal_bf16_bits((n, 3, 56, 128), seed=71)
    src = to_device(src_bits)
    heads = h3.head_split(56, world)
    bufs = _alloc_rank_bufs(n, heads, 3, [rank])
    info = h3.seq2head(src, bufs, world, rank=rank, max_chunk_bytes=heads[rank][1] * 128 * 2)
    torch.cuda.synchronize()
    assert info.chunk_tokens == 1 and info.chunks == n and info.launches == 3 * n
    ref = oracle.seq2head(src_bits, world, ranks=[rank])
    for p in range(3):
        assert np.array_equal(to_bits(bufs[rank][p]), ref[(rank, p)]), p


@pytest.mark.parametrize("name", ["128k_p4_qkvg", "250k_p8_qkvg"])
def test_head2seq_workload_full(name):
    h3 = _h3()
    w = WORKLOADS[name]
    say("head2seq workload", name)
    heads = h3.head_split(56, w.world)
    src = [normal_bf16((w.n_tokens, c, 128), seed=w.seed + 50 + j, device="cuda") for j, (_, c) in enumerate(heads)]
    dst = torch.empty((w.n_tokens, 56, 128), dtype=torch.bfloat16, device="cuda")
    h3.head2seq(src, dst, w.world, max_chunk_bytes=w.max_chunk_bytes)
    torch.cuda.synchronize()
    ref = oracle.head2seq([to_bits(s) for s in src], 56)
    assert np.array_equal(to_bits(dst), ref)
