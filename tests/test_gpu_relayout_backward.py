"""GPU parity of the relayout adjoints (the backward of seq2head and head2seq):
bit for bit against the oracle's backward exchange, with the forward's plan."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS
from synth.inputs import normal_bf16_bits
from tests.gpu_util import say, to_bits, to_device

pytestmark = pytest.mark.gpu


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _plan(info):
    return (info.launches, info.chunks, info.chunk_tokens, info.grid_x, info.block_x, info.max_launch_src_bytes,
            info.bytes_read, info.bytes_written)


@pytest.mark.parametrize("n,k,world", [(1, 3, 1), (7, 3, 2), (37, 4, 6), (300, 3, 8), (1000, 4, 7)])
@pytest.mark.parametrize("rank", [-1, "last"])
@pytest.mark.parametrize("chunk_rows", [0, 5])
def test_seq2head_backward_small(n, k, world, rank, chunk_rows):
    h3 = _h3()
    if n < world:
        pytest.skip("empty token partition")
    rank = world - 1 if rank == "last" else rank
    say("seq2head backward", n, k, world, rank, chunk_rows)
    heads = h3.head_split(56, world)
    ranks = list(range(world)) if rank < 0 else [rank]
    gbits = {(j, p): normal_bf16_bits((n, heads[j][1], 128), seed=500 + 13 * j + p + n) for j in ranks for p in range(k)}
    gdst = [[to_device(gbits[(j, p)]) for p in range(k)] if j in ranks else None for j in range(world)]
    sentinel = normal_bf16_bits((n, k, 56, 128), seed=599)
    gsrc = to_device(sentinel)
    chunk = chunk_rows * 56 * 128 * 2
    info = h3.seq2head_backward(gdst, gsrc, world, rank=rank, max_chunk_bytes=chunk)
    # the forward call of the same layout, for its plan
    fwd_dst = [[torch.empty((n, heads[j][1], 128), dtype=torch.bfloat16, device="cuda") for _ in range(k)]
               if j in ranks else None for j in range(world)]
    fwd = h3.seq2head(to_device(sentinel), fwd_dst, world, rank=rank, max_chunk_bytes=chunk)
    torch.cuda.synchronize()
    ref = oracle.seq2head_backward(gbits, n, k, 56, world, ranks=ranks, out=sentinel)
    assert np.array_equal(to_bits(gsrc), ref)
    assert _plan(info) == _plan(fwd)


@pytest.mark.parametrize("n,world", [(1, 1), (9, 2), (37, 6), (300, 8), (1000, 4)])
@pytest.mark.parametrize("rank", [-1, 0])
def test_head2seq_backward_small(n, world, rank):
    h3 = _h3()
    say("head2seq backward", n, world, rank)
    heads = h3.head_split(56, world)
    ranks = list(range(world)) if rank < 0 else [rank]
    gbits = normal_bf16_bits((n, 56, 128), seed=600 + n + world)
    gsrc = [torch.full((n, c, 128), 3.0, dtype=torch.bfloat16, device="cuda") for _, c in heads]
    chunk = 3 * 56 * 128 * 2 if n > 8 else 0
    info = h3.head2seq_backward(to_device(gbits), gsrc, world, rank=rank, max_chunk_bytes=chunk)
    fwd = h3.head2seq(gsrc, torch.empty((n, 56, 128), dtype=torch.bfloat16, device="cuda"), world, rank=rank,
                      max_chunk_bytes=chunk)
    torch.cuda.synchronize()
    ref = oracle.head2seq_backward(gbits, world, ranks=ranks)
    three = np.full(1, 3.0, np.float32).view(np.uint32)[0] >> 16
    for j in range(world):
        got = to_bits(gsrc[j])
        if j in ranks:
            assert np.array_equal(got, ref[j]), j
        else:
            assert (got == three).all(), j
    assert _plan(info) == _plan(fwd)


@pytest.mark.parametrize("world", [1, 4, 8])
def test_backward_undoes_forward(world):
    """seq2head_backward(seq2head(x)) == x and head2seq_backward(head2seq(b)) == b on the device."""
    h3 = _h3()
    n, k = 999, 4
    say("backward undoes forward", world)
    src_bits = normal_bf16_bits((n, k, 56, 128), seed=700 + world)
    heads = h3.head_split(56, world)
    bufs = [[torch.empty((n, c, 128), dtype=torch.bfloat16, device="cuda") for _ in range(k)] for _, c in heads]
    h3.seq2head(to_device(src_bits), bufs, world)
    back = torch.zeros((n, k, 56, 128), dtype=torch.bfloat16, device="cuda")
    h3.seq2head_backward(bufs, back, world)
    out = torch.empty((n, 56, 128), dtype=torch.bfloat16, device="cuda")
    h3.head2seq([b[1] for b in bufs], out, world)
    again = [torch.empty_like(b[1]) for b in bufs]
    h3.head2seq_backward(out, again, world)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(back), src_bits)
    for j in range(world):
        assert torch.equal(again[j].view(torch.int16), bufs[j][1].view(torch.int16))


@pytest.mark.parametrize("name", ["128k_p4_qkvg", "250k_p8_qkvg"])
def test_seq2head_backward_workload_rank_share(name):
    """The backward of one rank's share at full size, in the forward's bounded chunks."""
    h3 = _h3()
    w = WORKLOADS[name]
    j = w.relayout_rank
    say("seq2head backward workload", name, j)
    heads = h3.head_split(56, w.world)
    gbits = {(j, p): normal_bf16_bits((w.n_tokens, heads[j][1], 128), seed=w.seed + 40 + p) for p in range(w.planes)}
    gdst = [None] * w.world
    gdst[j] = [to_device(gbits[(j, p)]) for p in range(w.planes)]
    gsrc = torch.zeros((w.n_tokens, w.planes, 56, 128), dtype=torch.bfloat16, device="cuda")
    info = h3.seq2head_backward(gdst, gsrc, w.world, rank=j, max_chunk_bytes=w.max_chunk_bytes)
    torch.cuda.synchronize()
    if w.max_chunk_bytes:
        assert info.max_launch_src_bytes <= w.max_chunk_bytes
    got = to_bits(gsrc)
    hb, hn = heads[j]
    for p in range(w.planes):
        assert np.array_equal(got[:, p, hb:hb + hn], gbits[(j, p)]), p
    mask = np.ones(56, bool)
    mask[hb:hb + hn] = False
    assert not got[:, :, mask].any()
