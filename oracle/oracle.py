"""Plain CPU reference for the Ulysses H3 hot path.

TEST INFRASTRUCTURE ONLY.  This module, and the C file beside it, may be used
by ``tests/``, by ``__graft_entry__.smoke()`` and by the CPU-baseline leg of
``bench.py``.  The product library never imports, links or runs it, and it
imports nothing from the product package: the two share no code.

Every function here is the plain definition of one step of the method, written
for a reader to check against the pages by eye:

* ``partition``      -- balanced quotient/remainder split of heads or tokens
                        ("Distributed H3 Execution", Partition Contract: the
                        head-ownership table and the sentence that token ranges
                        use the same rule; empty parts are rejected, per the
                        same page's introduction).
* ``clip_segments``  -- segment boundaries clipped to a rank's token interval
                        and rebased (same page, Partition Contract).
* ``seq2head`` / ``head2seq`` -- the Ulysses all-to-all pair, simulated rank
                        by rank as the exchange of messages it is ("Distributed
                        H3 Execution", introduction: QKV sequence-to-head
                        all-to-all and its inverse around attention; "[perf]
                        Harden Ulysses agreement and tune bounded H3
                        transfers", Problem and behavior: one operand plane at
                        a time, outputs in storage of their own).
* ``seq2head_backward`` / ``head2seq_backward`` -- the same exchanges run
                        backwards: each message's gradient returns along its
                        edge ("[perf] Harden Ulysses ...", Problem and behavior:
                        backward reuses the forward's plan; Review and
                        validation: exact gradients).
* ``attention_rows`` -- segment-masked softmax attention in fp64 (C, threads).
* ``attention_backward`` -- its gradients (dq, dk, dv, dg) and log-sum-exp by
                        the chain rule of softmax attention, in fp64 (C).
* ``attention_dense`` -- the same result reached a second way: one dense
                        N x N logit matrix with -inf off the segment blocks.
* ``adaln_rows``     -- per-segment AdaLN modulation / residual gating in fp64.

Bit patterns of bfloat16 travel as ``numpy.uint16``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "h3_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


# ---------------------------------------------------------------------------
# build / load of the C part (plain gcc, no GPU toolchain)
# ---------------------------------------------------------------------------

def build(force: bool = False) -> str:
    """Compile ``h3_oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.h3o_attn_rows.restype = ctypes.c_int
        lib.h3o_attn_rows.argtypes = [ctypes.c_void_p] * 4 + [
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i64p, ctypes.c_int32, ctypes.c_double,
            i64p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32]
        bwd_args = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i64p, ctypes.c_int32,
                                            ctypes.c_double, i64p, ctypes.c_int64] + [ctypes.c_void_p] * 4 + [
                                            ctypes.c_int32]
        lib.h3o_attn_bwd_rows.restype = ctypes.c_int
        lib.h3o_attn_bwd_rows.argtypes = bwd_args
        lib.h3o_attn_bwd_keys.restype = ctypes.c_int
        lib.h3o_attn_bwd_keys.argtypes = bwd_args
        lib.h3o_adaln_rows.restype = ctypes.c_int
        lib.h3o_adaln_rows.argtypes = [ctypes.c_int32] + [ctypes.c_void_p] * 5 + [
            ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), i64p, i64p,
            ctypes.c_int32, ctypes.c_double, i64p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ---------------------------------------------------------------------------
# partition and clipping (integer work, pure Python)
# ---------------------------------------------------------------------------

class EmptyPartition(ValueError):
    """A split that would leave some rank without heads or tokens."""


def partition(total: int, parts: int) -> List[Tuple[int, int]]:
    """Balanced quotient/remainder split of ``total`` items over ``parts`` ranks.

    "Distributed H3 Execution", Partition Contract: head ownership is balanced
    and may be ragged (56 heads over 6 ranks gives 10,10,9,9,9,9, so the extra
    items go to the FIRST ranks), and token ranges follow the same rule.  The
    introduction of that page says empty token or head partitions are rejected.

    Returns ``[(begin, count), ...]`` for ranks 0..parts-1.
    """
    if parts < 1 or total < parts:
        raise EmptyPartition(f"cannot split {total} items over {parts} ranks without an empty part; "
                             f"legal rank counts are 1..{total}")
    q, r = divmod(total, parts)
    out = []
    begin = 0
    for i in range(parts):
        count = q + (1 if i < r else 0)
        out.append((begin, count))
        begin += count
    return out


def clip_segments(cu: Sequence[int], a: int, b: int) -> List[Tuple[int, int, int]]:
    """Clip the global segment table to the token interval ``[a, b)`` and rebase it.

    "Distributed H3 Execution", Partition Contract (the table a token-sharded
    rank's AdaLN ops use): local row ``i`` is global token ``a + i``, and each
    segment is intersected with ``[a, b)`` and shifted by ``-a``.  ``cu``
    holds the global offsets ``cu[0]=0 < ... <
    cu[S]=N``.  Returns ``(s, lo - a, hi - a)`` for every global segment ``s``
    whose clipped part ``[lo, hi) = [max(cu[s], a), min(cu[s+1], b))`` is not
    empty; ``s`` stays the GLOBAL segment id.
    """
    out = []
    for s in range(len(cu) - 1):
        lo = max(int(cu[s]), a)
        hi = min(int(cu[s + 1]), b)
        if lo < hi:
            out.append((s, lo - a, hi - a))
    return out


# ---------------------------------------------------------------------------
# relayouts: the all-to-all exchange, simulated rank by rank
# ---------------------------------------------------------------------------

def seq2head(src: np.ndarray, world: int, planes: Optional[Sequence[int]] = None,
             ranks: Optional[Sequence[int]] = None) -> dict:
    """Sequence-to-head all-to-all of a packed ``[N, K, H, D]`` operand.

    Before the exchange, rank ``i`` holds the tokens ``[a_i, b_i)`` of every
    head; afterwards rank ``j`` holds every token of its own heads
    ``[hb_j, hb_j + H_j)`` ("Distributed H3 Execution", introduction and
    Partition Contract).  For each plane, one at a time ("[perf] Harden Ulysses
    agreement ...", Problem and behavior), rank ``i`` sends rank ``j`` the
    message ``src[a_i:b_i, p, hb_j:hb_j+H_j, :]`` and rank ``j`` lays the
    received messages end to end in source-rank order, which gives a buffer
    ``[N, H_j, D]`` in global token order.

    Returns ``{(j, p): array [N, H_j, D]}``, each in storage of its own.
    """
    n, k, h, d = src.shape
    tokens = partition(n, world)
    heads = partition(h, world)
    planes = range(k) if planes is None else planes
    ranks = range(world) if ranks is None else ranks
    out = {}
    for p in planes:
        for j in ranks:
            hb, hn = heads[j]
            messages = []
            for i in range(world):
                a, cnt = tokens[i]
                messages.append(src[a:a + cnt, p, hb:hb + hn, :])
            out[(j, p)] = np.concatenate(messages, axis=0)
    return out


def head2seq(bufs: Sequence[np.ndarray], n_heads: int) -> np.ndarray:
    """Head-to-sequence all-to-all, the inverse exchange.

    Rank ``j`` holds ``bufs[j]`` = ``[N, H_j, D]`` (every token, its heads).
    It sends rank ``i`` the rows of rank ``i``'s tokens; rank ``i`` places the
    message from ``j`` at heads ``[hb_j, hb_j+H_j)`` of its token rows.  The
    token shards of all ranks, stacked in order, form the returned
    ``[N, H, D]`` array.
    """
    world = len(bufs)
    n, _, d = bufs[0].shape
    tokens = partition(n, world)
    heads = partition(n_heads, world)
    shards = []
    for i in range(world):
        a, cnt = tokens[i]
        shard = np.empty((cnt, n_heads, d), dtype=bufs[0].dtype)
        for j in range(world):
            hb, hn = heads[j]
            if bufs[j].shape != (n, hn, d):
                raise ValueError(f"rank {j} buffer has shape {bufs[j].shape}, expected {(n, hn, d)}")
            shard[:, hb:hb + hn, :] = bufs[j][a:a + cnt]
        shards.append(shard)
    return np.concatenate(shards, axis=0)


def seq2head_backward(grads: dict, n_tokens: int, n_planes: int, n_heads: int, world: int,
                      ranks: Optional[Sequence[int]] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Backward of ``seq2head``: every message's gradient travels back along its edge.

    In the forward exchange rank ``i`` sent rank ``j`` the message
    ``src[a_i:b_i, p, hb_j:hb_j+H_j, :]`` and rank ``j`` stacked the messages in
    source-rank order.  The backward pass ("[perf] Harden Ulysses agreement
    ...", Problem and behavior: backward reuses the plan of its forward; Review
    and validation: exact gradients) therefore cuts rank ``j``'s gradient
    ``grads[(j, p)]`` (``[N, H_j, D]``) back into the same messages and rank
    ``i`` writes each one where its forward message came from.

    Returns the ``[N, K, H, D]`` gradient of the packed operand.  Heads of ranks
    outside ``ranks`` keep the values of ``out`` (zeros when ``out`` is None).
    """
    d = next(iter(grads.values())).shape[2]
    tokens = partition(n_tokens, world)
    heads = partition(n_heads, world)
    ranks = range(world) if ranks is None else ranks
    res = (np.zeros((n_tokens, n_planes, n_heads, d), dtype=next(iter(grads.values())).dtype)
           if out is None else np.array(out, copy=True))
    for p in range(n_planes):
        for j in ranks:
            hb, hn = heads[j]
            g = grads[(j, p)]
            if g.shape != (n_tokens, hn, d):
                raise ValueError(f"gradient of rank {j}, plane {p} has shape {g.shape}, expected {(n_tokens, hn, d)}")
            for i in range(world):
                a, cnt = tokens[i]
                res[a:a + cnt, p, hb:hb + hn, :] = g[a:a + cnt]
    return res


def head2seq_backward(grad: np.ndarray, world: int, ranks: Optional[Sequence[int]] = None) -> dict:
    """Backward of ``head2seq``: rank ``i`` sends rank ``j`` the gradient of the
    rows it received from ``j`` -- heads ``[hb_j, hb_j+H_j)`` of its own token
    shard -- and rank ``j`` stacks them in rank order.  Returns ``{j: [N, H_j, D]}``.
    """
    n, n_heads, d = grad.shape
    tokens = partition(n, world)
    heads = partition(n_heads, world)
    ranks = range(world) if ranks is None else ranks
    res = {}
    for j in ranks:
        hb, hn = heads[j]
        res[j] = np.concatenate([grad[a:a + cnt, hb:hb + hn, :] for a, cnt in tokens], axis=0)
    return res


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# ragged collectives of the token-sharded blocks, simulated rank by rank
# ---------------------------------------------------------------------------

def reduce_scatter(partials: Sequence[np.ndarray], bias: Optional[np.ndarray] = None,
                   ranks: Optional[Sequence[int]] = None) -> dict:
    """Ragged reduce-scatter of per-rank partial outputs, bias added once.

    "Distributed H3 Execution", Partition Contract (tensor mode): every rank
    computes a partial output for all token rows, a ragged reduce-scatter sums
    the partials and hands each rank the rows of its own token interval
    (quotient/remainder split), and the projection bias, left out of the
    partials, is added exactly once after the reduction.  Simulated message by
    message: rank ``j`` sends rank ``i`` its partial rows ``[a_i, b_i)``; rank
    ``i`` adds the messages in source-rank order, then the bias.

    ``partials``: P arrays ``[N, C]`` of bf16 bits (or floats); ``bias``:
    ``[C]`` bf16 bits or None.  Returns ``{i: fp64 [N_i, C]}``.
    """
    world = len(partials)
    n, c = partials[0].shape
    for j, a in enumerate(partials):
        if a.shape != (n, c):
            raise ValueError(f"partial {j} has shape {a.shape}, expected {(n, c)}")
    if bias is not None and bias.shape != (c,):
        raise ValueError(f"bias has shape {bias.shape}, expected {(c,)}")
    tokens = partition(n, world)
    wide = lambda a: bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)  # noqa: E731
    out = {}
    for i in (range(world) if ranks is None else ranks):
        a, cnt = tokens[i]
        acc = np.zeros((cnt, c), np.float64)
        for j in range(world):                      # the message from rank j
            acc += wide(partials[j][a:a + cnt])
        if bias is not None:
            acc += wide(bias)[None, :]              # once, after the reduction
        out[i] = acc
    return out


def gather_rows(shards: Sequence[np.ndarray], pad_value: int = 0xFFFF) -> np.ndarray:
    """Ragged row gather with the collective's temporary padding removed.

    "Distributed H3 Execution", introduction: the collective that gathers the
    ragged token shards pads them to a common size, and that padding is
    removed before any model operation.  Simulated literally: every rank pads
    its ``[N_i, C]`` rows to ``M = max N_i`` with ``pad_value`` rows, the
    gather lays the P padded blocks end to end (``[P * M, C]``), and the first
    ``N_i`` rows of block ``i`` are kept.  Returns ``[sum N_i, C]``.
    """
    world = len(shards)
    c = shards[0].shape[1]
    m = max(a.shape[0] for a in shards)
    blocks = []
    for a in shards:
        pad = np.full((m - a.shape[0], c), pad_value, dtype=a.dtype)
        blocks.append(np.concatenate([a, pad], axis=0))
    gathered = np.concatenate(blocks, axis=0)
    keep = [i * m + r for i in range(world) for r in range(shards[i].shape[0])]
    return gathered[keep]


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bfloat16 operands travel as uint16 bit patterns")
    return a


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: Optional[np.ndarray],
                   cu: Sequence[int], scale: float, rows: Optional[Sequence[int]] = None,
                   threads: Optional[int] = None) -> np.ndarray:
    """Segment-masked attention of the given query rows, fp64 (see h3_oracle.c).

    ``q, k, v, g``: bf16 bits ``[N, H, D]``; ``g`` may be None (no gate).
    Returns fp64 ``[len(rows), H, D]``; ``rows`` defaults to every token.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    g = None if g is None else _u16(g)
    n, h, d = q.shape
    for a in (k, v) + ((g,) if g is not None else ()):
        if a.shape != (n, h, d):
            raise ValueError("q, k, v, g must share one [N, H, D] shape")
    rows = _i64(np.arange(n) if rows is None else rows)
    cu = _i64(cu)
    out = np.empty((rows.shape[0], h, d), dtype=np.float64)
    lib = _load()
    rc = lib.h3o_attn_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                           None if g is None else g.ctypes.data,
                           n, h, d, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(cu) - 1,
                           float(scale), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                           rows.shape[0], out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"h3o_attn_rows failed with {rc}")
    return out


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: Optional[np.ndarray], dout: np.ndarray,
                       cu: Sequence[int], scale: float, q_rows: Optional[Sequence[int]] = None,
                       k_rows: Optional[Sequence[int]] = None, threads: Optional[int] = None) -> dict:
    """Gradients of ``attention_rows`` for the incoming output gradient ``dout``, fp64 (see h3_oracle.c).

    The chain rule of softmax attention, term by term: for query rows, the
    log-sum-exp ``lse``, ``delta`` = <do * sig(g), a> and the gradients
    ``dq`` and ``dg`` (``dg`` only when ``g`` is given); for key rows, ``dk``
    and ``dv``, which need ``lse`` and ``delta`` of every query of their
    segment (computed here over those segments first).  Row lists default to
    every token.  Returns a dict of fp64 arrays ``[rows, H, D]`` (``[rows, H]``
    for ``lse`` and ``delta``).
    """
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    g = None if g is None else _u16(g)
    n, h, d = q.shape
    for a in (k, v, dout) + ((g,) if g is not None else ()):
        if a.shape != (n, h, d):
            raise ValueError("q, k, v, g, dout must share one [N, H, D] shape")
    cu = _i64(cu)
    lib = _load()
    nt = threads or default_threads()
    i64p = ctypes.POINTER(ctypes.c_int64)
    gp = None if g is None else g.ctypes.data

    def row_pass(rows, gradients=True):
        rows = _i64(rows)
        lse = np.empty((rows.shape[0], h), np.float64)
        delta = np.empty((rows.shape[0], h), np.float64)
        dq = np.empty((rows.shape[0], h, d), np.float64) if gradients else None
        dg = np.empty((rows.shape[0], h, d), np.float64) if g is not None and gradients else None
        rc = lib.h3o_attn_bwd_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, gp, dout.ctypes.data, n, h, d,
                                   cu.ctypes.data_as(i64p), len(cu) - 1, float(scale), rows.ctypes.data_as(i64p),
                                   rows.shape[0], lse.ctypes.data, delta.ctypes.data,
                                   None if dq is None else dq.ctypes.data, None if dg is None else dg.ctypes.data, nt)
        if rc != 0:
            raise ValueError(f"h3o_attn_bwd_rows failed with {rc}")
        return lse, delta, dq, dg

    out = {}
    q_rows = np.arange(n) if q_rows is None else np.asarray(q_rows)
    out["lse"], out["delta"], out["dq"], dg = row_pass(q_rows)
    if dg is not None:
        out["dg"] = dg
    k_rows = np.arange(n) if k_rows is None else np.asarray(k_rows)
    if len(k_rows):
        # lse and delta of every query of the segments the key rows fall in
        seg = np.searchsorted(cu, k_rows, side="right") - 1
        need = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in np.unique(seg)])
        lse_all = np.zeros((n, h), np.float64)
        delta_all = np.zeros((n, h), np.float64)
        have = np.zeros(n, bool)
        have[q_rows] = True
        if have[need].all():            # the query-side pass above already covers them
            lse_all[q_rows], delta_all[q_rows] = out["lse"], out["delta"]
        else:
            lse_n, delta_n, _, _ = row_pass(need, gradients=False)
            lse_all[need], delta_all[need] = lse_n, delta_n
        kr = _i64(k_rows)
        dk = np.empty((kr.shape[0], h, d), np.float64)
        dv = np.empty((kr.shape[0], h, d), np.float64)
        rc = lib.h3o_attn_bwd_keys(q.ctypes.data, k.ctypes.data, v.ctypes.data, gp, dout.ctypes.data, n, h, d,
                                   cu.ctypes.data_as(i64p), len(cu) - 1, float(scale), kr.ctypes.data_as(i64p),
                                   kr.shape[0], lse_all.ctypes.data, delta_all.ctypes.data, dk.ctypes.data,
                                   dv.ctypes.data, nt)
        if rc != 0:
            raise ValueError(f"h3o_attn_bwd_keys failed with {rc}")
        out["dk"], out["dv"] = dk, dv
    return out


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: Optional[np.ndarray],
                    cu: Sequence[int], scale: float) -> np.ndarray:
    """The same attention reached by brute force, for small N only.

    One dense ``N x N`` logit matrix per head, ``-inf`` wherever query and key
    lie in different segments, a row softmax over all N columns, then the
    product with V.  It takes no per-segment loop, so it checks the segment
    bookkeeping of :func:`attention_rows` from outside.
    """
    qf, kf, vf = (bf16_bits_to_f64(a) for a in (q, k, v))
    n, h, d = qf.shape
    seg = np.empty(n, dtype=np.int64)
    for s in range(len(cu) - 1):
        seg[cu[s]:cu[s + 1]] = s
    mask = seg[:, None] == seg[None, :]
    out = np.empty((n, h, d), dtype=np.float64)
    for hh in range(h):
        logits = scale * (qf[:, hh, :] @ kf[:, hh, :].T)
        logits = np.where(mask, logits, -np.inf)
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        out[:, hh, :] = w @ vf[:, hh, :]
    if g is not None:
        out *= 1.0 / (1.0 + np.exp(-bf16_bits_to_f64(g)))
    return out


# ---------------------------------------------------------------------------
# AdaLN
# ---------------------------------------------------------------------------

MODULATE = 0
GATE_RESIDUAL = 1
GATE_MODULATE = 2          # the gated residual, modulated by the next sub-block's parameters


def adaln_rows(mode: int, x: np.ndarray, b: Optional[np.ndarray], shift: Optional[np.ndarray],
               scale: Optional[np.ndarray], gate: Optional[np.ndarray], tok_begin: int, tok_end: int,
               cu: Sequence[int], eps: float, rows: Optional[Sequence[int]] = None,
               threads: Optional[int] = None) -> np.ndarray:
    """Per-segment AdaLN on the local rows of token interval ``[tok_begin, tok_end)``.

    The global segment table ``cu`` is first clipped and rebased to the
    interval with :func:`clip_segments`, exactly as the Partition Contract of
    "Distributed H3 Execution" orders; each local row then takes the
    parameters of its GLOBAL segment.  ``x`` (and ``b``) are ``[tok_end -
    tok_begin, C]`` bf16 bits; parameters are ``[S, C]``.  Returns fp64
    ``[len(rows), C]``.
    """
    x = _u16(x)
    n_local, c = x.shape
    if n_local != tok_end - tok_begin:
        raise ValueError("x must hold exactly the rows of the token interval")
    table = clip_segments(cu, tok_begin, tok_end)
    seg_id = np.ascontiguousarray([t[0] for t in table], dtype=np.int32)
    lb = _i64([t[1] for t in table])
    le = _i64([t[2] for t in table])
    rows = _i64(np.arange(n_local) if rows is None else rows)
    out = np.empty((rows.shape[0], c), dtype=np.float64)
    # contiguous copies stay referenced by these names until the call returns
    bb, sh, sc, gt = (None if a is None else _u16(a) for a in (b, shift, scale, gate))
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    lib = _load()
    rc = lib.h3o_adaln_rows(int(mode), x.ctypes.data, ptr(bb), ptr(sh), ptr(sc), ptr(gt),
                            n_local, c, seg_id.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            lb.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                            le.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(table), float(eps),
                            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.shape[0],
                            out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"h3o_adaln_rows failed with {rc}")
    return out


def adaln_gate_modulate(x: np.ndarray, b: np.ndarray, gate: np.ndarray, shift: np.ndarray, scale: np.ndarray,
                        tok_begin: int, tok_end: int, cu: Sequence[int], eps: float,
                        rows: Optional[Sequence[int]] = None, threads: Optional[int] = None):
    """Residual gating of one sub-block followed by the next sub-block's
    modulation, on the local rows of ``[tok_begin, tok_end)``.

    Returns ``(resid, y)``: ``resid = x + gate_s * b`` (mode GATE_RESIDUAL) and
    ``y`` = LayerNorm(resid) * (1 + scale_s) + shift_s (mode GATE_MODULATE),
    both fp64, with the clipped table of :func:`adaln_rows`.
    """
    resid = adaln_rows(GATE_RESIDUAL, x, b, None, None, gate, tok_begin, tok_end, cu, eps, rows, threads)
    y = adaln_rows(GATE_MODULATE, x, b, shift, scale, gate, tok_begin, tok_end, cu, eps, rows, threads)
    return resid, y


def attention_flops(cu: Sequence[int], n_heads: int, head_dim: int) -> int:
    """Algorithmic FLOPs of segment-masked attention: two products of 2*D per pair."""
    return 4 * head_dim * n_heads * sum((int(cu[s + 1]) - int(cu[s])) ** 2 for s in range(len(cu) - 1))


__all__ = ["build", "partition", "clip_segments", "seq2head", "head2seq", "seq2head_backward",
           "head2seq_backward", "attention_rows", "attention_backward",
           "attention_dense", "adaln_rows", "adaln_gate_modulate", "reduce_scatter", "gather_rows",
           "bf16_bits_to_f64", "EmptyPartition", "MODULATE", "GATE_RESIDUAL", "GATE_MODULATE",
           "default_threads", "attention_flops"]
