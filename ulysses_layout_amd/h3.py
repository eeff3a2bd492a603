"""ctypes binding of libh3.so -- argument marshalling only.

Every function here checks the torch tensors it is handed (device, dtype,
contiguity, shape), turns them into raw device pointers and calls the C entry
point of the same name on the current HIP stream.  All work of the hot path
runs in the library's HIP kernels; there is no fallback of any kind: if
libh3.so is missing or was built for another target, importing this module
fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
# H3_LIBRARY may name another build of the same library (e.g. the host-checking
# build of build_sanitized.py); by default the in-tree release build is used.
LIB_PATH = os.environ.get("H3_LIBRARY") or os.path.join(_PKG, "libh3.so")

H3_OK = 0
H3_ADALN_MODULATE = 0
H3_ADALN_GATE_RESIDUAL = 1
H3_ADALN_GATE_MODULATE = 2
HEAD_DIM = 128
NOALLOC_SCRATCH_BYTES = 64 << 20      # H3_NOALLOC_SCRATCH_BYTES
STATUS_NAMES = {0: "H3_OK", 1: "H3_ERR_ARG", 2: "H3_ERR_EMPTY_PARTITION", 3: "H3_ERR_SEGMENTS",
                4: "H3_ERR_UNSUPPORTED", 5: "H3_ERR_ALIAS", 6: "H3_ERR_HIP"}

# names every build of libh3.so must export (the declarations of include/h3.h)
EXPORTS = ("h3_seq2head", "h3_head2seq", "h3_seq2head_backward", "h3_head2seq_backward", "h3_packed_attn",
           "h3_packed_attn_lse", "h3_packed_attn_backward", "h3_packed_attn_backward_workspace",
           "h3_packed_attn_backward_noalloc", "h3_adaln_segment", "h3_adaln_gate_modulate", "h3_reduce_scatter",
           "h3_gather_rows", "h3_partition", "h3_clip_segments", "h3_status_string", "h3_last_error",
           "h3_version")


class H3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Layout(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_planes", ctypes.c_int32), ("world", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("max_chunk_bytes", ctypes.c_int64)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32), ("chunks", ctypes.c_int32), ("grid_x", ctypes.c_int32),
                ("block_x", ctypes.c_int32), ("chunk_tokens", ctypes.c_int64),
                ("max_launch_src_bytes", ctypes.c_int64), ("bytes_read", ctypes.c_int64),
                ("bytes_written", ctypes.c_int64), ("flops", ctypes.c_double), ("tiles", ctypes.c_int64)]


@dataclass(frozen=True)
class PlanInfo:
    """What one call actually enqueued (copied out of h3_plan_info)."""
    launches: int
    chunks: int
    grid_x: int
    block_x: int
    chunk_tokens: int
    max_launch_src_bytes: int
    bytes_read: int
    bytes_written: int
    flops: float
    tiles: int


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python ulysses_layout_amd/build.py` "
                          "(the hot path has no other implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    missing = [name for name in EXPORTS if not hasattr(lib, name)]
    if missing:
        raise ImportError(f"{LIB_PATH} is stale (does not export {', '.join(missing)}): rebuild it with "
                          "`python ulysses_layout_amd/build.py`")
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    i64p = ctypes.POINTER(ctypes.c_int64)
    lp = ctypes.POINTER(Layout)
    ip = ctypes.POINTER(_PlanInfo)
    lib.h3_seq2head.argtypes = [lp, vp, ctypes.POINTER(vp), vp, ip]
    lib.h3_head2seq.argtypes = [lp, ctypes.POINTER(vp), vp, vp, ip]
    lib.h3_seq2head_backward.argtypes = [lp, ctypes.POINTER(vp), vp, vp, ip]
    lib.h3_head2seq_backward.argtypes = [lp, vp, ctypes.POINTER(vp), vp, ip]
    lib.h3_packed_attn.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64p, i32, f32, vp, ip]
    lib.h3_packed_attn_lse.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i64p, i32, f32, vp, ip]
    lib.h3_packed_attn_backward.argtypes = [vp] * 11 + [vp, i64, i64, i32, i32, i64p, i32, f32, vp, ip]
    lib.h3_packed_attn_backward_noalloc.argtypes = [vp] * 11 + [i64, i32, i32, i64p, i32, f32, vp, ip]
    lib.h3_packed_attn_backward_workspace.argtypes = [i64, i32, i32]
    lib.h3_packed_attn_backward_workspace.restype = i64
    lib.h3_adaln_segment.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i64, i32, i64p, i32, f32, vp, ip]
    lib.h3_adaln_gate_modulate.argtypes = [vp] * 7 + [i64, i64, i32, i64p, i32, f32, vp, ip]
    lib.h3_reduce_scatter.argtypes = [ctypes.POINTER(vp), vp, ctypes.POINTER(vp), i64, i32, i32, i32, vp, ip]
    lib.h3_gather_rows.argtypes = [ctypes.POINTER(vp), vp, i64, i32, i32, vp, ip]
    lib.h3_partition.argtypes = [i64, i32, i32, i64p, i64p]
    lib.h3_clip_segments.argtypes = [i64p, i32, i64, i64, ctypes.POINTER(i32), i64p, i64p]
    lib.h3_clip_segments.restype = i32
    for name in ("h3_seq2head", "h3_head2seq", "h3_seq2head_backward", "h3_head2seq_backward",
                 "h3_packed_attn", "h3_packed_attn_lse", "h3_packed_attn_backward",
                 "h3_packed_attn_backward_noalloc", "h3_adaln_segment",
                 "h3_adaln_gate_modulate", "h3_reduce_scatter", "h3_gather_rows", "h3_partition"):
        getattr(lib, name).restype = ctypes.c_int
    lib.h3_status_string.argtypes = [ctypes.c_int]
    lib.h3_status_string.restype = ctypes.c_char_p
    lib.h3_last_error.argtypes = []
    lib.h3_last_error.restype = ctypes.c_char_p
    lib.h3_version.argtypes = []
    lib.h3_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def version() -> str:
    return _lib.h3_version().decode()


def _check(status: int) -> None:
    if status != H3_OK:
        raise H3Error(status, _lib.h3_last_error().decode())


def _info(raw: _PlanInfo) -> PlanInfo:
    return PlanInfo(**{name: getattr(raw, name) for name, _ in _PlanInfo._fields_})


def _i64_array(values: Sequence[int]):
    arr = (ctypes.c_int64 * len(values))(*[int(v) for v in values])
    return arr


# ---------------------------------------------------------------------------
# host-only helpers
# ---------------------------------------------------------------------------

def partition(total: int, parts: int, index: int) -> Tuple[int, int]:
    """(begin, count) of part ``index`` of the quotient/remainder split."""
    b, c = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.h3_partition(int(total), int(parts), int(index), ctypes.byref(b), ctypes.byref(c)))
    return b.value, c.value


def clip_segments(cu: Sequence[int], a: int, b: int) -> List[Tuple[int, int, int]]:
    """(global segment id, local begin, local end) of the clipped, rebased table."""
    n = len(cu) - 1
    cua = _i64_array(cu)
    sid = (ctypes.c_int32 * max(n, 1))()
    lb = (ctypes.c_int64 * max(n, 1))()
    le = (ctypes.c_int64 * max(n, 1))()
    m = _lib.h3_clip_segments(cua, n, int(a), int(b), sid, lb, le)
    if m < 0:
        raise H3Error(1, _lib.h3_last_error().decode())
    return [(sid[i], lb[i], le[i]) for i in range(m)]


# ---------------------------------------------------------------------------
# device entry points (torch tensors -> pointers)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev_tensor(t, name: str, dtype, shape: Optional[Tuple[int, ...]] = None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _dev_bf16(t, name: str, shape: Optional[Tuple[int, ...]] = None) -> int:
    return _dev_tensor(t, name, _torch().bfloat16, shape)


def _dev_f32(t, name: str, shape: Optional[Tuple[int, ...]] = None) -> int:
    return _dev_tensor(t, name, _torch().float32, shape)


def head_split(n_heads: int, world: int) -> List[Tuple[int, int]]:
    return [partition(n_heads, world, j) for j in range(world)]


def seq2head(src, dst: Sequence[Sequence], world: int, rank: int = -1, max_chunk_bytes: int = 0,
             stream=None) -> PlanInfo:
    """``src`` [N, K, H, 128] -> ``dst[j][p]`` [N, H_j, 128] for the selected ranks.

    ``dst`` is indexed ``dst[j][p]``; with ``rank = j`` only ``dst[j]`` is used
    (other entries may be None).
    """
    n, k, h, d = src.shape
    src_ptr = _dev_bf16(src, "src")
    ptrs = (ctypes.c_void_p * (world * k))()
    heads = head_split(h, world) if 1 <= world <= h else [(0, 0)] * max(world, 0)
    for j in range(world):
        if rank not in (-1, j):
            continue
        for p in range(k):
            ptrs[j * k + p] = _dev_bf16(dst[j][p], f"dst[{j}][{p}]", (n, heads[j][1], d))
    lay = Layout(n, h, d, k, world, rank, 0, max_chunk_bytes)
    info = _PlanInfo()
    _check(_lib.h3_seq2head(ctypes.byref(lay), src_ptr, ptrs, _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def head2seq(src: Sequence, dst, world: int, rank: int = -1, max_chunk_bytes: int = 0,
             stream=None) -> PlanInfo:
    """``src[j]`` [N, H_j, 128] -> ``dst`` [N, H, 128] for the selected ranks."""
    n, h, d = dst.shape
    dst_ptr = _dev_bf16(dst, "dst")
    ptrs = (ctypes.c_void_p * world)()
    heads = head_split(h, world) if 1 <= world <= h else [(0, 0)] * max(world, 0)
    for j in range(world):
        if rank not in (-1, j):
            continue
        ptrs[j] = _dev_bf16(src[j], f"src[{j}]", (n, heads[j][1], d))
    lay = Layout(n, h, d, 1, world, rank, 0, max_chunk_bytes)
    info = _PlanInfo()
    _check(_lib.h3_head2seq(ctypes.byref(lay), ptrs, dst_ptr, _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def seq2head_backward(grad_dst: Sequence[Sequence], grad_src, world: int, rank: int = -1,
                      max_chunk_bytes: int = 0, stream=None) -> PlanInfo:
    """Adjoint of ``seq2head``: ``grad_dst[j][p]`` [N, H_j, 128] -> ``grad_src`` [N, K, H, 128].

    Takes the forward call's ``world``, ``rank`` and ``max_chunk_bytes``; the
    returned plan equals the forward's.  Heads of unselected ranks in
    ``grad_src`` are left untouched.
    """
    n, k, h, d = grad_src.shape
    gs_ptr = _dev_bf16(grad_src, "grad_src")
    ptrs = (ctypes.c_void_p * (world * k))()
    heads = head_split(h, world) if 1 <= world <= h else [(0, 0)] * max(world, 0)
    for j in range(world):
        if rank not in (-1, j):
            continue
        for p in range(k):
            ptrs[j * k + p] = _dev_bf16(grad_dst[j][p], f"grad_dst[{j}][{p}]", (n, heads[j][1], d))
    lay = Layout(n, h, d, k, world, rank, 0, max_chunk_bytes)
    info = _PlanInfo()
    _check(_lib.h3_seq2head_backward(ctypes.byref(lay), ptrs, gs_ptr, _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def head2seq_backward(grad_dst, grad_src: Sequence, world: int, rank: int = -1, max_chunk_bytes: int = 0,
                      stream=None) -> PlanInfo:
    """Adjoint of ``head2seq``: ``grad_dst`` [N, H, 128] -> ``grad_src[j]`` [N, H_j, 128]."""
    n, h, d = grad_dst.shape
    gd_ptr = _dev_bf16(grad_dst, "grad_dst")
    ptrs = (ctypes.c_void_p * world)()
    heads = head_split(h, world) if 1 <= world <= h else [(0, 0)] * max(world, 0)
    for j in range(world):
        if rank not in (-1, j):
            continue
        ptrs[j] = _dev_bf16(grad_src[j], f"grad_src[{j}]", (n, heads[j][1], d))
    lay = Layout(n, h, d, 1, world, rank, 0, max_chunk_bytes)
    info = _PlanInfo()
    _check(_lib.h3_head2seq_backward(ctypes.byref(lay), gd_ptr, ptrs, _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def packed_attn(q, k, v, g, o, cu_seqlens: Sequence[int], scale: float, stream=None, lse=None) -> PlanInfo:
    """Segment-masked attention of [N, H, 128] operands; ``g`` may be None.

    With ``lse`` (a float32 [N, H] device tensor) the call also writes the
    per-row log-sum-exp of the scaled logits (``h3_packed_attn_lse``).
    """
    n, h, d = q.shape
    shp = (n, h, d)
    ptrs = [_dev_bf16(t, nm, shp) for t, nm in ((q, "q"), (k, "k"), (v, "v"))]
    gp = None if g is None else _dev_bf16(g, "g", shp)
    op = _dev_bf16(o, "o", shp)
    cu = _i64_array(cu_seqlens)
    info = _PlanInfo()
    if lse is None:
        _check(_lib.h3_packed_attn(ptrs[0], ptrs[1], ptrs[2], gp, op, n, h, d, cu, len(cu_seqlens) - 1,
                                   float(scale), _stream_ptr(stream), ctypes.byref(info)))
    else:
        lp = _dev_f32(lse, "lse", (n, h))
        _check(_lib.h3_packed_attn_lse(ptrs[0], ptrs[1], ptrs[2], gp, op, lp, n, h, d, cu, len(cu_seqlens) - 1,
                                       float(scale), _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def packed_attn_backward_workspace(n_tokens: int, n_heads: int, gated: bool) -> int:
    """Bytes of device scratch ``packed_attn_backward`` needs."""
    return int(_lib.h3_packed_attn_backward_workspace(int(n_tokens), int(n_heads), int(bool(gated))))


def packed_attn_backward(q, k, v, g, o, dout, lse, dq, dk, dv, dg, workspace, cu_seqlens: Sequence[int],
                         scale: float, stream=None) -> PlanInfo:
    """Gradients of ``packed_attn``: dq, dk, dv (and dg when ``g`` is given).

    ``o`` and ``lse`` come from the forward (``packed_attn(..., lse=lse)``);
    ``workspace`` is a uint8 device tensor of at least
    ``packed_attn_backward_workspace(N, H, g is not None)`` bytes.
    """
    torch = _torch()
    n, h, d = q.shape
    shp = (n, h, d)
    ins = [_dev_bf16(t, nm, shp) for t, nm in ((q, "q"), (k, "k"), (v, "v"))]
    gp = None if g is None else _dev_bf16(g, "g", shp)
    op, dop = _dev_bf16(o, "o", shp), _dev_bf16(dout, "dout", shp)
    lp = _dev_f32(lse, "lse", (n, h))
    outs = [_dev_bf16(t, nm, shp) for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    dgp = None if dg is None else _dev_bf16(dg, "dg", shp)
    wp = _dev_tensor(workspace, "workspace", torch.uint8)
    cu = _i64_array(cu_seqlens)
    info = _PlanInfo()
    _check(_lib.h3_packed_attn_backward(ins[0], ins[1], ins[2], gp, op, dop, lp, outs[0], outs[1], outs[2], dgp, wp,
                                        workspace.numel(), n, h, d, cu, len(cu_seqlens) - 1, float(scale),
                                        _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def packed_attn_backward_noalloc(q, k, v, g, o, dout, lse, dq, dk, dv, dg, cu_seqlens: Sequence[int],
                                 scale: float, stream=None) -> PlanInfo:
    """``packed_attn_backward`` without a workspace: the library's per-GPU
    scratch array (``NOALLOC_SCRATCH_BYTES``) stands in for it, so the call
    allocates nothing.  Calls that may overlap in time on one GPU race on
    that array."""
    n, h, d = q.shape
    shp = (n, h, d)
    ins = [_dev_bf16(t, nm, shp) for t, nm in ((q, "q"), (k, "k"), (v, "v"))]
    gp = None if g is None else _dev_bf16(g, "g", shp)
    op, dop = _dev_bf16(o, "o", shp), _dev_bf16(dout, "dout", shp)
    lp = _dev_f32(lse, "lse", (n, h))
    outs = [_dev_bf16(t, nm, shp) for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    dgp = None if dg is None else _dev_bf16(dg, "dg", shp)
    cu = _i64_array(cu_seqlens)
    info = _PlanInfo()
    _check(_lib.h3_packed_attn_backward_noalloc(ins[0], ins[1], ins[2], gp, op, dop, lp, outs[0], outs[1], outs[2],
                                                dgp, n, h, d, cu, len(cu_seqlens) - 1, float(scale),
                                                _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def adaln_segment(mode: int, x, branch, shift, scale, gate, y, tok_begin: int, tok_end: int,
                  cu_seqlens: Sequence[int], eps: float = 1e-6, stream=None) -> PlanInfo:
    """Per-segment AdaLN on rows ``[tok_begin, tok_end)``; x, branch, y are [rows, C]."""
    rows, c = x.shape
    n_seg = len(cu_seqlens) - 1
    xp = _dev_bf16(x, "x", (rows, c))
    yp = _dev_bf16(y, "y", (rows, c))
    bp = None if branch is None else _dev_bf16(branch, "branch", (rows, c))
    pp = [None if t is None else _dev_bf16(t, nm, (n_seg, c))
          for t, nm in ((shift, "shift"), (scale, "scale"), (gate, "gate"))]
    cu = _i64_array(cu_seqlens)
    info = _PlanInfo()
    _check(_lib.h3_adaln_segment(int(mode), xp, bp, pp[0], pp[1], pp[2], yp, int(tok_begin), int(tok_end), c,
                                 cu, n_seg, float(eps), _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def adaln_gate_modulate(x, branch, gate, shift, scale, resid, y, tok_begin: int, tok_end: int,
                        cu_seqlens: Sequence[int], eps: float = 1e-6, stream=None) -> PlanInfo:
    """``resid = x + gate[s] * branch`` and ``y`` = its modulation by the next
    sub-block's ``shift`` / ``scale``, on rows ``[tok_begin, tok_end)``; x,
    branch, resid, y are [rows, C], parameters [S, C]."""
    rows, c = x.shape
    n_seg = len(cu_seqlens) - 1
    xp, bp = _dev_bf16(x, "x", (rows, c)), _dev_bf16(branch, "branch", (rows, c))
    rp, yp = _dev_bf16(resid, "resid", (rows, c)), _dev_bf16(y, "y", (rows, c))
    gp, shp, scp = (_dev_bf16(t, nm, (n_seg, c)) for t, nm in ((gate, "gate"), (shift, "shift"), (scale, "scale")))
    cu = _i64_array(cu_seqlens)
    info = _PlanInfo()
    _check(_lib.h3_adaln_gate_modulate(xp, bp, gp, shp, scp, rp, yp, int(tok_begin), int(tok_end), c, cu, n_seg,
                                       float(eps), _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def reduce_scatter(partials: Sequence, bias, out: Sequence, rank: int = -1, stream=None) -> PlanInfo:
    """Sum the P partials ``[N, C]``, add ``bias`` ``[C]`` (or None) once, and
    write rank i's rows to ``out[i]`` ``[N_i, C]`` for the selected ranks
    (``rank = -1``: all; other entries of ``out`` may be None)."""
    world = len(partials)
    n, c = partials[0].shape
    pp = (ctypes.c_void_p * world)(*[_dev_bf16(t, f"partials[{j}]", (n, c)) for j, t in enumerate(partials)])
    op = (ctypes.c_void_p * world)()
    for i in range(world):
        if rank in (-1, i):
            op[i] = _dev_bf16(out[i], f"out[{i}]", (partition(n, world, i)[1], c))
    bp = None if bias is None else _dev_bf16(bias, "bias", (c,))
    info = _PlanInfo()
    _check(_lib.h3_reduce_scatter(pp, bp, op, n, c, world, int(rank), _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)


def gather_rows(shards: Sequence, dst, stream=None) -> PlanInfo:
    """Rank i's first N_i rows of ``shards[i]`` (``[>= N_i, C]``, e.g. one
    padded block of a gathered buffer) to rows ``[a_i, a_i + N_i)`` of ``dst``
    ``[N, C]``."""
    world = len(shards)
    n, c = dst.shape
    dp = _dev_bf16(dst, "dst", (n, c))
    sp = (ctypes.c_void_p * world)()
    for i, t in enumerate(shards):
        sp[i] = _dev_bf16(t, f"shards[{i}]")
        if 1 <= world <= n and (t.dim() != 2 or t.shape[1] != c or t.shape[0] < partition(n, world, i)[1]):
            raise ValueError(f"shards[{i}] has shape {tuple(t.shape)}; it needs at least "
                             f"{partition(n, world, i)[1]} rows of {c} channels")
    info = _PlanInfo()
    _check(_lib.h3_gather_rows(sp, dp, n, c, world, _stream_ptr(stream), ctypes.byref(info)))
    return _info(info)
