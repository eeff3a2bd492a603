"""Host-side contract of libh3.so, runnable without a GPU.

* the library loads and exports every function include/h3.h declares;
* the host helpers (partition, clip) equal the oracle exactly;
* every invalid call is rejected on the host with the documented status, before
  anything could be enqueued (fake device addresses are never dereferenced),
  and a rejected call leaves nothing behind for the next one.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import ulysses_layout_amd as h3
from ulysses_layout_amd.h3 import Layout, _PlanInfo
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3.h")

ARG, EMPTY, SEGS, UNSUP, ALIAS = 1, 2, 3, 4, 5
FAKE = 1 << 40     # a device-looking address that is never touched


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0      # counts devices without initialising HIP


# The rejection tests hand the library fake device addresses and rely on every
# case being refused on the host.  Where a GPU is visible a case that slipped
# through validation would launch on those addresses, so they run only on
# machines without one.
fake_addresses = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses; run where no GPU is visible")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) >= {"h3_seq2head", "h3_head2seq", "h3_packed_attn", "h3_adaln_segment"}
    lib = ctypes.CDLL(h3.h3.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), f"libh3.so does not export {name}"
    assert set(names) == set(h3.EXPORTS)


def test_library_is_built_for_gfx950():
    blob = open(h3.h3.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_partition_equals_oracle():
    for total in list(range(1, 40)) + [56, 8192, 131072, 250000]:
        for parts in range(1, min(total, 64) + 1):
            ref = oracle.partition(total, parts)
            for j in range(parts):
                assert h3.partition(total, parts, j) == ref[j]


@pytest.mark.parametrize("total,parts", [(56, 0), (56, 57), (5, 6), (0, 1)])
def test_partition_rejects_empty(total, parts):
    with pytest.raises(h3.H3Error) as e:
        h3.partition(total, parts, 0)
    assert e.value.status == EMPTY
    assert "legal" in e.value.message


def test_clip_equals_oracle():
    rng = np.random.default_rng(5)
    for w in WORKLOADS.values():
        for a, cnt in oracle.partition(w.n_tokens, w.world):
            assert h3.clip_segments(w.cu, a, a + cnt) == oracle.clip_segments(w.cu, a, a + cnt)
    for _ in range(300):
        n = int(rng.integers(2, 500))
        s = int(rng.integers(1, min(n, 30) + 1))
        cu = [0] + sorted(int(c) for c in rng.choice(np.arange(1, n), size=s - 1, replace=False)) + [n]
        a = int(rng.integers(0, n))
        b = int(rng.integers(a + 1, n + 1))
        assert h3.clip_segments(cu, a, b) == oracle.clip_segments(cu, a, b)


def test_clip_rejects_bad_input():
    with pytest.raises(h3.H3Error):
        h3.clip_segments([0, 5, 5, 9], 0, 9)      # empty segment
    with pytest.raises(h3.H3Error):
        h3.clip_segments([0, 5, 9], 3, 3)         # empty interval
    with pytest.raises(h3.H3Error):
        h3.clip_segments([0, 5, 9], 3, 10)        # past the end


# ---------------------------------------------------------------------------
# validation of the device entry points, straight through the C ABI
# ---------------------------------------------------------------------------

LIB = h3.library()


def _seq2head(layout, src=FAKE, dst=None):
    k, p = layout.n_planes, layout.world
    if dst is None:
        heads = [c for _, c in oracle.partition(layout.n_heads, p)] if 1 <= p <= layout.n_heads else []
        dst, addr = [], FAKE * 2
        for j in range(max(p, 0)):
            for _ in range(k):
                dst.append(addr)
                addr += layout.n_tokens * (heads[j] if heads else 1) * 256 + 4096
    arr = (ctypes.c_void_p * max(len(dst), 1))(*dst)
    info = _PlanInfo()
    return LIB.h3_seq2head(ctypes.byref(layout), src, arr, None, ctypes.byref(info)), info


def _layout(**kw):
    base = dict(n_tokens=512, n_heads=56, head_dim=128, n_planes=3, world=2, rank=-1, reserved=0,
                max_chunk_bytes=0)
    base.update(kw)
    return Layout(**base)


@fake_addresses
@pytest.mark.parametrize("kw,status", [
    (dict(world=0), EMPTY), (dict(world=57), EMPTY), (dict(n_tokens=3, world=4), EMPTY),
    (dict(n_tokens=0), EMPTY), (dict(head_dim=64), UNSUP), (dict(n_planes=0), ARG),
    (dict(n_planes=9), ARG), (dict(rank=2), ARG), (dict(rank=-2), ARG), (dict(reserved=1), ARG),
    (dict(max_chunk_bytes=-1), ARG), (dict(max_chunk_bytes=1000), ARG), (dict(n_heads=0), ARG),
])
def test_seq2head_rejects_bad_layout(kw, status):
    rc, info = _seq2head(_layout(**kw))
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0
    msg = LIB.h3_last_error().decode()
    assert msg
    if status == EMPTY and "world" in kw:
        assert "legal values are 1.." in msg


@fake_addresses
def test_seq2head_rejects_null_and_alias():
    lay = _layout()
    rc, _ = _seq2head(lay, src=None)
    assert rc == ARG
    # one destination placed inside the source
    src_bytes = 512 * 3 * 56 * 128 * 2
    dst = [FAKE * 2 + i * (1 << 24) for i in range(6)]
    dst[3] = FAKE + src_bytes // 2
    rc, _ = _seq2head(lay, dst=dst)
    assert rc == ALIAS
    # two destinations overlapping each other
    dst = [FAKE * 2 + i * (1 << 24) for i in range(6)]
    dst[4] = dst[1] + 256
    rc, _ = _seq2head(lay, dst=dst)
    assert rc == ALIAS
    dst = [FAKE * 2 + i * (1 << 24) for i in range(6)]
    dst[5] = None
    rc, _ = _seq2head(lay, dst=dst)
    assert rc == ARG


def _seq2head_bwd(layout, grad_src=FAKE, grad_dst=None):
    k, p = layout.n_planes, layout.world
    if grad_dst is None:
        heads = [c for _, c in oracle.partition(layout.n_heads, p)] if 1 <= p <= layout.n_heads else []
        grad_dst, addr = [], FAKE * 2
        for j in range(max(p, 0)):
            for _ in range(k):
                grad_dst.append(addr)
                addr += layout.n_tokens * (heads[j] if heads else 1) * 256 + 4096
    arr = (ctypes.c_void_p * max(len(grad_dst), 1))(*grad_dst)
    info = _PlanInfo()
    return LIB.h3_seq2head_backward(ctypes.byref(layout), arr, grad_src, None, ctypes.byref(info)), info


@fake_addresses
@pytest.mark.parametrize("kw,status", [
    (dict(world=0), EMPTY), (dict(world=57), EMPTY), (dict(n_tokens=0), EMPTY), (dict(head_dim=64), UNSUP),
    (dict(n_planes=9), ARG), (dict(rank=2), ARG), (dict(max_chunk_bytes=1000), ARG),
])
def test_seq2head_backward_rejects_bad_layout(kw, status):
    rc, info = _seq2head_bwd(_layout(**kw))
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0
    assert LIB.h3_last_error().decode()


@fake_addresses
def test_seq2head_backward_rejects_null_and_alias():
    lay = _layout()
    assert _seq2head_bwd(lay, grad_src=None)[0] == ARG
    gd = [FAKE * 2 + i * (1 << 24) for i in range(6)]
    gd[2] = None
    assert _seq2head_bwd(lay, grad_dst=gd)[0] == ARG
    # a gradient input inside the output
    gd = [FAKE * 2 + i * (1 << 24) for i in range(6)]
    gd[0] = FAKE + 4096
    assert _seq2head_bwd(lay, grad_dst=gd)[0] == ALIAS


def _head2seq_bwd(layout, grad_dst=FAKE, grad_src=None):
    p = layout.world
    if grad_src is None:
        grad_src = [FAKE * 2 + j * (1 << 28) for j in range(max(p, 0))]
    arr = (ctypes.c_void_p * max(len(grad_src), 1))(*grad_src)
    info = _PlanInfo()
    return LIB.h3_head2seq_backward(ctypes.byref(layout), grad_dst, arr, None, ctypes.byref(info)), info


@fake_addresses
@pytest.mark.parametrize("kw,status", [
    (dict(n_planes=3), ARG), (dict(world=57), EMPTY), (dict(head_dim=64), UNSUP), (dict(rank=5), ARG),
])
def test_head2seq_backward_rejects_bad_layout(kw, status):
    base = dict(n_planes=1)
    base.update(kw)
    rc, info = _head2seq_bwd(_layout(**base))
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0


@fake_addresses
def test_head2seq_backward_rejects_null_and_alias():
    lay = _layout(n_planes=1)
    assert _head2seq_bwd(lay, grad_dst=None)[0] == ARG
    assert _head2seq_bwd(lay, grad_src=[FAKE * 2, None])[0] == ARG
    assert _head2seq_bwd(lay, grad_src=[FAKE * 2, FAKE + 256])[0] == ALIAS


@fake_addresses
def test_rejected_call_leaves_no_state():
    rc, _ = _seq2head(_layout(world=57))
    assert rc == EMPTY
    assert h3.partition(56, 6, 0) == (0, 10)           # next valid call works
    assert LIB.h3_last_error().decode() == ""


def _attn(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), g=None, o=FAKE + (3 << 32), n=512, h=4, d=128,
          cu=(0, 96, 256, 512), scale=0.088):
    cua = (ctypes.c_int64 * len(cu))(*cu)
    info = _PlanInfo()
    rc = LIB.h3_packed_attn(q, k, v, g, o, n, h, d, cua, len(cu) - 1, scale, None, ctypes.byref(info))
    return rc, info


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ARG), (dict(o=None), ARG), (dict(d=64), UNSUP), (dict(h=0), EMPTY), (dict(n=0), EMPTY),
    (dict(cu=(0, 96, 96, 512)), SEGS), (dict(cu=(1, 96, 512)), SEGS), (dict(cu=(0, 96, 500)), SEGS),
    (dict(scale=0.0), ARG), (dict(scale=float("nan")), ARG), (dict(o=FAKE + 256), ALIAS),
    (dict(g=FAKE + (3 << 32) + 64), ALIAS), (dict(cu=tuple(range(0, 2 * 300, 2)) + (600,), n=600), SEGS),
])
@fake_addresses
def test_packed_attn_rejects(kw, status):
    rc, info = _attn(**kw)
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0


def _adaln(mode=0, x=FAKE, b=None, shift=FAKE + (1 << 32), scale=FAKE + (2 << 32), gate=None,
           y=FAKE + (3 << 32), a=0, e=256, c=7168, cu=(0, 96, 256, 512), eps=1e-6):
    cua = (ctypes.c_int64 * len(cu))(*cu)
    info = _PlanInfo()
    rc = LIB.h3_adaln_segment(mode, x, b, shift, scale, gate, y, a, e, c, cua, len(cu) - 1, eps, None,
                              ctypes.byref(info))
    return rc, info


@pytest.mark.parametrize("kw,status", [
    (dict(mode=2), ARG), (dict(x=None), ARG), (dict(shift=None), ARG), (dict(mode=1), ARG),
    (dict(a=10, e=10), EMPTY), (dict(a=-1), EMPTY), (dict(c=7170), UNSUP), (dict(c=0), UNSUP),
    (dict(c=16392), UNSUP), (dict(e=600), SEGS), (dict(cu=(0, 300, 200, 512)), SEGS),
    (dict(y=FAKE + 1024), ALIAS), (dict(eps=float("nan")), ARG),
])
@fake_addresses
def test_adaln_rejects(kw, status):
    rc, info = _adaln(**kw)
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0


def test_status_strings():
    for code, name in h3.h3.STATUS_NAMES.items():
        LIB.h3_status_string.restype = ctypes.c_char_p
        assert LIB.h3_status_string(code).decode() == name


def _chain(x=FAKE, b=FAKE + (1 << 32), gate=FAKE + (2 << 32), shift=FAKE + (3 << 32), scale=FAKE + (4 << 32),
           resid=FAKE + (5 << 32), y=FAKE + (6 << 32), a=0, e=256, c=7168, cu=(0, 96, 256, 512), eps=1e-6):
    cua = (ctypes.c_int64 * len(cu))(*cu)
    info = _PlanInfo()
    rc = LIB.h3_adaln_gate_modulate(x, b, gate, shift, scale, resid, y, a, e, c, cua, len(cu) - 1, eps, None,
                                    ctypes.byref(info))
    return rc, info


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ARG), (dict(b=None), ARG), (dict(gate=None), ARG), (dict(shift=None), ARG),
    (dict(scale=None), ARG), (dict(resid=None), ARG), (dict(y=None), ARG), (dict(a=5, e=5), EMPTY),
    (dict(c=7170), UNSUP), (dict(e=600), SEGS), (dict(eps=-1.0), ARG),
    (dict(resid=FAKE + (6 << 32) + 512), ALIAS),          # resid overlaps y
    (dict(y=FAKE + (1 << 32) + 4096), ALIAS),             # y overlaps the branch
    (dict(resid=FAKE + (2 << 32)), ALIAS),                # resid overlaps the gate rows
])
@fake_addresses
def test_adaln_gate_modulate_rejects(kw, status):
    rc, info = _chain(**kw)
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0


def _ptrs(values):
    return (ctypes.c_void_p * len(values))(*values)


def _rs(n=1003, c=64, world=3, rank=-1, partials=None, out=None, bias=FAKE + (9 << 32)):
    partials = [FAKE + (j << 32) for j in range(world)] if partials is None else partials
    out = [FAKE + ((20 + i) << 32) for i in range(world)] if out is None else out
    info = _PlanInfo()
    rc = LIB.h3_reduce_scatter(_ptrs(partials), bias, _ptrs(out), n, c, world, rank, None, ctypes.byref(info))
    return rc, info


@pytest.mark.parametrize("kw,status", [
    (dict(world=0), EMPTY), (dict(world=1004), EMPTY), (dict(n=0), EMPTY), (dict(n=100, world=65), UNSUP),
    (dict(c=60), UNSUP), (dict(c=0), UNSUP), (dict(rank=3), ARG), (dict(rank=-2), ARG),
    (dict(partials=[FAKE, None, FAKE + (2 << 32)]), ARG), (dict(out=[FAKE + (20 << 32), None, FAKE + (22 << 32)]), ARG),
    (dict(partials=[FAKE, FAKE + (1 << 32) + 8, FAKE + (2 << 32)]), ARG),          # misaligned
    (dict(bias=FAKE + (9 << 32) + 2), ARG),
    (dict(out=[FAKE + (20 << 32), FAKE + 1003 * 128 - 128, FAKE + (22 << 32)]), ALIAS),   # inside partial 0
    (dict(out=[FAKE + (20 << 32), FAKE + (20 << 32) + 334 * 128, FAKE + (22 << 32)]), ALIAS),  # out 0 / out 1
    (dict(bias=FAKE + (21 << 32) + 256), ALIAS),
    (dict(n=1 << 22, c=8192, world=1), UNSUP),             # one rank's range passes 2^31 vectors
])
@fake_addresses
def test_reduce_scatter_rejects(kw, status):
    rc, info = _rs(**kw)
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0


@fake_addresses
def test_reduce_scatter_unselected_outputs_may_be_null():
    # rank 1 only: the NULL out[0] and out[2] are not looked at; the call is
    # refused for the selected output, which overlaps partial 0
    rc, info = _rs(rank=1, out=[None, FAKE, None])
    assert rc == ALIAS, LIB.h3_last_error()
    assert info.launches == 0


def _gather(n=1003, c=64, world=3, shards=None, dst=FAKE + (30 << 32)):
    shards = [FAKE + (j << 32) for j in range(world)] if shards is None else shards
    info = _PlanInfo()
    rc = LIB.h3_gather_rows(_ptrs(shards), dst, n, c, world, None, ctypes.byref(info))
    return rc, info


@pytest.mark.parametrize("kw,status", [
    (dict(world=0), EMPTY), (dict(world=1004), EMPTY), (dict(c=12), UNSUP), (dict(dst=None), ARG),
    (dict(shards=[FAKE, None, FAKE]), ARG), (dict(dst=FAKE + (30 << 32) + 4), ARG),
    (dict(dst=FAKE + (1 << 32) - 64), ALIAS),
    (dict(shards=[FAKE, FAKE + (30 << 32) + 1003 * 128 - 16, FAKE]), ALIAS),
])
@fake_addresses
def test_gather_rows_rejects(kw, status):
    rc, info = _gather(**kw)
    assert rc == status, LIB.h3_last_error()
    assert info.launches == 0


# ---------------------------------------------------------------------------
# alignment: every device pointer a kernel reads or writes in 16-byte vectors
# is refused when it does not start on a 16-byte boundary (the fp32 lse on a
# 4-byte one), before anything is enqueued
# ---------------------------------------------------------------------------

MIS = 2          # one bf16 element past an aligned address


def _h2s(layout, dst=FAKE, src=None):
    p = layout.world
    if src is None:
        src = [FAKE * 2 + j * (1 << 28) for j in range(p)]
    arr = (ctypes.c_void_p * max(len(src), 1))(*src)
    info = _PlanInfo()
    return LIB.h3_head2seq(ctypes.byref(layout), arr, dst, None, ctypes.byref(info)), info


def _six(i=None):
    """Six well-separated fake destination pointers, entry i misaligned."""
    out = [FAKE * 2 + j * (1 << 28) for j in range(6)]
    if i is not None:
        out[i] += MIS
    return out


@fake_addresses
@pytest.mark.parametrize("case", ["src", "dst0", "dst5"])
def test_seq2head_rejects_misaligned(case):
    lay = _layout()
    if case == "src":
        rc, info = _seq2head(lay, src=FAKE + MIS, dst=_six())
    else:
        rc, info = _seq2head(lay, dst=_six(int(case[3:])))
    assert rc == ARG, LIB.h3_last_error()
    assert "aligned" in LIB.h3_last_error().decode()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("case", ["dst", "src1"])
def test_head2seq_rejects_misaligned(case):
    lay = _layout(n_planes=1)
    if case == "dst":
        rc, info = _h2s(lay, dst=FAKE + MIS)
    else:
        rc, info = _h2s(lay, src=[FAKE * 2, FAKE * 2 + (1 << 28) + MIS])
    assert rc == ARG, LIB.h3_last_error()
    assert "aligned" in LIB.h3_last_error().decode()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("case", ["grad_src", "grad_dst2"])
def test_seq2head_backward_rejects_misaligned(case):
    lay = _layout()
    if case == "grad_src":
        rc, info = _seq2head_bwd(lay, grad_src=FAKE + 8, grad_dst=_six())
    else:
        rc, info = _seq2head_bwd(lay, grad_dst=_six(2))
    assert rc == ARG, LIB.h3_last_error()
    assert "aligned" in LIB.h3_last_error().decode()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("case", ["grad_dst", "grad_src0"])
def test_head2seq_backward_rejects_misaligned(case):
    lay = _layout(n_planes=1)
    if case == "grad_dst":
        rc, info = _head2seq_bwd(lay, grad_dst=FAKE + MIS)
    else:
        rc, info = _head2seq_bwd(lay, grad_src=[FAKE * 2 + 4, FAKE * 2 + (1 << 28)])
    assert rc == ARG, LIB.h3_last_error()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("name", ["q", "k", "v", "g", "o"])
def test_packed_attn_rejects_misaligned(name):
    kw = dict(g=FAKE + (4 << 32))
    kw[name] = (kw.get(name) or dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), o=FAKE + (3 << 32))[name]) + MIS
    rc, info = _attn(**kw)
    assert rc == ARG, LIB.h3_last_error()
    assert name in LIB.h3_last_error().decode() and "aligned" in LIB.h3_last_error().decode()
    assert info.launches == 0


def _attn_lse(lse, n=512, h=4, cu=(0, 96, 256, 512)):
    cua = (ctypes.c_int64 * len(cu))(*cu)
    info = _PlanInfo()
    rc = LIB.h3_packed_attn_lse(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), None, FAKE + (3 << 32), lse, n, h, 128,
                                cua, len(cu) - 1, 0.088, None, ctypes.byref(info))
    return rc, info


@fake_addresses
@pytest.mark.parametrize("off", [1, 2, 3])
def test_packed_attn_lse_rejects_misaligned(off):
    rc, info = _attn_lse(FAKE + (5 << 32) + off)
    assert rc == ARG, LIB.h3_last_error()
    assert "lse" in LIB.h3_last_error().decode()
    assert info.launches == 0


BWD_NAMES = ["q", "k", "v", "g", "o", "dout", "lse", "dq", "dk", "dv", "dg", "workspace"]


def _attn_bwd(mis=None, off=MIS, n=512, h=4, cu=(0, 96, 256, 512)):
    ptr = {name: FAKE + (i << 32) for i, name in enumerate(BWD_NAMES)}
    if mis is not None:
        ptr[mis] += off
    ws = LIB.h3_packed_attn_backward_workspace(n, h, 1)
    cua = (ctypes.c_int64 * len(cu))(*cu)
    info = _PlanInfo()
    rc = LIB.h3_packed_attn_backward(*[ptr[x] for x in BWD_NAMES], ws, n, h, 128, cua, len(cu) - 1, 0.088, None,
                                     ctypes.byref(info))
    return rc, info


@fake_addresses
@pytest.mark.parametrize("name", BWD_NAMES)
def test_packed_attn_backward_rejects_misaligned(name):
    rc, info = _attn_bwd(name)
    assert rc == ARG, LIB.h3_last_error()
    assert name in LIB.h3_last_error().decode() and "aligned" in LIB.h3_last_error().decode()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("name", ["x", "shift", "scale", "y"])
def test_adaln_modulate_rejects_misaligned(name):
    kw = dict(x=FAKE, shift=FAKE + (1 << 32), scale=FAKE + (2 << 32), y=FAKE + (3 << 32))
    kw[name] += MIS
    rc, info = _adaln(**kw)
    assert rc == ARG, LIB.h3_last_error()
    assert name in LIB.h3_last_error().decode()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("name", ["b", "gate"])
def test_adaln_gate_rejects_misaligned(name):
    kw = dict(mode=1, shift=None, scale=None, b=FAKE + (4 << 32), gate=FAKE + (5 << 32))
    kw[name] += 8
    rc, info = _adaln(**kw)
    assert rc == ARG, LIB.h3_last_error()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("name", ["x", "b", "gate", "shift", "scale", "resid", "y"])
def test_adaln_gate_modulate_rejects_misaligned(name):
    base = dict(x=FAKE, b=FAKE + (1 << 32), gate=FAKE + (2 << 32), shift=FAKE + (3 << 32), scale=FAKE + (4 << 32),
                resid=FAKE + (5 << 32), y=FAKE + (6 << 32))
    base[name] += MIS
    rc, info = _chain(**base)
    assert rc == ARG, LIB.h3_last_error()
    assert info.launches == 0


@fake_addresses
def test_misaligned_call_leaves_no_state():
    rc, _ = _attn(q=FAKE + MIS)
    assert rc == ARG
    assert h3.partition(56, 6, 0) == (0, 10)
    assert LIB.h3_last_error().decode() == ""


# ---------------------------------------------------------------------------
# h3_packed_attn_backward_noalloc: every check runs before the scratch array
# is looked up, so all rejections are visible without a GPU
# ---------------------------------------------------------------------------

NOALLOC_NAMES = ["q", "k", "v", "g", "o", "dout", "lse", "dq", "dk", "dv", "dg"]


def _attn_bwd_noalloc(mis=None, off=MIS, null=None, n=512, h=4, cu=(0, 96, 256, 512), gated=True):
    ptr = {name: FAKE + (i << 32) for i, name in enumerate(NOALLOC_NAMES)}
    if not gated:
        ptr["g"] = ptr["dg"] = None
    if mis is not None:
        ptr[mis] += off
    if null is not None:
        ptr[null] = None
    cua = (ctypes.c_int64 * len(cu))(*cu)
    info = _PlanInfo()
    rc = LIB.h3_packed_attn_backward_noalloc(*[ptr[x] for x in NOALLOC_NAMES], n, h, 128, cua, len(cu) - 1, 0.088,
                                             None, ctypes.byref(info))
    return rc, info


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define H3_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == h3.NOALLOC_SCRATCH_BYTES


@fake_addresses
@pytest.mark.parametrize("name", NOALLOC_NAMES)
def test_noalloc_backward_rejects_misaligned(name):
    rc, info = _attn_bwd_noalloc(mis=name)
    assert rc == ARG, LIB.h3_last_error()
    assert name in LIB.h3_last_error().decode()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("name", ["q", "lse", "dq", "dg"])
def test_noalloc_backward_rejects_null(name):
    rc, info = _attn_bwd_noalloc(null=name)
    assert rc == ARG, LIB.h3_last_error()
    assert info.launches == 0


@fake_addresses
@pytest.mark.parametrize("n,h,gated", [(16384, 16, True), (131072, 14, True), (1 << 21, 9, False)])
def test_noalloc_backward_rejects_beyond_scratch(n, h, gated):
    need = LIB.h3_packed_attn_backward_workspace(n, h, int(gated))
    assert need > h3.NOALLOC_SCRATCH_BYTES
    rc, info = _attn_bwd_noalloc(n=n, h=h, cu=(0, n), gated=gated)
    assert rc == UNSUP, LIB.h3_last_error()
    msg = LIB.h3_last_error().decode()
    assert str(need) in msg and str(h3.NOALLOC_SCRATCH_BYTES) in msg
    assert info.launches == 0


@fake_addresses
def test_noalloc_backward_rejects_alias_and_segments():
    rc, _ = _attn_bwd_noalloc(cu=(0, 96, 96, 512))
    assert rc == SEGS
    rc, _ = _attn_bwd_noalloc(mis="dq", off=-(7 << 32) + 256)     # dq moved inside q
    assert rc == ALIAS, LIB.h3_last_error()


# ---------------------------------------------------------------------------
# valid calls on a machine without a GPU: validation passes, the whole launch
# plan is built (and, in a build with H3_DEBUG_BOUNDS, every kernel-argument
# table is re-checked), and only the launch itself fails with H3_ERR_HIP
# ---------------------------------------------------------------------------

HIP_ERR = 6


def _apart(n, base=FAKE, step=1 << 36):
    return [base + (i + 1) * step for i in range(n)]


def _expect_launch_failure(rc):
    assert rc == HIP_ERR, (rc, LIB.h3_last_error())
    msg = LIB.h3_last_error().decode()
    assert "launch" in msg or "hipGetDevice" in msg, msg


@fake_addresses
@pytest.mark.parametrize("n,world,rank,planes,cap", [
    (512, 2, -1, 3, 0), (8192, 6, 3, 3, 0), (250000, 8, 0, 4, 896_000_000), (250000, 8, -1, 4, 896_000_000),
    (1000, 7, -1, 4, 5 * 56 * 256), (64, 56, 55, 1, 0),
])
def test_relayouts_reach_launch(n, world, rank, planes, cap):
    lay = _layout(n_tokens=n, world=world, rank=rank, n_planes=planes, max_chunk_bytes=cap)
    dst = _apart(world * planes)
    rc, _ = _seq2head(lay, src=FAKE, dst=dst)
    _expect_launch_failure(rc)
    rc, _ = _seq2head_bwd(lay, grad_src=FAKE, grad_dst=dst)
    _expect_launch_failure(rc)
    lay1 = _layout(n_tokens=n, world=world, rank=rank, n_planes=1, max_chunk_bytes=cap)
    rc, _ = _h2s(lay1, dst=FAKE, src=_apart(world))
    _expect_launch_failure(rc)
    rc, _ = _head2seq_bwd(lay1, grad_dst=FAKE, grad_src=_apart(world))
    _expect_launch_failure(rc)


@fake_addresses
@pytest.mark.parametrize("cu", [(0, 96, 256, 512), (0, 98304, 131072), tuple(range(0, 257 * 3, 3)), (0, 1)])
def test_attention_reaches_launch(cu):
    n = cu[-1]
    cua = (ctypes.c_int64 * len(cu))(*cu)
    ptr = _apart(13)
    info = _PlanInfo()
    rc = LIB.h3_packed_attn(ptr[0], ptr[1], ptr[2], ptr[3], ptr[4], n, 14, 128, cua, len(cu) - 1, 0.088, None,
                            ctypes.byref(info))
    _expect_launch_failure(rc)
    rc = LIB.h3_packed_attn_lse(ptr[0], ptr[1], ptr[2], None, ptr[4], ptr[5], n, 14, 128, cua, len(cu) - 1, 0.088,
                                None, ctypes.byref(info))
    _expect_launch_failure(rc)
    ws = LIB.h3_packed_attn_backward_workspace(n, 14, 1)
    rc = LIB.h3_packed_attn_backward(*ptr[:11], ptr[11], ws, n, 14, 128, cua, len(cu) - 1, 0.088, None,
                                     ctypes.byref(info))
    _expect_launch_failure(rc)
    if ws <= h3.NOALLOC_SCRATCH_BYTES:
        rc = LIB.h3_packed_attn_backward_noalloc(*ptr[:11], n, 14, 128, cua, len(cu) - 1, 0.088, None,
                                                 ctypes.byref(info))
        _expect_launch_failure(rc)


@fake_addresses
@pytest.mark.parametrize("a,e,c", [(0, 256, 7168), (256, 512, 7168), (100, 400, 1000), (0, 512, 8)])
def test_token_sharded_ops_reach_launch(a, e, c):
    cu = (0, 96, 256, 512)
    for mode in (0, 1):
        rc, _ = _adaln(mode=mode, x=FAKE, b=FAKE + (4 << 32) if mode else None,
                       shift=None if mode else FAKE + (1 << 32), scale=None if mode else FAKE + (2 << 32),
                       gate=FAKE + (5 << 32) if mode else None, y=FAKE + (3 << 32), a=a, e=e, c=c, cu=cu)
        _expect_launch_failure(rc)
    rc, _ = _chain(a=a, e=e, c=c, cu=cu)
    _expect_launch_failure(rc)
    for rank in (-1, 1):
        rc, _ = _rs(n=e, c=c, world=3, rank=rank, partials=_apart(3), out=_apart(3, base=FAKE << 4))
        _expect_launch_failure(rc)
    rc, _ = _gather(n=e, c=c, world=3, shards=_apart(3), dst=FAKE)
    _expect_launch_failure(rc)
