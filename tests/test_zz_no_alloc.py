"""h3_packed_attn_backward_noalloc against h3_packed_attn_backward: the same
gradients, bit for bit, from the library's per-GPU scratch array instead of a
caller workspace, on two calls in a row, the second smaller than the first."""
import pytest
import torch

from synth import segment_offsets
from synth.inputs import normal_bf16
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
SCALE = 128 ** -0.5


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _case(lengths, heads, gated, seed):
    h3 = _h3()
    cu = segment_offsets(lengths)
    n = cu[-1]
    shp = (n, heads, 128)
    q, k, v, g, dout = (normal_bf16(shp, seed=seed + i, device="cuda") for i in range(5))
    g = g if gated else None
    o = torch.empty_like(q)
    lse = torch.empty((n, heads), dtype=torch.float32, device="cuda")
    h3.packed_attn(q, k, v, g, o, cu, SCALE, lse=lse)
    return h3, cu, (q, k, v, g, o, dout, lse)


def _grads(like, gated):
    out = [torch.full_like(like, float("nan")) for _ in range(3)]
    out.append(torch.full_like(like, float("nan")) if gated else None)
    return out


def _same(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


@pytest.mark.parametrize("gated", [True, False])
def test_noalloc_backward_equals_workspace_backward(gated):
    cases = [([3000, 1, 4191, 1000], 8, 11), ([129, 700, 171], 3, 23)]     # second call smaller
    assert sum(cases[1][0]) * cases[1][1] < sum(cases[0][0]) * cases[0][1]
    for lengths, heads, seed in cases:
        say("noalloc backward", lengths, heads, "gated" if gated else "ungated")
        h3, cu, (q, k, v, g, o, dout, lse) = _case(lengths, heads, gated, seed)
        ref = _grads(q, gated)
        ws = torch.empty(h3.packed_attn_backward_workspace(q.shape[0], heads, gated), dtype=torch.uint8, device="cuda")
        info_ref = h3.packed_attn_backward(q, k, v, g, o, dout, lse, *ref, ws, cu, SCALE)
        got = _grads(q, gated)
        info = h3.packed_attn_backward_noalloc(q, k, v, g, o, dout, lse, *got, cu, SCALE)
        torch.cuda.synchronize()
        assert info == info_ref
        for name, a, b in zip(("dq", "dk", "dv", "dg"), got, ref):
            if b is not None:
                assert torch.isfinite(a.float()).all(), name
                _same(a, b, f"{name} {lengths} x {heads}")


def test_noalloc_backward_rejects_oversize_on_gpu():
    h3 = _h3()
    n, heads = 16384, 16                       # gated scratch need 68,157,440 bytes > 64 MiB
    say("noalloc oversize", n, heads)
    t = torch.zeros((n, heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((n, heads), dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(t) for _ in range(4)]
    with pytest.raises(h3.H3Error) as e:
        h3.packed_attn_backward_noalloc(t, t.clone(), t.clone(), t.clone(), t.clone(), t.clone(), lse, *outs,
                                        [0, n], SCALE)
    assert "64 MiB" in str(e.value) or str(h3.NOALLOC_SCRATCH_BYTES) in str(e.value)
