"""GPU parity of the gated AdaLN chain (one sub-block's gated residual, modulated
by the next sub-block's parameters) against the fp64 oracle; its stored
residual is bit-equal to the unfused gate call, and for a zero gate its output
is bit-equal to the plain modulation."""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, segment_offsets
from synth.inputs import normal_bf16, normal_bf16_bits
from tests.gpu_util import compare, say, sample_rows, to_bits, to_device

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _h3():
    import ulysses_layout_amd as h3
    return h3


def _inputs(n, c, s, seed):
    x = normal_bf16_bits((n, c), seed)
    b = normal_bf16_bits((n, c), seed + 1)
    shift, scale, gate = (normal_bf16_bits((s, c), seed + 2 + i, std=0.1) for i in range(3))
    return x, b, gate, shift, scale


def _chain(x, b, gate, shift, scale, a, e, cu):
    """The fused call, and the unfused gate call, on the same device inputs."""
    h3 = _h3()
    resid, y = torch.empty_like(x), torch.empty_like(x)
    info = h3.adaln_gate_modulate(x, b, gate, shift, scale, resid, y, a, e, cu, EPS)
    r2 = torch.empty_like(x)
    h3.adaln_segment(h3.H3_ADALN_GATE_RESIDUAL, x, b, None, None, gate, r2, a, e, cu, 0.0)
    torch.cuda.synchronize()
    return resid, y, r2, info


@pytest.mark.parametrize("c", [512, 1000, 7168, 8192])
def test_chain_intervals(c):
    cu = segment_offsets([96, 160, 1, 255])
    n = cu[-1]
    x, b, gate, shift, scale = _inputs(n, c, 4, seed=1200 + c)
    gd, shd, scd = to_device(gate), to_device(shift), to_device(scale)
    for a, e in [(0, n), (0, 256), (256, 512), (50, 300), (95, 97), (256, 257)]:
        say("adaln chain", c, a, e)
        resid, y, r2, info = _chain(to_device(x[a:e]), to_device(b[a:e]), gd, shd, scd, a, e, cu)
        r_ref, y_ref = oracle.adaln_gate_modulate(x[a:e], b[a:e], gate, shift, scale, a, e, cu, EPS)
        compare(to_bits(resid), r_ref, f"chain resid c={c} [{a},{e})")
        compare(to_bits(y), y_ref, f"chain y c={c} [{a},{e})")
        assert torch.equal(resid.view(torch.int16), r2.view(torch.int16))
        assert info.launches == 1
        assert info.bytes_written == 2 * (e - a) * c * 2


def test_chain_zero_gate_is_modulation_of_x():
    h3 = _h3()
    cu = segment_offsets([40, 60])
    x, b, gate, shift, scale = _inputs(100, 7168, 2, seed=1250)
    xd = to_device(x)
    resid, y, _, _ = _chain(xd, to_device(b), to_device(np.zeros_like(gate)), to_device(shift),
                               to_device(scale), 0, 100, cu)
    ym = torch.empty_like(xd)
    h3.adaln_segment(h3.H3_ADALN_MODULATE, xd, None, to_device(shift), to_device(scale), None, ym, 0, 100, cu, EPS)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(resid), x)
    assert torch.equal(y.view(torch.int16), ym.view(torch.int16))


@pytest.mark.parametrize("name", ["8k_p6", "128k_p4_qkvg", "250k_p8_qkvg"])
def test_chain_workload(name):
    """[N, 7168] at the workload's size, every virtual rank's interval: the
    residual bit-equal to the unfused gate call on every row, both outputs
    against the oracle on sampled rows."""
    h3 = _h3()
    w = WORKLOADS[name]
    n, c = w.n_tokens, 7168
    say("adaln chain workload", name)
    x = normal_bf16((n, c), seed=w.seed + 30, device="cuda")
    b = normal_bf16((n, c), seed=w.seed + 31, device="cuda")
    prm = [normal_bf16((w.n_segments, c), seed=w.seed + 32 + i, std=0.1, device="cuda") for i in range(3)]
    resid, y = torch.empty_like(x), torch.empty_like(x)
    r2 = torch.empty_like(x)
    parts = [h3.partition(n, w.world, i) for i in range(w.world)]
    for a, cnt in parts:
        s = slice(a, a + cnt)
        h3.adaln_gate_modulate(x[s], b[s], prm[0], prm[1], prm[2], resid[s], y[s], a, a + cnt, w.cu, EPS)
        h3.adaln_segment(h3.H3_ADALN_GATE_RESIDUAL, x[s], b[s], None, None, prm[0], r2[s], a, a + cnt, w.cu, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(resid.view(torch.int16), r2.view(torch.int16))
    pb = [to_bits(t) for t in prm]
    for a, cnt in parts:
        rows = sample_rows([0] + [e for _, _, e in oracle.clip_segments(w.cu, a, a + cnt)],
                           seed=w.seed + a + 1, per_tile=512, limit=300)
        idx = torch.from_numpy(rows + a).cuda()
        xs, bs = to_bits(x.index_select(0, idx)), to_bits(b.index_select(0, idx))
        # the oracle over the sampled rows only: pass them as the interval's rows they are
        xr = np.zeros((cnt, c), np.uint16)
        br = np.zeros((cnt, c), np.uint16)
        xr[rows], br[rows] = xs, bs
        r_ref, y_ref = oracle.adaln_gate_modulate(xr, br, pb[0], pb[1], pb[2], a, a + cnt, w.cu, EPS, rows=rows)
        compare(to_bits(resid.index_select(0, idx)), r_ref, f"{name} chain resid rank@{a}")
        compare(to_bits(y.index_select(0, idx)), y_ref, f"{name} chain y rank@{a}")
