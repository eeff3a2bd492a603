"""GPU parity of per-segment AdaLN (modulate and gate-residual) against the fp64 oracle."""
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
    shift = normal_bf16_bits((s, c), seed + 2, std=0.1)
    scale = normal_bf16_bits((s, c), seed + 3, std=0.1)
    gate = normal_bf16_bits((s, c), seed + 4, std=0.1)
    return x, b, shift, scale, gate


def _run(mode, bits, a, e, cu):
    h3 = _h3()
    x, b, shift, scale, gate = bits
    xd = to_device(x[a:e])
    y = torch.empty_like(xd)
    if mode == 0:
        h3.adaln_segment(0, xd, None, to_device(shift), to_device(scale), None, y, a, e, cu, EPS)
    else:
        h3.adaln_segment(1, xd, to_device(b[a:e]), None, None, to_device(gate), y, a, e, cu, 0.0)
    torch.cuda.synchronize()
    return to_bits(y)


@pytest.mark.parametrize("c", [512, 1000, 7168, 8192])
@pytest.mark.parametrize("mode", [0, 1])
def test_adaln_intervals(c, mode):
    cu = segment_offsets([96, 160, 1, 255])
    n = cu[-1]
    bits = _inputs(n, c, 4, seed=900 + c)
    for a, e in [(0, n), (0, 256), (256, 512), (50, 300), (95, 97), (256, 257)]:
        say("adaln", c, mode, a, e)
        got = _run(mode, bits, a, e, cu)
        ref = oracle.adaln_rows(mode, bits[0][a:e], bits[1][a:e], bits[2], bits[3], bits[4], a, e, cu, EPS)
        compare(got, ref, f"adaln c={c} mode={mode} [{a},{e})")


def test_adaln_gate_zero_is_identity():
    cu = segment_offsets([40, 60])
    x, b, shift, scale, gate = _inputs(100, 7168, 2, seed=950)
    got = _run(1, (x, b, shift, scale, np.zeros_like(gate)), 0, 100, cu)
    assert np.array_equal(got, x)


def test_adaln_per_rank_equals_global():
    """Applying per virtual rank with clipped tables gives the global result bit for bit."""
    w = WORKLOADS["8k_p6"]
    bits = _inputs(w.n_tokens, 7168, w.n_segments, seed=960)
    for mode in (0, 1):
        whole = _run(mode, bits, 0, w.n_tokens, w.cu)
        for a, cnt in oracle.partition(w.n_tokens, w.world):
            assert np.array_equal(_run(mode, bits, a, a + cnt, w.cu), whole[a:a + cnt])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_adaln_workload(name):
    """[N, 7168] at the workload's real size, every virtual rank's interval, sampled rows
    (every clipped-segment edge included)."""
    h3 = _h3()
    w = WORKLOADS[name]
    n, c = w.n_tokens, 7168
    say("adaln workload", name)
    x = normal_bf16((n, c), seed=w.seed + 20, device="cuda")
    b = normal_bf16((n, c), seed=w.seed + 21, device="cuda")
    prm = [normal_bf16((w.n_segments, c), seed=w.seed + 22 + i, std=0.1, device="cuda") for i in range(3)]
    y = torch.empty_like(x)
    yg = torch.empty_like(x)
    parts = [h3.partition(n, w.world, i) for i in range(w.world)]
    for a, cnt in parts:
        h3.adaln_segment(0, x[a:a + cnt], None, prm[0], prm[1], None, y[a:a + cnt], a, a + cnt, w.cu, EPS)
        h3.adaln_segment(1, x[a:a + cnt], b[a:a + cnt], None, None, prm[2], yg[a:a + cnt], a, a + cnt, w.cu, 0.0)
    torch.cuda.synchronize()
    xb, bb = to_bits(x), to_bits(b)
    pb = [to_bits(t) for t in prm]
    for a, cnt in parts:
        rows = sample_rows([0] + [e for _, _, e in oracle.clip_segments(w.cu, a, a + cnt)],
                           seed=w.seed + a, per_tile=512, limit=600)
        for mode, out in ((0, y), (1, yg)):
            ref = oracle.adaln_rows(mode, xb[a:a + cnt], bb[a:a + cnt], pb[0], pb[1], pb[2], a, a + cnt, w.cu,
                                    EPS if mode == 0 else 0.0, rows=rows)
            compare(to_bits(out[a:a + cnt])[rows], ref, f"{name} mode {mode} rank@{a}")
