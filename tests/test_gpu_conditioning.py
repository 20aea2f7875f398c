"""How close fp32 arithmetic comes to the literal gate on the BERT-shaped LION-S workload (marked gpu).

The workload's inputs are exact bf16 values.  Here every form computes in fp32 (phi, the products on the
fp32 matrix cores, the states): the bf16 inputs with LION_FP32_ARITH (the RNN form's own arithmetic is
fp32), and the same values upcast to fp32 inputs -- the most accurate arithmetic the library has -- and
writes fp32 outputs.  Every row of the full workload (B32 H16 L512) is compared with the
fp64 oracle.  Asserted: the condition-aware gate with fp32's own unit roundoff, which every correct fp32
evaluation meets.  Reported, not asserted: the literal error max |dY| / RMS(Y) against the workload's 2e-2,
and, for the worst-conditioned row, its condition number kappa = sum_j |P_ij| / |den_i|, its |y| / RMS and
the first-order fp32 rounding bound u (sum_j |P_ij| |v_j| + |y_i| sum_j |P_ij|) / |den_i| / RMS with
u = 2^-24 -- on this workload that bound is about 0.3 RMS, so whether an fp32 evaluation lands under 2e-2
depends on how its roundings happen to cancel, not on the method."""
from __future__ import annotations

import numpy as np
import pytest

from bidirectional_linear_attention_lion_amd import inputs as lin
from tests.gpu_util import oracle_full, report, to_device
from tests.parity import compare

pytestmark = pytest.mark.gpu


def test_fp32_arithmetic_on_bert_large_s():
    import torch
    import bidirectional_linear_attention_lion_amd as lion
    wl = lin.WORKLOADS["bert_large_s"]
    inp = lin.make_inputs(wl)
    yr, dr, an, ad = oracle_full(inp, wl.eps)
    rms = float(np.sqrt(np.mean(yr ** 2)))
    kappa = ad / np.abs(dr)
    bound = 2.0 ** -24 * (an + np.abs(yr) * ad[..., None]) / np.abs(dr)[..., None]
    worst = np.unravel_index(np.argmax(bound.max(-1)), bound.shape[:-1])
    report(f"[fp32 arithmetic] bert_large_s B{wl.B} H{wl.H} L{wl.L}: worst row {tuple(int(x) for x in worst)} "
           f"kappa={kappa[worst]:.4g} |y|/RMS={np.abs(yr[worst]).max() / rms:.4g} "
           f"fp32 first-order bound/RMS={bound[worst].max() / rms:.3g}; kappa max={kappa.max():.4g} "
           f"median={np.median(kappa):.3g}")
    # the workload's bf16 inputs with fp32 arithmetic, and the same values upcast to fp32 inputs
    qb, kb, vb, ll = to_device(inp)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    S32 = lin.S | lion.FP32_ARITH
    f32 = torch.float32
    runs = {
        "full (bf16 in, fp32 arithmetic)": lambda: lion.lion_attn_full(qb, kb, vb, ll, S32, wl.eps, y_dtype=f32),
        "chunk C=64 (bf16 in, fp32 arithmetic)": lambda: lion.lion_attn_chunk(qb, kb, vb, ll, S32, 64, wl.eps, y_dtype=f32),
        "chunk C=128 (bf16 in, fp32 arithmetic)": lambda: lion.lion_attn_chunk(qb, kb, vb, ll, S32, 128, wl.eps,
                                                                               y_dtype=f32),
        "birnn (bf16 in)": lambda: lion.lion_attn_birnn(qb, kb, vb, ll, "s", wl.eps, y_dtype=f32),
        "full (fp32 in)": lambda: lion.lion_attn_full(q, k, v, ll, "s", wl.eps),
        "chunk C=128 (fp32 in)": lambda: lion.lion_attn_chunk(q, k, v, ll, "s", 128, wl.eps),
        "birnn (fp32 in)": lambda: lion.lion_attn_birnn(q, k, v, ll, "s", wl.eps),
    }
    for name, fn in runs.items():
        y = fn()
        torch.cuda.synchronize()
        yg = y.cpu().numpy().astype(np.float64)
        rep = compare(yg, yr, dr, an, ad, "f32", "f32", wl.d, wl.L)
        lit = float(np.max(np.abs(yg - yr)) / rms)
        report(f"[fp32 arithmetic] {name}: literal max|dY|/RMS={lit:.3e} (workload gate 2e-2) {rep}")
        assert np.all(np.isfinite(yg))
        assert rep.gate_c <= 1.0, f"{name}: {rep}"
