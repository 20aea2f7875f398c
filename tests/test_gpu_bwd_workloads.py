"""GPU parity of both backward passes on the workloads' own inputs (marked gpu).

For each bf16 workload, the inputs of its recipe (q, k, v ~ N(0, 1) rounded to bf16 and its decay
recipe; fewer batch entries and heads, full length and head dimension) and a seeded incoming gradient
dy go through the full form's backward and the chunkwise one (chunks of 64; on the longer sequences
also 128, and 32 -- the fp32 path -- on the longest), each held to the condition-aware gate of
``tests.test_gpu_bwd`` against one fp64 oracle evaluation.  The report lines are those of the parity report's backward rows at workload shapes.
"""
from __future__ import annotations

import numpy as np
import pytest

from bidirectional_linear_attention_lion_amd import inputs as lin
from tests.test_gpu_bwd import run_inputs

pytestmark = pytest.mark.gpu

# (workload, batch entries, heads, chunkwise chunk sizes)
CASES = [("vit_tiny_lit", 2, 3, (64,)), ("vit_base_d", 2, 2, (64,)), ("bert_large_s", 1, 2, (64, 128)),
         ("hires_d", 1, 2, (32, 64, 128))]


@pytest.mark.parametrize("name,B,H,Cs", CASES, ids=[c[0] for c in CASES])
def test_bwd_workload_inputs(name, B, H, Cs):
    wl = lin.WORKLOADS[name]
    inp = lin.make_inputs(wl, B=B, H=H)
    rng = np.random.default_rng(wl.seed + 1000)
    g32 = (rng.standard_normal((B, H, wl.L, wl.d), dtype=np.float32) * np.float32(0.1))
    gb = lin.round_bf16_bits(g32)
    dy = lin.bf16_bits_to_f64(gb)
    label = f"{name} B{B} H{H} L{wl.L} d{wl.d} kind={lin.KIND_NAME[wl.kind]} workload inputs"
    run_inputs((inp.q_dev, inp.k_dev, inp.v_dev, gb), (inp.q, inp.k, inp.v, dy), inp.log_lambda, wl.kind, False,
               wl.eps, (None,) + tuple(Cs), label)
