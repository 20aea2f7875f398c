"""The chunkwise form's no-allocation entry point (lion_attn_chunk_noalloc: scratch from the library's
built-in per-GPU array) against the workspace entry point (lion_attn_chunk), through the C ABI (marked
gpu).  Both run the same kernels on the same inputs, so their outputs and row sums must agree bit for
bit.  Two calls in a row, the second with a smaller input, then one that needs no scratch: the array
keeps the earlier call's contents, which the later calls must not read."""
from __future__ import annotations

import numpy as np
import pytest

from bidirectional_linear_attention_lion_amd import inputs as lin
from tests.gpu_util import report, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # (workload recipe, B, H, L, C): the first two take scratch (the long-sequence paths); the last, at
    # most 256 rows, runs in one launch with its states in LDS
    ("hires_d", 2, 12, 4097, 128),
    ("bert_large_s", 1, 4, 777, 64),
    ("vit_tiny_lit", 3, 3, 197, 64),
]


def _pair(name, B, H, L, C):
    import torch
    import bidirectional_linear_attention_lion_amd as lion
    wl = lin.WORKLOADS[name]
    need = lion.lion_attn_workspace_bytes(lion.FORM_CHUNK, B, H, L, wl.d, C, 1)
    print(f"no-alloc case {name} B{B} H{H} L{L} C{C}: workspace {need} bytes", flush=True)
    inp = lin.make_inputs(wl, B=B, H=H, L=L)
    q, k, v, ll = to_device(inp)
    den_a = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    den_b = torch.empty_like(den_a)
    y_a = lion.lion_attn_chunk(q, k, v, ll, wl.kind, C, wl.eps, den_out=den_a)
    y_b = torch.full_like(y_a, float("nan"))
    lion.lion_attn_chunk_noalloc(q, k, v, ll, wl.kind, C, wl.eps, y=y_b, den_out=den_b)
    torch.cuda.synchronize()
    return need, y_a, y_b, den_a, den_b


def test_noalloc_matches_workspace_entry_point():
    import torch
    needs = []
    for case in CASES:
        need, y_a, y_b, den_a, den_b = _pair(*case)
        needs.append(need)
        ya = y_a.view(torch.int16).cpu().numpy()
        yb = y_b.view(torch.int16).cpu().numpy()
        mism = int(np.count_nonzero(ya != yb))
        dmism = int(np.count_nonzero(den_a.cpu().numpy().view(np.int32) != den_b.cpu().numpy().view(np.int32)))
        report(f"[chunk_noalloc] {case}: {mism} output and {dmism} row-sum mismatches (bitwise) vs lion_attn_chunk")
        assert torch.isfinite(y_b.float()).all()
        assert mism == 0 and dmism == 0
    # the workspace query answers for every way the form can run (fp32 arithmetic included), an upper
    # bound of what these bf16 calls take
    assert needs[0] > needs[1] > 0
