"""Helpers of the GPU tests: device copies of seeded inputs, oracle references, report lines."""
from __future__ import annotations

import os

import numpy as np

import oracle
from bidirectional_linear_attention_lion_amd import inputs as lin


def to_device(inp: "lin.Inputs"):
    import torch
    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ll = None if inp.log_lambda is None else torch.from_numpy(inp.log_lambda).cuda()
    return dev(inp.q_dev), dev(inp.k_dev), dev(inp.v_dev), ll


def oracle_full(inp: "lin.Inputs", eps: float, causal: bool = False):
    kind = inp.wl.kind | (oracle.CAUSAL if causal else 0)
    return oracle.full(inp.q, inp.k, inp.v, inp.log_lambda_f64, kind, eps, want_abs=True)


def oracle_rows(inp: "lin.Inputs", eps: float, rows, causal: bool = False):
    kind = inp.wl.kind | (oracle.CAUSAL if causal else 0)
    return oracle.rows(inp.q, inp.k, inp.v, inp.log_lambda_f64, kind, eps, rows, want_abs=True)


def sample_rows(B, H, L, n, seed=0):
    """Row ids (bh * L + i): first/last rows, tile and chunk boundaries, plus random rows."""
    rng = np.random.default_rng(seed)
    special = sorted({0, 1, 15, 16, 31, 32, 63, 64, 127, 128, 255, 256, L // 2, L - 2, L - 1})
    special = [i for i in special if 0 <= i < L]
    bhs = rng.integers(0, B * H, size=len(special))
    ids = [int(b) * L + i for b, i in zip(bhs, special)]
    ids += list(rng.integers(0, B * H * L, size=max(0, n - len(ids))))
    return np.unique(np.array(ids, dtype=np.int64))


def report(line: str):
    print(line, flush=True)
    path = os.environ.get("LION_PARITY_REPORT")
    if path:
        with open(path, "a") as fh:
            fh.write(line + "\n")
