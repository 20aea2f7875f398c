"""GPU parity of the full form's backward pass against the fp64 backward oracle (marked gpu).

The oracle's backward is pinned by finite differences of the forward definition
(``oracle_pins.pin_bwd_finite_differences``).  Every GPU call goes through the C ABI: the forward
(y, den) first, then ``lion_attn_full_bwd`` with fp32 gradients.

Gate (condition-aware, every element of dq, dk, dv and dlog(lambda)):
    |G_gpu - G_ref| <= tol RMS(G_ref) + C u A,
A the oracle's absolute-value companion of G (the same chain rule with every term replaced by its
magnitude and every difference by a sum; the forward's den and y enter with their own first-order
error, so a nearly cancelling row sum widens the bound as in the forward's gate), u = 2^-8 (twice
bf16's unit roundoff), C = 4: the terms a gradient is summed from carry the bf16 rounding of phi(q) or
phi(k) and of dS or P / den (u/2 each), the forward's row sum and y (3u per term, bounded inside the
companion) and the bf16 rounding of y that delta reads (u/2).  The companion matters most for dq: y does
not change when phi(q_i) is scaled, so the exact dphi(q_i) is orthogonal to phi(q_i) and its two parts
(through the numerator and through delta) cancel along that direction -- completely at L = 1.
A literal report (max |dG| / RMS) is printed for every case; inputs with positive q and k (every score
positive, no row sum cancels) and the workloads' signed inputs are both covered.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bidirectional_linear_attention_lion_amd import inputs as lin
from tests.gpu_util import report

pytestmark = pytest.mark.gpu

BWD_TOL, BWD_U, BWD_C = 2e-2, 2.0 ** -8, 4.0


def _bf16(rng, shape, positive=False):
    x = rng.standard_normal(shape, dtype=np.float32)
    if positive:
        x = np.abs(x) + np.float32(0.05)
    bits = lin.round_bf16_bits(x)
    return bits, lin.bf16_bits_to_f64(bits)


def _dev(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def run_case(B, H, L, d, kind, causal=False, positive=True, seed=0, eps=1e-6, tag="", C=None):
    """One case through the C ABI against the oracle; C given: the chunkwise backward with chunks of C."""
    rng = np.random.default_rng(seed)
    shape = (B, H, L, d)
    qb, q = _bf16(rng, shape, positive)
    kb, k = _bf16(rng, shape, positive)
    vb, v = _bf16(rng, shape)
    gb, dy = _bf16(rng, shape)
    ll32 = lin.random_inputs(B, H, L, d, kind, dtype="bf16", seed=seed + 1).log_lambda
    form = "bwd" if C is None else f"chunk_bwd C{C}"
    label = (f"B{B} H{H} L{L} d{d} kind={lin.KIND_NAME[kind]}{' causal' if causal else ''} "
             f"{'positive' if positive else 'signed'} {tag}")
    return run_inputs((qb, kb, vb, gb), (q, k, v, dy), ll32, kind, causal, eps, (C,), label)[form]


def run_inputs(bits, vals, ll32, kind, causal, eps, Cs, label):
    """The forward and the backward passes through the C ABI on given bf16 inputs (bit patterns and their
    exact values: q, k, v, dy), each held to the condition-aware gate against one oracle evaluation.
    Cs lists the passes: None the full form's backward, an integer the chunkwise one with chunks of it.
    Returns {form: literal errors}."""
    import torch
    import bidirectional_linear_attention_lion_amd as lion
    qb, kb, vb, gb = bits
    q, k, v, dy = vals
    B, H, L, d = q.shape
    ll = None if ll32 is None else torch.from_numpy(ll32).cuda()
    mk = kind | (lion.CAUSAL if causal else 0)
    qd, kd, vd, gd = _dev(qb), _dev(kb), _dev(vb), _dev(gb)
    den = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    y = lion.lion_attn_full(qd, kd, vd, ll, mk, eps, den_out=den)
    got_all = {}
    for C in Cs:
        if C is None:
            out = lion.lion_attn_full_bwd(qd, kd, vd, ll, mk, y, den, gd, grad_dtype=torch.float32)
        else:
            out = lion.lion_attn_chunk_bwd(qd, kd, vd, ll, mk, C, y, den, gd, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        got_all["bwd" if C is None else f"chunk_bwd C{C}"] = dict(zip(("dq", "dk", "dv", "dll"), out))
    res = oracle.full_bwd(q, k, v, None if ll32 is None else ll32.astype(np.float64),
                          kind | (oracle.CAUSAL if causal else 0), eps, dy, want_abs=True)
    names = ("dq", "dk", "dv", "dll")
    ref, absc = dict(zip(names, res[:4])), dict(zip(names, res[4:]))
    out_errs = {}
    for form, got in got_all.items():
        errs, gates = {}, {}
        for name in names:
            if ref[name] is None:
                continue
            g = got[name].cpu().numpy().astype(np.float64).reshape(ref[name].shape)
            assert np.all(np.isfinite(g)), f"{form} {name}: non-finite gradients"
            rms = float(np.sqrt(np.mean(ref[name] ** 2)))
            err = np.abs(g - ref[name])
            errs[name] = float(np.max(err)) / max(rms, 1e-300)
            bound = BWD_TOL * rms + BWD_C * BWD_U * absc[name]
            # a zero bound (an exactly zero gradient, e.g. dlog(lambda) at L = 1) admits only a zero error
            ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
            gates[name] = float(np.max(ratio))
        report(f"[{form}] {label}: literal " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + " | gate "
               + " ".join(f"{n}={e:.3f}" for n, e in gates.items()))
        for name, gv in gates.items():
            assert gv <= 1.0, f"{form} {name}: condition-aware gate {gv:.3f} > 1 ({label})"
        out_errs[form] = errs
    return out_errs


CASES_L = [1, 17, 64, 100, 197, 300, 600]


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_positive(kind, causal):
    for L in CASES_L:
        run_case(1, 2, L, 64, kind, causal=causal, seed=1000 + L)


@pytest.mark.parametrize("d", [32, 128])
def test_bwd_head_dims(d):
    for kind in (lin.LIT, lin.D, lin.S):
        run_case(1, 2, 150, d, kind, seed=2000 + d)


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
def test_bwd_sides_apart(kind):
    # L <= 256, more than 256 (batch, head) pairs: the query and key sides of a pair run in workgroups of
    # their own (B H = 272 leaves the last group of 16 workgroups partly empty); the small cases of the
    # tests above take the same route
    for B, H, L, d, causal in ((64, 5, 197, 64, False), (32, 9, 256, 64, True), (128, 3, 37, 32, False),
                               (257, 1, 1, 64, False), (16, 17, 100, 64, False), (64, 5, 129, 32, True)):
        run_case(B, H, L, d, kind, causal=causal, positive=False, seed=5000 + L, tag="sides apart")


@pytest.mark.parametrize("kind", [lin.LIT, lin.S])
def test_bwd_one_workgroup_per_pair(kind):
    # L <= 256 and 128 < B H <= 256, LION-LIT or LION-S: one workgroup per (batch, head) with all four
    # tiles (chunks of 64, 128 and 256; two tiles per wave at 256)
    for B, H, L, d, causal in ((64, 3, 197, 64, False), (32, 8, 256, 64, True), (129, 1, 37, 32, False),
                               (200, 1, 1, 64, False), (16, 16, 100, 64, False), (43, 3, 129, 32, True)):
        run_case(B, H, L, d, kind, causal=causal, positive=False, seed=6000 + L, tag="one workgroup per pair")


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
def test_bwd_signed(kind):
    for L in (64, 197, 512):
        run_case(2, 3, L, 64, kind, positive=False, seed=3000 + L)
    run_case(1, 2, 300, 64, kind, causal=True, positive=False, seed=3999)
