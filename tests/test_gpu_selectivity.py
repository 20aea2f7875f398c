"""GPU parity of the LION-S selectivity prologue (lion_selectivity) against the fp64 oracle (marked gpu).

log(lambda) = log sigmoid(x . w_h + b_h), key scale = lambda - 1, scaled keys = scale * k (the reading in
``oracle/lion_oracle.c``).  The device forms z from bf16 x and w on the matrix cores: each product is exact
in fp32 and the sum carries at most Dm 2^-24 sum_c |x_c w_c| of rounding; the fp32 log/exp add about
2^-20 relative.  That bound, computed per element from the oracle's inputs, is the tolerance.  The
prologue then feeds the attention (BERT-shaped LION-S workload) with the attention's own gates.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bidirectional_linear_attention_lion_amd import inputs as lin
from tests.gpu_util import report
from tests.parity import assert_parity, compare

pytestmark = pytest.mark.gpu


def _bf16(a32):
    bits = lin.round_bf16_bits(a32)
    return bits, lin.bf16_bits_to_f64(bits)


def _dev(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def run_case(B, L, H, Dm, d=64, bias=None, seed=0, in_place=False):
    import torch
    import bidirectional_linear_attention_lion_amd as lion
    rng = np.random.default_rng(seed)
    xb, x = _bf16(rng.standard_normal((B, L, Dm), dtype=np.float32))
    wb, w = _bf16((rng.standard_normal((H, Dm)) / np.sqrt(Dm)).astype(np.float32))
    bias = (rng.standard_normal(H) * 2).astype(np.float32) if bias is None else np.full(H, bias, np.float32)
    kb, k = _bf16(rng.standard_normal((B, H, L, d), dtype=np.float32))
    kd = _dev(kb)
    ll, ks, ko = lion.lion_selectivity(_dev(xb), _dev(wb), torch.from_numpy(bias).cuda(), k=kd,
                                       k_out=kd if in_place else None, want_key_scale=True)
    torch.cuda.synchronize()
    rll, rks, rko = oracle.selectivity(x, w, bias.astype(np.float64), k)
    zb = Dm * 2.0 ** -24 * np.einsum("blc,hc->bhl", np.abs(x), np.abs(w))
    ll_g = ll.cpu().numpy().astype(np.float64)
    ks_g = ks.cpu().numpy().astype(np.float64)
    ko_g = ko.float().cpu().numpy().astype(np.float64)
    e_ll = np.abs(ll_g - rll) / (zb + 2.0 ** -20 * (1 + np.abs(rll)))
    e_ks = np.abs(ks_g - rks) / (0.25 * zb + 2.0 ** -20)
    e_ko = np.abs(ko_g - rko) / (2.0 ** -8 * np.abs(rko) + np.abs(k) * (0.25 * zb + 2.0 ** -20)[..., None] + 1e-30)
    report(f"[selectivity] B{B} L{L} H{H} Dm{Dm} d{d}{' in place' if in_place else ''}: "
           f"log_lambda {e_ll.max():.3f}  key_scale {e_ks.max():.3f}  k_out {e_ko.max():.3f} (of the bound)")
    assert e_ll.max() <= 1.0 and e_ks.max() <= 1.0 and e_ko.max() <= 1.0
    return ll


@pytest.mark.parametrize("B,L,H,Dm", [(2, 17, 3, 64), (1, 1, 1, 32), (2, 64, 16, 1024), (1, 130, 20, 96),
                                      (3, 199, 12, 256)])
def test_selectivity(B, L, H, Dm):
    run_case(B, L, H, Dm, seed=B * 1000 + L)


def test_selectivity_in_place_keys():
    run_case(2, 33, 4, 64, in_place=True, seed=5)


def test_selectivity_feeds_attention():
    """The BERT-shaped LION-S workload with its decays made on the device from x, w, b = 3 (the
    workload's recipe), then the full form against the oracle fed the oracle's own decays."""
    import torch
    import bidirectional_linear_attention_lion_amd as lion
    B, L, H, Dm, d = 2, 512, 16, 1024, 64
    rng = np.random.default_rng(44)
    xb, x = _bf16(rng.standard_normal((B, L, Dm), dtype=np.float32))
    wb, w = _bf16((rng.standard_normal((H, Dm)) / np.sqrt(Dm)).astype(np.float32))
    bias = np.full(H, 3.0, np.float32)
    qb, q = _bf16(rng.standard_normal((B, H, L, d), dtype=np.float32))
    kb, k = _bf16(rng.standard_normal((B, H, L, d), dtype=np.float32))
    vb, v = _bf16(rng.standard_normal((B, H, L, d), dtype=np.float32))
    ll, _, _ = lion.lion_selectivity(_dev(xb), _dev(wb), torch.from_numpy(bias).cuda())
    den = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    y = lion.lion_attn_full(_dev(qb), _dev(kb), _dev(vb), ll, lion.MASK_S, 1e-6, den_out=den)
    torch.cuda.synchronize()
    rll, _, _ = oracle.selectivity(x, w, bias.astype(np.float64))
    yr, dr, an, ad = oracle.full(q, k, v, rll, lin.S, 1e-6, want_abs=True)
    rep = compare(y.float().cpu().numpy(), yr, dr, an, ad, "bf16", "bf16", d, L)
    report(f"[selectivity -> full] B{B} H{H} L{L} Dm{Dm}: {rep}")
    assert_parity(rep, "selectivity then full form")
