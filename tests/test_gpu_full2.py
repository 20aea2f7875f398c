"""GPU parity of the two-order full form (lion_attn_full2: the masks of the tokens' own order and of a
second order averaged) against the fp64 oracle ``oracle.full2`` (marked gpu).  Gates as for the other
forms (``parity.py``); the chunkwise two-order form (lion_attn_chunk2) is held to the same oracle.  Orders: the column-major raster of an image's patch grid (class token first),
the reversed order and random permutations."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bidirectional_linear_attention_lion_amd import inputs as lin
from tests.gpu_util import report, to_device
from tests.parity import assert_parity, compare

pytestmark = pytest.mark.gpu


def check(inp, order, eps=1e-6, tag=""):
    import torch
    import bidirectional_linear_attention_lion_amd as lion
    wl = inp.wl
    q, k, v, ll = to_device(inp)
    o = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).cuda()
    den = torch.empty((wl.B, wl.H, wl.L), dtype=torch.float32, device="cuda")
    y = lion.lion_attn_full2(q, k, v, ll, wl.kind, o, eps, den_out=den)
    torch.cuda.synchronize()
    yr, dr, an, ad = oracle.full2(inp.q, inp.k, inp.v, inp.log_lambda_f64, wl.kind, eps, order, want_abs=True)
    out_dtype = "f32" if wl.dtype == "f32" else "bf16"
    rep = compare(y.float().cpu().numpy(), yr, dr, an, ad, wl.dtype, out_dtype, wl.d, wl.L)
    den_err = float(np.max(np.abs(den.cpu().numpy() - dr) / (ad + 1e-30)))
    report(f"[full2] B{wl.B} H{wl.H} L{wl.L} d{wl.d} {wl.dtype} kind={lin.KIND_NAME[wl.kind]} {tag}: {rep} "
           f"den_relerr={den_err:.2e}")
    assert_parity(rep, f"full2 {tag}", require_literal=wl.kind == lin.LIT)
    u = 2.0 ** -8 if wl.dtype == "bf16" else (wl.d + wl.L) * 2.0 ** -24
    assert den_err <= 3 * u


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_full2_image_orders(kind, dtype):
    for rows, cols in ((4, 4), (8, 8), (14, 14)):
        L = 1 + rows * cols
        inp = lin.random_inputs(2, 3, L, 64, kind, dtype=dtype, seed=600 + L)
        check(inp, lin.column_major_order(rows, cols), tag=f"column-major {rows}x{cols}")


@pytest.mark.parametrize("kind", [lin.D, lin.S])
def test_full2_permutations(kind):
    rng = np.random.default_rng(61)
    for L in (1, 2, 33, 100, 600):
        inp = lin.random_inputs(1, 2, L, 64, kind, dtype="bf16", seed=700 + L)
        check(inp, rng.permutation(L), tag=f"random permutation L={L}")
        check(inp, np.arange(L)[::-1], tag=f"reversed L={L}")


@pytest.mark.parametrize("d", [32, 128])
def test_full2_head_dims(d):
    for kind in (lin.D, lin.S):
        inp = lin.random_inputs(1, 2, 197, d, kind, dtype="bf16", seed=800 + d)
        check(inp, lin.column_major_order(14, 14), tag=f"column-major d={d}")


def test_full2_vit_base_shape():
    """The ViT-Base-shaped LION-D workload with its 14 x 14 patches in both raster orders (LION-D natural)."""
    wl = lin.WORKLOADS["vit_base_d"]
    inp = lin.make_inputs(wl, B=4)
    check(inp, lin.column_major_order(14, 14), eps=wl.eps, tag="vit_base_d B4 column-major")


def check_chunk2(inp, order, C, eps=1e-6, tag=""):
    """The chunkwise two-order form (lion_attn_chunk2) against the same oracle and gates."""
    import torch
    import bidirectional_linear_attention_lion_amd as lion
    wl = inp.wl
    q, k, v, ll = to_device(inp)
    o = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).cuda()
    den = torch.empty((wl.B, wl.H, wl.L), dtype=torch.float32, device="cuda")
    y = lion.lion_attn_chunk2(q, k, v, ll, wl.kind, o, C, eps, den_out=den)
    torch.cuda.synchronize()
    yr, dr, an, ad = oracle.full2(inp.q, inp.k, inp.v, inp.log_lambda_f64, wl.kind, eps, order, want_abs=True)
    out_dtype = "f32" if wl.dtype == "f32" else "bf16"
    rep = compare(y.float().cpu().numpy(), yr, dr, an, ad, wl.dtype, out_dtype, wl.d, wl.L)
    den_err = float(np.max(np.abs(den.cpu().numpy() - dr) / (ad + 1e-30)))
    report(f"[chunk2 C{C}] B{wl.B} H{wl.H} L{wl.L} d{wl.d} {wl.dtype} kind={lin.KIND_NAME[wl.kind]} {tag}: {rep} "
           f"den_relerr={den_err:.2e}")
    assert_parity(rep, f"chunk2 {tag}", require_literal=wl.kind == lin.LIT)
    u = 2.0 ** -8 if wl.dtype == "bf16" else (wl.d + wl.L) * 2.0 ** -24
    assert den_err <= 3 * u


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk2_image_orders(kind, dtype):
    for rows, cols in ((4, 4), (14, 14)):
        L = 1 + rows * cols
        inp = lin.random_inputs(2, 3, L, 64, kind, dtype=dtype, seed=650 + L)
        check_chunk2(inp, lin.column_major_order(rows, cols), 64, tag=f"column-major {rows}x{cols}")


@pytest.mark.parametrize("kind", [lin.D, lin.S])
def test_chunk2_permutations_and_chunk_sizes(kind):
    rng = np.random.default_rng(62)
    for L, C in ((1, 64), (33, 16), (100, 32), (600, 128), (600, 256)):
        inp = lin.random_inputs(1, 2, L, 64, kind, dtype="bf16", seed=750 + L)
        check_chunk2(inp, rng.permutation(L), C, tag=f"random permutation L={L}")
        check_chunk2(inp, np.arange(L)[::-1], C, tag=f"reversed L={L}")


def test_chunk2_head_dims():
    for d in (32, 128):
        inp = lin.random_inputs(1, 2, 197, d, lin.S, dtype="bf16", seed=850 + d)
        check_chunk2(inp, lin.column_major_order(14, 14), 64, tag=f"column-major d={d}")
