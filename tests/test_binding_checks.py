"""The Python binding rejects, before any call into the library, every tensor argument the C ABI
cannot take as given: the ABI sees only pointers and sizes, so a transposed view, a wrong shape or
dtype, or a tensor on another device would otherwise be misread silently (CPU only: CPU tensors hit
every check that comes before the device check, and the device check itself)."""
import pytest
import torch

import bidirectional_linear_attention_lion_amd as lion
from bidirectional_linear_attention_lion_amd import binding

B, H, L, D = 2, 3, 17, 32
BF, F32 = torch.bfloat16, torch.float32


def qkv(dtype=BF):
    return [torch.zeros(B, H, L, D, dtype=dtype) for _ in range(3)]


def _raises(match, fn, *a, **kw):
    with pytest.raises(lion.LionArgumentError, match=match):
        fn(*a, **kw)


FORWARD = {
    "full": lambda q, k, v, ll, kind, **kw: lion.lion_attn_full(q, k, v, ll, kind, **kw),
    "chunk": lambda q, k, v, ll, kind, **kw: lion.lion_attn_chunk(q, k, v, ll, kind, 64, **kw),
    "birnn": lambda q, k, v, ll, kind, **kw: lion.lion_attn_birnn(q, k, v, ll, kind, **kw),
    "full2": lambda q, k, v, ll, kind, **kw: lion.lion_attn_full2(q, k, v, ll, kind, torch.arange(L, dtype=torch.int32), **kw),
    "chunk2": lambda q, k, v, ll, kind, **kw: lion.lion_attn_chunk2(q, k, v, ll, kind, torch.arange(L, dtype=torch.int32), 64, **kw),
}


@pytest.mark.parametrize("form", list(FORWARD))
def test_transposed_projection_is_rejected(form):
    # the usual model layout [B, L, H, d] viewed as [B, H, L, d]: same shape, wrong strides
    q = torch.zeros(B, L, H, D, dtype=BF).transpose(1, 2)
    _, k, v = qkv()
    _raises("q is not contiguous", FORWARD[form], q, k, v, None, "lit")


@pytest.mark.parametrize("form", list(FORWARD))
def test_forward_rejections(form):
    fn = FORWARD[form]
    q, k, v = qkv()
    _raises("k has shape", fn, q, k[:, :, :-1], v, None, "lit")
    _raises("v has dtype", fn, q, k, v.float(), None, "lit")
    _raises("k is not contiguous", fn, q, k.transpose(2, 3).contiguous().transpose(2, 3), v, None, "lit")
    _raises("unsupported dtype", fn, q.double(), k.double(), v.double(), None, "lit")
    _raises("4-D", fn, q[0], k, v, None, "lit")
    _raises("log_lambda must be None", fn, q, k, v, torch.zeros(H), "lit")
    _raises("log_lambda is required", fn, q, k, v, None, "d")
    _raises("log_lambda has shape", fn, q, k, v, torch.zeros(B, H, L), "d")
    _raises("log_lambda has shape", fn, q, k, v, torch.zeros(H), "s")
    _raises("log_lambda has dtype", fn, q, k, v, torch.zeros(H, dtype=torch.float64), "d")
    _raises("log_lambda has dtype", fn, q, k, v, torch.zeros(B, H, L, dtype=BF), "s")
    _raises("log_lambda is not contiguous", fn, q, k, v, torch.zeros(B, L, H).transpose(1, 2), "s")
    _raises("unknown mask kind", fn, q, k, v, None, "x")
    _raises("unknown mask kind", fn, q, k, v, None, 3)
    _raises("y has shape", fn, q, k, v, None, "lit", y=torch.zeros(B, H, L, D - 1, dtype=BF))
    _raises("y has dtype", fn, q, k, v, None, "lit", y=torch.zeros(B, H, L, D, dtype=torch.float16))
    _raises("y_dtype", fn, q, k, v, None, "lit", y_dtype=torch.float16)
    _raises("y_dtype", fn, *qkv(F32), None, "lit", y_dtype=BF)
    _raises("den_out has shape", fn, q, k, v, None, "lit", den_out=torch.zeros(B, H, L + 1))
    _raises("den_out has dtype", fn, q, k, v, None, "lit", den_out=torch.zeros(B, H, L, dtype=BF))
    # everything valid but on the CPU: the library has no CPU path
    _raises("GPU only", fn, q, k, v, None, "lit")
    _raises("GPU only", fn, q, k, v, torch.zeros(H), "d")


def test_device_mismatch_is_rejected():
    q, k, v = qkv()
    km = torch.zeros(B, H, L, D, dtype=BF, device="meta")
    _raises("k is on meta", lion.lion_attn_full, q, km, v, None, "lit")


def test_order_rejections():
    q, k, v = qkv()
    _raises("order has dtype", lion.lion_attn_full2, q, k, v, None, "lit", torch.arange(L))          # int64
    _raises("order has shape", lion.lion_attn_full2, q, k, v, None, "lit", torch.arange(L - 1, dtype=torch.int32))
    _raises("order is required", lion.lion_attn_chunk2, q, k, v, None, "lit", None)


def test_workspace_rejections():
    q, k, v = qkv()
    ws = torch.zeros(64, 2, dtype=torch.uint8).t()
    _raises("workspace must be a contiguous", binding._workspace, lion.FORM_CHUNK, B, H, L, D, 64, 1, ws, q.device)
    _raises("workspace is on meta", binding._workspace, lion.FORM_CHUNK, B, H, L, D, 64, 1,
            torch.zeros(64, dtype=torch.uint8, device="meta"), q.device)


BACKWARD = {
    "full_bwd": lambda *a, **kw: lion.lion_attn_full_bwd(*a, **kw),
    "chunk_bwd": lambda q, k, v, ll, kind, y, den, dy, **kw: lion.lion_attn_chunk_bwd(q, k, v, ll, kind, 32, y, den,
                                                                                       dy, **kw),
}


@pytest.mark.parametrize("form", list(BACKWARD))
def test_backward_rejections(form):
    fn = BACKWARD[form]
    q, k, v = qkv()
    y, dy = torch.zeros_like(q), torch.zeros_like(q)
    den = torch.ones(B, H, L)
    ll = torch.zeros(B, H, L)
    _raises("y has shape", fn, q, k, v, ll, "s", y[:, :, 1:], den, dy)
    _raises("den has dtype", fn, q, k, v, ll, "s", y, den.double(), dy)
    _raises("den is required", fn, q, k, v, ll, "s", y, None, dy)
    _raises("dy is not contiguous", fn, q, k, v, ll, "s", y, den, dy.transpose(2, 3).contiguous().transpose(2, 3))
    _raises("dq has dtype", fn, q, k, v, ll, "s", y, den, dy, dq=torch.zeros(B, H, L, D))
    _raises("dv has shape", fn, q, k, v, ll, "s", y, den, dy, dv=torch.zeros(B, H, L, D + 1, dtype=BF))
    _raises("grad_dtype", fn, q, k, v, ll, "s", y, den, dy, grad_dtype=torch.float16)
    _raises("dlog_lambda has shape", fn, q, k, v, ll, "s", y, den, dy, dlog_lambda=torch.zeros(H))
    _raises("dlog_lambda must be None", fn, q, k, v, None, "lit", y, den, dy, dlog_lambda=torch.zeros(H))
    _raises("GPU only", fn, q, k, v, ll, "s", y, den, dy)


def test_selectivity_rejections():
    Dm = 64
    x = torch.zeros(B, L, Dm, dtype=BF)
    w = torch.zeros(H, Dm, dtype=BF)
    bias = torch.zeros(H)
    k = torch.zeros(B, H, L, D, dtype=BF)
    _raises("x must be a 3-D", lion.lion_selectivity, x[0], w, bias)
    _raises("w has shape", lion.lion_selectivity, x, torch.zeros(H, Dm + 32, dtype=BF), bias)
    _raises("x has dtype", lion.lion_selectivity, x.float(), w, bias)
    _raises("bias has dtype", lion.lion_selectivity, x, w, bias.double())
    _raises("k has shape", lion.lion_selectivity, x, w, bias, k=torch.zeros(B, H + 1, L, D, dtype=BF))
    _raises("k_out given without k", lion.lion_selectivity, x, w, bias, k_out=k)
    _raises("x is not contiguous", lion.lion_selectivity, torch.zeros(L, B, Dm, dtype=BF).transpose(0, 1), w, bias)
    _raises("GPU only", lion.lion_selectivity, x, w, bias, k=k)
