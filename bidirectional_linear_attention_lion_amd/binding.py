"""ctypes binding of liblion_attn.so: the same entry points as include/lion_attn.h, taking torch
tensors.  Argument marshalling only -- every step of the computation runs in the HIP kernels.
PyTorch supplies device memory and the stream; outputs (and the workspace, if the caller passes
none) are allocated with torch."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblion_attn.so")

MASK_LIT, MASK_D, MASK_S = 0, 1, 2
CAUSAL = 4   # OR-ed into a mask kind: the causal (unidirectional) variant
FP32_ARITH = 8   # OR-ed into a mask kind: fp32 arithmetic throughout for bf16 inputs (full and chunk forms)
DTYPE_F32, DTYPE_BF16 = 0, 1
FORM_FULL, FORM_CHUNK, FORM_BIRNN, FORM_FULL_BWD, FORM_CHUNK_BWD, FORM_CHUNK2 = 0, 1, 2, 3, 4, 5
_KINDS = {"lit": MASK_LIT, "d": MASK_D, "s": MASK_S}


class LionError(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({lion_status_str(status)})")


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i, f, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    common = [vp, vp, vp, fp, i]
    lib.lion_attn_full.argtypes = common + [f, i, i, i, i, i, vp, i, fp, vp]
    lib.lion_attn_chunk.argtypes = common + [i, f, i, i, i, i, i, vp, i, fp, vp, sz, vp]
    lib.lion_attn_birnn.argtypes = common + [f, i, i, i, i, i, vp, i, fp, vp, sz, vp]
    lib.lion_attn_full_bwd.argtypes = common + [i, i, i, i, i, vp, fp, vp, vp, vp, vp, i, fp, vp, sz, vp]
    lib.lion_attn_chunk_bwd.argtypes = common + [i, i, i, i, i, i, vp, fp, vp, vp, vp, vp, i, fp, vp, sz, vp]
    lib.lion_selectivity.argtypes = [vp, vp, fp, i, i, i, i, fp, fp, vp, vp, i, vp]
    lib.lion_attn_full2.argtypes = common + [f, vp, i, i, i, i, i, vp, i, fp, vp]
    lib.lion_attn_chunk2.argtypes = common + [i, f, vp, i, i, i, i, i, vp, i, fp, vp, sz, vp]
    lib.lion_attn_chunk_noalloc.argtypes = common + [i, f, i, i, i, i, i, vp, i, fp, vp]
    for fn in ("lion_attn_full", "lion_attn_chunk", "lion_attn_birnn", "lion_attn_full_bwd", "lion_attn_chunk_bwd",
               "lion_selectivity",
               "lion_attn_full2", "lion_attn_chunk2", "lion_attn_chunk_noalloc", "lion_attn_abi_version"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.lion_attn_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.lion_attn_workspace_bytes.restype = sz
    lib.lion_status_str.argtypes = [i]
    lib.lion_status_str.restype = ctypes.c_char_p
    lib.lion_attn_abi_version.argtypes = []
    _lib = lib
    return lib


def lion_status_str(status: int) -> str:
    return library().lion_status_str(int(status)).decode()


def lion_attn_abi_version() -> int:
    return library().lion_attn_abi_version()


def lion_attn_workspace_bytes(form: int, B: int, H: int, L: int, d: int, C: int = 0, dtype: int = DTYPE_BF16) -> int:
    return int(library().lion_attn_workspace_bytes(form, B, H, L, d, C, dtype))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise LionArgumentError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class LionArgumentError(ValueError):
    """A tensor argument the C ABI cannot take as given (shape, dtype, device, layout).

    The ABI sees only pointers and sizes, so these checks can only live here; they all run before
    any call into the library."""


def _tensor(name, t, shape, dtypes, device=None, optional=False):
    """Check that ``t`` is a contiguous tensor of ``shape`` with a dtype in ``dtypes`` on ``device``."""
    import torch
    if t is None:
        if optional:
            return
        raise LionArgumentError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise LionArgumentError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        want = " or ".join(str(x).replace("torch.", "") for x in dtypes)
        raise LionArgumentError(f"{name} has dtype {str(t.dtype).replace('torch.', '')}, expected {want}")
    if tuple(t.shape) != tuple(shape):
        raise LionArgumentError(f"{name} has shape {list(t.shape)}, expected {list(shape)}")
    if not t.is_contiguous():
        raise LionArgumentError(f"{name} is not contiguous (strides {t.stride()}): the kernels read it as "
                                f"row-major {list(shape)}; call .contiguous() first")
    if device is not None and t.device != device:
        raise LionArgumentError(f"{name} is on {t.device}, expected {device}")


def _device_of(q):
    """q's device, which must be a GPU: the library has no CPU path."""
    if q.device.type != "cuda":
        raise LionArgumentError(f"q is on {q.device}; the library computes on the GPU only (no CPU path)")
    return q.device


def _decay_shape(kind, B, H, L):
    base = kind & 3
    return None if base == MASK_LIT else ((H,) if base == MASK_D else (B, H, L))


def _kind_code(mask_kind) -> int:
    if isinstance(mask_kind, str):
        if mask_kind not in _KINDS:
            raise LionArgumentError(f"unknown mask kind {mask_kind!r} (lit, d or s)")
        return _KINDS[mask_kind]
    return int(mask_kind)


def _check_attn_inputs(q, k, v, log_lambda, kind):
    """Validate q, k, v and log_lambda of an attention call; returns (B, H, L, d, dtype code).

    Device placement is checked last (``_device_of``), so every other rejection can be exercised
    with CPU tensors."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise LionArgumentError("q must be a 4-D tensor [B, H, L, d]")
    B, H, L, d = q.shape
    dt = _dtype_code(q)
    _tensor("q", q, (B, H, L, d), (q.dtype,))
    _tensor("k", k, (B, H, L, d), (q.dtype,), q.device)
    _tensor("v", v, (B, H, L, d), (q.dtype,), q.device)
    if kind < 0 or (kind & ~(3 | CAUSAL | FP32_ARITH)) or (kind & 3) == 3:
        raise LionArgumentError(f"unknown mask kind {kind}")
    want = _decay_shape(kind, B, H, L)
    if want is None:
        if log_lambda is not None:
            raise LionArgumentError("log_lambda must be None for LION-LIT (lambda = 1)")
    else:
        _tensor("log_lambda", log_lambda, want, (torch.float32,), q.device)
    return B, H, L, d, dt


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _prepare(q, k, v, log_lambda, mask_kind, y, y_dtype, den_out, stream, order=None, need_order=False):
    """Validate the arguments of a forward call and allocate y if not given."""
    import torch
    kind = _kind_code(mask_kind)
    B, H, L, d, dt = _check_attn_inputs(q, k, v, log_lambda, kind)
    ydts = (q.dtype,) if q.dtype == torch.float32 else (torch.bfloat16, torch.float32)
    if y is not None:
        _tensor("y", y, (B, H, L, d), ydts, q.device)
    elif y_dtype is not None and y_dtype not in ydts:
        raise LionArgumentError(f"y_dtype {y_dtype} is not available for {q.dtype} inputs")
    _tensor("den_out", den_out, (B, H, L), (torch.float32,), q.device, optional=True)
    if need_order:
        _tensor("order", order, (L,), (torch.int32,), q.device)
    dev = _device_of(q)
    if y is None:
        y = torch.empty((B, H, L, d), dtype=q.dtype if y_dtype is None else y_dtype, device=dev)
    return kind, B, H, L, d, dt, y, _dtype_code(y), _stream_ptr(stream, dev)


def _workspace(form, B, H, L, d, C, dt, workspace, device):
    """The caller's workspace (checked) or a new one of the size the library asks for."""
    import torch
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
            raise LionArgumentError("workspace must be a contiguous tensor")
        if workspace.device != device:
            raise LionArgumentError(f"workspace is on {workspace.device}, expected {device}")
        return workspace, workspace.numel() * workspace.element_size()
    need = lion_attn_workspace_bytes(form, B, H, L, d, C, dt)
    if need == (1 << 64) - 1:    # the library rejects these sizes; its call reports why
        return None, 0
    if need == 0:
        return None, 0
    return torch.empty(need, dtype=torch.uint8, device=device), need


def _call(fn: str, *args):
    rc = getattr(library(), fn)(*args)
    if rc != 0:
        raise LionError(fn, rc)


def lion_attn_full(q, k, v, log_lambda, mask_kind, eps: float = 1e-6, *, y=None, y_dtype=None, den_out=None,
                   stream=None):
    """Full form; returns y.  q, k, v: contiguous [B, H, L, d] bf16/fp32 cuda tensors."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, log_lambda, mask_kind, y, y_dtype, den_out, stream)
    _call("lion_attn_full", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, float(eps), B, H, L, d, dt,
          _ptr(y), ydt, _ptr(den_out), sptr)
    return y


def lion_attn_full2(q, k, v, log_lambda, mask_kind, order, eps: float = 1e-6, *, y=None, y_dtype=None,
                    den_out=None, stream=None):
    """Full form with the masks of the tokens' own order and of ``order`` (int32 cuda tensor [L]) averaged."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, log_lambda, mask_kind, y, y_dtype, den_out, stream,
                                                  order=order, need_order=True)
    _call("lion_attn_full2", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, float(eps), _ptr(order), B, H,
          L, d, dt, _ptr(y), ydt, _ptr(den_out), sptr)
    return y


def lion_attn_chunk2(q, k, v, log_lambda, mask_kind, order, C: int = 64, eps: float = 1e-6, *, y=None, y_dtype=None,
                     den_out=None, workspace=None, stream=None):
    """Chunkwise form with the masks of the tokens' own order and of ``order`` (int32 cuda tensor [L])
    averaged (the definition of lion_attn_full2)."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, log_lambda, mask_kind, y, y_dtype, den_out, stream,
                                                  order=order, need_order=True)
    ws, nbytes = _workspace(FORM_CHUNK2, B, H, L, d, int(C), dt, workspace, q.device)
    _call("lion_attn_chunk2", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, int(C), float(eps), _ptr(order),
          B, H, L, d, dt, _ptr(y), ydt, _ptr(den_out), _ptr(ws), nbytes, sptr)
    return y


def lion_attn_chunk(q, k, v, log_lambda, mask_kind, C: int = 64, eps: float = 1e-6, *, y=None, y_dtype=None,
                    den_out=None, workspace=None, stream=None):
    """Chunkwise form with chunk size C; returns y."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, log_lambda, mask_kind, y, y_dtype, den_out, stream)
    ws, nbytes = _workspace(FORM_CHUNK, B, H, L, d, int(C), dt, workspace, q.device)
    _call("lion_attn_chunk", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, int(C), float(eps), B, H, L,
          d, dt, _ptr(y), ydt, _ptr(den_out), _ptr(ws), nbytes, sptr)
    return y


def lion_attn_chunk_noalloc(q, k, v, log_lambda, mask_kind, C: int = 64, eps: float = 1e-6, *, y=None, y_dtype=None,
                            den_out=None, stream=None):
    """Chunkwise form whose scratch is the library's built-in per-GPU array (no workspace argument; the
    library allocates nothing).  Pass ``y`` to allocate nothing here either; calls overlapping in time on
    one GPU race for the array."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, log_lambda, mask_kind, y, y_dtype, den_out, stream)
    _call("lion_attn_chunk_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, int(C), float(eps), B, H, L,
          d, dt, _ptr(y), ydt, _ptr(den_out), sptr)
    return y


def lion_attn_birnn(q, k, v, log_lambda, mask_kind, eps: float = 1e-6, *, y=None, y_dtype=None, den_out=None,
                    workspace=None, stream=None):
    """Bidirectional RNN form; returns y."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, log_lambda, mask_kind, y, y_dtype, den_out, stream)
    ws, nbytes = _workspace(FORM_BIRNN, B, H, L, d, 0, dt, workspace, q.device)
    _call("lion_attn_birnn", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, float(eps), B, H, L, d, dt,
          _ptr(y), ydt, _ptr(den_out), _ptr(ws), nbytes, sptr)
    return y


def _prepare_bwd(q, k, v, log_lambda, mask_kind, y, den, dy, grad_dtype, dq, dk, dv, dlog_lambda):
    """Validate a backward call's arguments and allocate the gradients not given."""
    import torch
    kind = _kind_code(mask_kind)
    B, H, L, d, dt = _check_attn_inputs(q, k, v, log_lambda, kind)
    shape = (B, H, L, d)
    _tensor("y", y, shape, (q.dtype,), q.device)
    _tensor("den", den, (B, H, L), (torch.float32,), q.device)
    _tensor("dy", dy, shape, (q.dtype,), q.device)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    if gdt not in (torch.bfloat16, torch.float32):
        raise LionArgumentError(f"grad_dtype {gdt} (bf16 or fp32)")
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        _tensor(name, g, shape, (gdt,), q.device, optional=True)
    want = _decay_shape(kind, B, H, L)
    if want is None:
        if dlog_lambda is not None:
            raise LionArgumentError("dlog_lambda must be None for LION-LIT")
    else:
        _tensor("dlog_lambda", dlog_lambda, want, (torch.float32,), q.device, optional=True)
    dev = _device_of(q)
    dq = torch.empty(shape, dtype=gdt, device=dev) if dq is None else dq
    dk = torch.empty(shape, dtype=gdt, device=dev) if dk is None else dk
    dv = torch.empty(shape, dtype=gdt, device=dev) if dv is None else dv
    if dlog_lambda is None and want is not None:
        dlog_lambda = torch.empty(want, dtype=torch.float32, device=dev)
    return kind, B, H, L, d, dt, dq, dk, dv, dlog_lambda, dev


def lion_attn_full_bwd(q, k, v, log_lambda, mask_kind, y, den, dy, *, grad_dtype=None, dq=None, dk=None, dv=None,
                       dlog_lambda=None, workspace=None, stream=None):
    """Backward pass of the full form; returns (dq, dk, dv, dlog_lambda).

    y and den are the forward call's output and den_out; dy the incoming gradient (bf16)."""
    kind, B, H, L, d, dt, dq, dk, dv, dll, dev = _prepare_bwd(q, k, v, log_lambda, mask_kind, y, den, dy,
                                                              grad_dtype, dq, dk, dv, dlog_lambda)
    ws, nbytes = _workspace(FORM_FULL_BWD, B, H, L, d, 0, dt, workspace, dev)
    _call("lion_attn_full_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, B, H, L, d, dt, _ptr(y),
          _ptr(den), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq), _ptr(dll), _ptr(ws), nbytes,
          _stream_ptr(stream, dev))
    return dq, dk, dv, dll


def lion_attn_chunk_bwd(q, k, v, log_lambda, mask_kind, C, y, den, dy, *, grad_dtype=None, dq=None, dk=None,
                        dv=None, dlog_lambda=None, workspace=None, stream=None):
    """Backward pass computed chunkwise (chunks of C tokens); returns (dq, dk, dv, dlog_lambda).

    Same gradients and arguments as lion_attn_full_bwd, plus the chunk size C."""
    kind, B, H, L, d, dt, dq, dk, dv, dll, dev = _prepare_bwd(q, k, v, log_lambda, mask_kind, y, den, dy,
                                                              grad_dtype, dq, dk, dv, dlog_lambda)
    ws, nbytes = _workspace(FORM_CHUNK_BWD, B, H, L, d, int(C), dt, workspace, dev)
    _call("lion_attn_chunk_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, int(C), B, H, L, d, dt,
          _ptr(y), _ptr(den), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq), _ptr(dll), _ptr(ws),
          nbytes, _stream_ptr(stream, dev))
    return dq, dk, dv, dll


def lion_selectivity(x, w, bias, *, k=None, k_out=None, want_key_scale=False, stream=None):
    """LION-S decays from the layer input x [B, L, Dm] (bf16), w [H, Dm] (bf16), bias [H] (fp32).

    Returns (log_lambda [B, H, L], key_scale or None, k_out or None); with k [B, H, L, d] the scaled keys
    are written to k_out (allocated if not given; may be k itself)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise LionArgumentError("x must be a 3-D tensor [B, L, Dm]")
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise LionArgumentError("w must be a 2-D tensor [H, Dm]")
    B, L, Dm = x.shape
    H = w.shape[0]
    _tensor("x", x, (B, L, Dm), (torch.bfloat16,))
    _tensor("w", w, (H, Dm), (torch.bfloat16,), x.device)
    _tensor("bias", bias, (H,), (torch.float32,), x.device)
    d = 0
    if k is not None:
        if not isinstance(k, torch.Tensor) or k.dim() != 4:
            raise LionArgumentError("k must be a 4-D tensor [B, H, L, d]")
        d = k.shape[-1]
        _tensor("k", k, (B, H, L, d), (torch.bfloat16,), x.device)
        _tensor("k_out", k_out, (B, H, L, d), (torch.bfloat16,), x.device, optional=True)
    elif k_out is not None:
        raise LionArgumentError("k_out given without k")
    if x.device.type != "cuda":
        raise LionArgumentError(f"x is on {x.device}; the library computes on the GPU only (no CPU path)")
    dev = x.device
    ll = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    ks = torch.empty((B, H, L), dtype=torch.float32, device=dev) if want_key_scale else None
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    _call("lion_selectivity", _ptr(x), _ptr(w), _ptr(bias), B, L, H, Dm, _ptr(ll), _ptr(ks), _ptr(k),
          _ptr(k_out), d, _stream_ptr(stream, dev))
    return ll, ks, k_out
