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
    for fn in ("lion_attn_full", "lion_attn_chunk", "lion_attn_birnn", "lion_attn_full_bwd", "lion_attn_chunk_bwd",
               "lion_selectivity",
               "lion_attn_full2", "lion_attn_chunk2", "lion_attn_abi_version"):
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
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _prepare(q, k, v, mask_kind, y, y_dtype, den_out, stream):
    import torch
    kind = _KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, d = q.shape
    dt = _dtype_code(q)
    if y is None:
        out_dtype = q.dtype if y_dtype is None else y_dtype
        y = torch.empty((B, H, L, d), dtype=out_dtype, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return kind, B, H, L, d, dt, y, _dtype_code(y), sptr


def lion_attn_full(q, k, v, log_lambda, mask_kind, eps: float = 1e-6, *, y=None, y_dtype=None, den_out=None,
                   stream=None):
    """Full form; returns y.  q, k, v: contiguous [B, H, L, d] bf16/fp32 cuda tensors."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, mask_kind, y, y_dtype, den_out, stream)
    rc = library().lion_attn_full(_ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, float(eps), B, H, L, d, dt,
                                  _ptr(y), ydt, _ptr(den_out), sptr)
    if rc != 0:
        raise LionError("lion_attn_full", rc)
    return y


def lion_attn_full2(q, k, v, log_lambda, mask_kind, order, eps: float = 1e-6, *, y=None, y_dtype=None,
                    den_out=None, stream=None):
    """Full form with the masks of the tokens' own order and of ``order`` (int32 cuda tensor [L]) averaged."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, mask_kind, y, y_dtype, den_out, stream)
    rc = library().lion_attn_full2(_ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, float(eps), _ptr(order), B, H,
                                   L, d, dt, _ptr(y), ydt, _ptr(den_out), sptr)
    if rc != 0:
        raise LionError("lion_attn_full2", rc)
    return y


def lion_attn_chunk2(q, k, v, log_lambda, mask_kind, order, C: int = 64, eps: float = 1e-6, *, y=None, y_dtype=None,
                     den_out=None, workspace=None, stream=None):
    """Chunkwise form with the masks of the tokens' own order and of ``order`` (int32 cuda tensor [L])
    averaged (the definition of lion_attn_full2)."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, mask_kind, y, y_dtype, den_out, stream)
    ws, nbytes = _workspace(FORM_CHUNK2, B, H, L, d, C, dt, workspace, q.device)
    rc = library().lion_attn_chunk2(_ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, C, float(eps), _ptr(order), B,
                                    H, L, d, dt, _ptr(y), ydt, _ptr(den_out), _ptr(ws), nbytes, sptr)
    if rc != 0:
        raise LionError("lion_attn_chunk2", rc)
    return y


def _workspace(form, B, H, L, d, C, dt, workspace, device):
    import torch
    need = lion_attn_workspace_bytes(form, B, H, L, d, C, dt)
    if need == (1 << 64) - 1:
        return None, 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, nbytes


def lion_attn_chunk(q, k, v, log_lambda, mask_kind, C: int = 64, eps: float = 1e-6, *, y=None, y_dtype=None,
                    den_out=None, workspace=None, stream=None):
    """Chunkwise form with chunk size C; returns y."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, mask_kind, y, y_dtype, den_out, stream)
    ws, nbytes = _workspace(FORM_CHUNK, B, H, L, d, C, dt, workspace, q.device)
    rc = library().lion_attn_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, int(C), float(eps), B, H, L,
                                   d, dt, _ptr(y), ydt, _ptr(den_out), _ptr(ws), nbytes, sptr)
    if rc != 0:
        raise LionError("lion_attn_chunk", rc)
    return y


def lion_attn_birnn(q, k, v, log_lambda, mask_kind, eps: float = 1e-6, *, y=None, y_dtype=None, den_out=None,
                    workspace=None, stream=None):
    """Bidirectional RNN form; returns y."""
    kind, B, H, L, d, dt, y, ydt, sptr = _prepare(q, k, v, mask_kind, y, y_dtype, den_out, stream)
    ws, nbytes = _workspace(FORM_BIRNN, B, H, L, d, 0, dt, workspace, q.device)
    rc = library().lion_attn_birnn(_ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, float(eps), B, H, L, d, dt,
                                   _ptr(y), ydt, _ptr(den_out), _ptr(ws), nbytes, sptr)
    if rc != 0:
        raise LionError("lion_attn_birnn", rc)
    return y


def lion_attn_full_bwd(q, k, v, log_lambda, mask_kind, y, den, dy, *, grad_dtype=None, dq=None, dk=None, dv=None,
                       dlog_lambda=None, workspace=None, stream=None):
    """Backward pass of the full form; returns (dq, dk, dv, dlog_lambda).

    y and den are the forward call's output and den_out; dy the incoming gradient (bf16)."""
    import torch
    kind = _KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    B, H, L, d = q.shape
    dt = _dtype_code(q)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty((B, H, L, d), dtype=gdt, device=q.device) if dq is None else dq
    dk = torch.empty((B, H, L, d), dtype=gdt, device=q.device) if dk is None else dk
    dv = torch.empty((B, H, L, d), dtype=gdt, device=q.device) if dv is None else dv
    base = kind & 3
    if dlog_lambda is None and base != MASK_LIT:
        shape = (H,) if base == MASK_D else (B, H, L)
        dlog_lambda = torch.empty(shape, dtype=torch.float32, device=q.device)
    ws, nbytes = _workspace(FORM_FULL_BWD, B, H, L, d, 0, dt, workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    rc = library().lion_attn_full_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, B, H, L, d, dt, _ptr(y),
                                      _ptr(den), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq),
                                      _ptr(dlog_lambda), _ptr(ws), nbytes, sptr)
    if rc != 0:
        raise LionError("lion_attn_full_bwd", rc)
    return dq, dk, dv, dlog_lambda


def lion_attn_chunk_bwd(q, k, v, log_lambda, mask_kind, C, y, den, dy, *, grad_dtype=None, dq=None, dk=None,
                        dv=None, dlog_lambda=None, workspace=None, stream=None):
    """Backward pass computed chunkwise (chunks of C tokens); returns (dq, dk, dv, dlog_lambda).

    Same gradients and arguments as lion_attn_full_bwd, plus the chunk size C."""
    import torch
    kind = _KINDS[mask_kind] if isinstance(mask_kind, str) else int(mask_kind)
    B, H, L, d = q.shape
    dt = _dtype_code(q)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty((B, H, L, d), dtype=gdt, device=q.device) if dq is None else dq
    dk = torch.empty((B, H, L, d), dtype=gdt, device=q.device) if dk is None else dk
    dv = torch.empty((B, H, L, d), dtype=gdt, device=q.device) if dv is None else dv
    base = kind & 3
    if dlog_lambda is None and base != MASK_LIT:
        shape = (H,) if base == MASK_D else (B, H, L)
        dlog_lambda = torch.empty(shape, dtype=torch.float32, device=q.device)
    ws, nbytes = _workspace(FORM_CHUNK_BWD, B, H, L, d, C, dt, workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    rc = library().lion_attn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_lambda), kind, C, B, H, L, d, dt, _ptr(y),
                                       _ptr(den), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq),
                                       _ptr(dlog_lambda), _ptr(ws), nbytes, sptr)
    if rc != 0:
        raise LionError("lion_attn_chunk_bwd", rc)
    return dq, dk, dv, dlog_lambda


def lion_selectivity(x, w, bias, *, k=None, k_out=None, want_key_scale=False, stream=None):
    """LION-S decays from the layer input x [B, L, Dm] (bf16), w [H, Dm] (bf16), bias [H] (fp32).

    Returns (log_lambda [B, H, L], key_scale or None, k_out or None); with k [B, H, L, d] the scaled keys
    are written to k_out (allocated if not given; may be k itself)."""
    import torch
    B, L, Dm = x.shape
    H = w.shape[0]
    ll = torch.empty((B, H, L), dtype=torch.float32, device=x.device)
    ks = torch.empty((B, H, L), dtype=torch.float32, device=x.device) if want_key_scale else None
    d = 0
    if k is not None:
        d = k.shape[-1]
        if k_out is None:
            k_out = torch.empty_like(k)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    rc = library().lion_selectivity(_ptr(x), _ptr(w), _ptr(bias), B, L, H, Dm, _ptr(ll), _ptr(ks), _ptr(k),
                                    _ptr(k_out), d, sptr)
    if rc != 0:
        raise LionError("lion_selectivity", rc)
    return ll, ks, k_out
