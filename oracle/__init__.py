"""fp64 CPU oracle of LION bidirectional masked linear attention.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` are the only callers.  The GPU library never imports, links or runs anything here,
and nothing here imports the GPU package.

``lion_oracle.c`` holds the definition (the full form, see its header for the passages it follows);
``forms.py`` holds the chunkwise and recurrent forms in numpy, used only to cross-check the
definition in the oracle's own tests.  This module builds the C file with gcc and wraps it for
numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lion_oracle.c")
LIB = os.path.join(HERE, "liblion_oracle.so")

MASK_LIT, MASK_D, MASK_S = 0, 1, 2
CAUSAL = 4   # OR-ed into a kind: keys after the query masked out (see lion_oracle.c)
KIND_NAMES = {"lit": MASK_LIT, "d": MASK_D, "s": MASK_S}

CFLAGS = ["-O2", "-fno-fast-math", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra_flags: list[str] | None = None) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


_libs: dict[str, ctypes.CDLL] = {}


def load(path: str = LIB) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library at ``path``."""
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        if path != LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_long)
    i, d_ = ctypes.c_int, ctypes.c_double
    lib.lion_oracle_phi_f64.argtypes = [i, dp, ctypes.c_long, i, dp]
    lib.lion_oracle_mask_f64.argtypes = [dp, i, dp]
    lib.lion_oracle_attn_f64.argtypes = [dp, dp, dp, dp, d_, i, i, i, i, dp, dp, dp, dp]
    lib.lion_oracle_full_f64.argtypes = [dp, dp, dp, dp, i, d_, i, i, i, i, dp, dp, dp, dp]
    lib.lion_oracle_rows_f64.argtypes = [dp, dp, dp, dp, i, d_, i, i, i, i, lp, ctypes.c_long, dp, dp, dp, dp]
    lib.lion_oracle_full_bwd_f64.argtypes = [dp, dp, dp, dp, i, d_, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.lion_oracle_selectivity_f64.argtypes = [dp, dp, dp, i, i, i, i, i, dp, dp, dp, dp]
    lib.lion_oracle_full2_f64.argtypes = [dp, dp, dp, dp, i, d_, lp, i, i, i, i, dp, dp, dp, dp]
    for f in ("phi", "mask", "attn", "full", "rows", "full_bwd", "selectivity", "full2"):
        getattr(lib, f"lion_oracle_{f}_f64").restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _kind(kind) -> int:
    return KIND_NAMES[kind] if isinstance(kind, str) else int(kind)


def phi(kind, x, lib_path: str = LIB) -> np.ndarray:
    """phi of every row of ``x`` (last axis = channels)."""
    x = _f64(x)
    out = np.empty_like(x)
    d = x.shape[-1]
    rc = load(lib_path).lion_oracle_phi_f64(_kind(kind), _p(x), x.size // d, d, _p(out))
    if rc != 0:
        raise ValueError(f"lion_oracle_phi_f64 returned {rc}")
    return out


def mask(lam, lib_path: str = LIB) -> np.ndarray:
    """L x L mask of one sequence of per-token decays."""
    lam = _f64(lam)
    L = lam.shape[0]
    M = np.empty((L, L), dtype=np.float64)
    rc = load(lib_path).lion_oracle_mask_f64(_p(lam), L, _p(M))
    if rc != 0:
        raise ValueError(f"lion_oracle_mask_f64 returned {rc}")
    return M


def attn(phq, phk, v, lam, eps=0.0, want_abs=False, lib_path: str = LIB):
    """Masked, row-normalised attention on phi-applied inputs [B,H,L,d] and decays [B,H,L].

    Returns (y, den) or (y, den, absnum, absden)."""
    phq, phk, v, lam = _f64(phq), _f64(phk), _f64(v), _f64(lam)
    B, H, L, d = phq.shape
    y = np.empty_like(phq)
    den = np.empty((B, H, L))
    an = np.empty_like(phq) if want_abs else None
    ad = np.empty((B, H, L)) if want_abs else None
    rc = load(lib_path).lion_oracle_attn_f64(_p(phq), _p(phk), _p(v), _p(lam), float(eps), B, H, L, d, _p(y),
                                             _p(den), _p(an), _p(ad))
    if rc != 0:
        raise ValueError(f"lion_oracle_attn_f64 returned {rc}")
    return (y, den, an, ad) if want_abs else (y, den)


def full(q, k, v, log_lambda, kind, eps=0.0, want_abs=False, lib_path: str = LIB):
    """The full-form definition on raw q, k, v [B,H,L,d]; log_lambda None / [H] / [B,H,L].

    Returns (y, den) or (y, den, absnum, absden); den is the divisor (row sum + eps)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    ll = None if log_lambda is None else _f64(log_lambda)
    B, H, L, d = q.shape
    y = np.empty_like(q)
    den = np.empty((B, H, L))
    an = np.empty_like(q) if want_abs else None
    ad = np.empty((B, H, L)) if want_abs else None
    rc = load(lib_path).lion_oracle_full_f64(_p(q), _p(k), _p(v), _p(ll), _kind(kind), float(eps), B, H, L, d,
                                             _p(y), _p(den), _p(an), _p(ad))
    if rc != 0:
        raise ValueError(f"lion_oracle_full_f64 returned {rc}")
    return (y, den, an, ad) if want_abs else (y, den)


def rows(q, k, v, log_lambda, kind, eps, row_ids, want_abs=False, lib_path: str = LIB):
    """The full-form definition at selected rows ``row_ids`` (flat index bh * L + i)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    ll = None if log_lambda is None else _f64(log_lambda)
    B, H, L, d = q.shape
    rid = np.ascontiguousarray(row_ids, dtype=np.int64)
    n = rid.shape[0]
    y = np.empty((n, d))
    den = np.empty((n,))
    an = np.empty((n, d)) if want_abs else None
    ad = np.empty((n,)) if want_abs else None
    rc = load(lib_path).lion_oracle_rows_f64(_p(q), _p(k), _p(v), _p(ll), _kind(kind), float(eps), B, H, L, d,
                                             rid.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), n, _p(y), _p(den),
                                             _p(an), _p(ad))
    if rc != 0:
        raise ValueError(f"lion_oracle_rows_f64 returned {rc}")
    return (y, den, an, ad) if want_abs else (y, den)


def full_bwd(q, k, v, log_lambda, kind, eps, dy, want_abs=False, lib_path: str = LIB):
    """Gradients of the full-form definition for a loss with dL/dy = dy.

    Returns (dq, dk, dv, dll), then (adq, adk, adv, adll) if want_abs (the absolute-value companions
    of the condition-aware gate); dll is None (LIT), [H] (D) or [B, H, L] (S)."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    ll = None if log_lambda is None else _f64(log_lambda)
    B, H, L, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    base = _kind(kind) & 3
    dll = None if base == 0 else (np.empty((H,)) if base == 1 else np.empty((B, H, L)))
    adq = adk = adv = adll = None
    if want_abs:
        adq, adk, adv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        adll = None if dll is None else np.empty_like(dll)
    rc = load(lib_path).lion_oracle_full_bwd_f64(_p(q), _p(k), _p(v), _p(ll), _kind(kind), float(eps), B, H, L, d,
                                                 _p(dy), _p(dq), _p(dk), _p(dv), _p(dll), _p(adq), _p(adk), _p(adv),
                                                 _p(adll))
    if rc != 0:
        raise ValueError(f"lion_oracle_full_bwd_f64 returned {rc}")
    if want_abs:
        return dq, dk, dv, dll, adq, adk, adv, adll
    return dq, dk, dv, dll


def selectivity(x, w, bias, k=None, lib_path: str = LIB):
    """LION-S's decay and key scale from the layer input: x [B, L, Dm], w [H, Dm], bias [H], optional
    k [B, H, L, d].  Returns (log_lambda [B, H, L], key_scale [B, H, L], k_out or None)."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    B, L, Dm = x.shape
    H = w.shape[0]
    ll = np.empty((B, H, L))
    ks = np.empty((B, H, L))
    kk = None if k is None else _f64(k)
    d = 0 if kk is None else kk.shape[-1]
    ko = None if kk is None else np.empty_like(kk)
    rc = load(lib_path).lion_oracle_selectivity_f64(_p(x), _p(w), _p(bias), B, L, H, Dm, d, _p(kk), _p(ll), _p(ks),
                                                    _p(ko))
    if rc != 0:
        raise ValueError(f"lion_oracle_selectivity_f64 returned {rc}")
    return ll, ks, ko


def full2(q, k, v, log_lambda, kind, eps, order, want_abs=False, lib_path: str = LIB):
    """The full definition with the average of two masks: the tokens' own order and ``order`` ([L], the
    tokens listed in a second order).  Returns (y, den) or (y, den, absnum, absden)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    ll = None if log_lambda is None else _f64(log_lambda)
    B, H, L, d = q.shape
    o = np.ascontiguousarray(order, dtype=np.int64)
    y = np.empty_like(q)
    den = np.empty((B, H, L))
    an = np.empty_like(q) if want_abs else None
    ad = np.empty((B, H, L)) if want_abs else None
    rc = load(lib_path).lion_oracle_full2_f64(_p(q), _p(k), _p(v), _p(ll), _kind(kind), float(eps),
                                              o.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), B, H, L, d, _p(y),
                                              _p(den), _p(an), _p(ad))
    if rc != 0:
        raise ValueError(f"lion_oracle_full2_f64 returned {rc}")
    return (y, den, an, ad) if want_abs else (y, den)
