"""Seeded synthetic inputs for LION attention workloads.

This module is the only code both the GPU path's tests/bench and the oracle's tests share.  It
holds no attention arithmetic: it draws q, k, v and the decay inputs from a seeded PCG64 stream,
rounds to bf16 where the workload asks for bf16, and forms log(lambda) by each workload's recipe.
The result carries the exact values the device receives (``*_dev``) and their exact fp64 upcast
(``*_f64``), so the oracle consumes precisely what the kernels consume.

Recipes (draw order q -> k -> v -> decay inputs; fp32 draws; bf16 by round-to-nearest-even), with
the forms each is quoted with:
  lion_s_unit   B1  H1  L64   d16 fp32  LION-S:   log lam = log sigmoid(z + 2), z ~ N(0,1) [B,H,L]
                                                  full, chunk (C=16), RNN
  vit_tiny_lit  B64 H3  L197  d64 bf16  LION-LIT: lambda = 1 (no decay input);  full, chunk (C=64)
  vit_base_d    B64 H12 L197  d64 bf16  LION-D:   log lam_h = log(1 - 2^(-5-h)), h = 0..H-1
                                                  full, chunk (C=64), RNN
  bert_large_s  B32 H16 L512  d64 bf16  LION-S:   log lam = log sigmoid(x_i . w_h + 3),
                                                  x ~ N(0,1) [B,L,1024] shared by heads, w ~ N(0,1/1024) [H,1024]
                                                  full, chunk (C=64)
  hires_d       B8  H12 L4097 d64 bf16  LION-D:   per-head lambda as vit_base_d;  chunk (C=64/128/256), RNN

The shapes stand in for the pages' workloads (ViT-Tiny at 224 px: 196 patches + cls; ViT-Base
with 12 heads; BERT-Large with 16 heads at 512 tokens; a 1024 x 1024 image in 16-pixel patches
plus cls = 4097 tokens); no dataset or trained weight is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

LIT, D, S = 0, 1, 2
KIND_NAME = {LIT: "lit", D: "d", S: "s"}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: str          # "f32" or "bf16": storage and MFMA input type of q, k, v, y
    kind: int           # LIT / D / S
    lam_recipe: str     # "none", "per_head", "sigmoid_noise", "sigmoid_proj"
    forms: tuple        # the forms the workload is quoted with (every form runs on every workload in tests)
    chunks: tuple = (64,)
    eps: float = 1e-6
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.B * self.L


WORKLOADS = {
    "lion_s_unit": Workload("lion_s_unit", 1, 1, 64, 16, "f32", S, "sigmoid_noise",
                            ("full", "chunk", "birnn"), chunks=(16,), seed=1),
    "vit_tiny_lit": Workload("vit_tiny_lit", 64, 3, 197, 64, "bf16", LIT, "none",
                             ("full", "chunk"), chunks=(64,), seed=2),
    "vit_base_d": Workload("vit_base_d", 64, 12, 197, 64, "bf16", D, "per_head",
                           ("full", "chunk", "birnn"), chunks=(64,), seed=3),
    "bert_large_s": Workload("bert_large_s", 32, 16, 512, 64, "bf16", S, "sigmoid_proj",
                             ("full", "chunk"), chunks=(64,), seed=4),
    "hires_d": Workload("hires_d", 8, 12, 4097, 64, "bf16", D, "per_head",
                        ("chunk", "birnn"), chunks=(64, 128, 256), seed=5),
}


def round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.  Inputs are finite."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns, as fp64."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclass
class Inputs:
    wl: Workload
    q_dev: np.ndarray           # device-ready: float32 array, or uint16 bf16 bit patterns
    k_dev: np.ndarray
    v_dev: np.ndarray
    log_lambda: np.ndarray | None   # float32 (what the device receives): None, [H] or [B,H,L]
    q: np.ndarray = field(repr=False, default=None)   # exact fp64 values of the device inputs
    k: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)
    log_lambda_f64: np.ndarray | None = field(repr=False, default=None)


def _dev(x32: np.ndarray, dtype: str):
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    bits = round_bf16_bits(x32)
    return bits, bf16_bits_to_f64(bits)


def _log_sigmoid(t: np.ndarray) -> np.ndarray:
    # log sigmoid(t) = -log(1 + exp(-t)), evaluated without overflow
    return -np.logaddexp(0.0, -t)


def make_inputs(wl: Workload, B: int | None = None, H: int | None = None, L: int | None = None,
                d: int | None = None, seed: int | None = None) -> Inputs:
    """Draw one input set for ``wl`` (optionally with overridden sizes or seed)."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    L = wl.L if L is None else L
    d = wl.d if d is None else d
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    shape = (B, H, L, d)
    q32 = rng.standard_normal(shape, dtype=np.float32)
    k32 = rng.standard_normal(shape, dtype=np.float32)
    v32 = rng.standard_normal(shape, dtype=np.float32)
    qd, qf = _dev(q32, wl.dtype)
    kd, kf = _dev(k32, wl.dtype)
    vd, vf = _dev(v32, wl.dtype)
    if wl.lam_recipe == "none":
        ll = None
    elif wl.lam_recipe == "per_head":
        h = np.arange(H, dtype=np.float64)
        ll = np.log1p(-np.exp2(-5.0 - h)).astype(np.float32)
    elif wl.lam_recipe == "sigmoid_noise":
        z = rng.standard_normal((B, H, L), dtype=np.float32).astype(np.float64)
        ll = _log_sigmoid(z + 2.0).astype(np.float32)
    elif wl.lam_recipe == "sigmoid_proj":
        width = 1024
        x = rng.standard_normal((B, L, width), dtype=np.float32).astype(np.float64)
        w = rng.standard_normal((H, width), dtype=np.float32).astype(np.float64) / np.sqrt(width)
        a = np.einsum("blw,hw->bhl", x, w) + 3.0
        ll = _log_sigmoid(a).astype(np.float32)
    else:
        raise ValueError(wl.lam_recipe)
    return Inputs(wl=Workload(**{**wl.__dict__, "B": B, "H": H, "L": L, "d": d}), q_dev=qd, k_dev=kd, v_dev=vd,
                  log_lambda=ll, q=qf, k=kf, v=vf,
                  log_lambda_f64=None if ll is None else ll.astype(np.float64))


def random_inputs(B, H, L, d, kind, dtype="bf16", seed=0, lam_recipe=None, eps=1e-6) -> Inputs:
    """Seeded inputs of an arbitrary shape with the decay recipe of ``kind`` (for edge cases)."""
    recipe = lam_recipe or {LIT: "none", D: "per_head", S: "sigmoid_noise"}[kind]
    wl = Workload(f"random_{KIND_NAME[kind]}", B, H, L, d, dtype, kind, recipe, ("full", "chunk", "birnn"),
                  eps=eps, seed=seed)
    return make_inputs(wl)


def column_major_order(rows: int, cols: int, cls: bool = True) -> np.ndarray:
    """Tokens of an image in column-major patch order: the class token (if any) first, then patch (r, c)
    of the row-major grid -- token cls + r * cols + c -- listed column by column.  int32 [L]."""
    off = 1 if cls else 0
    grid = np.arange(rows * cols, dtype=np.int32).reshape(rows, cols) + off
    head = np.zeros(off, dtype=np.int32)
    return np.concatenate([head, grid.T.reshape(-1)]).astype(np.int32)
