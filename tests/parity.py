"""Parity gates between a GPU result and the fp64 oracle.

Gate L (literal): max |Y_gpu - Y_ref| / RMS(Y_ref) <= 2e-2 for bf16 inputs, 1e-4 for fp32 inputs.

Gate C (condition-aware): elementwise
    |Y_gpu - Y_ref|_ic <= tol * RMS(Y_ref) + beta_ic,
    beta_ic = 3 u (sum_j Pbar_ij |v_jc| + |y_ic| sum_j Pbar_ij) / |den_i| + u_out |y_ic|,
with Pbar_ij = M_ij |phi(q_i)|.|phi(k_j)| (the oracle's absolute-value sums), den_i the exact divisor.
This is the first-order forward-error bound of a ratio of two sums whose terms each carry a
relative error of at most 3u: phi(q), phi(k) and the masked score are each rounded once to the
matrix-core input type (u = 2^-8, twice bf16's unit roundoff, for bf16 inputs; (d + L) 2^-24 for
fp32 inputs, a bound on fp32 accumulation), and the output is rounded once (u_out).  On a row
whose exact denominator nearly cancels (condition number kappa_i = sum_j Pbar_ij / |den_i| large)
every result within beta of the exact one is as correct as any other an implementation in that
arithmetic can give.  So Gate C is asserted everywhere, and Gate L on every row of the
well-conditioned workloads (LION-LIT, whose positive phi makes kappa = 1, and the fp32 LION-S unit
case) and on the well-conditioned rows (kappa_i <= 2) of all the others.

Row scale (``row_scale=True``, the causal variant): a causal row i averages i + 1 values, so output
magnitudes fall by up to sqrt(L) from the first rows to the last, while every rounding above is
relative to the row's own terms.  There RMS(Y_ref) in both gates is taken per row, over its d
channels, instead of over the whole output.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BF16_TOL, F32_TOL = 2e-2, 1e-4
KAPPA_WELL = 2.0


def unit_roundoff(in_dtype: str, d: int, L: int) -> float:
    return 2.0 ** -8 if in_dtype == "bf16" else (d + L) * 2.0 ** -24


def out_roundoff(out_dtype: str) -> float:
    return 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -23


@dataclass
class ParityReport:
    gate_l: float            # max |dY| / RMS over all rows
    gate_l_wellcond: float   # the same over rows with kappa_i <= KAPPA_WELL
    wellcond_rows: float     # fraction of rows with kappa_i <= KAPPA_WELL
    gate_c: float            # max over elements of |dY| / (tol RMS + beta); pass if <= 1
    kappa_max: float
    kappa_median: float
    tol: float

    def __str__(self):
        return (f"gateL={self.gate_l:.3e} gateL(kappa<={KAPPA_WELL:g} rows, {100 * self.wellcond_rows:.1f}%)="
                f"{self.gate_l_wellcond:.3e} gateC={self.gate_c:.3f} kappa max={self.kappa_max:.3g} "
                f"median={self.kappa_median:.3g} tol={self.tol:g}")


def compare(y_gpu, y_ref, den_ref, absnum, absden, in_dtype: str, out_dtype: str, d: int, L: int,
            row_scale: bool = False) -> ParityReport:
    """All arrays are per-row views: y [..., d], den/absden [...]. Values fp64."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(-1, d)
    y_ref = np.asarray(y_ref, dtype=np.float64).reshape(-1, d)
    den = np.asarray(den_ref, dtype=np.float64).reshape(-1)
    an = np.asarray(absnum, dtype=np.float64).reshape(-1, d)
    ad = np.asarray(absden, dtype=np.float64).reshape(-1)
    tol = BF16_TOL if in_dtype == "bf16" else F32_TOL
    u, uo = unit_roundoff(in_dtype, d, L), out_roundoff(out_dtype)
    if row_scale:
        rms = np.sqrt(np.mean(y_ref ** 2, axis=1))[:, None]
    else:
        rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = np.abs(y_gpu - y_ref)
    if not np.all(np.isfinite(y_gpu)):
        err = np.where(np.isfinite(y_gpu), err, np.inf)
    absden_ = np.abs(den)
    beta = 3 * u * (an + np.abs(y_ref) * ad[:, None]) / absden_[:, None] + uo * np.abs(y_ref)
    gate_c = float(np.max(err / (tol * rms + beta)))
    row_err = np.max(err, axis=1) / (rms[:, 0] if row_scale else rms)
    kappa = ad / absden_
    well = kappa <= KAPPA_WELL
    gl_well = float(np.max(row_err[well])) if np.any(well) else 0.0
    return ParityReport(gate_l=float(np.max(row_err)), gate_l_wellcond=gl_well,
                        wellcond_rows=float(np.mean(well)), gate_c=gate_c,
                        kappa_max=float(np.max(kappa)), kappa_median=float(np.median(kappa)), tol=tol)


def assert_parity(rep: ParityReport, what: str, require_literal: bool = False):
    """Gate C always; Gate L on the well-conditioned rows; Gate L on every row if asked."""
    assert rep.gate_c <= 1.0, f"{what}: Gate C failed: {rep}"
    assert rep.gate_l_wellcond <= rep.tol, f"{what}: Gate L failed on well-conditioned rows: {rep}"
    if require_literal:
        assert rep.gate_l <= rep.tol, f"{what}: Gate L failed: {rep}"
