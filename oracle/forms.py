"""The other computational forms of LION, in plain numpy fp64, for the oracle's own tests.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  These are not the definition: they are
the recurrent and chunkwise forms the pages state are equivalent to it, written here so the
definition in ``lion_oracle.c`` can be checked against algorithms that reach the same numbers by a
different route.  All functions take one (batch, head) problem: ``phq, phk`` [L, d] with phi
already applied, ``v`` [L, dv], per-token decays ``lam`` [L] (lam[0] never enters), ``eps``.

Sources:
  [RB] "LION: A bidirectional framework that trains like a Transformer and infers like an RNN",
       author-reviewer discussion (paperhub copy of the ICLR 2025 forum).
  [BL] "LION Part IV - Results" (blog), section "LION Architecture Variants and Trade-offs".
"""
from __future__ import annotations

import numpy as np


def naive_birnn(phq, phk, v, lam, eps=0.0):
    """Forward and backward matrix-state recurrences kept for every token, then combined.

    Forward  S^F_i = lam_i S^F_{i-1} + k_i v_i^T,  z^F_i = lam_i z^F_{i-1} + k_i
    Backward S^B_i = lam_{i+1} S^B_{i+1} + k_i v_i^T,  z^B_i likewise
    y_i = q_i^T (S^F_i + S^B_i - k_i v_i^T) / (q_i^T (z^F_i + z^B_i - k_i) + eps)

    The recurrences are the bidirectional RNN of Theorem 3.3 Eq. 20-24 [RB, reply "Concern 1"]; the
    output with the diagonal subtracted once is the naive extension of linear attention [RB, reply
    "1: Recurrence Form of Linear Attention"], here with the decays of the mask.  The backward decay
    index (lam_{i+1}) is the reading that makes the recurrence reproduce the symmetric mask.
    Memory O(L d^2), as the pages say of this variant."""
    L, d = phq.shape
    dv = v.shape[1]
    SF = np.zeros((L, d, dv))
    zF = np.zeros((L, d))
    SB = np.zeros((L, d, dv))
    zB = np.zeros((L, d))
    S = np.zeros((d, dv))
    z = np.zeros(d)
    for i in range(L):
        S = lam[i] * S + np.outer(phk[i], v[i])
        z = lam[i] * z + phk[i]
        SF[i], zF[i] = S, z
    S = np.zeros((d, dv))
    z = np.zeros(d)
    for i in range(L - 1, -1, -1):
        decay = lam[i + 1] if i + 1 < L else 0.0
        S = decay * S + np.outer(phk[i], v[i])
        z = decay * z + phk[i]
        SB[i], zB[i] = S, z
    y = np.empty((L, dv))
    den = np.empty(L)
    for i in range(L):
        num = phq[i] @ (SF[i] + SB[i] - np.outer(phk[i], v[i]))
        den[i] = phq[i] @ (zF[i] + zB[i] - phk[i]) + eps
        y[i] = num / den[i]
    return y, den


def memory_efficient_birnn(phq, phk, v, lam, eps=0.0):
    """The bidirectional RNN that keeps only a vector y^F_i and a scalar c^F_i per token.

    A forward sweep stores y^F_i = q_i^T S^F_i and c^F_i = q_i^T z^F_i (O(L d + L) memory); the
    backward sweep carries S^B, z^B and emits
      y_i = (y^F_i + q_i^T S^B_i - (q_i.k_i) v_i) / (c^F_i + q_i^T z^B_i - q_i.k_i + eps)
    [RB, reply "1: Recurrence Form of Linear Attention", the per-token scalars c and vectors y]."""
    L, d = phq.shape
    dv = v.shape[1]
    yF = np.empty((L, dv))
    cF = np.empty(L)
    S = np.zeros((d, dv))
    z = np.zeros(d)
    for i in range(L):
        S = lam[i] * S + np.outer(phk[i], v[i])
        z = lam[i] * z + phk[i]
        yF[i] = phq[i] @ S
        cF[i] = phq[i] @ z
    y = np.empty((L, dv))
    den = np.empty(L)
    S = np.zeros((d, dv))
    z = np.zeros(d)
    for i in range(L - 1, -1, -1):
        decay = lam[i + 1] if i + 1 < L else 0.0
        S = decay * S + np.outer(phk[i], v[i])
        z = decay * z + phk[i]
        diag = phq[i] @ phk[i]
        den[i] = cF[i] + phq[i] @ z - diag + eps
        y[i] = (yF[i] + phq[i] @ S - diag * v[i]) / den[i]
    return y, den


def chunkwise(phq, phk, v, lam, eps=0.0, C=64):
    """Chunkwise form: masked attention inside each chunk of C tokens plus two d x (dv+1) states
    carried across chunks, forward and backward [RB, reply "4: Practicality of Recurrent
    Inference"; BL, "LION Chunk"].  The pages print no chunk equations; these follow from the mask:

      A_t = sum_{s<=t} log lam_s  (prefix sums, the cumsum the pages build the mask with)
      M_ij = exp(-|A_i - A_j|)
      chunk c = tokens s_c..e_c;  [v, 1] appends the denominator column
      F_c = exp(A_{e_c} - A_{e_{c-1}}) F_{c-1} + sum_{j in c} exp(A_{e_c} - A_j) k_j [v_j, 1]^T
      G_c = exp(A_{e_c} - A_{e_{c-1}}) G_{c+1} + sum_{j in c} exp(A_j - A_{e_{c-1}}) k_j [v_j, 1]^T
      out_i = sum_{j in c} M_ij (q_i.k_j) [v_j, 1]
              + exp(A_i - A_{e_{c-1}}) q_i^T F_{c-1} + exp(A_{e_c} - A_i) q_i^T G_{c+1}
      y_i = out_i[:dv] / (out_i[dv] + eps)

    Every exponent is <= 0.  The mask here comes from logarithms and prefix sums, unlike the
    definition in lion_oracle.c, which multiplies the decays directly."""
    L, d = phq.shape
    dv = v.shape[1]
    A = np.cumsum(np.log(lam))
    v1 = np.concatenate([v, np.ones((L, 1))], axis=1)
    starts = list(range(0, L, C))
    ends = [min(s + C, L) - 1 for s in starts]
    n = len(starts)

    def a_before(c):  # A at the last token of the previous chunk (0 before the first chunk)
        return A[starts[c] - 1] if starts[c] > 0 else 0.0

    Fex = [None] * n
    F = np.zeros((d, dv + 1))
    for c in range(n):
        s, e = starts[c], ends[c]
        Fex[c] = F
        w = np.exp(A[e] - A[s:e + 1])
        F = np.exp(A[e] - a_before(c)) * F + (phk[s:e + 1] * w[:, None]).T @ v1[s:e + 1]
    Gex = [None] * n
    G = np.zeros((d, dv + 1))
    for c in range(n - 1, -1, -1):
        s, e = starts[c], ends[c]
        Gex[c] = G
        w = np.exp(A[s:e + 1] - a_before(c))
        G = np.exp(A[e] - a_before(c)) * G + (phk[s:e + 1] * w[:, None]).T @ v1[s:e + 1]
    out = np.empty((L, dv + 1))
    for c in range(n):
        s, e = starts[c], ends[c]
        Ai = A[s:e + 1]
        Mc = np.exp(-np.abs(Ai[:, None] - Ai[None, :]))
        P = (phq[s:e + 1] @ phk[s:e + 1].T) * Mc
        intra = P @ v1[s:e + 1]
        fwd = np.exp(Ai - a_before(c))[:, None] * (phq[s:e + 1] @ Fex[c])
        bwd = np.exp(A[e] - Ai)[:, None] * (phq[s:e + 1] @ Gex[c])
        out[s:e + 1] = intra + fwd + bwd
    den = out[:, dv] + eps
    return out[:, :dv] / den[:, None], den

