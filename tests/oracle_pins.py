"""Pins of the fp64 oracle: checks against what the pages and mathematics fix, not against itself.

Each ``pin_*`` function takes the path of an oracle shared library and raises AssertionError if
the oracle built there disagrees with the pin.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with planted mistakes and
requires every mistake to be caught by at least one pin.

Pages: "LION: A bidirectional framework that trains like a Transformer and infers like an RNN"
(author-reviewer discussion), cited below as [RB] with the reply each passage sits in.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import forms

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / scale if a.size else 0.0
    assert err <= rtol, f"{what}: max rel err {err:.3e} > {rtol:.1e}"


# ---------------------------------------------------------------------------------------------
# phi against library routines [RB, item 4: elu()+1 for LION-LIT, silu normalized for LION-S]

def pin_phi_lit_is_elu_plus_one(lib):
    x = np.random.default_rng(11).standard_normal((257, 24)) * 3
    x[0, :4] = [0.0, -0.0, 1e-300, -1e-300]
    ref = (F.elu(torch.from_numpy(x), alpha=1.0) + 1.0).numpy()
    _close(oracle.phi("lit", x, lib_path=lib), ref, 1e-15, "phi lit vs torch elu+1")


def pin_phi_s_is_normalised_silu(lib):
    x = np.random.default_rng(12).standard_normal((257, 24)) * 3
    x[1] = 0.0                                   # silu(0) = 0 everywhere -> phi = 0 (no epsilon)
    ref = F.normalize(F.silu(torch.from_numpy(x)), p=2.0, dim=-1).numpy()
    got = oracle.phi("s", x, lib_path=lib)
    _close(got, ref, 2e-15, "phi s vs torch normalize(silu)")
    assert np.all(got[1] == 0.0)
    # special value: equal positive entries t -> each 1/sqrt(d)
    row = np.full((1, 16), 0.75)
    _close(oracle.phi("s", row, lib_path=lib), np.full((1, 16), 0.25), 1e-15, "phi s of a constant row")


def pin_phi_d_is_identity(lib):
    x = np.random.default_rng(13).standard_normal((33, 8))
    assert np.array_equal(oracle.phi("d", x, lib_path=lib), x)


# ---------------------------------------------------------------------------------------------
# the mask: invariants and the product definition in exact rationals

def pin_mask_invariants(lib):
    rng = np.random.default_rng(21)
    L = 37
    lam = rng.uniform(0.3, 1.0, L)
    M = oracle.mask(lam, lib_path=lib)
    # symmetric up to rounding: row i multiplies outward from i, so M_ij and M_ji take the same
    # factors in opposite orders
    assert np.all(np.abs(M - M.T) <= 1e-14 * M), "mask not symmetric"
    assert np.all(np.diag(M) == 1.0), "mask diagonal not 1"
    assert np.all(M > 0.0) and np.all(M <= 1.0), "mask outside (0, 1]"
    # semiseparable: M_ij = M_ik M_kj for i <= k <= j
    for i, k, j in [(0, 5, 36), (3, 3, 20), (10, 17, 17), (2, 30, 31)]:
        assert abs(M[i, j] - M[i, k] * M[k, j]) <= 1e-14 * M[i, j], (i, k, j)
    # lam = 1 -> all ones [RB, item 5]
    assert np.all(oracle.mask(np.ones(9), lib_path=lib) == 1.0)


def pin_mask_is_product_of_decays(lib):
    lam_q = [Fraction(1), Fraction(1, 2), Fraction(3, 4), Fraction(5, 8), Fraction(7, 8), Fraction(1, 4)]
    L = len(lam_q)
    M = oracle.mask(np.array([float(t) for t in lam_q]), lib_path=lib)
    for i in range(L):
        for j in range(L):
            exact = Fraction(1)
            for t in range(min(i, j) + 1, max(i, j) + 1):
                exact *= lam_q[t]
            assert M[i, j] == float(exact), (i, j, M[i, j], exact)


# ---------------------------------------------------------------------------------------------
# the whole definition against exact rational brute force and hand-worked cases

def _brute_rational(q, k, v, lam, eps):
    """Exact rational evaluation for phi = identity: products of decays multiplied out directly."""
    L, d = len(q), len(q[0])
    ys, dens = [], []
    for i in range(L):
        num = [Fraction(0)] * d
        den = Fraction(0)
        for j in range(L):
            m = Fraction(1)
            for t in range(min(i, j) + 1, max(i, j) + 1):
                m *= lam[t]
            p = sum((q[i][c] * k[j][c] for c in range(d)), Fraction(0)) * m
            den += p
            for c in range(d):
                num[c] += p * v[j][c]
        ys.append([n / (den + eps) for n in num])
        dens.append(den + eps)
    return ys, dens


def pin_brute_force_rational(lib):
    rng = np.random.default_rng(31)
    for trial in range(12):
        L = int(rng.integers(1, 8))
        d = int(rng.integers(1, 4))
        # dyadic values: exact in binary, so the rational result is the exact result for these inputs
        q = [[Fraction(int(rng.integers(1, 9)), 4) for _ in range(d)] for _ in range(L)]
        k = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(d)] for _ in range(L)]
        v = [[Fraction(int(rng.integers(-16, 17)), 2) for _ in range(d)] for _ in range(L)]
        lam = [Fraction(int(rng.integers(1, 17)), 16) for _ in range(L)]
        eps = Fraction(1, 1024) if trial % 2 else Fraction(0)
        ys, dens = _brute_rational(q, k, v, lam, eps)
        f = lambda a: np.array([[float(t) for t in r] for r in a])[None, None]
        y, den = oracle.attn(f(q), f(k), f(v), np.array([[[float(t) for t in lam]]]), float(eps), lib_path=lib)
        _close(y[0, 0], np.array([[float(t) for t in r] for r in ys]), 1e-13, f"brute force trial {trial}")
        _close(den[0, 0], np.array([float(t) for t in dens]), 1e-13, f"brute force den trial {trial}")


def _read_golden():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "hand_worked.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest}
                cases.append(cur)
            elif key == "kind":
                cur["kind"] = rest
            else:
                cur[key] = [[Fraction(t) for t in row.split()] for row in rest.split("|")]
    return cases


def pin_hand_worked_golden(lib):
    for case in _read_golden():
        arr = lambda key: np.array([[float(t) for t in r] for r in case[key]])
        q, k, v = arr("q")[None, None], arr("k")[None, None], arr("v")[None, None]
        lam = arr("lam")[:, 0]
        if case["kind"] == "lit":
            y, den = oracle.full(q, k, v, None, "lit", 0.0, lib_path=lib)
        else:
            # phi = identity with per-token decays, through the attention entry
            y, den = oracle.attn(q, k, v, lam[None, None], 0.0, lib_path=lib)
        _close(y[0, 0], arr("y"), 1e-15, f"golden case {case['name']} y")
        _close(den[0, 0], arr("den")[:, 0], 1e-15, f"golden case {case['name']} den")


# ---------------------------------------------------------------------------------------------
# closed forms of special cases

def pin_lit_closed_form(lib):
    """lambda = 1: plain non-causal linear attention, O(L d^2) by associativity [RB, item 5]."""
    rng = np.random.default_rng(41)
    B, H, L, d = 2, 3, 45, 12
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    eps = 1e-3
    y, den = oracle.full(q, k, v, None, "lit", eps, lib_path=lib)
    phq = (F.elu(torch.from_numpy(q)) + 1.0).numpy()
    phk = (F.elu(torch.from_numpy(k)) + 1.0).numpy()
    for b in range(B):
        for h in range(H):
            S = phk[b, h].T @ v[b, h]
            z = phk[b, h].sum(axis=0)
            dref = phq[b, h] @ z + eps
            _close(y[b, h], (phq[b, h] @ S) / dref[:, None], 1e-12, "lit closed form")
            _close(den[b, h], dref, 1e-12, "lit closed form den")


def pin_d_toeplitz_closed_form(lib):
    """LION-D: fixed per-head decay, so M_ij = lambda_h^|i-j| (a Toeplitz matrix of powers)."""
    rng = np.random.default_rng(42)
    B, H, L, d = 2, 3, 40, 8
    q, k = np.abs(rng.standard_normal((B, H, L, d))), np.abs(rng.standard_normal((B, H, L, d)))
    v = rng.standard_normal((B, H, L, d))
    lam_h = np.array([0.97, 0.8, 0.5])
    y, den = oracle.full(q, k, v, np.log(lam_h), "d", 0.0, lib_path=lib)
    idx = np.arange(L)
    for b in range(B):
        for h in range(H):
            M = np.power(lam_h[h], np.abs(idx[:, None] - idx[None, :]).astype(np.float64))
            P = (q[b, h] @ k[b, h].T) * M
            _close(y[b, h], (P @ v[b, h]) / P.sum(axis=1)[:, None], 1e-12, "d toeplitz")


def pin_lambda_to_zero_gives_v(lib):
    """lambda -> 0: M -> I, so y_i = v_i (eps = 0) for any phi with phi(q_i).phi(k_i) != 0."""
    rng = np.random.default_rng(43)
    B, H, L, d = 1, 2, 17, 6
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    ll = np.full((B, H, L), -1000.0)
    y, _ = oracle.full(q, k, v, ll, "s", 0.0, lib_path=lib)
    _close(y, v, 1e-12, "lambda -> 0")


# ---------------------------------------------------------------------------------------------
# invariants of the operator

def pin_constant_v_and_linearity(lib):
    rng = np.random.default_rng(51)
    B, H, L, d = 2, 2, 23, 5
    q, k = rng.standard_normal((B, H, L, d)), rng.standard_normal((B, H, L, d))
    ll = np.log(rng.uniform(0.5, 1.0, (B, H, L)))
    for kind in ("lit", "s"):
        lam_arg = None if kind == "lit" else ll
        c = rng.standard_normal(d)
        vc = np.broadcast_to(c, (B, H, L, d)).copy()
        y, _ = oracle.full(q, k, vc, lam_arg, kind, 0.0, lib_path=lib)
        _close(y, vc, 1e-11, f"constant v ({kind})")
        v1, v2 = rng.standard_normal((B, H, L, d)), rng.standard_normal((B, H, L, d))
        ya, _ = oracle.full(q, k, v1, lam_arg, kind, 1e-3, lib_path=lib)
        yb, _ = oracle.full(q, k, v2, lam_arg, kind, 1e-3, lib_path=lib)
        yc, _ = oracle.full(q, k, 2.0 * v1 - 3.0 * v2, lam_arg, kind, 1e-3, lib_path=lib)
        _close(yc, 2.0 * ya - 3.0 * yb, 1e-11, f"linearity in v ({kind})")


def pin_reversal(lib):
    """Reversing the sequence with decays lam'_t = lam_{L-t} (t >= 1) reverses the output: the mask
    of the reversed problem is the reversed mask.  Fixes which decays sit between i and j."""
    rng = np.random.default_rng(52)
    B, H, L, d = 1, 2, 29, 6
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    ll = np.log(rng.uniform(0.3, 1.0, (B, H, L)))
    y, _ = oracle.full(q, k, v, ll, "s", 1e-3, lib_path=lib)
    llr = np.empty_like(ll)
    llr[..., 0] = ll[..., 0]
    llr[..., 1:] = ll[..., :0:-1]
    yr, _ = oracle.full(q[:, :, ::-1], k[:, :, ::-1], v[:, :, ::-1], llr, "s", 1e-3, lib_path=lib)
    _close(yr[:, :, ::-1], y, 1e-11, "reversal")
    # an asymmetric sequence of decays really changes the answer when not reversed alongside
    yw, _ = oracle.full(q[:, :, ::-1], k[:, :, ::-1], v[:, :, ::-1], ll, "s", 1e-3, lib_path=lib)
    assert np.max(np.abs(yw[:, :, ::-1] - y)) > 1e-3


def pin_query_scale_invariance(lib):
    """phi = identity, eps = 0: scaling q_i by alpha > 0 scales numerator and row sum alike."""
    rng = np.random.default_rng(53)
    B, H, L, d = 1, 3, 19, 7
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    ll = np.log(np.array([0.9, 0.7, 0.99]))
    y, _ = oracle.full(q, k, v, ll, "d", 0.0, lib_path=lib)
    alpha = rng.uniform(0.1, 10.0, (B, H, L, 1))
    y2, _ = oracle.full(q * alpha, k, v, ll, "d", 0.0, lib_path=lib)
    _close(y2, y, 1e-9, "query scale")


def pin_decay_indexing_per_head_and_batch(lib):
    """Each (batch, head) uses its own decays: compare against one-problem calls."""
    rng = np.random.default_rng(54)
    B, H, L, d = 2, 3, 11, 4
    q, k, v = (np.abs(rng.standard_normal((B, H, L, d))) for _ in range(3))
    lls = np.log(rng.uniform(0.2, 1.0, (B, H, L)))
    lld = np.log(np.array([0.9, 0.5, 0.7]))
    ys, _ = oracle.full(q, k, v, lls, "s", 0.0, lib_path=lib)
    yd, _ = oracle.full(q, k, v, lld, "d", 0.0, lib_path=lib)
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            y1, _ = oracle.full(q[sl], k[sl], v[sl], lls[sl], "s", 0.0, lib_path=lib)
            _close(ys[sl], y1, 0.0, "per-(b,h) S decays")
            y2, _ = oracle.full(q[sl], k[sl], v[sl], lld[h:h + 1], "d", 0.0, lib_path=lib)
            _close(yd[sl], y2, 0.0, "per-head D decays")
    # and the two kinds give different answers (decays really enter)
    assert np.max(np.abs(ys - yd)) > 1e-3


# ---------------------------------------------------------------------------------------------
# equivalence of the forms the pages state compute the same thing

def pin_forms_equivalent(lib):
    """Full = chunkwise (several C) = naive bidirectional RNN = memory-efficient RNN, in fp64
    [RB, "Concern 1": Theorem 3.3 Eq. 20-25; "4: Practicality of Recurrent Inference"]."""
    rng = np.random.default_rng(61)
    B, H, L, d = 1, 2, 23, 5
    q = np.abs(rng.standard_normal((B, H, L, d)))
    k = np.abs(rng.standard_normal((B, H, L, d)))
    v = rng.standard_normal((B, H, L, d))
    lam = rng.uniform(0.4, 1.0, (B, H, L))
    eps = 1e-4
    y, den = oracle.attn(q, k, v, lam, eps, lib_path=lib)
    for h in range(H):
        a = (q[0, h], k[0, h], v[0, h], lam[0, h], eps)
        for name, (yf, df) in [("naive rnn", forms.naive_birnn(*a)),
                               ("mem-efficient rnn", forms.memory_efficient_birnn(*a))] + \
                              [(f"chunk C={C}", forms.chunkwise(*a, C=C)) for C in (1, 2, 3, 5, 8, L)]:
            _close(yf, y[0, h], 1e-12, f"{name} head {h}")
            _close(df, den[0, h], 1e-12, f"{name} den head {h}")


def pin_rows_entry_matches_full(lib):
    rng = np.random.default_rng(71)
    B, H, L, d = 2, 2, 31, 6
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    ll = np.log(rng.uniform(0.5, 1.0, (B, H, L)))
    y, den, an, ad = oracle.full(q, k, v, ll, "s", 1e-6, want_abs=True, lib_path=lib)
    rid = np.array([0, 5, 30, 31, 62, 123, 100])
    yr, dr, anr, adr = oracle.rows(q, k, v, ll, "s", 1e-6, rid, want_abs=True, lib_path=lib)
    _close(yr, y.reshape(-1, d)[rid], 0.0, "rows y")
    _close(dr, den.reshape(-1)[rid], 0.0, "rows den")
    _close(anr, an.reshape(-1, d)[rid], 0.0, "rows absnum")
    _close(adr, ad.reshape(-1)[rid], 0.0, "rows absden")


def pin_abs_sums(lib):
    """The absolute-value sums of the parity bound are the row sums of |phi q| |phi k|^T (.) M."""
    rng = np.random.default_rng(72)
    B, H, L, d = 1, 1, 13, 4
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    lam = rng.uniform(0.5, 1.0, (B, H, L))
    _, _, an, ad = oracle.attn(q, k, v, lam, 0.0, want_abs=True, lib_path=lib)
    idx = np.arange(L)
    A = np.cumsum(np.log(lam[0, 0]))
    M = np.exp(-np.abs(A[:, None] - A[None, :]))
    Pbar = (np.abs(q[0, 0]) @ np.abs(k[0, 0]).T) * M
    _close(ad[0, 0], Pbar.sum(axis=1), 1e-13, "absden")
    _close(an[0, 0], Pbar @ np.abs(v[0, 0]), 1e-13, "absnum")
    assert idx.size == L


# ---------------------------------------------------------------------------------------------
# the causal variant (keys after the query masked out) against the forward recurrence written out
# here: causal linear attention S_i = S_{i-1} + k_i v_i^T, z_i = z_{i-1} + k_i, y_i = q_i^T S_i / q_i^T z_i
# [RB, reply "1: Recurrence Form of Linear Attention", Eq. 4a-4c], with the decay lambda_i applied to
# the carried state for LION-D and LION-S

def _phi_ref(kind, x):
    t = torch.from_numpy(x)
    if kind == "lit":
        return (F.elu(t, alpha=1.0) + 1.0).numpy()
    if kind == "s":
        return F.normalize(F.silu(t), p=2.0, dim=-1).numpy()
    return x.copy()


def _causal_recurrence(q, k, v, lam, eps):
    L, d = q.shape
    S = np.zeros((d, v.shape[1]))
    z = np.zeros(d)
    y = np.empty_like(v)
    den = np.empty(L)
    for i in range(L):
        S = lam[i] * S + np.outer(k[i], v[i])
        z = lam[i] * z + k[i]
        den[i] = q[i] @ z + eps
        y[i] = (q[i] @ S) / den[i]
    return y, den


def pin_causal_is_forward_recurrence(lib):
    rng = np.random.default_rng(81)
    B, H, L, d = 2, 2, 23, 5
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    for kind, ll in (("lit", None), ("d", np.log(rng.uniform(0.6, 0.99, H))),
                     ("s", np.log(rng.uniform(0.3, 1.0, (B, H, L))))):
        y, den = oracle.full(q, k, v, ll, oracle.KIND_NAMES[kind] | oracle.CAUSAL, 1e-6, lib_path=lib)
        for b in range(B):
            for h in range(H):
                lam = np.ones(L) if kind == "lit" else np.exp(ll[h] if kind == "d" else ll[b, h]) * np.ones(L)
                yr, dr = _causal_recurrence(_phi_ref(kind, q[b, h]), _phi_ref(kind, k[b, h]), v[b, h], lam, 1e-6)
                _close(y[b, h], yr, 1e-12, f"causal {kind} b{b} h{h} vs forward recurrence")
                _close(den[b, h], dr, 1e-12, f"causal {kind} den b{b} h{h}")


def pin_causal_ends(lib):
    """The last row sees every key either way; the first row sees only itself."""
    rng = np.random.default_rng(82)
    B, H, L, d = 1, 3, 17, 4
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    ll = np.log(rng.uniform(0.4, 1.0, (B, H, L)))
    yc, dc = oracle.full(q, k, v, ll, oracle.MASK_S | oracle.CAUSAL, 1e-3, lib_path=lib)
    yb, db = oracle.full(q, k, v, ll, oracle.MASK_S, 1e-3, lib_path=lib)
    _close(yc[:, :, -1], yb[:, :, -1], 1e-14, "causal last row vs bidirectional")
    pq, pk = _phi_ref("s", q[0]), _phi_ref("s", k[0])
    s00 = np.einsum("hc,hc->h", pq[:, 0], pk[:, 0])
    _close(yc[0, :, 0], v[0, :, 0] * (s00 / (s00 + 1e-3))[:, None], 1e-14, "causal first row")
    # and the causal rows never depend on later keys: change the last key and value
    k2, v2 = k.copy(), v.copy()
    k2[:, :, -1] += 1.0
    v2[:, :, -1] -= 2.0
    y2, _ = oracle.full(q, k2, v2, ll, oracle.MASK_S | oracle.CAUSAL, 1e-3, lib_path=lib)
    assert np.array_equal(y2[:, :, :-1], yc[:, :, :-1]), "causal rows depend on a later token"


def pin_bwd_finite_differences(lib):
    """The backward oracle against central differences of the (pinned) forward definition.

    Loss = sum(y * R) for a fixed random R, so dL/dy = R.  Every element of q, k, v and log(lambda) is
    perturbed by +-h; the forward oracle alone gives the slope.  Covers every kind, the causal variant,
    LION-D's per-head decay shared by two batch entries, and eps."""
    rng = np.random.default_rng(91)
    B, H, L, d, eps, h = 2, 2, 6, 3, 0.05, 1e-6
    for kind in (oracle.MASK_LIT, oracle.MASK_D, oracle.MASK_S, oracle.MASK_S | oracle.CAUSAL,
                 oracle.MASK_D | oracle.CAUSAL):
        q, k, v, R = (rng.standard_normal((B, H, L, d)) for _ in range(4))
        base = kind & 3
        ll = None if base == 0 else (np.log(rng.uniform(0.3, 0.95, (H,))) if base == 1
                                     else np.log(rng.uniform(0.2, 1.0, (B, H, L))))
        dq, dk, dv, dll = oracle.full_bwd(q, k, v, ll, kind, eps, R, lib_path=lib)

        def loss(q_, k_, v_, ll_):
            y, _ = oracle.full(q_, k_, v_, ll_, kind, eps, lib_path=lib)
            return float(np.sum(y * R))

        def fd(x, which):
            g = np.empty_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v, ll]
                args_m = [q, k, v, ll]
                args_p[which], args_m[which] = xp, xm
                g[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            return g

        for name, an, which in (("dq", dq, 0), ("dk", dk, 1), ("dv", dv, 2)):
            num = fd([q, k, v][which], which)
            _close(an, num, 1e-6 * max(1.0, float(np.max(np.abs(num)))), f"{name} kind={kind}")
        if base:
            num = fd(ll, 3)
            _close(dll, num, 1e-6 * max(1.0, float(np.max(np.abs(num)))), f"dlog_lambda kind={kind}")


def pin_bwd_abs_companions(lib):
    """The backward's absolute-value companions bound their gradients (triangle inequality) and do not
    change when dy or v flip sign -- what makes them a bound on rounding, not another gradient."""
    rng = np.random.default_rng(92)
    B, H, L, d = 2, 2, 9, 4
    for kind in (oracle.MASK_LIT, oracle.MASK_D, oracle.MASK_S, oracle.MASK_S | oracle.CAUSAL):
        q, k, v, dy = (rng.standard_normal((B, H, L, d)) for _ in range(4))
        base = kind & 3
        ll = None if base == 0 else (np.log(rng.uniform(0.3, 0.95, (H,))) if base == 1
                                     else np.log(rng.uniform(0.2, 1.0, (B, H, L))))
        r = oracle.full_bwd(q, k, v, ll, kind, 1e-3, dy, want_abs=True, lib_path=lib)
        r2 = oracle.full_bwd(q, k, -v, ll, kind, 1e-3, -dy, want_abs=True, lib_path=lib)
        for name, gr, ab, ab2 in zip(("dq", "dk", "dv", "dll"), r[:4], r[4:], r2[4:]):
            if gr is None:
                continue
            assert np.all(np.abs(gr) <= ab * (1 + 1e-12)), f"{name} companion does not bound it (kind={kind})"
            _close(ab2, ab, 1e-13, f"{name} companion under sign flips (kind={kind})")


def pin_selectivity(lib):
    """log(lambda) = log sigmoid(x . w_h + b_h) and the key scale lambda - 1, against scipy's log_expit
    and expit on a numpy matmul, with closed-form values at z = 0 and the far tails."""
    from scipy.special import expit, log_expit
    rng = np.random.default_rng(93)
    B, L, H, Dm, d = 2, 7, 3, 40, 5
    x = rng.standard_normal((B, L, Dm))
    w = rng.standard_normal((H, Dm)) / np.sqrt(Dm)
    bias = np.array([3.0, -1.0, 0.0])
    k = rng.standard_normal((B, H, L, d))
    ll, ks, ko = oracle.selectivity(x, w, bias, k, lib_path=lib)
    z = np.einsum("blc,hc->bhl", x, w) + bias[None, :, None]
    _close(ll, log_expit(z), 1e-14, "log lambda vs log_expit")
    _close(ks, expit(z) - 1.0, 1e-14, "key scale vs expit - 1")
    _close(ko, ks[..., None] * k, 1e-15, "scaled keys")
    # closed forms: z = 0 -> log(1/2), -1/2; z = +-40 -> -exp(-40), 40 + log... (no overflow, no underflow to 0)
    xz = np.zeros((1, 3, 1))
    wz = np.ones((1, 1))
    for bb, ll_ref, ks_ref in ((0.0, -np.log(2.0), -0.5), (40.0, -np.exp(-40.0), -np.exp(-40.0)),
                               (-40.0, -40.0 - np.log1p(np.exp(-40.0)), -1.0 / (1.0 + np.exp(-40.0)))):
        l1, k1, _ = oracle.selectivity(xz, wz, np.array([bb]), lib_path=lib)
        _close(l1, np.full_like(l1, ll_ref), 1e-15, f"log lambda at z = {bb}")
        _close(k1, np.full_like(k1, ks_ref), 1e-15, f"key scale at z = {bb}")


def _brute_rational_two(q, k, v, lam, eps, order):
    """Exact rational evaluation of the two-order mask (phi = identity): the decay products taken along
    the tokens' own order and along ``order``, averaged."""
    L, d = len(q), len(q[0])
    pos = {t: p for p, t in enumerate(order)}
    ys = []
    for i in range(L):
        num = [Fraction(0)] * d
        den = Fraction(0)
        for j in range(L):
            mb = Fraction(1)
            for t in range(min(i, j) + 1, max(i, j) + 1):
                mb *= lam[t]
            mc = Fraction(1)
            for p in range(min(pos[i], pos[j]) + 1, max(pos[i], pos[j]) + 1):
                mc *= lam[order[p]]
            s = sum((q[i][c] * k[j][c] for c in range(d)), Fraction(0)) * (mb + mc) / 2
            den += s
            for c in range(d):
                num[c] += s * v[j][c]
        ys.append([n / (den + eps) for n in num])
    return ys


def pin_two_order_mask(lib):
    """Averaged masks of two token orders: brute force on tiny inputs with arbitrary permutations
    (per-token decays, LION-S), exact rationals for LION-D; the identity order (and, for LION-D, the
    reversed order, which keeps every distance) reduce to the one-order definition; LIT is unchanged by
    any order."""
    rng = np.random.default_rng(94)
    # LION-S: phi from the (separately pinned) phi routine, the two masks as explicit decay products
    for trial in range(8):
        L = int(rng.integers(1, 8))
        d = int(rng.integers(1, 4))
        q, k, v = (rng.standard_normal((1, 1, L, d)) for _ in range(3))
        lam = rng.uniform(0.2, 1.0, L)
        order = [int(t) for t in rng.permutation(L)]
        pos = {t: p for p, t in enumerate(order)}
        M = np.zeros((L, L))
        for i in range(L):
            for j in range(L):
                mb = 1.0
                for t in range(min(i, j) + 1, max(i, j) + 1):
                    mb *= lam[t]
                mc = 1.0
                for p in range(min(pos[i], pos[j]) + 1, max(pos[i], pos[j]) + 1):
                    mc *= lam[order[p]]
                M[i, j] = 0.5 * (mb + mc)
        phq = oracle.phi("s", q[0, 0], lib_path=lib)
        phk = oracle.phi("s", k[0, 0], lib_path=lib)
        P = M * (phq @ phk.T)
        ref = (P @ v[0, 0]) / (P.sum(1) + 1e-3)[:, None]
        y, _ = oracle.full2(q, k, v, np.log(lam)[None, None], "s", 1e-3, order, lib_path=lib)
        _close(y[0, 0], ref, 1e-12, f"two-order mask, per-token decays, trial {trial}")
    # kind D (phi = identity, one decay per head) against exact rationals
    for trial in range(6):
        L = int(rng.integers(2, 7))
        d = 2
        q = [[Fraction(int(rng.integers(1, 9)), 4) for _ in range(d)] for _ in range(L)]
        k = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(d)] for _ in range(L)]
        v = [[Fraction(int(rng.integers(-16, 17)), 2) for _ in range(d)] for _ in range(L)]
        lam1 = Fraction(int(rng.integers(2, 16)), 16)
        lam = [lam1] * L
        order = [int(t) for t in rng.permutation(L)]
        ys = _brute_rational_two(q, k, v, lam, Fraction(1, 512), order)
        f = lambda a: np.array([[float(t) for t in r] for r in a])[None, None]
        y, _ = oracle.full2(f(q), f(k), f(v), np.array([np.log(float(lam1))]), "d", 1 / 512, order, lib_path=lib)
        _close(y[0, 0], np.array([[float(t) for t in r] for r in ys]), 1e-13, f"two-order D trial {trial}")
    # reductions
    B, H, L, d = 2, 2, 23, 5
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    ll_s = np.log(rng.uniform(0.3, 1.0, (B, H, L)))
    ll_d = np.log(np.array([0.9, 0.6]))
    ident = np.arange(L)
    for kind, ll in (("s", ll_s), ("d", ll_d)):
        y1, d1 = oracle.full(q, k, v, ll, kind, 1e-3, lib_path=lib)
        y2, d2 = oracle.full2(q, k, v, ll, kind, 1e-3, ident, lib_path=lib)
        _close(y2, y1, 1e-14, f"identity second order, kind {kind}")
    yr, _ = oracle.full2(q, k, v, ll_d, "d", 1e-3, ident[::-1], lib_path=lib)
    y1, _ = oracle.full(q, k, v, ll_d, "d", 1e-3, lib_path=lib)
    _close(yr, y1, 1e-13, "reversed order keeps LION-D's distances")
    perm = rng.permutation(L)
    yl, _ = oracle.full2(q, k, v, None, "lit", 1e-3, perm, lib_path=lib)
    y1, _ = oracle.full(q, k, v, None, "lit", 1e-3, lib_path=lib)
    _close(yl, y1, 1e-14, "LIT under any order")


ALL_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_abs_companions,
    pin_selectivity,
    pin_two_order_mask,
    pin_phi_lit_is_elu_plus_one,
    pin_phi_s_is_normalised_silu,
    pin_phi_d_is_identity,
    pin_mask_invariants,
    pin_mask_is_product_of_decays,
    pin_brute_force_rational,
    pin_hand_worked_golden,
    pin_lit_closed_form,
    pin_d_toeplitz_closed_form,
    pin_lambda_to_zero_gives_v,
    pin_constant_v_and_linearity,
    pin_reversal,
    pin_query_scale_invariance,
    pin_decay_indexing_per_head_and_batch,
    pin_forms_equivalent,
    pin_rows_entry_matches_full,
    pin_abs_sums,
    pin_causal_is_forward_recurrence,
    pin_causal_ends,
]
