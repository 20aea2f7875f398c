"""The C ABI on the host (CPU only): the library loads, exports every symbol the header declares,
and rejects every invalid argument with the documented status before any HIP call.

Only argument combinations that validation must reject are passed here (with fake, aligned,
non-null pointers); nothing in this file can reach a kernel launch.
"""
import ctypes
import os
import re

import pytest

import bidirectional_linear_attention_lion_amd as lion
from bidirectional_linear_attention_lion_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lion_attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
P = 0x10000          # fake aligned device address: never dereferenced by the calls below
MIS = 0x10008        # misaligned by 8 bytes
SIZE_MAX = (1 << 64) - 1


def header_symbols():
    with open(HEADER) as fh:
        text = fh.read()
    return re.findall(r"LION_API\s+[\w\s\*]+?\b(lion_\w+)\s*\(", text)


def test_library_exports_every_declared_symbol():
    lib = lion.library()
    names = header_symbols()
    assert set(names) == {"lion_attn_full", "lion_attn_full2", "lion_attn_chunk", "lion_attn_birnn",
                          "lion_attn_full_bwd", "lion_attn_chunk_bwd", "lion_attn_chunk2", "lion_selectivity", "lion_attn_workspace_bytes",
                          "lion_attn_chunk_noalloc",
                          "lion_status_str", "lion_attn_abi_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert lion.lion_attn_abi_version() == 1


def test_status_strings():
    assert lion.lion_status_str(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert lion.lion_status_str(s) not in ("ok", "unknown status")
    assert lion.lion_status_str(-99) == "unknown status"


def full(q=P, k=P, v=P, ll=None, kind=0, eps=1e-6, B=2, H=3, L=17, d=64, dt=1, y=P, ydt=1, den=None):
    return lion.library().lion_attn_full(q, k, v, ll, kind, eps, B, H, L, d, dt, y, ydt, den, None)


def chunk(C=64, ws=None, wsb=0, **kw):
    a = dict(q=P, k=P, v=P, ll=None, kind=0, eps=1e-6, B=2, H=3, L=17, d=64, dt=1, y=P, ydt=1, den=None)
    a.update(kw)
    return lion.library().lion_attn_chunk(a["q"], a["k"], a["v"], a["ll"], a["kind"], C, a["eps"], a["B"], a["H"],
                                          a["L"], a["d"], a["dt"], a["y"], a["ydt"], a["den"], ws, wsb, None)


def birnn(ws=None, wsb=0, **kw):
    a = dict(q=P, k=P, v=P, ll=None, kind=0, eps=1e-6, B=2, H=3, L=17, d=64, dt=1, y=P, ydt=1, den=None)
    a.update(kw)
    return lion.library().lion_attn_birnn(a["q"], a["k"], a["v"], a["ll"], a["kind"], a["eps"], a["B"], a["H"],
                                          a["L"], a["d"], a["dt"], a["y"], a["ydt"], a["den"], ws, wsb, None)


INVALID_CASES = [
    ("null q", dict(q=None)), ("null k", dict(k=None)), ("null v", dict(v=None)), ("null y", dict(y=None)),
    ("misaligned q", dict(q=MIS)), ("misaligned y", dict(y=MIS)), ("misaligned den", dict(den=MIS)),
    ("bad kind", dict(kind=3)), ("negative kind", dict(kind=-1)),
    ("unknown flag bit", dict(kind=16)), ("causal bad kind", dict(kind=3 | 4)),
    ("causal LIT with log_lambda", dict(kind=4, ll=P)), ("causal S without log_lambda", dict(kind=2 | 4, ll=None)),
    ("LIT with log_lambda", dict(kind=0, ll=P)), ("D without log_lambda", dict(kind=1, ll=None)),
    ("S without log_lambda", dict(kind=2, ll=None)), ("misaligned log_lambda", dict(kind=1, ll=MIS)),
    ("negative eps", dict(eps=-1e-3)), ("nan eps", dict(eps=float("nan"))), ("inf eps", dict(eps=float("inf"))),
    ("B=0", dict(B=0)), ("H=0", dict(H=0)), ("L=0", dict(L=0)), ("d=0", dict(d=0)), ("L negative", dict(L=-5)),
    ("L too large", dict(L=(1 << 22) + 1)), ("rows too many", dict(B=1 << 12, H=1 << 10, L=1 << 10)),
    ("bad dtype", dict(dt=2)), ("bad y dtype", dict(ydt=7)),
]
UNSUPPORTED_CASES = [("d=48", dict(d=48)), ("d=256", dict(d=256)), ("d=8", dict(d=8)),
                     ("f32 in, bf16 out", dict(dt=0, ydt=1))]


def chunk_noalloc(C=64, **kw):
    a = dict(q=P, k=P, v=P, ll=None, kind=0, eps=1e-6, B=2, H=3, L=17, d=64, dt=1, y=P, ydt=1, den=None)
    a.update(kw)
    return lion.library().lion_attn_chunk_noalloc(a["q"], a["k"], a["v"], a["ll"], a["kind"], C, a["eps"], a["B"],
                                                  a["H"], a["L"], a["d"], a["dt"], a["y"], a["ydt"], a["den"], None)


ENTRIES = [full, chunk, birnn, chunk_noalloc]
ENTRY_IDS = ["full", "chunk", "birnn", "chunk_noalloc"]


@pytest.mark.parametrize("name,kw", INVALID_CASES, ids=[c[0] for c in INVALID_CASES])
@pytest.mark.parametrize("entry", ENTRIES, ids=ENTRY_IDS)
def test_invalid_arguments(entry, name, kw):
    assert entry(**kw) == INVALID


@pytest.mark.parametrize("name,kw", UNSUPPORTED_CASES, ids=[c[0] for c in UNSUPPORTED_CASES])
@pytest.mark.parametrize("entry", ENTRIES, ids=ENTRY_IDS)
def test_unsupported_combinations(entry, name, kw):
    assert entry(**kw) == UNSUPPORTED


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """The no-allocation chunkwise entry point serves sizes whose workspace fits its built-in array and
    rejects larger ones (before any HIP call) with LION_ERR_WORKSPACE."""
    cap = 64 << 20
    sizes = [(8, 12, 4097, 16), (8, 12, 4097, 32), (64, 12, 197, 16), (32, 16, 512, 16), (16, 12, 4097, 64)]
    seen_reject = False
    for (B, H, L, C) in sizes:
        need = lion.lion_attn_workspace_bytes(lion.FORM_CHUNK, B, H, L, 64, C, 1)
        if need > cap:
            seen_reject = True
            assert chunk_noalloc(C=C, B=B, H=H, L=L, kind=1, ll=P) == WORKSPACE, (B, H, L, C)
    assert seen_reject
    assert chunk_noalloc(C=48) == UNSUPPORTED and chunk_noalloc(C=0) == INVALID


@pytest.mark.parametrize("C,status", [(0, INVALID), (-64, INVALID), (48, UNSUPPORTED), (512, UNSUPPORTED),
                                      (8, UNSUPPORTED)])
def test_chunk_size_checks(C, status):
    assert chunk(C=C) == status


def test_chunk_size_limit_for_d128():
    assert chunk(C=256, d=128) == UNSUPPORTED
    assert lion.lion_attn_workspace_bytes(lion.FORM_CHUNK, 1, 1, 100, 128, 256, 1) == SIZE_MAX


def test_workspace_query():
    wb = lion.lion_attn_workspace_bytes
    assert wb(lion.FORM_FULL, 2, 3, 17, 64, 0, 1) == 0
    for bad in [(lion.FORM_FULL, 0, 3, 17, 64, 0, 1), (lion.FORM_CHUNK, 2, 3, 17, 64, 48, 1),
                (lion.FORM_BIRNN, 2, 3, 17, 48, 0, 1), (7, 2, 3, 17, 64, 64, 1), (lion.FORM_FULL, 2, 3, 17, 64, 0, 5)]:
        assert wb(*bad) == SIZE_MAX, bad
    for form in (lion.FORM_CHUNK, lion.FORM_BIRNN):
        for L in (1, 197, 512, 4097):
            n = wb(form, 8, 12, L, 64, 64, 1)
            assert 0 <= n < (1 << 40)


@pytest.mark.parametrize("form,entry", [(binding.FORM_CHUNK, chunk), (binding.FORM_BIRNN, birnn)])
def test_workspace_too_small(form, entry):
    """Sizes for which the form needs scratch memory must reject a missing or short workspace."""
    for (B, H, L) in [(8, 12, 4097), (64, 12, 197), (1, 1, 100000)]:
        need = lion.lion_attn_workspace_bytes(form, B, H, L, 64, 64, 1)
        if need == 0:
            continue
        # the query answers for every way the form can run; fp32 arithmetic (flag 8) needs the most
        kw = dict(kind=1 | 8, ll=P, B=B, H=H, L=L)
        assert entry(ws=None, wsb=need, **kw) == WORKSPACE
        assert entry(ws=P, wsb=need - 1, **kw) == WORKSPACE
        return
    pytest.skip("form needs no workspace at any tested size")


def bwd(ws=P, wsb=1 << 30, **kw):
    a = dict(q=P, k=P, v=P, ll=None, kind=0, B=2, H=3, L=17, d=64, dt=1, y=P, den=P, dy=P, dq=P, dk=P, dv=P, gdt=0,
             dll=None)
    a.update(kw)
    return lion.library().lion_attn_full_bwd(a["q"], a["k"], a["v"], a["ll"], a["kind"], a["B"], a["H"], a["L"],
                                             a["d"], a["dt"], a["y"], a["den"], a["dy"], a["dq"], a["dk"], a["dv"],
                                             a["gdt"], a["dll"], ws, wsb, None)


BWD_INVALID = [
    ("null q", dict(q=None)), ("null y", dict(y=None)), ("null den", dict(den=None)), ("null dy", dict(dy=None)),
    ("null dq", dict(dq=None)), ("null dk", dict(dk=None)), ("null dv", dict(dv=None)),
    ("misaligned dy", dict(dy=MIS)), ("misaligned dv", dict(dv=MIS)), ("misaligned den", dict(den=MIS)),
    ("LIT with dlog_lambda", dict(dll=P)), ("S without dlog_lambda", dict(kind=2, ll=P, dll=None)),
    ("D without log_lambda", dict(kind=1, ll=None, dll=P)), ("misaligned dlog_lambda", dict(kind=1, ll=P, dll=MIS)),
    ("bad grad dtype", dict(gdt=3)), ("bad kind", dict(kind=3)), ("L=0", dict(L=0)), ("misaligned workspace", dict(ws=MIS)),
]


@pytest.mark.parametrize("name,kw", BWD_INVALID, ids=[c[0] for c in BWD_INVALID])
def test_bwd_invalid_arguments(name, kw):
    assert bwd(**kw) == INVALID


def test_bwd_unsupported_and_workspace():
    assert bwd(dt=0) == UNSUPPORTED                 # fp32 inputs
    assert bwd(d=16) == UNSUPPORTED
    assert bwd(kind=0 | 8) == UNSUPPORTED           # fp32 arithmetic: forward only
    need = lion.lion_attn_workspace_bytes(lion.FORM_FULL_BWD, 2, 3, 17, 64, 0, 1)
    assert need == 12 * 2 * 3 * 17
    assert lion.lion_attn_workspace_bytes(lion.FORM_FULL_BWD, 2, 3, 17, 64, 0, 0) == SIZE_MAX
    assert bwd(ws=None, wsb=need) == WORKSPACE
    assert bwd(ws=P, wsb=need - 1) == WORKSPACE


def cbwd(C=64, ws=P, wsb=1 << 30, **kw):
    a = dict(q=P, k=P, v=P, ll=None, kind=0, B=2, H=3, L=17, d=64, dt=1, y=P, den=P, dy=P, dq=P, dk=P, dv=P, gdt=0,
             dll=None)
    a.update(kw)
    return lion.library().lion_attn_chunk_bwd(a["q"], a["k"], a["v"], a["ll"], a["kind"], C, a["B"], a["H"], a["L"],
                                              a["d"], a["dt"], a["y"], a["den"], a["dy"], a["dq"], a["dk"], a["dv"],
                                              a["gdt"], a["dll"], ws, wsb, None)


@pytest.mark.parametrize("name,kw", BWD_INVALID, ids=[c[0] for c in BWD_INVALID])
def test_chunk_bwd_invalid_arguments(name, kw):
    assert cbwd(**kw) == INVALID


def test_chunk_bwd_unsupported_and_workspace():
    assert cbwd(dt=0) == UNSUPPORTED                 # fp32 inputs
    assert cbwd(d=16) == UNSUPPORTED
    for C in (8, 256, 0):
        assert cbwd(C=C) == UNSUPPORTED
    assert cbwd(C=128, d=128) == UNSUPPORTED         # chunks of 128 need d <= 64
    assert lion.lion_attn_workspace_bytes(lion.FORM_CHUNK_BWD, 2, 3, 17, 128, 128, 1) == SIZE_MAX
    assert lion.lion_attn_workspace_bytes(lion.FORM_CHUNK_BWD, 2, 3, 17, 64, 64, 0) == SIZE_MAX
    B, H, L, d = 2, 3, 150, 64
    da = 4 * 2 * ((B * H * L + 3) // 4) * 4          # the two dA halves
    # chunks of 16 and 32: four d x (d+1) fp32 states (rows padded to d + 4) per chunk and (batch, head)
    for C in (16, 32):
        nch = (L + C - 1) // C
        want = 4 * 4 * B * H * nch * d * (d + 4) + da
        need = lion.lion_attn_workspace_bytes(lion.FORM_CHUNK_BWD, B, H, L, d, C, 1)
        assert need == want
        assert cbwd(C=C, B=B, H=H, L=L, ws=None, wsb=need) == WORKSPACE
        assert cbwd(C=C, B=B, H=H, L=L, ws=P, wsb=need - 1) == WORKSPACE
    # chunks of 64 and 128: four bf16 d x d blocks and four fp32 last columns per chunk
    for C in (64, 128):
        nch = (L + C - 1) // C
        want = B * H * nch * 4 * (2 * d * d + 4 * d) + da
        assert lion.lion_attn_workspace_bytes(lion.FORM_CHUNK_BWD, B, H, L, d, C, 1) == want
        assert cbwd(C=C, B=B, H=H, L=L, ws=P, wsb=want - 1) == WORKSPACE


def chunk2(order=P, C=64, ws=P, wsb=1 << 40, **kw):
    a = dict(q=P, k=P, v=P, ll=P, kind=1, eps=1e-6, B=2, H=3, L=17, d=64, dt=1, y=P, ydt=1, den=None)
    a.update(kw)
    return lion.library().lion_attn_chunk2(a["q"], a["k"], a["v"], a["ll"], a["kind"], C, a["eps"], order, a["B"],
                                           a["H"], a["L"], a["d"], a["dt"], a["y"], a["ydt"], a["den"], ws, wsb, None)


def test_chunk2_arguments():
    assert chunk2(order=None) == INVALID
    assert chunk2(order=MIS) == INVALID
    assert chunk2(q=None) == INVALID
    assert chunk2(ws=MIS) == INVALID
    assert chunk2(kind=1 | 4) == UNSUPPORTED
    assert chunk2(C=48) == UNSUPPORTED
    need = lion.lion_attn_workspace_bytes(lion.FORM_CHUNK2, 2, 3, 17, 64, 64, 1)
    assert need != SIZE_MAX and need > 2 * 3 * 17 * 64 * (3 * 2 + 2 * 4)
    # the size query answers for LION-S (the largest: its rearranged log(lambda) too)
    assert chunk2(kind=2, ws=None, wsb=need) == WORKSPACE
    assert chunk2(kind=2, ws=P, wsb=need - 1) == WORKSPACE


def full2(order=P, **kw):
    a = dict(q=P, k=P, v=P, ll=P, kind=1, eps=1e-6, B=2, H=3, L=17, d=64, dt=1, y=P, ydt=1, den=None)
    a.update(kw)
    return lion.library().lion_attn_full2(a["q"], a["k"], a["v"], a["ll"], a["kind"], a["eps"], order, a["B"],
                                          a["H"], a["L"], a["d"], a["dt"], a["y"], a["ydt"], a["den"], None)


def test_full2_arguments():
    assert full2(order=None) == INVALID
    assert full2(order=MIS) == INVALID
    assert full2(q=None) == INVALID
    assert full2(kind=1 | 4) == UNSUPPORTED
    assert full2(d=48) == UNSUPPORTED


def sel(x=P, w=P, bias=P, B=2, L=17, H=3, Dm=64, ll=P, ks=None, k=None, ko=None, d=64):
    return lion.library().lion_selectivity(x, w, bias, B, L, H, Dm, ll, ks, k, ko, d, None)


SEL_INVALID = [
    ("null x", dict(x=None)), ("null w", dict(w=None)), ("null bias", dict(bias=None)), ("null out", dict(ll=None)),
    ("misaligned x", dict(x=MIS)), ("misaligned key scale", dict(ks=MIS)), ("k without k_out", dict(k=P)),
    ("k_out without k", dict(ko=P)), ("misaligned k_out", dict(k=P, ko=MIS)), ("k with d=0", dict(k=P, ko=P, d=0)),
    ("B=0", dict(B=0)), ("L=0", dict(L=0)), ("H=0", dict(H=0)), ("Dm=0", dict(Dm=0)),
]


@pytest.mark.parametrize("name,kw", SEL_INVALID, ids=[c[0] for c in SEL_INVALID])
def test_selectivity_invalid_arguments(name, kw):
    assert sel(**kw) == INVALID


def test_selectivity_unsupported():
    assert sel(Dm=48) == UNSUPPORTED
    assert sel(k=P, ko=P, d=12) == UNSUPPORTED


def test_binding_requires_built_library(monkeypatch, tmp_path):
    """No fallback: a missing library is an error, not a silent CPU path."""
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError):
        binding.library()


def test_fp32_arith_flag():
    """LION_FP32_ARITH is accepted by the full, chunkwise and RNN forms and refused (unsupported) by the
    two-order forms; the chunkwise workspace query covers the fp32 states it needs."""
    F = 8
    lib = lion.library()
    for C in (64, 128):
        for L in (197, 4097):
            wf = lion.lion_attn_workspace_bytes(lion.FORM_CHUNK, 2, 3, L, 64, C, 1)
            w32 = lion.lion_attn_workspace_bytes(lion.FORM_CHUNK, 2, 3, L, 64, C, 0)
            assert wf >= w32, (C, L, wf, w32)   # bf16 inputs may take fp32 states
    assert lib.lion_attn_full2(P, P, P, P, 1 | F, 1e-6, P, 2, 3, 17, 64, 1, P, 0, None, None) == UNSUPPORTED
    assert lib.lion_attn_chunk2(P, P, P, P, 1 | F, 64, 1e-6, P, 2, 3, 17, 64, 1, P, 0, None, None, 0, None) == UNSUPPORTED
    assert full(kind=3 | F) == INVALID and full(kind=16 | F) == INVALID
