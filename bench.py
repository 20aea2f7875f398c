"""Throughput of LION bidirectional masked linear attention (forward) on one MI355X.

Default workload: the high-resolution LION-D inference shape (a 1024 x 1024 image in 16-pixel patches
plus the class token: B8 H12 L4097 d64, bf16), the largest configuration that fits one GPU, with every
form it is quoted with: the chunkwise form at C = 64, 128 and 256, the bidirectional RNN, and the full
form as the memory-bound reference.  Form keys: ``full``, ``chunk<C>`` (``chunk`` alone means the
workload's chunk sizes, or --chunk), ``birnn``; and, off the default, ``full_bwd``, ``chunk_bwd<C>``,
``selectivity``, ``full2``, ``chunk2_<C>``.

One step = one call of every form over one batch of the workload's synthetic inputs; each call writes
the attention output of all B x L tokens (every head).  The timed region runs the K steps form by form:
K back-to-back calls of each form between one pair of HIP events on the launch stream, so each form's
average call duration is its events' span / K.  Input sets are rotated so that more than --rotate-gib
of distinct buffers stream through HBM: the 256 MB last-level cache cannot hold them, so kernels read
HBM, not cache.

Prints one JSON line:
  value         tokens/s (B x L per call) of the fastest forward form of the step -- the form a user
                would run this workload with (``config.value_form`` names it; the pages find the
                chunkwise form the fastest at inference).  Each form's own rate is in ``forms``.
  ms_per_step   the step (every form once); ``step_tokens_per_s`` = B x L / ms_per_step.
  forms         per form: tokens/s, average call time, algorithmic GB/s and TFLOP/s, the binding roof
                and the fraction of it, memory (inputs + output + workspace), single-call spread.
  roofline      for the form with the largest share of the step (the dominant kernel).
  cpu_baseline  the fp64 oracle on the host, on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LION attention fwd tokens/s per form (full/chunk/RNN) + % of MFMA or HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense
VALU_FP32_PEAK_TFLOPS = 157.3   # fp32 vector
CSRC = os.path.join(ROOT, "bidirectional_linear_attention_lion_amd", "csrc")
KERNEL_FILES = {"full": "lion_full.hip", "chunk": "lion_chunk.hip", "birnn": "lion_birnn.hip",
                "full_bwd": ("lion_full_bwd.hip", "lion_chunk_bwd_mfma.hip", "lion_bwd_tiles.h"),
                "chunk_bwd": ("lion_chunk_bwd_mfma.hip", "lion_bwd_tiles.h"), "selectivity": "lion_selectivity.hip",
                "full2": "lion_full.hip", "chunk2": "lion_chunk2.hip"}
SEL_WIDTH = 1024   # layer-input width of the selectivity prologue (the BERT-Large-shaped recipe)
FORWARD_FORMS = ("full", "chunk", "birnn", "full2", "chunk2")


def split_form(key: str, default_c: int = 64):
    """Form key -> (form, C): ``chunk128`` -> ("chunk", 128), ``chunk_bwd32``, ``chunk2_128`` (two orders);
    chunkwise keys without a size take default_c (chunk_bwd: 64)."""
    for form, pat in (("chunk2", r"chunk2(?:_(\d+))?"), ("chunk_bwd", r"chunk_bwd(\d*)"), ("chunk", r"chunk(\d*)")):
        m = re.fullmatch(pat, key)
        if m:
            c = m.group(1)
            return form, int(c) if c else (64 if form == "chunk_bwd" else default_c)
    if key in ("full", "full2", "full_bwd", "birnn", "selectivity"):
        return key, default_c
    raise SystemExit(f"bench.py: unknown form key {key!r}")


def default_forms(wl, chunk=None):
    """The workload's forms, the chunkwise one at each of its chunk sizes (or at ``chunk``); the
    4097-token workload adds the full form as the memory-bound reference."""
    keys = []
    for f in wl.forms:
        if f == "chunk":
            keys += [f"chunk{c}" for c in ((chunk,) if chunk else wl.chunks)]
        else:
            keys.append(f)
    if wl.L > 2048 and "full" not in keys:
        keys.append("full")
    return keys


def memory_bytes(form: str, wl, C: int, workspace_bytes: int) -> dict:
    """Device memory a call touches: inputs, output and workspace (the full form never forms the L x L
    score or mask matrix; the pages' PyTorch full form does)."""
    esz = 2 if wl.dtype == "bf16" else 4
    io = 4 * wl.B * wl.H * wl.L * wl.d * esz
    io += {0: 0, 1: 4 * wl.H, 2: 4 * wl.B * wl.H * wl.L}[wl.kind]
    return {"io_MB": io / 1e6, "workspace_MB": workspace_bytes / 1e6, "total_MB": (io + workspace_bytes) / 1e6}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="hires_d")
    ap.add_argument("--forms", default=None,
                    help="comma-separated form keys (default: the workload's forms, the chunkwise form at each of "
                         "its chunk sizes; the 4097-token workload adds the full form as a reference): full, "
                         "chunk<C>, birnn; full_bwd (the full form's backward pass, bf16 gradients; y, den and a "
                         "random dy prepared beforehand), chunk_bwd<C> (the same gradients computed chunkwise; C = 16, "
                         "32 on fp32 matrix cores, 64, 128 on bf16 ones; default 64), selectivity (the LION-S "
                         "prologue: log lambda from a [B, L, 1024] "
                         "layer input, keys scaled), full2 / chunk2 (the masks of the raster and the "
                         "column-major patch order averaged; image workloads, L = 1 + n^2; the chunkwise one is keyed "
                         "chunk2_<C>)")
    ap.add_argument("--chunk", type=int, default=None,
                    help="chunk size C for form keys given without one (default: the workload's chunk sizes)")
    ap.add_argument("--causal", action="store_true",
                    help="the causal variant (keys after the query masked out) of the workload's mask")
    ap.add_argument("--fp32-arith", action="store_true",
                    help="fp32 arithmetic throughout for the bf16 inputs (LION_FP32_ARITH; full and chunkwise "
                         "forms), fp32 outputs")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0,
                    help="wall-time budget of the oracle sample (0 disables)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run plain device copies of this many MiB (reference for "
                         "HBM byte counters) and print their rate")
    return ap.parse_args()


def copy_calibration(mib: int, reps: int = 5):
    """Device-to-device copies of a known size: reads and writes exactly mib MiB each."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    print(json.dumps({"copy_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4, "ms": ms,
                      "GBps_read_plus_write": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)


def spin_cycles_for(seconds: float) -> int:
    """Argument of torch.cuda._sleep that keeps the GPU busy for about `seconds`."""
    import torch
    n = 1 << 20
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(n)
    b.record()
    torch.cuda.synchronize()
    per_cycle = a.elapsed_time(b) * 1e-3 / n
    return int(seconds / max(per_cycle, 1e-12))


def host_seconds_per_call(call, forms, start):
    """Host time to enqueue one launch (measured after warm-up, GPU work not waited for)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(5):
        for f in forms:
            call(f, start + s)
    t = (time.perf_counter() - t0) / (5 * len(forms))
    torch.cuda.synchronize()
    return t


def kernel_hash(form: str) -> str:
    """Hash of the sources a form's kernels are built from (its own files, then the shared headers)."""
    own = KERNEL_FILES[form]
    h = hashlib.sha256()
    for f in ((own,) if isinstance(own, str) else own) + ("lion_device.h", "lion_mask.h", "lion_stage.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic(form: str, wl, C: int, causal: bool = False):
    """Algorithmic bytes and flops of one launch (what the method must read, write and compute).
    Causal: the L (L + 1) / 2 query-key pairs of the lower triangle, the intra-chunk triangles plus
    the forward states only, one recurrence."""
    B, H, L, d = wl.B, wl.H, wl.L, wl.d
    esz = 2 if wl.dtype == "bf16" else 4
    nbytes = 4 * B * H * L * d * esz                      # read q, k, v; write y
    if wl.kind == 2:
        nbytes += 4 * B * H * L                           # per-token log(lambda)
    elif wl.kind == 1:
        nbytes += 4 * H
    bh = B * H
    if form == "selectivity":
        # read x [B, L, 1024] and w, write log(lambda); read and write the keys
        nbytes = B * L * SEL_WIDTH * 2 + H * SEL_WIDTH * 2 + 4 * H + 4 * B * H * L + 2 * B * H * L * d * 2
        return nbytes, 2 * B * L * H * SEL_WIDTH + B * H * L * (d + 8)
    if form == "full_bwd":
        # read q, k, v, y, dy and den (and log(lambda)); write dq, dk, dv (bf16) and dlog(lambda)
        nbytes = 8 * B * H * L * d * esz + 4 * B * H * L
        if wl.kind == 2:
            nbytes += 4 * B * H * L
        elif wl.kind == 1:
            nbytes += 4 * H
        pairs = L * (L + 1) / 2 if causal else L * L
        # S, dY V^T, dV, dphi(Q), dphi(K): five L x L x d products; mask, dp, dS and dA per pair
        return nbytes, bh * (10 * pairs * d + 8 * pairs)
    if form == "chunk_bwd":
        nbytes = 8 * B * H * L * d * esz + 4 * B * H * L
        if wl.kind == 2:
            nbytes += 4 * B * H * L
        elif wl.kind == 1:
            nbytes += 4 * H
        cpairs = L * (C + 1) / 2 if causal else L * C
        # the five products inside chunks; per token, the chunk's states summed (four d x (d+1), two
        # when causal) and applied (dphi(q), dphi(k) and dv from them)
        per_tok = (10 if causal else 20) * d * d
        return nbytes, bh * (10 * cpairs * d + 8 * cpairs + L * per_tok)
    if form == "full2":
        return nbytes, bh * (4 * L * L * d + 4 * L * L)   # as the full form, two mask terms per score
    if form == "chunk2":
        # the chunkwise form's work once per order; bytes are the method's (the rearranged copies of
        # q, k, v and the fp32 partial results are this implementation's own traffic)
        return nbytes, 2 * bh * (4 * L * C * d + 8 * L * d * d + 2 * L * C)
    if form == "full":
        pairs = L * (L + 1) / 2 if causal else L * L
        flops = bh * (4 * pairs * d + 2 * pairs)          # phi(Q)phi(K)^T, P V, mask and row sums
    elif form == "chunk":
        cpairs = L * (C + 1) / 2 if causal else L * C
        flops = bh * (4 * cpairs * d + (4 if causal else 8) * L * d * d + 2 * cpairs)   # intra-chunk + states
    else:
        per_dir = (4 * d * d + 3 * d) if wl.kind == 0 else (5 * d * d + 4 * d)
        flops = bh * L * (1 if causal else 2) * per_dir   # recurrences: state update + q^T S, q.z
    return nbytes, flops


def fp32_form(form: str, C: int) -> bool:
    """Forms whose products run in fp32 (the RNN form's vector ALUs; the chunkwise backward's fp32 matrix
    cores for chunks of 16 and 32), priced against the fp32 peak."""
    return form == "birnn" or (form == "chunk_bwd" and C < 64)


def bound_of(form: str, wl, C: int, causal: bool = False) -> str:
    """The roof that binds a form on a workload: fp32 work (fp32_form) is priced on the fp32 peak; the
    bf16 matrix-core forms are bound by HBM below the bf16 ridge (peak flops / peak bytes) and by the
    matrix cores above it."""
    if fp32_form(form, C):
        return "alu"
    nbytes, flops = algorithmic(form, wl, C, causal)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "mfma" if flops / nbytes > ridge else "hbm"


def peak_of(bound: str):
    return {"hbm": (HBM_PEAK_GBS, "GB/s"), "mfma": (MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"),
            "alu": (VALU_FP32_PEAK_TFLOPS, "TFLOP/s")}[bound]


def read_traffic(key: str, workload: str, causal: bool = False):
    """HBM bytes per call of form key ``key`` from a committed counter summary, if it was taken on
    the current kernel source."""
    form = split_form(key)[0]
    path = os.path.join(ROOT, "profiles", f"traffic_{key}_{workload}{'_causal' if causal else ''}.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*(\w+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_h or not m_b or m_h.group(1) != kernel_hash(form):
        return None
    return float(m_b.group(1))


def cpu_baseline(wl, budget_s: float, causal: bool = False):
    """The fp64 oracle (the full-form definition) on the host: the whole workload if it fits the
    budget, else as many leading batch entries as do; tokens/s over the sample."""
    import oracle
    from bidirectional_linear_attention_lion_amd import inputs as lin
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    kind = wl.kind | (oracle.CAUSAL if causal else 0)
    inp1 = lin.make_inputs(wl, B=1)
    t0 = time.perf_counter()
    oracle.full(inp1.q, inp1.k, inp1.v, inp1.log_lambda_f64, kind, wl.eps)
    t1 = time.perf_counter() - t0
    nb = int(max(1, min(wl.B, budget_s / max(t1, 1e-6))))
    inp = lin.make_inputs(wl, B=nb) if nb > 1 else inp1
    # a workload smaller than the budget is run repeatedly, until the budget is spent, for a stable rate
    reps, dt = 0, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.full(inp.q, inp.k, inp.v, inp.log_lambda_f64, kind, wl.eps)
        dt += time.perf_counter() - t0
        reps += 1
        if dt + dt / reps > budget_s:
            break
    return {"value": reps * nb * wl.L / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{nb} of {wl.B} batch entries x {wl.H} heads x L={wl.L}, run {reps} time(s) "
                      f"(fp64 C oracle, OpenMP over (batch, head)), {dt:.2f} s"}


def main():
    args = parse_args()
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the (batch, head) problems are independent, see the design notes for sharding)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bidirectional_linear_attention_lion_amd as lion
    from bidirectional_linear_attention_lion_amd import inputs as lin

    wl = lin.WORKLOADS[args.workload]
    keys = default_forms(wl, args.chunk) if args.forms is None else [f for f in args.forms.split(",") if f]
    if args.forms is not None and args.chunk is None:
        # a key without a size takes each of the workload's chunk sizes
        expanded = []
        for key in keys:
            form, c = split_form(key)
            if form == "chunk" and key == form:
                expanded += [f"chunk{cc}" for cc in wl.chunks]
            elif form == "chunk2" and key == form:
                expanded += [f"chunk2_{cc}" for cc in wl.chunks]
            else:
                expanded.append(key)
        keys = expanded
    spec = {key: split_form(key, args.chunk or wl.chunks[0]) for key in keys}
    causal = args.causal
    kind = wl.kind | (lion.CAUSAL if causal else 0)
    if args.fp32_arith:
        if wl.dtype != "bf16" or any(f not in ("full", "chunk", "birnn") for f, _ in spec.values()):
            raise SystemExit("bench.py: --fp32-arith applies to the full, chunkwise and RNN forms of bf16 workloads")
        kind |= lion.FP32_ARITH
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    inp = lin.make_inputs(wl)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q0, k0, v0 = to_dev(inp.q_dev), to_dev(inp.k_dev), to_dev(inp.v_dev)
    ll = None if inp.log_lambda is None else torch.from_numpy(inp.log_lambda).to(dev)
    set_bytes = 4 * q0.numel() * q0.element_size()
    nsets = max(2, int(np.ceil(args.rotate_gib * (1 << 30) / set_bytes)))
    ydt = torch.float32 if args.fp32_arith else q0.dtype
    sets = [(q0.clone(), k0.clone(), v0.clone(), torch.empty(q0.shape, dtype=ydt, device=dev)) for _ in range(nsets)]
    del q0, k0, v0
    forms_used = {f for f, _ in spec.values()}
    bwd_sets = []
    if forms_used & {"full_bwd", "chunk_bwd"}:
        if wl.dtype != "bf16":
            raise SystemExit("bench.py: full_bwd and chunk_bwd need bf16 inputs")
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed)
        for (q, k, v, _) in sets:
            den = torch.empty((wl.B, wl.H, wl.L), dtype=torch.float32, device=dev)
            yb = lion.lion_attn_full(q, k, v, ll, kind, wl.eps, den_out=den, stream=stream)
            dy = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            grads = tuple(torch.empty_like(q) for _ in range(3))
            dll = None if wl.kind == 0 else torch.empty(
                (wl.H,) if wl.kind == 1 else (wl.B, wl.H, wl.L), dtype=torch.float32, device=dev)
            bwd_sets.append((yb, den, dy, grads, dll))
    order = None
    if forms_used & {"full2", "chunk2"}:
        side = int(round((wl.L - 1) ** 0.5))
        if side * side + 1 != wl.L:
            raise SystemExit("bench.py: full2 and chunk2 need an image workload (L = 1 + n^2)")
        order = torch.from_numpy(lin.column_major_order(side, side)).to(dev)
    sel = None
    if "selectivity" in forms_used:
        if wl.dtype != "bf16":
            raise SystemExit("bench.py: selectivity needs bf16 inputs")
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed + 1)
        # one layer input per input set, so x streams from HBM like the other operands
        xs = [torch.randn((wl.B, wl.L, SEL_WIDTH), generator=gen, device=dev).to(torch.bfloat16) for _ in range(nsets)]
        ws_ = (torch.randn((wl.H, SEL_WIDTH), generator=gen, device=dev) / SEL_WIDTH ** 0.5).to(torch.bfloat16)
        bs = torch.full((wl.H,), 3.0, dtype=torch.float32, device=dev)
        sel = (xs, ws_, bs)
    form_ids = {"chunk": lion.FORM_CHUNK, "birnn": lion.FORM_BIRNN, "full_bwd": lion.FORM_FULL_BWD,
                "chunk_bwd": lion.FORM_CHUNK_BWD, "chunk2": lion.FORM_CHUNK2}
    ws, ws_bytes = {}, {}
    for key, (f, C) in spec.items():
        nb = 0
        if f in form_ids:
            nb = lion.lion_attn_workspace_bytes(form_ids[f], wl.B, wl.H, wl.L, wl.d, C,
                                                1 if wl.dtype == "bf16" else 0)
            if nb == (1 << 64) - 1:
                raise SystemExit(f"bench.py: form {key} does not support this workload")
            ws[key] = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        ws_bytes[key] = nb

    def call(key, s):
        f, C = spec[key]
        q, k, v, y = sets[s % nsets]
        if f == "full":
            lion.lion_attn_full(q, k, v, ll, kind, wl.eps, y=y, stream=stream)
        elif f == "full2":
            lion.lion_attn_full2(q, k, v, ll, kind, order, wl.eps, y=y, stream=stream)
        elif f == "chunk2":
            lion.lion_attn_chunk2(q, k, v, ll, kind, order, C, wl.eps, y=y, workspace=ws[key], stream=stream)
        elif f == "selectivity":
            lion.lion_selectivity(sel[0][s % nsets], sel[1], sel[2], k=k, k_out=y, stream=stream)
        elif f == "full_bwd":
            yb, den, dy, (dq, dk, dv), dll = bwd_sets[s % nsets]
            lion.lion_attn_full_bwd(q, k, v, ll, kind, yb, den, dy, dq=dq, dk=dk, dv=dv, dlog_lambda=dll,
                                    workspace=ws[key], stream=stream)
        elif f == "chunk_bwd":
            yb, den, dy, (dq, dk, dv), dll = bwd_sets[s % nsets]
            lion.lion_attn_chunk_bwd(q, k, v, ll, kind, C, yb, den, dy, dq=dq, dk=dk, dv=dv,
                                     dlog_lambda=dll, workspace=ws[key], stream=stream)
        elif f == "chunk":
            lion.lion_attn_chunk(q, k, v, ll, kind, C, wl.eps, y=y, workspace=ws[key], stream=stream)
        else:
            lion.lion_attn_birnn(q, k, v, ll, kind, wl.eps, y=y, workspace=ws[key], stream=stream)

    for s in range(args.warmup):
        for key in keys:
            call(key, s)
    torch.cuda.synchronize()

    ev = {key: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for key in keys}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # Hold the GPU in a spin kernel while the host enqueues every timed launch, so the kernels then run
    # back to back and the events bracket kernel execution, not host submission time.
    host_s = host_seconds_per_call(call, keys, args.warmup)
    sleep_cycles = spin_cycles_for(1.5 * host_s * len(keys) * args.steps + 2e-3)
    torch.cuda.synchronize()
    torch.cuda._sleep(sleep_cycles)
    t_start.record(stream)
    for key in keys:
        ev[key][0].record(stream)
        for s in range(args.steps):
            call(key, args.warmup + 5 + s)
        ev[key][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    print(f"bench.py: timed {args.steps} steps of {','.join(keys)} on {wl.name}: {ms_per_step:.4f} ms/step",
          file=sys.stderr, flush=True)

    # per-call spread (outside the timed region): each call between its own pair of events
    spread = {}
    for key in keys:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for s, (e0, e1) in enumerate(evs):
            e0.record(stream)
            call(key, args.warmup + 5 + args.steps + s)
            e1.record(stream)
        torch.cuda.synchronize()
        us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
        spread[key] = {"p10": float(np.percentile(us, 10)), "p50": float(np.median(us)),
                       "p90": float(np.percentile(us, 90))}

    tokens = wl.B * wl.L
    per_form = {}
    for key in keys:
        f, C = spec[key]
        avg = ev[key][0].elapsed_time(ev[key][1]) / args.steps
        nbytes, flops = algorithmic(f, wl, C, causal)
        bound = bound_of(f, wl, C, causal)
        pk, _ = peak_of(bound)
        gbps, tflops = nbytes / (avg * 1e-3) / 1e9, flops / (avg * 1e-3) / 1e12
        per_form[key] = {
            "tokens_per_s": tokens / (avg * 1e-3),
            "ms_avg": avg,
            "alg_GBps": gbps,
            "alg_TFLOPs": tflops,
            "bound": bound,
            "frac_of_roof": (gbps if bound == "hbm" else tflops) / pk,
            "frac_hbm": gbps / HBM_PEAK_GBS,
            "frac_mfma_bf16": None if fp32_form(f, C) else tflops / MFMA_BF16_PEAK_TFLOPS,
            "memory": memory_bytes(f, wl, C, ws_bytes[key]),
            "launch_us": spread[key],
        }
        if f in ("chunk", "chunk2", "chunk_bwd"):
            per_form[key]["C"] = C
    fwd = [key for key in keys if spec[key][0] in FORWARD_FORMS] or keys
    best = max(fwd, key=lambda key: per_form[key]["tokens_per_s"])
    dom = max(keys, key=lambda key: per_form[key]["ms_avg"])
    f_dom, c_dom = spec[dom]
    nbytes, flops = algorithmic(f_dom, wl, c_dom, causal)
    avg_s = per_form[dom]["ms_avg"] * 1e-3
    dom_bound = per_form[dom]["bound"]
    peak, unit = peak_of(dom_bound)
    achieved = nbytes / avg_s / 1e9 if dom_bound == "hbm" else flops / avg_s / 1e12
    traffic = read_traffic(dom, wl.name, causal)

    out = {
        "metric": METRIC,
        "value": per_form[best]["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "L": wl.L, "d": wl.d,
                   "mask": lin.KIND_NAME[wl.kind] + ("+causal" if causal else "") + ("+fp32arith" if args.fp32_arith else ""),
                   "forms": keys,
                   "value_form": best, "input_sets": nsets, "host_us_per_launch": host_s * 1e6},
        "step_tokens_per_s": tokens / (ms_per_step * 1e-3),
        "forms": per_form,
        "roofline": {"bound": dom_bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic},
    }
    if args.cpu_baseline_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_baseline_seconds, causal)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
