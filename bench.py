"""Throughput of the WKV7 forward + backward on one MI355X.

One step = the whole hot path over one batch: the per-chunk operands (shared
by forward and backward), the forward scan (y, checkpoints, final state), the
backward scan (state gradient at every chunk boundary, dv), then the per-token
input gradients, for a loss gradient dy.  Inputs are seeded synthetic tensors
of the workload's shape, resident in HBM before timing starts.

Prints one JSON line.  Default workload: B12 T1024 H6 D64, bf16 inputs
(the 36M "debug" training layer).

--prologue times the layer with its time-mix prologue fused into the kernels
(wkv7_fwd_proj + wkv7_bwd_proj: w, a, b formed from raw projections inside the
loads), and beside it the same two calls without the prologue (wkv7_fwd +
wkv7_bwd on w, a, b) and with the prologue as separate torch operations.

--division times the diagnostic division-walk backward (wkv7_bwd_division,
restarting from the exact state at every chunk end) beside the recompute
backward (wkv7_bwd) on the same forward's checkpoints.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "WKV7 fwd+bwd tokens/s and % HBM peak, B12 T1024 H6 D64 (1 MI355X)"
HBM_PEAK_GBS = 8000.0
D = 64
CSRC = os.path.join(ROOT, "linear_rnn_lm_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
FLUSH_BYTES = 1 << 30   # read before every timed step: more than the L2s and the 256 MB MALL
MIN_WARMUP_S = 0.5      # warm-up lasts at least this long (the clocks settle under sustained load)


class Flush:
    """Evicts the L2s and the MALL by reading a 1 GiB buffer (a sum).  A read
    is used rather than a write: a write leaves 256 MB of dirty lines whose
    write-back would land in the first timed kernels; a read writes back
    whatever is dirty during the flush itself and leaves clean lines."""

    def __init__(self, torch, dev):
        self.buf = torch.zeros(FLUSH_BYTES // 4, device=dev, dtype=torch.float32)
        self.acc = torch.zeros((), device=dev, dtype=torch.float32)
        self.torch = torch

    def __call__(self):
        self.torch.sum(self.buf, dim=0, out=self.acc)


def warm_up(torch, fn, steps, min_s=None):
    """At least `steps` calls and at least `min_s` (default MIN_WARMUP_S)
    seconds of them."""
    min_s = MIN_WARMUP_S if min_s is None else min_s
    t0 = time.perf_counter()
    n = 0
    while n < steps or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n
OPS_BYTES = 36864      # transition operands P, M, E, F of one chunk of one head


def source_digest() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def kernel_bytes(wl, in_bytes: int) -> dict:
    """Algorithmic bytes of each kernel per launch: its share of what the
    method itself must move (each input read once per pass, y, the gradients,
    hT and dh0 written once, the checkpoints written once by the forward and
    read once by the backward, dy read once).  Per head-token with bf16
    inputs: chunk_prepare 640 (r, w, k, a, b: the forward's read), fwd_scan
    896 (v, y, checkpoints), bwd_scan 256 (dv), bwd_inputs 2,816 (the six
    inputs, dy, the checkpoints, five gradients); they add up to the path's
    1,536 B forward + 3,072 B backward.  Everything else a kernel moves --
    the chunk operands and inverses, the state gradients at chunk boundaries,
    the backward scan's read of dy -- is recompute or hand-off traffic of this
    design, reported separately by `extra_bytes`."""
    ht = wl.B * wl.T * wl.H          # head-tokens
    heads = wl.B * wl.H
    nc = (wl.T + 31) // 32
    tok_in = ht * D * in_bytes
    tok32 = ht * D * 4
    st = heads * D * D * 4
    ck = heads * nc * D * D * 4
    h0 = st if wl.with_h0 else 0
    alg = {
        "chunk_prepare": 5 * tok_in,
        "fwd_scan": tok_in + tok32 + ck + h0 + st,
        "bwd_scan": tok32 + st,
        "bwd_inputs": 6 * tok_in + tok32 + ck + 5 * tok32,
    }
    alg["path"] = sum(alg.values())
    return alg


def extra_bytes(wl) -> dict:
    """Bytes each kernel moves beyond its algorithmic share: intermediates of
    the chunked design (written once, read back) and re-reads."""
    heads = wl.B * wl.H
    nc = (wl.T + 31) // 32
    tok32 = wl.B * wl.T * wl.H * D * 4
    ck = heads * nc * D * D * 4
    inv = heads * nc * 32 * 32 * 4
    ops = heads * nc * OPS_BYTES
    ex = {
        "chunk_prepare": inv + ops,          # chunk inverses and operands written
        "fwd_scan": ops,                     # operands read
        "bwd_scan": tok32 + ops + ck,        # dy read again, operands read, state gradients written
        "bwd_inputs": inv + ck,              # inverses and state gradients read
    }
    ex["path"] = sum(ex.values())
    return ex


def kernel_key(name: str):
    """bench key of a kernel name as the profiler prints it (None: not ours)."""
    if "chunk_prepare_kernel" in name:
        return "chunk_prepare"
    if "scan_kernel" in name:
        return "bwd_scan" if ", true>(" in name else "fwd_scan"
    if "grad_kernel" in name:
        return "bwd_inputs"
    return None


KERNEL_KEYS = ("chunk_prepare", "fwd_scan", "bwd_scan", "bwd_inputs")
COPY_MIB = 256


def copy_calibration(dev, reps: int = 3) -> None:
    """A plain device copy of known size (256 MiB read, 256 MiB written, as a
    negation so that it is one elementwise kernel and not a DMA): the reference
    that scales the HBM byte counters of the other kernels."""
    import torch
    src = torch.ones(COPY_MIB << 18, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _pmc_rows(d: str):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def traffic_from(d: str, workload: str) -> dict:
    """HBM bytes per launch of every kernel from two rocprofv3 --pmc runs
    (d/fetch: FETCH_SIZE, d/write: WRITE_SIZE, KiB per dispatch), each scaled
    by what the same counter reads for the 256 MiB copy."""
    from linear_rnn_lm_amd.inputs import WORKLOADS
    wl = WORKLOADS[workload]
    meas = {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        vals = {}
        for r in _pmc_rows(os.path.join(d, sub)):
            if r["Counter_Name"] != ctr:
                continue
            name = r["Kernel_Name"]
            key = "copy" if "neg" in name else kernel_key(name)
            if key:
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
        if "copy" not in vals:
            raise RuntimeError(f"no copy kernel in the {ctr} run under {d}")
        scale = (COPY_MIB * 1024) / (sum(vals["copy"]) / len(vals["copy"]))
        meas[ctr] = {k: sum(v) / len(v) * 1024 * scale for k, v in vals.items() if k != "copy"}
        meas[ctr + "_copy_scale"] = scale
    kb = kernel_bytes(wl, 2 if str(wl.dtype).endswith("bfloat16") else 4)
    ex = extra_bytes(wl)
    out = {"copy_scale": {"FETCH_SIZE": meas["FETCH_SIZE_copy_scale"], "WRITE_SIZE": meas["WRITE_SIZE_copy_scale"]},
           "source_digest": source_digest(), "kernels": {}}
    for k in KERNEL_KEYS:
        fb, wb = meas["FETCH_SIZE"].get(k), meas["WRITE_SIZE"].get(k)
        if fb is None or wb is None:
            continue
        out["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                             "algorithmic_bytes": kb[k], "extra_bytes": ex[k], "ratio": (fb + wb) / kb[k],
                             "ratio_to_alg_plus_extra": (fb + wb) / (kb[k] + ex[k])}
    ks = out["kernels"]
    if all(k in ks for k in KERNEL_KEYS):
        tot = sum(ks[k]["bytes_per_launch"] for k in KERNEL_KEYS)
        out["step"] = {"bytes": tot, "algorithmic_bytes": kb["path"], "extra_bytes": ex["path"],
                       "ratio": tot / kb["path"]}
    return out


def trace_summary(d: str, steps: int) -> str:
    """Markdown table of a rocprofv3 --kernel-trace of bench.py: per kernel,
    every launch, and the launches of the two timed flushed passes (the last
    2 x steps launches that follow the flush's reduction within their step;
    the warm-up steps before them are flushed too but not timed), in
    microseconds."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    stats = {}
    flushed = False
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        key = kernel_key(name) or ("step_kernel" if "step_kernel" in name else
                                   "fwd_sequential" if "fwd_sequential_kernel" in name else None)
        if key is None:
            if "reduce_kernel" in name:
                flushed = True
            continue
        short = name.rsplit("(", 1)[0].split("::")[-1].replace("unsigned short", "bf16")
        st = stats.setdefault(key, {"all": [], "flushed": [], "name": short})
        st["all"].append(dur)
        if flushed:
            st["flushed"].append(dur)
        if key == "bwd_inputs":   # the last kernel of a step
            flushed = False
    out = ["| kernel | calls | avg us | min us | max us | timed flushed calls | their avg us | their max/min |",
           "|---|---|---|---|---|---|---|---|"]
    for key, st in sorted(stats.items(), key=lambda kv: -sum(kv[1]["all"])):
        a, fl = st["all"], st["flushed"][-2 * steps:]
        fcol = (f"{len(fl)} | {sum(fl) / len(fl):.1f} | {max(fl) / min(fl):.3f}" if fl else "0 | - | -")
        out.append(f"| `{st['name']}` ({key}) | {len(a)} | {sum(a) / len(a):.1f} | {min(a):.1f} | {max(a):.1f} | {fcol} |")
    return "\n".join(out)


# Utilisation counters of every kernel, one rocprofv3 --pmc pass each (at most
# four SQ counters per pass): the derived metrics' own definitions, averaged
# over the dispatches of each kernel.
UTIL_PASSES = (("valu", "VALUBusy MfmaUtil"), ("lds", "LdsUtil LDSBankConflict"))


def counters_from(d: str) -> dict:
    """Utilisation per kernel from rocprofv3 --pmc runs in d/valu, d/lds."""
    vals = {}
    for sub, _ in UTIL_PASSES:
        for r in _pmc_rows(os.path.join(d, sub)):
            key = kernel_key(r["Kernel_Name"])
            if key:
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    kern = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    return {"source_digest": source_digest(), "kernels": kern,
            "definitions": {"VALUBusy": "100 * SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE",
                            "MfmaUtil": "100 * SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs)",
                            "LdsUtil": "100 * SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE * CUs)",
                            "LDSBankConflict": "100 * SQ_LDS_BANK_CONFLICT / GRBM_GUI_ACTIVE / CUs"}}


def host_cpu() -> dict:
    """The host's CPU model and core counts."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": avail, "os_cpu_count": os.cpu_count()}


def cpu_baseline(wl, budget_s: float) -> dict:
    """The oracle, as it stands, on the host cores: whole fwd+bwd passes of the
    workload (a subset of heads if one pass would exceed the budget).  One
    worker thread per available core, at most 16 (this process's share of a
    shared GPU host)."""
    import oracle
    from linear_rnn_lm_amd.inputs import make_inputs
    threads = oracle.default_threads()
    # probe with a few heads to size the sample
    probe_heads = min(wl.heads, threads)
    xb = make_inputs(1, wl.T, probe_heads, wl.dtype, seed=wl.seed, with_h0=wl.with_h0)
    t0 = time.perf_counter()
    oracle.fwd(*xb.tensors(), xb.h0, threads=threads)
    oracle.bwd(*xb.tensors(), xb.dy, xb.h0, None, threads=threads)
    per_head = (time.perf_counter() - t0) / probe_heads
    heads = max(probe_heads, min(wl.heads, int(budget_s / max(per_head, 1e-9))))
    B = max(1, heads // wl.H) if heads >= wl.H else 1
    H = wl.H if heads >= wl.H else heads
    x = make_inputs(B, wl.T, H, wl.dtype, seed=wl.seed, with_h0=wl.with_h0)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd(*x.tensors(), x.h0, threads=threads)
        oracle.bwd(*x.tensors(), x.dy, x.h0, None, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s * 0.5 or reps >= 1000:
            break
    tokens = B * wl.T * reps * (H / wl.H)    # tokens of the full-width layer
    return {"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on B{B} T{wl.T} H{H} ({B * H} of {wl.heads} heads), "
                      f"{reps} pass(es) in {el:.1f} s, {threads} threads; tokens scaled by {H}/{wl.H} heads",
            **host_cpu()}


STEP_METRIC = "WKV7 recurrent step tokens/s and % HBM peak, 32 layers x B256 T1 H64 D64 (1 MI355X)"
PROLOGUE_METRIC = "WKV7 layer with fused time-mix prologue, fwd+bwd tokens/s (1 MI355X)"
STEP_PROLOGUE_METRIC = "WKV7 recurrent step with fused time-mix prologue tokens/s, 32 layers x B256 T1 H64 D64 (1 MI355X)"


def _time_steps(torch, stream, fn, warmup, steps):
    """Milliseconds per call of fn, from two events on the launch stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


DIVISION_METRIC = "WKV7 backward by division (diagnostic), tokens/s (1 MI355X)"


def bench_division(args, wl) -> int:
    """One step = wkv7_bwd_division (restart at every chunk end) on the
    checkpoints of one forward; wkv7_bwd on the same checkpoints beside it."""
    import torch
    import linear_rnn_lm_amd as L
    from linear_rnn_lm_amd.inputs import workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = workload_inputs(wl)
    ins = [t.to(dev) for t in x.tensors()]
    h0 = None if x.h0 is None else x.h0.to(dev)
    dy = x.dy.to(dev)
    y, ck, hT = L.fwd(*ins, h0)
    stream = torch.cuda.current_stream(dev)
    steps, warmup = max(1, min(args.steps, 5)), min(args.warmup, 1)
    ms_div = _time_steps(torch, stream, lambda: L.bwd_division(dy, *ins, ck, hT, None, restart=True),
                         warmup, steps)
    ms_rec = _time_steps(torch, stream, lambda: L.bwd(dy, *ins, ck, None), args.warmup, args.steps)
    tokens = wl.B * wl.T
    out = {
        "metric": DIVISION_METRIC,
        "value": tokens / (ms_div * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_div,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: backward only, {wl.description}", "B": wl.B, "T": wl.T, "H": wl.H,
                   "D": D},
        "ms_recompute_bwd": ms_rec,
        "slowdown_vs_recompute": ms_div / ms_rec,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_prologue(args, wl) -> int:
    """One step = wkv7_fwd_proj then wkv7_bwd_proj (each runs the chunk
    preparation itself, as a training framework calling forward and backward
    separately would).  Also timed: wkv7_fwd + wkv7_bwd on w, a, b (the layer
    without a prologue), and the prologue as torch operations around them."""
    import torch
    import linear_rnn_lm_amd as L
    from linear_rnn_lm_amd.inputs import make_proj_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, H = wl.B, wl.T, wl.H
    x = make_proj_inputs(B, T, H, wl.dtype, wl.seed, wl.with_h0)
    r, w_raw, k, v, kappa, alpha = (t.to(dev) for t in x.tensors())
    h0 = None if x.h0 is None else x.h0.to(dev)
    dy = x.dy.to(dev)
    f32 = dict(device=dev, dtype=torch.float32)
    nc = L.num_chunks(T)
    y = torch.empty(B, T, H, D, **f32)
    ck = torch.empty(B, H, nc, D, D, **f32)
    hT = torch.empty(B, H, D, D, **f32)
    grads = [torch.empty(B, T, H, D, **f32) for _ in range(6)]
    fws = torch.empty(L.chunk_ops_bytes(B, T, H) // 4, **f32)
    bws = torch.empty(L.workspace_bytes(B, T, H) // 4, **f32)
    stream = torch.cuda.current_stream(dev)

    def fused_fwd():
        L.fwd_proj(r, w_raw, k, v, kappa, alpha, h0, y=y, ckpt=ck, hT=hT, workspace=fws)

    def fused_bwd():
        L.bwd_proj(dy, r, w_raw, k, v, kappa, alpha, ck, None, workspace=bws, out=grads)

    def fused():
        fused_fwd()
        fused_bwd()

    # the layer without a prologue, on w, a, b of the same values' dtype
    c = -0.6065306597126334
    sw = torch.sigmoid(w_raw.float())
    kf = kappa.float()
    nrm = kf.norm(dim=-1, keepdim=True)
    kh = kf / nrm
    sa = torch.sigmoid(alpha.float())
    wd, ad, bd = (t.to(wl.dtype) for t in (torch.exp(c * sw), -kh, kh * sa))

    def core():
        L.fwd(r, wd, k, v, ad, bd, h0, y=y, ckpt=ck, hT=hT, workspace=fws)
        L.bwd(dy, r, wd, k, v, ad, bd, ck, None, workspace=bws, out=grads)

    def unfused():
        s1 = torch.sigmoid(w_raw.float())
        w1 = torch.exp(c * s1)
        k1 = kappa.float()
        n1 = k1.norm(dim=-1, keepdim=True)
        h1 = k1 / n1
        a1 = torch.sigmoid(alpha.float())
        wb, ab, bb = w1.to(wl.dtype), (-h1).to(wl.dtype), (h1 * a1).to(wl.dtype)
        L.fwd(r, wb, k, v, ab, bb, h0, y=y, ckpt=ck, hT=hT, workspace=fws)
        dr, dw, dk, dv, da, db, _ = L.bwd(dy, r, wb, k, v, ab, bb, ck, None, workspace=bws, out=grads)
        g = db * a1 - da
        return (dw * w1 * c * s1 * (1 - s1), (g - h1 * (h1 * g).sum(-1, keepdim=True)) / n1,
                db * h1 * a1 * (1 - a1))

    ms = _time_steps(torch, stream, fused, args.warmup, args.steps)
    ms_fwd = _time_steps(torch, stream, fused_fwd, args.warmup, args.steps)
    ms_bwd = _time_steps(torch, stream, fused_bwd, args.warmup, args.steps)
    ms_core = _time_steps(torch, stream, core, args.warmup, args.steps)
    ms_unfused = _time_steps(torch, stream, unfused, args.warmup, args.steps)
    in_bytes = 2 if wl.dtype == torch.bfloat16 else 4
    kb = kernel_bytes(wl, in_bytes)
    tokens = B * T
    out = {
        "metric": PROLOGUE_METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(in_bytes),
        "data": "synthetic",
        "config": {"workload": f"{wl.name} with raw projections w_raw, kappa, alpha: {wl.description}",
                   "B": B, "T": T, "H": H, "D": D,
                   "in_dtype": "bf16" if in_bytes == 2 else "f32", "state_dtype": "f32"},
        "ms_fwd_proj": ms_fwd,
        "ms_bwd_proj": ms_bwd,
        "ms_without_prologue": ms_core,
        "ms_prologue_in_torch": ms_unfused,
        "path_hbm": {"algorithmic_bytes": kb["path"],
                     "achieved_GBs": kb["path"] / (ms * 1e-3) / 1e9,
                     "frac_of_peak": kb["path"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    print(json.dumps(out), flush=True)
    return 0


def step_bytes(wl, in_bytes: int) -> int:
    """Bytes one layer call of the one-token step must move: the state read and
    written once (in place), six input rows read, y written."""
    heads = wl.B * wl.H
    return 2 * heads * D * D * 4 + 6 * heads * D * in_bytes + heads * D * 4


def bench_step(args, wl) -> int:
    """The one-token recurrent step (forward only): one call per layer, each
    updating that layer's (B,H,64,64) fp32 state in place.  A step is all
    layers; tokens/s counts the B sequences' tokens per step.  With --prologue
    the layers take raw projections (wkv7_fwd_proj), and the same step on
    precomputed w, a, b and with the prologue as torch operations is timed
    beside it."""
    import torch
    import linear_rnn_lm_amd as L
    from linear_rnn_lm_amd.inputs import make_inputs, make_proj_inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    in_bytes = 2 if wl.dtype == torch.bfloat16 else 4
    layers = []
    gen = torch.Generator(device=dev)
    for layer in range(wl.layers):
        make = make_proj_inputs if args.prologue else make_inputs
        x = make(wl.B, 1, wl.H, wl.dtype, wl.seed + layer, with_h0=False)
        gen.manual_seed(wl.seed + layer)
        # the states: N(0, 0.1), drawn on the device (8.6 GB for 32 layers)
        state = torch.randn(wl.B, wl.H, D, D, generator=gen, device=dev, dtype=torch.float32) * 0.1
        layers.append(([t.to(dev) for t in x.tensors()], state,
                       torch.empty(wl.B, 1, wl.H, D, device=dev, dtype=torch.float32)))
    lib = L.lib()
    code = 1 if wl.dtype == torch.bfloat16 else 0
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    calls = [([t.data_ptr() for t in ins], st.data_ptr(), y.data_ptr()) for ins, st, y in layers]

    entry = lib.wkv7_fwd_proj if args.prologue else lib.wkv7_fwd

    def call(c):
        p, ps, py = c
        st = entry(wl.B, 1, wl.H, D, code, *p, ps, py, None, ps, None, 0, sh)
        assert st == 0, lib.wkv7_status_str(st)

    def step():
        for c in calls:
            call(c)

    warm_up(torch, step, args.warmup, args.min_warmup_s)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    # per-launch duration of the layer kernel, from events around each call
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    launch_ms = []
    for _ in range(args.steps):
        evs[0].record(stream)
        for i, c in enumerate(calls):
            call(c)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        launch_ms += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(calls))]
    per_launch_ms = sum(launch_ms) / len(launch_ms)
    kb = step_bytes(wl, in_bytes)
    achieved = kb / (per_launch_ms * 1e-3) / 1e9
    out = {
        "metric": STEP_METRIC,
        "value": wl.B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "B": wl.B, "T": 1, "H": wl.H, "D": D,
                   "layers": wl.layers, "in_dtype": "bf16" if in_bytes == 2 else "f32", "state_dtype": "f32"},
        "layer_tokens_per_s": wl.B * wl.layers / (ms_per_step * 1e-3),
        "kernel_ms": {"fwd_sequential": per_launch_ms},
        "roofline": {"kernel": "fwd_sequential", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None},
    }
    if args.prologue:
        out["metric"] = STEP_PROLOGUE_METRIC
        c = -0.6065306597126334
        pre = []
        for ins, st, y in layers:
            r, w_raw, k, v, kappa, alpha = ins
            kf = kappa.float()
            kh = kf / kf.norm(dim=-1, keepdim=True)
            wd = torch.exp(c * torch.sigmoid(w_raw.float())).to(wl.dtype)
            pre.append(([r, wd, k, v, (-kh).to(wl.dtype), (kh * torch.sigmoid(alpha.float())).to(wl.dtype)], st, y))

        def core():
            for ins, st, y in pre:
                L.fwd(*ins, st, want_ckpt=False, y=y, hT=st)

        def unfused():
            for ins, st, y in layers:
                r, w_raw, k, v, kappa, alpha = ins
                kf = kappa.float()
                kh = kf / kf.norm(dim=-1, keepdim=True)
                wd = torch.exp(c * torch.sigmoid(w_raw.float())).to(wl.dtype)
                L.fwd(r, wd, k, v, (-kh).to(wl.dtype), (kh * torch.sigmoid(alpha.float())).to(wl.dtype), st,
                      want_ckpt=False, y=y, hT=st)

        out["ms_without_prologue"] = _time_steps(torch, stream, core, args.warmup, args.steps)
        out["ms_prologue_in_torch"] = _time_steps(torch, stream, unfused, args.warmup, args.steps)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="debug_36m")
    ap.add_argument("--min-warmup-s", type=float, default=MIN_WARMUP_S,
                    help="warm-up lasts at least this many seconds (short runs under a profiler: 0)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prologue", action="store_true",
                    help="time the layer with its fused time-mix prologue (see the module docstring)")
    ap.add_argument("--division", action="store_true",
                    help="time the diagnostic division-walk backward (see the module docstring)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy, the reference for HBM byte counters")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="no GPU work: write profiles/traffic.json from rocprofv3 --pmc runs in DIR/fetch, DIR/write")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="no GPU work: write profiles/counters.json from rocprofv3 --pmc runs in DIR/valu, DIR/lds")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="no GPU work: print a markdown table of a rocprofv3 --kernel-trace of bench.py in DIR")
    ap.add_argument("--fwd-ab", action="store_true",
                    help="time the chunked forward against the token-by-token forward on the workload")
    args = ap.parse_args()

    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.steps))
        return 0

    if args.counters_from:
        cf = {}
        if os.path.exists(COUNTERS_FILE):
            with open(COUNTERS_FILE) as f:
                cf = json.load(f)
        cf[args.workload] = counters_from(args.counters_from)
        with open(COUNTERS_FILE, "w") as f:
            json.dump(cf, f, indent=1, sort_keys=True)
        print(json.dumps(cf[args.workload], indent=1))
        return 0

    if args.traffic_from:
        tr = {}
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                tr = json.load(f)
        tr[args.workload] = traffic_from(args.traffic_from, args.workload)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(tr, f, indent=1, sort_keys=True)
        print(json.dumps(tr[args.workload], indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py: measures exactly one GPU; --gpus {args.gpus} is not supported. "
              "The WKV7 op shards over heads with no exchange, so N GPUs each run this same "
              "single-GPU step on their share.", file=sys.stderr)
        return 2

    import torch
    import linear_rnn_lm_amd as L
    from linear_rnn_lm_amd.inputs import WORKLOADS, workload_inputs

    wl = WORKLOADS[args.workload]
    if args.copy_calibration:
        copy_calibration(torch.device("cuda:0"))
    if wl.T == 1:
        return bench_step(args, wl)
    if args.prologue:
        return bench_prologue(args, wl)
    if args.division:
        return bench_division(args, wl)
    if args.fwd_ab:
        return bench_fwd_ab(args, wl)
    return bench_train_step(args, wl)


def _digest_entry(path, workload):
    """The workload's entry of a counters file, if it was taken on the current sources."""
    try:
        with open(path) as f:
            ent = json.load(f).get(workload, {})
    except (OSError, ValueError):
        return None
    return ent if ent.get("source_digest") == source_digest() else None


def _stats(xs):
    ys = sorted(xs)
    n = len(ys)
    med = ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])
    return {"mean": sum(ys) / n, "median": med, "min": ys[0], "max": ys[-1], "n": n}


def bench_train_step(args, wl) -> int:
    """One step = chunk_prepare, fwd_scan, bwd_scan, bwd_inputs on the current
    stream.  Timing: before every timed step a 1 GiB buffer is written, which
    evicts the L2s and the 256 MB MALL, so each step starts from HBM; the step
    is bracketed by two events (flush outside).  A second flushed pass puts
    events between the kernels for per-kernel durations.  The same steps back
    to back without flushes are timed as well (the 'unflushed' figures)."""
    import torch
    import linear_rnn_lm_amd as L
    from linear_rnn_lm_amd.inputs import workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = workload_inputs(wl)
    ins = [t.to(dev) for t in x.tensors()]
    h0 = None if x.h0 is None else x.h0.to(dev)
    dy = x.dy.to(dev)
    B, T, H = wl.B, wl.T, wl.H
    nc = L.num_chunks(T)
    f32 = dict(device=dev, dtype=torch.float32)
    y = torch.empty(B, T, H, D, **f32)
    ck = torch.empty(B, H, nc, D, D, **f32)
    hT = torch.empty(B, H, D, D, **f32)
    dck = torch.empty(B, H, nc, D, D, **f32)
    ops = torch.empty(L.chunk_ops_bytes(B, T, H) // 4, **f32)
    dv = torch.empty(B, T, H, D, **f32)
    dh0 = torch.empty(B, H, D, D, **f32)
    grads = [torch.empty(B, T, H, D, **f32) for _ in range(5)]
    flush = Flush(torch, dev)
    lib = L.lib()
    code = 1 if wl.dtype == torch.bfloat16 else 0
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    p = [t.data_ptr() for t in ins]
    ph0 = None if h0 is None else h0.data_ptr()
    pops = ops.data_ptr()

    def k_prep():
        st = lib.wkv7_chunk_prepare(B, T, H, D, code, p[0], p[1], p[2], p[4], p[5], pops, sh)
        assert st == 0, lib.wkv7_status_str(st)

    def k_fwd():
        st = lib.wkv7_fwd_scan(B, T, H, D, code, p[3], pops, ph0, y.data_ptr(), ck.data_ptr(), hT.data_ptr(), sh)
        assert st == 0, lib.wkv7_status_str(st)

    def k_bscan():
        st = lib.wkv7_bwd_scan(B, T, H, D, code, dy.data_ptr(), None, pops, dck.data_ptr(), dv.data_ptr(),
                               dh0.data_ptr(), sh)
        assert st == 0, lib.wkv7_status_str(st)

    def k_inputs():
        st = lib.wkv7_bwd_inputs(B, T, H, D, code, dy.data_ptr(), None, *p, pops, ck.data_ptr(), dck.data_ptr(),
                                 *[g.data_ptr() for g in grads], sh)
        assert st == 0, lib.wkv7_status_str(st)

    # one training step: the chunk operands (shared by forward and backward),
    # the forward scan, the backward scan, the input gradients
    kernels = [("chunk_prepare", k_prep), ("fwd_scan", k_fwd), ("bwd_scan", k_bscan), ("bwd_inputs", k_inputs)]

    def step():
        for _, fn in kernels:
            fn()

    def flushed_step():
        flush()
        step()

    n_warm = warm_up(torch, flushed_step, args.warmup, args.min_warmup_s)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    # pass 1, the timed region: exactly `steps` steps, each flushed first and
    # bracketed by two events on the launch stream
    marks = [(ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in marks:
        flush()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in marks]
    # pass 2: per-kernel durations, events between the launches of every flushed step
    kev = [[ev() for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    for s in range(args.steps):
        flush()
        kev[s][0].record(stream)
        for i, (_, fn) in enumerate(kernels):
            fn()
            kev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    kernel_ms = {name: _stats([kev[s][i].elapsed_time(kev[s][i + 1]) for s in range(args.steps)])
                 for i, (name, _) in enumerate(kernels)}
    # pass 3: the same steps back to back, no flushes
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    unflushed_ms = e0.elapsed_time(e1) / args.steps

    in_bytes = 2 if wl.dtype == torch.bfloat16 else 4
    kb = kernel_bytes(wl, in_bytes)
    ex = extra_bytes(wl)
    st_ms = _stats(step_ms)
    ms_per_step = st_ms["mean"]
    dom = max(kernel_ms, key=lambda k: kernel_ms[k]["mean"])
    dom_ms = kernel_ms[dom]["mean"]
    achieved = kb[dom] / (dom_ms * 1e-3) / 1e9
    traffic = None
    tr = _digest_entry(TRAFFIC_FILE, wl.name)
    if tr and dom in tr.get("kernels", {}):
        traffic = tr["kernels"][dom]["bytes_per_launch"]
    util = _digest_entry(COUNTERS_FILE, wl.name)

    tokens = B * T
    out = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(in_bytes),
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: WKV7 fwd+bwd {wl.description}, chunk 32",
                   "B": B, "T": T, "H": H, "D": D,
                   "in_dtype": "bf16" if in_bytes == 2 else "f32", "state_dtype": "f32"},
        "timing": {"protocol": f"each timed step preceded by a {FLUSH_BYTES >> 30} GiB read (L2 and MALL "
                               "flushed); ms_per_step = mean of the flushed steps",
                   "warmup_steps_run": n_warm,
                   "flushed_ms": st_ms,
                   "unflushed_ms_per_step": unflushed_ms,
                   "unflushed_tokens_per_s": tokens / (unflushed_ms * 1e-3)},
        "fwd_tokens_per_s": tokens / ((kernel_ms["fwd_scan"]["mean"] + kernel_ms["chunk_prepare"]["mean"]) * 1e-3),
        "kernel_ms": {k: v["mean"] for k, v in kernel_ms.items()},
        "kernel_ms_stats": kernel_ms,
        "path_hbm": {"algorithmic_bytes": kb["path"],
                     "extra_bytes": ex["path"],
                     "achieved_GBs": kb["path"] / (ms_per_step * 1e-3) / 1e9,
                     "frac_of_peak": kb["path"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": kb[dom], "extra_bytes": ex[dom],
                     "traffic_over_algorithmic": None if traffic is None else traffic / kb[dom]},
    }
    if tr and "step" in tr:
        out["path_hbm"]["counter_bytes"] = tr["step"]["bytes"]
        out["path_hbm"]["counter_over_algorithmic"] = tr["step"]["ratio"]
    if util:
        out["utilization_pct"] = util["kernels"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


def compute_dtype(in_bytes: int) -> str:
    """What the path computes in: bf16 inputs take bf16 MFMA products of a
    two-term (hi + lo) split of every fp32 operand, three products per term
    pair, accumulated in fp32; fp32 inputs take fp32 MFMA products."""
    return "bf16x3-split-mfma/f32-acc" if in_bytes == 2 else "f32-mfma/f32-acc"


FWD_AB_METRIC = "WKV7 forward tokens/s: chunked (matrix cores) vs token-by-token (vector units) (1 MI355X)"


def bench_fwd_ab(args, wl) -> int:
    """The forward two ways on the same inputs and outputs: the chunked form
    (chunk_prepare + fwd_scan, the matrix-core path wkv7_fwd takes for T > 1)
    and the token-by-token kernel (wkv7_fwd_sequential, vector units only).
    Each timed call is preceded by the 1 GiB flush."""
    import torch
    import linear_rnn_lm_amd as L
    from linear_rnn_lm_amd.inputs import workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = workload_inputs(wl)
    ins = [t.to(dev) for t in x.tensors()]
    h0 = None if x.h0 is None else x.h0.to(dev)
    B, T, H = wl.B, wl.T, wl.H
    f32 = dict(device=dev, dtype=torch.float32)
    y = torch.empty(B, T, H, D, **f32)
    ck = torch.empty(B, H, L.num_chunks(T), D, D, **f32)
    hT = torch.empty(B, H, D, D, **f32)
    ws = torch.empty(L.fwd_workspace_bytes(B, T, H) // 4, **f32)
    flush = Flush(torch, dev)
    stream = torch.cuda.current_stream(dev)

    def chunked():
        L.fwd(*ins, h0, y=y, ckpt=ck, hT=hT, workspace=ws)

    def sequential():
        L.fwd_sequential(*ins, h0, y=y, ckpt=ck, hT=hT)

    res = {}
    for name, fn in (("chunked", chunked), ("sequential", sequential)):
        warm_up(torch, fn, args.warmup, args.min_warmup_s)
        times = []
        for _ in range(args.steps):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        res[name] = _stats(times)
    tokens = B * T
    out = {
        "metric": FWD_AB_METRIC,
        "value": tokens / (res["chunked"]["mean"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["chunked"]["mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(2 if wl.dtype == torch.bfloat16 else 4),
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: forward only, {wl.description}", "B": B, "T": T, "H": H, "D": D},
        "chunked_ms": res["chunked"],
        "sequential_ms": res["sequential"],
        "sequential_tokens_per_s": tokens / (res["sequential"]["mean"] * 1e-3),
        "speedup_chunked_over_sequential": res["sequential"]["mean"] / res["chunked"]["mean"],
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
