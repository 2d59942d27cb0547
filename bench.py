"""Benchmark: fused SDPA forward + backward on one MI355X.

One step = one pass of the whole hot path over one batch of the headline
workload (bf16, causal, B=4 H=16 S_q=S_kv=2048 d=128, scale 1/sqrt(128)):
sdpa_fwd, then the backward's two kernels in the order sdpa_bwd runs them
(dQ with the D preprocess of its rows, then dK/dV).
Inputs are seeded synthetic N(0,1) tensors, resident in HBM before timing.

Throughput uses the workload's algorithmic flop count: forward
4*b*h*s_q*s_kv*d (2*b*h*s_q*s_kv*(d_qk+d_v) in general), backward 2.5x that,
both halved under the causal mask.  Prints one JSON line (rank 0, N = 1).

The line also carries a "decode" object: the thin-query forward (split-KV)
on the decode workload (bf16, B=16, 32 query heads over 8 key/value heads,
one query row per sequence, S_kv=8192, d=128), timed the same way and
reported as algorithmic HBM bytes (K, V, Q, O, LSE) per second against the
8 TB/s peak; "decode_int8": the same step over an int8 K/V cache with fp32
scales per token and group of 32 head-dim elements (bytes: codes, scales,
Q, O, LSE); and "decode_int4": over signed 4-bit codes, two per byte.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-suite]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "SDPA fwd/bwd TFLOP/s (bf16 causal B4 H16 S2048 d128) + % MFMA peak"
KERNEL_SOURCES = ("sdpa_fwd.hip", "sdpa_bwd.hip", "sdpa_device.h", "sdpa_kcommon.h")


def flops(wl):
    f = 2.0 * wl.b * wl.h * wl.s_q * wl.s_kv * (wl.d_qk + wl.d_v)
    b = 2.0 * wl.b * wl.h * wl.s_q * wl.s_kv * (3 * wl.d_qk + 2 * wl.d_v)
    if wl.causal:
        f, b = f / 2, b / 2
    return f, b


def source_hash():
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "scaled_dot_product_13_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            d = json.load(f)
        if d.get("source_hash") != source_hash():
            return None
        return d.get("kernels", {}).get(kernel, {}).get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_info():
    """Host facts for the CPU baseline: logical CPUs and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(wl, x, budget_heads):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: the first `budget_heads` (batch, head) slices in batch-major
    order (by default all of them, i.e. the whole workload)."""
    import numpy as np
    import oracle.sdpa_oracle as O
    nthreads = min(16, os.cpu_count() or 1)
    heads = [(b, h) for b in range(wl.b) for h in range(wl.h)][:budget_heads]
    q, k, v, do = (x[n].double().numpy() for n in ("q", "k", "v", "dout"))
    kw = dict(scale=wl.softmax_scale, causal=wl.causal, heads=heads, threads=nthreads)
    t0 = time.perf_counter()
    O.fwd(q, k, v, **kw)
    O.bwd(q, k, v, do, **kw)
    dt = time.perf_counter() - t0
    f, b = flops(wl)
    frac = len(heads) / (wl.b * wl.h)
    return {"value": round((f + b) * frac / dt / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads,
            "kind": "oracle", **cpu_info(),
            "sample": f"fwd+bwd of {len(heads)} of {wl.b * wl.h} (batch, head) slices of the "
                      f"same workload, fp64, {dt:.1f} s wall"}


class CacheFlush:
    """Writes a 512 MiB device buffer, so that neither the 256 MB Infinity
    Cache nor the L2s hold any input of the next call, then reads a second
    512 MiB buffer, so that the lines the write left dirty are written back
    to HBM before the call instead of during it (the caches then hold clean
    lines of the read buffer, which the call's own reads evict for free).
    Called before each timed iteration of the memory-bound measurements,
    outside the interval the events bracket."""

    def __init__(self, torch, dev, mib=512):
        self.buf = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
        self.clean = torch.ones((mib << 20) // 4, dtype=torch.int32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xFF)
        self.clean.sum()


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def decode_bench(S, torch, steps, warmup, wl, flush):
    """Time the thin-query forward on a decode workload: HIP events on the
    launch stream around each sdpa_fwd call (the split kernel and, when the
    keys are split, the combine kernel), the caches flushed before each
    call; the median is reported."""
    from scaled_dot_product_13_amd import inputs
    x = inputs.make_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kw = dict(scale=wl.softmax_scale, causal=wl.causal, bottom_right=wl.bottom_right)
    hk = wl.h_kv or wl.h
    kv_elems = wl.b * hk * wl.s_kv * (wl.d_qk + wl.d_v)
    if wl.kv_quant is not None:
        gs, with_zp = wl.kv_quant[:2]
        fmt = wl.kv_quant[2] if len(wl.kv_quant) > 2 else "s8"
        kw.update(kv_scales=(x["k_scales"].to(dev), x["v_scales"].to(dev)), kv_group_size=gs,
                  kv_zero_points=(x["k_zp"].to(dev), x["v_zp"].to(dev)) if with_zp else None,
                  kv_format=fmt)
        code_bytes = kv_elems if fmt == "s8" else kv_elems // 2
        kv_bytes = code_bytes + kv_elems // gs * (4 + (1 if with_zp else 0))
    else:
        kv_bytes = 2 * kv_elems
    del x
    o = torch.empty((wl.b, wl.h, wl.s_q, wl.d_v), dtype=q.dtype, device=dev)
    lse = torch.empty((wl.b, wl.h, wl.s_q), dtype=torch.float32, device=dev)
    ws = torch.empty(max(S.fwd_workspace_size(q, k, v, **kw), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ms = _timed(torch, stream, lambda: S.sdpa_fwd(q, k, v, out=o, lse=lse, workspace=ws, **kw),
                steps, warmup, flush)
    byts = (kv_bytes                                             # K, V (+ scales)
            + 2 * wl.b * wl.h * wl.s_q * (wl.d_qk + wl.d_v)      # Q, O (bf16)
            + 4 * wl.b * wl.h * wl.s_q)                          # LSE
    gbs = byts / (ms * 1e-3) / 1e9
    return {"workload": wl.name, "ms": round(ms, 5), "bytes": byts, "timing": "median, flushed",
            "roofline": {"kernel": "fwd_decode (+ combine)", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def _timed(torch, stream, fn, steps, warmup, flush):
    """Median ms of fn() over `steps` calls, each bracketed by HIP events on
    the launch stream with the caches flushed just before (outside the
    bracket), after `warmup` untimed calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return _median([a.elapsed_time(b) for a, b in ev])


def suite_bench(S, torch, steps, warmup, flush):
    """The other workloads of the suite (fp16 with bias and dBias; bf16 packed
    variable-length causal; bf16 causal with dropout): sdpa_fwd and the whole
    sdpa_bwd, each timed with HIP events per call.  Reported as TFLOP/s of
    the workload's algorithmic flop count and as GB/s of algorithmic HBM
    bytes (inputs read once, outputs written once).  Also the standalone
    backward preprocess (D = rowsum(dO o O) and LSE*log2(e)), an HBM-bound
    kernel, on the headline and the variable-length shapes."""
    from scaled_dot_product_13_amd import inputs
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    for idx in (3, 4, 5):
        wl = inputs.WORKLOADS[idx]
        x = inputs.make_inputs(wl)
        q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
        kw = dict(scale=wl.softmax_scale, causal=wl.causal)
        e2 = q.element_size()
        if wl.varlen is not None:
            lens = [int(t) for t in x["lengths"]]
            kw.update(cu_seqlens_q=x["cu_seqlens"].to(dev), cu_seqlens_kv=x["cu_seqlens_kv"].to(dev),
                      max_seqlen_q=x["max_seqlen"], max_seqlen_kv=x["max_seqlen_kv"])
            pairs = sum(wl.h * L * L for L in lens)
            rows = wl.h * sum(lens)
            rows_kv = rows
        else:
            pairs = wl.b * wl.h * wl.s_q * wl.s_kv
            rows = wl.b * wl.h * wl.s_q
            rows_kv = wl.b * (wl.h_kv or wl.h) * wl.s_kv
        if wl.causal:
            pairs /= 2
        if wl.dropout_p:
            kw.update(dropout_p=wl.dropout_p, seed=inputs.DROPOUT_SEED, offset=0)
        bias = x["bias"].to(dev) if wl.bias else None
        del x
        o, lse, _ = S.sdpa_fwd(q, k, v, bias=bias, **kw)
        ws = torch.empty(max(1, S.bwd_workspace_size(q, k, v, **kw)), dtype=torch.uint8, device=dev)
        f_ms = _timed(torch, stream, lambda: S.sdpa_fwd(q, k, v, bias=bias, out=o, lse=lse, **kw),
                      steps, warmup, flush)
        b_ms = _timed(torch, stream, lambda: S.sdpa_bwd(q, k, v, o, do, lse, bias=bias,
                                                        want_dbias=bias is not None,
                                                        workspace=ws, **kw), steps, warmup, flush)
        f_fl = 2.0 * pairs * (wl.d_qk + wl.d_v)
        b_fl = 2.0 * pairs * (3 * wl.d_qk + 2 * wl.d_v)
        bias_b = bias.numel() * bias.element_size() if bias is not None else 0
        f_by = (rows * wl.d_qk + rows_kv * (wl.d_qk + wl.d_v)) * e2 + bias_b + rows * wl.d_v * e2 + 4 * rows
        b_by = ((rows * wl.d_qk + rows_kv * (wl.d_qk + wl.d_v) + 2 * rows * wl.d_v) * e2 + 4 * rows
                + bias_b                                                         # in
                + (rows * wl.d_qk + rows_kv * (wl.d_qk + wl.d_v)) * e2 + bias_b)  # dQ, dK, dV, dBias
        out[str(idx)] = {
            "workload": wl.name, "timing": "median, flushed",
            "fwd": {"ms": round(f_ms, 5), "tflops": round(f_fl / f_ms / 1e9, 2),
                    "hbm_gbs": round(f_by / f_ms / 1e6, 1), "bytes": int(f_by)},
            "bwd": {"ms": round(b_ms, 5), "tflops": round(b_fl / b_ms / 1e9, 2),
                    "hbm_gbs": round(b_by / b_ms / 1e6, 1), "bytes": int(b_by)},
            "tflops": round((f_fl + b_fl) / (f_ms + b_ms) / 1e9, 2),
        }
        if idx == 4:
            # the standalone preprocess in group mode
            n_st, off_st = S.stats_layout(len(lens), wl.h, kw["max_seqlen_q"])
            st = torch.empty(off_st + n_st, dtype=torch.float32, device=dev)
            p_ms = _timed(torch, stream, lambda: S.sdpa_bwd_preprocess(
                o, do, lse, cu_seqlens_q=kw["cu_seqlens_q"], max_seqlen_q=kw["max_seqlen_q"], out=st),
                steps, warmup, flush)
            p_by = 2 * rows * wl.d_v * e2 + 4 * rows + 8 * rows
            out[str(idx)]["bwd_preprocess"] = {"ms": round(p_ms, 5), "bytes": int(p_by),
                                               "hbm_gbs": round(p_by / p_ms / 1e6, 1)}
        del q, k, v, do, o, lse, bias, ws
        torch.cuda.empty_cache()
    return out


def preprocess_bench(S, torch, steps, warmup, flush, q, o, do, lse, stats):
    """The standalone backward preprocess on the headline shape (HBM-bound):
    reads O, dO (io type) and LSE, writes D and LSE*log2(e) (fp32)."""
    stream = torch.cuda.current_stream()
    ms = _timed(torch, stream, lambda: S.sdpa_bwd_preprocess(o, do, lse, out=stats), steps, warmup,
                flush)
    rows = lse.numel()
    by = 2 * o.numel() * o.element_size() + 4 * rows + 8 * rows
    gbs = by / ms / 1e6
    return {"ms": round(ms, 5), "bytes": int(by), "timing": "median, flushed",
            "roofline": {"kernel": "bwd_pre", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=2, help="workload index (2 = headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the thin-query (decode) line")
    ap.add_argument("--no-suite", action="store_true",
                    help="skip the other workloads and the standalone preprocess")
    ap.add_argument("--cpu-heads", type=int, default=1 << 30,
                    help="(batch, head) slices the CPU baseline times (default: all)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for calibrating HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world}): the "
              "attention heads shard across GPUs with no exchange, so the one-GPU number is "
              "the per-GPU figure; multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from scaled_dot_product_13_amd import inputs
    from scaled_dot_product_13_amd import sdpa as S

    wl = inputs.WORKLOADS[args.workload]
    assert wl.varlen is None and not wl.bias and wl.dropout_p == 0.0, "bench runs batch workloads"
    x = inputs.make_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    kw = dict(scale=wl.softmax_scale, causal=wl.causal)
    # preallocated outputs: the timed region runs kernels only
    o = torch.empty((wl.b, wl.h, wl.s_q, wl.d_v), dtype=q.dtype, device=dev)
    lse = torch.empty((wl.b, wl.h, wl.s_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    n, off = S.stats_layout(wl.b, wl.h, wl.s_q)
    stats = torch.empty(off + n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    # The decode lines and the other workloads are measured first (their
    # inputs drawn on the CPU in turn), right before the headline, so that
    # the GPU runs the headline's warm-up and timed steps near its steady
    # clocks: from an idle GPU, 10 warm-up steps (a few milliseconds of work)
    # leave the timed steps ~7% slower than 200 warm-up steps do.
    def extra(fn, *a):
        """A secondary measurement: an exception is reported in its place
        rather than stopping the headline measurement."""
        try:
            return fn(*a)
        except Exception as e:  # noqa: BLE001 - reported in the JSON line
            print(f"bench.py: {fn.__name__} failed: {e!r}", file=sys.stderr, flush=True)
            return {"error": repr(e)}

    flush = CacheFlush(torch, dev)
    ns, nw = max(args.steps, 50), min(args.warmup, 5)  # secondary lines: medians of >= 50
    decode = {}
    if not args.no_decode:
        decode["decode"] = extra(decode_bench, S, torch, ns, min(args.warmup, 10), inputs.DECODE,
                                 flush)
        decode["decode_int8"] = extra(decode_bench, S, torch, ns, min(args.warmup, 10),
                                      inputs.DECODE_Q8, flush)
        decode["decode_int4"] = extra(decode_bench, S, torch, ns, min(args.warmup, 10),
                                      inputs.DECODE_Q4, flush)
    suite = extra(suite_bench, S, torch, ns, nw, flush) if not args.no_suite else None

    names = ("fwd", "bwd_dq", "bwd_dkdv")
    calls = (lambda: S.sdpa_fwd(q, k, v, out=o, lse=lse, **kw),
             lambda: S.sdpa_bwd_dq_preprocess(q, k, v, o, do, lse, dq=dq, stats=stats, **kw),
             lambda: S.sdpa_bwd_dkdv(q, k, v, do, stats, dk=dk, dv=dv, **kw))

    def step(bracket, ev):
        """fwd, then the backward's kernels.  HIP events on the launch stream
        bracket the kernels named in `bracket` (each event record also costs
        the step a few microseconds, so the timed steps bracket only the
        dominant kernel)."""
        for n, c in zip(names, calls):
            if n in bracket:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                c()
                e1.record(stream)
                ev[n].append((e0, e1))
            else:
                c()

    def averages(ev):
        return {n: sum(a.elapsed_time(b) for a, b in ev[n]) / len(ev[n]) for n in ev if ev[n]}

    def medians(ev):
        out = {}
        for n in ev:
            if ev[n]:
                t = sorted(a.elapsed_time(b) for a, b in ev[n])
                out[n] = t[len(t) // 2]
        return out

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # warm-up steps, every kernel bracketed: they name the dominant kernel
    # (by median: the first launch of each kernel also loads its code)
    warm = {n: [] for n in names}
    for _ in range(args.warmup):
        step(names, warm)
    torch.cuda.synchronize()
    dom = max(names, key=lambda n: medians(warm).get(n, 0.0)) if args.warmup else "bwd_dkdv"
    # the timed steps
    ev = {n: [] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step((dom,), ev)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    dom_ms = averages(ev)[dom]
    # per-kernel breakdown (diagnostic, after the timed region): the same
    # number of steps with every kernel bracketed
    diag = {n: [] for n in names}
    for _ in range(args.steps):
        step(names, diag)
    torch.cuda.synchronize()
    avg = averages(diag)
    # and with the caches flushed before each step (outside the brackets):
    # the inputs then come from HBM, not from the Infinity Cache
    fl = {n: [] for n in names}
    for _ in range(args.steps):
        flush()
        step(names, fl)
    torch.cuda.synchronize()
    fl_med = medians(fl)

    f_fl, b_fl = flops(wl)
    fwd_ms = avg["fwd"]
    bwd_ms = avg["bwd_dq"] + avg["bwd_dkdv"]
    value = (f_fl + b_fl) / (ms_step * 1e-3) / 1e12
    fwd_tf = f_fl / (fwd_ms * 1e-3) / 1e12
    bwd_tf = b_fl / (bwd_ms * 1e-3) / 1e12

    # dominant kernel and its roofline (algorithmic work per launch)
    s2 = wl.b * wl.h * wl.s_q * wl.s_kv * (0.5 if wl.causal else 1.0)
    per_kernel_flops = {
        "fwd": 2.0 * s2 * (wl.d_qk + wl.d_v),                 # Q K^T and P V
        "bwd_dkdv": 2.0 * s2 * (2 * wl.d_qk + 2 * wl.d_v),    # S, dP, dV, dK
        "bwd_dq": 2.0 * s2 * (2 * wl.d_qk + wl.d_v),          # S, dP, dQ (+ the D preprocess)
    }
    ach = per_kernel_flops[dom] / (dom_ms * 1e-3) / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": stored_traffic(dom), "avg_launch_ms": round(dom_ms, 5)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + " fwd+bwd", "b": wl.b, "h": wl.h, "s_q": wl.s_q,
                   "s_kv": wl.s_kv, "d_qk": wl.d_qk, "d_v": wl.d_v, "causal": wl.causal,
                   "io": wl.dtype},
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 5), "tflops": round(fwd_tf, 2),
                "pct_mfma_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2)},
        "bwd": {"ms": round(bwd_ms, 5), "tflops": round(bwd_tf, 2),
                "pct_mfma_peak": round(100 * bwd_tf / PEAK_BF16_TFLOPS, 2),
                "kernels_ms": {n: round(avg[n], 5) for n in ("bwd_dq", "bwd_dkdv")}},
        "flushed_median_ms": {n: round(fl_med[n], 5) for n in names},
        "breakdown_note": "fwd/bwd ms: a diagnostic pass after the timed steps with every "
                          "kernel bracketed by HIP events; the timed steps bracket only the "
                          "roofline kernel; flushed_median_ms: one more pass with a 512 MiB "
                          "write before each step, medians per kernel",
        "roofline": roof,
    }
    if not args.no_suite:
        out["bwd_preprocess"] = extra(preprocess_bench, S, torch, ns, nw, flush, q, o, do, lse,
                                      stats)
        out["suite"] = suite
    if not args.no_decode:
        out.update(decode)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_heads)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
