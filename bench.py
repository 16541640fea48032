#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload NAME] [--cpu-seconds 15]

One step is the whole path over one batch: the forward pass (fa_fwd) and the
backward pass (fa_bwd's three phases: the D pre-pass, the key-block sweep for
dK and dV, the query-block sweep for dQ) on the causal bf16 workload B=8, H=32,
T=4096, d=128, with every input already resident in device memory.  FLOPs
follow the pages' convention: forward 4 B H Tq Tk d (halved when causal),
backward 2.5 x forward (five tile products against two); the two products the
backward sweeps form twice are not counted.  The value is total FLOPs per step
/ time per step.

Printed: one JSON line on stdout (progress goes to stderr), with
  roofline      the dominant kernel's algorithmic TFLOP/s (the FLOPs of the
                tile products it forms, per launch, / its mean duration from HIP
                events recorded on the launch stream over the timed steps)
                against the bf16 dense MFMA peak;
                `traffic` comes from the committed rocprofv3 counter summary
                when that summary matches the current kernel source, else null
  roofline_fwd  the same for the forward kernel alone
  cpu_baseline  the float64 NumPy oracle, fwd+bwd on a sample of heads of the
                same workload, timed on the host cores (a reported baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s and % bf16 MFMA peak (causal, T=4096, d=128)"
DEFAULT_WORKLOAD = "causal_bf16_b8h32_t4096_d128"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}     # MI355X published dense MFMA peaks
PROFILES = os.path.join(ROOT, "profiles")
# Oracle worker threads: the host cores one GPU's share of the box provides (16 on the
# MI355X boxes measured here, whose os.cpu_count() reports the whole host); the
# cpu_baseline object reports both this and os.cpu_count().
CPU_SHARE = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """SHA-256 over the HIP sources; a traffic summary names the digest it was taken at."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "io_aware_exact_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt (key = value
    lines written from two rocprofv3 --pmc runs), or None when absent or stale."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if "=" in line and not line.startswith("#"):
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = v
    if vals.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def mask_pairs(m, Tq: int, Tk: int, causal: bool):
    """Visible (query, key) pairs per head under a block mask [heads][nqb][nkb] of
    128 x 128 blocks (and the causal rule l <= r when asked for)."""
    import numpy as np
    nq, nk = m.shape[1], m.shape[2]
    kstart = 128 * np.arange(nk)
    kend = np.minimum(kstart + 128, Tk)
    if causal:
        r = np.arange(Tq)
        cnt = np.clip(np.minimum(r[:, None] + 1, kend[None, :]) - kstart[None, :], 0, None)
        blk = np.add.reduceat(cnt, 128 * np.arange(nq), axis=0)
    else:
        rows = np.minimum(128, Tq - 128 * np.arange(nq))
        blk = rows[:, None] * (kend - kstart)[None, :]
    return (np.asarray(m, np.int64) * blk[None]).sum(axis=(1, 2))


ORACLE_HEAD_BYTES = 1 << 30                     # largest T x T float64 matrix timed on whole heads


def window_pairs(Tq: int, Tk: int, window) -> float:
    """Visible (query, key) pairs of one head under a sliding window (wl, wr)."""
    import numpy as np
    wl, wr = window
    r = np.arange(Tq, dtype=np.int64)
    lo = np.maximum(0, r - wl) if wl >= 0 else np.zeros_like(r)
    hi = np.minimum(Tk - 1, r + wr) if wr >= 0 else np.full_like(r, Tk - 1)
    return float(np.maximum(0, hi - lo + 1).sum())


def doc_pairs(cu, causal: bool, rows=None) -> float:
    """Visible (query, key) pairs of one head under document offsets cu (of the listed
    query rows only, when given): a row sees its document, up to itself when causal."""
    import numpy as np
    cu = np.asarray(cu, np.int64)
    r = np.arange(int(cu[-1])) if rows is None else np.asarray(rows, np.int64)
    doc = np.searchsorted(cu, r, side="right") - 1
    start, end = cu[doc], cu[doc + 1]
    return float(((r - start + 1) if causal else (end - start)).sum())


def cpu_baseline_rows(w, raw, seconds: float, cores: int, docs=None):
    """For heads too large for the oracle's backward (its T x T matrices): time the
    oracle's forward on sampled query rows, one head per thread."""
    import numpy as np
    from oracle import naive
    from io_aware_exact_02_amd.inputs import as_f64
    scale = 1.0 / math.sqrt(w.d)
    rng = np.random.default_rng(w.seed)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    nrows = max(1, (ORACLE_HEAD_BYTES // 8) // w.Tk // cores)     # rows per head, all threads together ~1 GiB
    done, rounds, t_total, flops = 0, 0, 0.0, 0.0
    while t_total < seconds and rounds < 16:
        batch = [heads[(done + i) % len(heads)] for i in range(cores)]
        bi, hi = [b for b, _ in batch], [h for _, h in batch]
        q, k, v = (as_f64(raw[x][bi, hi], w.dtype)[None] for x in ("q", "k", "v"))
        rows = np.sort(rng.choice(w.Tq, size=min(nrows, w.Tq), replace=False))
        t0 = time.perf_counter()
        naive.forward(q, k, v, scale, w.causal, rows=rows, workers=cores, window=w.window, docs=docs)
        t_total += time.perf_counter() - t0
        if docs is not None:
            pairs = doc_pairs(docs, w.causal, rows)
        elif w.window is not None:
            pairs = float(naive.window_allowed(w.Tk, rows, w.window).sum())
        else:
            pairs = float(np.sum(np.minimum(rows + 1, w.Tk))) if w.causal else float(len(rows)) * w.Tk
        flops += 4.0 * w.d * pairs * len(batch)
        done += len(batch)
        rounds += 1
        log(f"[cpu_baseline] {rounds} rounds of {len(batch)} heads x {len(rows)} rows in {t_total:.1f} s")
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle, forward only, {rounds} rounds of {cores} (batch, head) slices x "
                      f"{nrows} random query rows of the same workload (T={w.Tq}, d={w.d}, causal={w.causal}, "
                      f"window={w.window}{', packed documents' if docs is not None else ''}), "
                      f"{t_total:.1f} s on {cores} threads with one BLAS thread each; its backward needs whole "
                      f"T x T matrices per head ({w.Tq * w.Tk * 8 / 2**30:.0f} GiB each in float64), so only the "
                      f"forward is timed; FLOPs counted as for the GPU"}


def cpu_baseline(w, raw, seconds: float, bmask=None, docs=None):
    """Time the float64 oracle's forward+backward on whole heads of the workload
    (with the workload's block mask when it has one)."""
    from oracle import naive
    from io_aware_exact_02_amd.inputs import as_f64
    cores = max(1, min(CPU_SHARE, os.cpu_count() or 1))
    if w.Tq * w.Tk * 8 > ORACLE_HEAD_BYTES and bmask is None:
        return cpu_baseline_rows(w, raw, seconds, cores, docs)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    scale = 1.0 / math.sqrt(w.d)
    pairs = mask_pairs(bmask, w.Tq, w.Tk, w.causal) if bmask is not None else None
    done, t_total, flops = 0, 0.0, 0.0
    while done < len(heads) and t_total < seconds:
        batch = heads[done:done + cores]
        bi, hi = [b for b, _ in batch], [h for _, h in batch]
        q, k, v, do = (as_f64(raw[x][bi, hi], w.dtype)[None] for x in ("q", "k", "v", "do"))
        bm = None if bmask is None else bmask[hi]
        t0 = time.perf_counter()
        naive.backward(q, k, v, do, scale, w.causal, workers=cores, block_mask=bm)
        t_total += time.perf_counter() - t0
        done += len(batch)
        if pairs is None:
            flops += len(batch) / (w.B * w.H) * (w.flops_fwd() + w.flops_bwd())
        else:
            flops += 3.5 * 4.0 * w.d * float(sum(pairs[h] for h in hi))
        log(f"[cpu_baseline] {done} heads in {t_total:.1f} s")
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle, forward+backward of {done} of {w.B * w.H} (batch, head) slices of "
                      f"the same workload (T={w.Tq}, d={w.d}, causal={w.causal}), {t_total:.1f} s on {cores} "
                      f"threads with one BLAS thread each; FLOPs counted as for the GPU"}


HBM_PEAK_GBS = 8000.0                           # MI355X published HBM3E bandwidth


def bench_decode(a, w):
    """Split-key forward on a decoding workload (few query rows, long key cache).

    Bound by the HBM read of K and V: the value is algorithmic bytes per step
    (Q, K, V read once; O and lse written once) / time per step, against the HBM
    peak.  One step = fa_fwd_splitkv (partials pass + merge pass)."""
    import torch
    import io_aware_exact_02_amd as fa
    from io_aware_exact_02_amd.inputs import draw_workload
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] drawing inputs for {w.name}")
    raw = draw_workload(w, with_do=False)
    q, k, v = (torch.from_numpy(raw[n].view("int16")).view(torch.bfloat16).to(dev) for n in ("q", "k", "v"))
    B, H, Tq, Tk, d = w.B, w.H, w.Tq, w.Tk, w.d
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    nbytes = fa.fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    step = lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, ws, causal=w.causal, stream=stream)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    ms_ev = e0.elapsed_time(e1) / a.steps
    alg_bytes = 2 * (2 * B * H * Tk * d + 2 * B * H * Tq * d) + 4 * B * H * Tq
    gbs = alg_bytes / (ms_ev * 1e-3) / 1e9
    out = {
        "metric": f"split-key decode HBM GB/s ({w.name})", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1))",
        "config": {"workload": w.name, "B": B, "H": H, "Tq": Tq, "Tk": Tk, "d": d, "causal": w.causal,
                   "pass": "forward (split-key)", "partials": nbytes // (4 * B * H * Tq * (d + 4))},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "decode_partial_kernel+merge"},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time budget (0 = skip)")
    ap.add_argument("--density", type=float, default=None,
                    help="block-sparse workloads: fraction of kept blocks (default: the workload's)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (a known-size "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange). Use --gpus 1.",
              file=sys.stderr)
        return 2
    import torch
    import io_aware_exact_02_amd as fa
    from io_aware_exact_02_amd.inputs import WORKLOADS, draw_workload, workload_docs, workload_mask

    w = WORKLOADS[a.workload]
    if w.Tq <= 32 and w.dtype == "bf16" and not w.backward:
        return bench_decode(a, w)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] drawing inputs for {w.name}")
    raw = draw_workload(w, with_do=True)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v, do = (up(raw[n]) for n in ("q", "k", "v", "do"))
    B, H, Tq, Tk, d = w.B, w.H, w.Tq, w.Tk, w.d
    # Large logits (Q, K spread > 1): O is carried between the passes in float32
    # and the gradients are float32 -- the path whose results meet the gradient
    # tolerance on that workload (rounding O to bf16 moves D = dO . O, and the
    # gradients reach magnitudes where bf16's own step nears the tolerance)
    wide = w.qk_spread > 1.0 and w.dtype == "bf16"
    o = torch.empty(q.shape, dtype=torch.float32, device=dev) if wide else torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    gdt = torch.float32 if wide else q.dtype
    dq, dk, dv = (torch.empty(x.shape, dtype=gdt, device=dev) for x in (q, k, v))
    nws = fa.fa_bwd_workspace_bytes(B, H, Tq, Tk, d, fa._dtype_code(q), fa._dtype_code(dq))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    phases = [fa.FA_BWD_PRE, fa.FA_BWD_MAIN, fa.FA_BWD_POST]
    bmask_np = bmask = None
    if w.mask_density is not None:
        bmask_np = workload_mask(w, a.density)
        bmask = torch.from_numpy(bmask_np).to(dev)
    cu_np = cu = None
    if w.doc_len is not None:
        cu_np = workload_docs(w)
        cu = torch.from_numpy(cu_np).to(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if cu is not None:
            fa.fa_fwd_docs(q, k, v, o, lse, cu, causal=w.causal, stream=stream)
        elif w.window is not None:
            fa.fa_fwd_window(q, k, v, o, lse, w.window, stream=stream)
        elif bmask is None:
            fa.fa_fwd(q, k, v, o, lse, causal=w.causal, stream=stream)
        else:
            fa.fa_fwd_masked(q, k, v, o, lse, bmask, causal=w.causal, stream=stream)
        for i, ph in enumerate(phases):
            if ev is not None:
                ev[i + 1].record(stream)
            if cu is not None:
                fa.fa_bwd_docs_phases(q, k, v, o, do, lse, dq, dk, dv, cu, ws, ph, causal=w.causal, stream=stream)
            elif w.window is not None:
                fa.fa_bwd_window_phases(q, k, v, o, do, lse, dq, dk, dv, w.window, ws, ph, stream=stream)
            elif bmask is None:
                fa.fa_bwd_phases(q, k, v, o, do, lse, dq, dk, dv, ws, ph, causal=w.causal, stream=stream)
            else:
                fa.fa_bwd_masked_phases(q, k, v, o, do, lse, dq, dk, dv, bmask, ws, ph, causal=w.causal,
                                        stream=stream)
        if ev is not None:
            ev[4].record(stream)

    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    log(f"[bench] timing {a.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / a.steps
    names = ["fwd", "bwd_pre", "bwd_main", "bwd_post"]
    dur = {n: sum(events[s][i].elapsed_time(events[s][i + 1]) for s in range(a.steps)) / a.steps
           for i, n in enumerate(names)}
    # per-step times from the events on the launch stream: median and spread
    per_step = sorted(events[s][0].elapsed_time(events[s][4]) for s in range(a.steps))
    step_stats = {"median_ms": round(per_step[len(per_step) // 2] if len(per_step) % 2 else
                                     0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2]), 4),
                  "min_ms": round(per_step[0], 4), "max_ms": round(per_step[-1], 4)}
    f_fwd, f_bwd = w.flops_fwd(), w.flops_bwd()
    if bmask_np is not None:                    # kept pairs only: 4 d per visible (query, key) pair
        f_fwd = 4.0 * d * B * float(mask_pairs(bmask_np, Tq, Tk, w.causal).sum())
        f_bwd = 2.5 * f_fwd
    if w.window is not None:                    # pairs inside the window only
        f_fwd = 4.0 * d * B * H * window_pairs(Tq, Tk, w.window)
        f_bwd = 2.5 * f_fwd
    if cu_np is not None:                       # pairs inside each document only
        f_fwd = 4.0 * d * B * H * doc_pairs(cu_np, w.causal)
        f_bwd = 2.5 * f_fwd
    total = f_fwd + f_bwd
    value = total / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    # FLOPs of the tile products each kernel forms (2 d per visible pair each):
    # the key-block sweep forms S, dP, dV, dK; the query-block sweep S, dP, dQ.
    kflops = {"fwd": f_fwd, "bwd_main": 0.8 * f_bwd, "bwd_post": 0.6 * f_bwd}
    kernels = {}
    for n in names:
        entry = {"ms": round(dur[n], 4)}
        if n in kflops:
            tf = kflops[n] / (dur[n] * 1e-3) / 1e12
            entry.update(tflops=round(tf, 1), frac_of_peak=round(tf / peak, 4))
        kernels[n] = entry
    dom = max(kflops, key=lambda n: dur[n])
    ach = kflops[dom] / (dur[dom] * 1e-3) / 1e12
    # the kernels each phase launches: d = 256 runs the forward (plain masks) and the dQ
    # sweep in two wave roles, the key-block sweep in its four-wave form
    plain = bmask_np is None and w.window is None and cu_np is None
    knames = {"fwd": "fwd_split_kernel" if d == 256 and plain else "fwd_bf16_kernel",
              "bwd_main": "bwd_kv_w4_kernel" if d == 256 else "bwd_kv_kernel",
              "bwd_post": "bwd_dq_split_kernel" if d == 256 else "bwd_dq_kernel"}
    kernel_name = knames[dom]
    roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": read_traffic(kernel_name, w.name),
                "kernel": kernel_name}
    # the forward's own roofline (the kernel the 60%-of-peak target is set on)
    ach_f = kflops["fwd"] / (dur["fwd"] * 1e-3) / 1e12
    roofline_fwd = {"bound": "mfma", "achieved": round(ach_f, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach_f / peak, 4), "traffic": read_traffic(knames["fwd"], w.name),
                    "kernel": knames["fwd"]}
    cpu = None
    if a.cpu_seconds > 0:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(w, raw, a.cpu_seconds, bmask_np, cu_np)
    out = {
        "metric": METRIC if w.name == DEFAULT_WORKLOAD else f"attention fwd+bwd TFLOP/s ({w.name})",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1), see io_aware_exact_02_amd/inputs.py)",
        "config": {"workload": f"{w.name}_fwd_bwd", "B": B, "H": H, "Tq": Tq, "Tk": Tk, "d": d,
                   "causal": w.causal, "pass": "forward+backward"},
        "pct_of_peak": round(100 * value / peak, 2),
        "step_events": step_stats,
        "roofline": roofline, "roofline_fwd": roofline_fwd, "kernels": kernels, "cpu_baseline": cpu,
    }
    if wide:
        out["config"].update(o_dtype="f32", grad_dtype="f32")
    if w.window is not None:
        out["config"].update(window=list(w.window),
                             flops="4 d per (query, key) pair inside the window forward, 2.5 x that backward")
    if cu_np is not None:
        out["config"].update(documents=len(cu_np) - 1, doc_len=list(w.doc_len),
                             doc_offsets="seeded, lengths log-uniform in doc_len, laid end to end",
                             flops="4 d per (query, key) pair inside a document forward, 2.5 x that backward")
    if bmask_np is not None:
        out["config"].update(block_mask="seeded Bernoulli per 128 x 128 block, one per head, diagonal kept",
                             kept_blocks=round(float(bmask_np.mean()), 4),
                             flops="4 d per kept (query, key) pair forward, 2.5 x that backward")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
