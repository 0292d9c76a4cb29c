#!/usr/bin/env python3
"""Throughput of the fused attention path on one MI355X.

One step = the whole hot path on one batch: forward (fa_fwd) then backward
(fa_bwd: the (L*log2 e, -D) preprocess, the dK/dV kernel, which also stores
dS on this workload, and the dQ kernel, which reads it) on the long-sequence
workload B=1, H=32, N=8192, d=128, causal, bf16 (Q and K
scaled by 3).  Inputs are synthetic (seeded normal draws on the GPU) and
resident in HBM before timing starts.  Prints ONE JSON line on stdout;
progress goes to stderr.

FLOP convention: forward 2 GEMMs = 4*d per unmasked (query, key) pair,
backward 5 GEMMs = 10*d per pair; pairs = N(N+1)/2 per head when causal.

`--write-traffic FETCH_CSV WRITE_CSV` turns two rocprofv3 counter runs of this
script (one with --pmc FETCH_SIZE, one with --pmc WRITE_SIZE, both with
--copy-calibration-mib) into profiles/hbm_traffic.json and exits.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s (bf16) at B·H·N·d, and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # dense bf16 MFMA: 256 CUs x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def unmasked_pairs(Nq, Nk, causal):
    if not causal:
        return Nq * Nk
    off = Nk - Nq  # key j visible to row i iff j <= i + off
    # rows i with i + off + 1 >= Nk see all keys; the others see i + off + 1
    full_from = max(0, Nk - off - 1)
    part = sum(min(Nk, i + off + 1) for i in range(min(Nq, full_from)))
    return part + max(0, Nq - full_from) * Nk


KERNEL_SOURCES = {
    "fwd_kernel": "fa_fwd.hip",
    "bwd_fused_kernel": "fa_bwd.hip",
    "bwd_dkdv_kernel": "fa_bwd.hip",
    "bwd_dq_kernel": "fa_bwd.hip",
    "bwd_dq_ds_kernel": "fa_bwd.hip",
    "bwd_pre_kernel": "fa_bwd.hip",
}
KERNEL_RE = r"(fwd_kernel|bwd_fused_kernel|bwd_dkdv_kernel|bwd_dq_kernel|bwd_dq_ds_kernel|bwd_pre_kernel)"


def stores_ds(fa, w, code):
    """True where fa_bwd takes the stored-dS path (dK/dV, then dQ from dS)."""
    return fa.bwd_stores_ds(w.B, w.H, w.Nq, w.Nk, w.d, w.causal, code)


def source_sha(path):
    """sha256 over a kernel's source file and the device header it includes."""
    h = hashlib.sha256()
    for p in (path, os.path.join(os.path.dirname(path), "fa_common.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def write_traffic(fetch_csv, write_csv, copy_mib):
    """profiles/hbm_traffic.json from two rocprofv3 --pmc runs of this script.

    Each counter is scaled by what it reads for the calibration copy (a plain
    elementwise kernel reading and writing copy_mib MiB): HBM bytes per launch
    = counter KiB * 1024 * (true copy bytes / counter bytes of the copy)."""
    import csv
    import re
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            m = re.search(KERNEL_RE, r["Kernel_Name"])
            name = m.group(1) if m else ("copy" if int(r["Grid_Size"]) == (copy_mib << 20) // 16
                                         else None)
            if name:
                vals.setdefault(name, []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = float(copy_mib << 10)
    fscale = copy_kib / max(fetch["copy"])  # max: the copy's source fill shares its grid size
    wscale = copy_kib / max(write["copy"])
    csrc = os.path.join(ROOT, "exact_attention_118_amd", "csrc")
    kernels = {}
    for name, src in KERNEL_SOURCES.items():
        if name not in fetch or name not in write:
            continue
        fk, wk = statistics.mean(fetch[name]), statistics.mean(write[name])
        kernels[name] = {"source": f"exact_attention_118_amd/csrc/{src} + fa_common.h",
                         "source_sha256": source_sha(os.path.join(csrc, src)),
                         "fetch_kib_raw": fk, "write_kib_raw": wk,
                         "fetch_bytes": fk * 1024 * fscale, "write_bytes": wk * 1024 * wscale,
                         "bytes_per_launch": fk * 1024 * fscale + wk * 1024 * wscale,
                         "launches": len(fetch[name])}
    rec = {"about": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE "
                    "(KiB per dispatch, mean over the launches), each scaled by what the same "
                    f"counter reads for a plain elementwise copy of {copy_mib} MiB in the same run. "
                    "A kernel's entry is valid while its source and fa_common.h hash to "
                    "source_sha256.",
           "fetch_scale": fscale, "write_scale": wscale, "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({k: round(v["bytes_per_launch"] / 2**20, 1) for k, v in kernels.items()}))


def measured_traffic(kernel_name, source):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel_name)
    if not k or k.get("source_sha256") != source_sha(source):
        return None
    return k.get("bytes_per_launch")


def cpu_baseline(w, x, heads):
    """The float64 oracle, untuned, on the first `heads` heads at full size."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = os.cpu_count() or 1
    BH = w.B * w.H
    flat = {k: v.reshape(BH, v.shape[2], w.d) for k, v in x.items()}
    t0 = time.perf_counter()
    for h in range(heads):
        Q, K, V, dO = (flat[k][h].float().cpu().double().numpy() for k in ("Q", "K", "V", "dO"))
        t_in = time.perf_counter()
        oracle.attention_forward(Q, K, V, w.scale, w.causal)
        oracle.attention_backward(Q, K, V, dO, w.scale, w.causal)
        log(f"oracle head {h}: {time.perf_counter() - t_in:.1f} s")
        del Q, K, V, dO
    dt = time.perf_counter() - t0
    flops = 14 * w.d * unmasked_pairs(w.Nq, w.Nk, w.causal) * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"forward+backward of {heads} of {BH} heads of {w.name} at full size "
                      f"(float64 numpy, {dt:.1f} s)", "seconds": dt}


SETTLE_S = 0.3  # seconds of untimed repetitions before each measurement


def settle(torch, fn, seconds=SETTLE_S):
    """Run fn repeatedly for about `seconds` before a measurement: after a
    pause the GPU needs a few hundred milliseconds of load before its clock
    and power settle (a forward timed after 3 warm-up steps ran 4-5% slower
    than after 100 on the long-sequence workload), and a training loop keeps
    it under load."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()


def bench_decode(fa, torch, steps):
    from exact_attention_118_amd import synth

    w = synth.WORKLOADS["decode_b16h32k16384d128"]
    x = synth.make_inputs(w, seed=0, device="cuda")
    O = torch.empty_like(x["Q"])
    L = torch.empty(w.B, w.H, 1, dtype=torch.float32, device="cuda")
    splits = fa.fwd_num_splits(w.B, w.H, 1, w.Nk, w.d, fa.FA_BF16, 0)
    ws = torch.empty(fa.fwd_workspace_size(w.B, w.H, 1, w.Nk, w.d, fa.FA_BF16, 0),
                     dtype=torch.uint8, device="cuda")
    settle(torch, lambda: fa.fa_fwd(x["Q"], x["K"], x["V"], O, L, w.scale, False, workspace=ws))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fa.fa_fwd(x["Q"], x["K"], x["V"], O, L, w.scale, False, workspace=ws)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    kv_bytes = 2 * w.B * w.H * w.Nk * w.d * 2
    all_bytes = kv_bytes + 2 * w.B * w.H * w.d * 2 + w.B * w.H * 4
    # What the HBM delivers to a plain device copy of the same K (2 GiB read,
    # 2 GiB written) in this run: a reference rate for the split path.
    buf = torch.empty_like(x["K"])
    settle(torch, lambda: buf.copy_(x["K"]))
    ev[0].record()
    for i in range(steps):
        buf.copy_(x["K"])
        ev[i + 1].record()
    torch.cuda.synchronize()
    copy_ms = ev[0].elapsed_time(ev[-1]) / steps
    copy_gbs = 2 * x["K"].numel() * x["K"].element_size() / (copy_ms * 1e-3) / 1e9
    del x, buf
    return {"workload": w.name, "ms": ms, "splits": splits,
            "GB/s": all_bytes / (ms * 1e-3) / 1e9,
            "hbm_frac": all_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "algorithmic_bytes": all_bytes,
            "reference_copy_GB/s": copy_gbs}


def bench_rows_split(fa, torch, steps):
    """A few query rows against a long key range (B=4, H=32, Nq=16, Nk=16384,
    d=128, causal): the key-split path against the tiled path (num_splits=1)."""
    from exact_attention_118_amd import synth

    w = synth.Workload("rows_b4h32q16k16384d128_causal", 4, 32, 16, 16384, 128, True,
                       torch.bfloat16, backward=False)
    x = synth.make_inputs(w, seed=0, device="cuda")
    O = torch.empty_like(x["Q"])
    L = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device="cuda")
    out = {"workload": w.name}
    kv_bytes = 2 * w.B * w.H * w.Nk * w.d * 2
    for label, ns in (("split", 0), ("tiled", 1)):
        nsplit = fa.fwd_num_splits(w.B, w.H, w.Nq, w.Nk, w.d, fa.FA_BF16, ns)
        nb = fa.fwd_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, fa.FA_BF16, ns)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
        settle(torch, lambda: fa.fa_fwd(x["Q"], x["K"], x["V"], O, L, w.scale, True, num_splits=ns,
                                        workspace=ws))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            fa.fa_fwd(x["Q"], x["K"], x["V"], O, L, w.scale, True, num_splits=ns, workspace=ws)
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[-1]) / steps
        out[label] = {"ms": ms, "splits": nsplit, "kv_GB/s": kv_bytes / (ms * 1e-3) / 1e9}
    del x
    return out


def _time_fwd_bwd(fa, torch, w, Q, K, V, dO, ws, steps, bias=None, dropout_p=0.0, tile_map=None):
    """Mean forward and backward milliseconds of fa_fwd + fa_bwd (the bias or
    the dropout entry points when given)."""
    O = torch.empty_like(Q)
    L = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device="cuda")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)

    def run(ev=None):
        if dropout_p or tile_map is not None:
            fa.fa_fwd_ex(Q, K, V, O, L, w.scale, w.causal, bias=bias, dropout_p=dropout_p, seed=1,
                         tile_map=tile_map)
        elif bias is None:
            fa.fa_fwd(Q, K, V, O, L, w.scale, w.causal)
        else:
            fa.fa_fwd_bias(Q, K, V, bias, O, L, w.scale, w.causal)
        if ev is not None:
            ev.record()
        if dropout_p or tile_map is not None:
            fa.fa_bwd_ex(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, bias=bias,
                         dropout_p=dropout_p, seed=1, workspace=ws, tile_map=tile_map)
        elif bias is None:
            fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws)
        else:
            fa.fa_bwd_bias(Q, K, V, bias, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws)

    settle(torch, run)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        run(e[1])
        e[2].record()
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    pairs = unmasked_pairs(w.Nq, w.Nk, w.causal) * w.B * w.H
    return {"fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
            "fwd_TFLOP/s": 4 * w.d * pairs / (fwd_ms * 1e-3) / 1e12,
            "bwd_TFLOP/s": 10 * w.d * pairs / (bwd_ms * 1e-3) / 1e12}


def bench_fp16(fa, torch, w, x, ws, steps):
    """The same forward and backward on fp16 copies of the inputs."""
    Q, K, V, dO = (x[k].to(torch.float16) for k in ("Q", "K", "V", "dO"))
    return _time_fwd_bwd(fa, torch, w, Q, K, V, dO, ws, steps)


def _time_fwd_bwd_graph(fa, torch, w, Q, K, V, dO, ws, reps, replays=20):
    """Mean forward and backward milliseconds of fa_fwd + fa_bwd, each captured
    `reps` times into a HIP graph and replayed (`replays` times back to back,
    after settling), so that host-side launch latency does not count: a
    kernel of a few microseconds would otherwise wait for the host between
    launches."""
    O = torch.empty_like(Q)
    L = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device="cuda")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)

    def fwd():
        fa.fa_fwd(Q, K, V, O, L, w.scale, w.causal)

    def bwd():
        fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
        bwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for fn in (fwd, bwd):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        graphs.append(g)
    ms = []
    for g in graphs:
        settle(torch, g.replay)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / (reps * replays))
    del graphs
    pairs = unmasked_pairs(w.Nq, w.Nk, w.causal) * w.B * w.H
    return {"fwd_ms": ms[0], "bwd_ms": ms[1],
            "fwd_TFLOP/s": 4 * w.d * pairs / (ms[0] * 1e-3) / 1e12,
            "bwd_TFLOP/s": 10 * w.d * pairs / (ms[1] * 1e-3) / 1e12,
            "timing": f"HIP graph of {reps} calls, replayed {replays} times after {SETTLE_S} s of replays"}


def bench_other_configs(fa, torch, steps):
    """Forward and backward of the other bf16 workloads, each against both
    roofs: MFMA (4*d and 10*d flop per unmasked pair) and HBM (algorithmic
    bytes: Q, K, V read and O, L written forward; Q, K, V, O, dO, L, D read
    and dQ, dK, dV written backward)."""
    from exact_attention_118_amd import synth

    out = {}
    for name in ("b4h16n1024d64_causal", "b2h16n4096d128_causal", "b2h16n4096d128"):
        w = synth.WORKLOADS[name]
        x = synth.make_inputs(w, seed=0, device="cuda")
        ws = torch.empty(fa.bwd_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, fa.FA_BF16),
                         dtype=torch.uint8, device="cuda")
        r = _time_fwd_bwd_graph(fa, torch, w, x["Q"], x["K"], x["V"], x["dO"], ws, steps)
        t = w.B * w.H * w.Nq * w.d * 2  # bytes of one bf16 tensor
        rows = w.B * w.H * w.Nq
        fwd_bytes, bwd_bytes = 4 * t + 4 * rows, 8 * t + 8 * rows
        r["fwd_mfma_frac"] = r["fwd_TFLOP/s"] / PEAK_BF16_TFLOPS
        r["bwd_mfma_frac"] = r["bwd_TFLOP/s"] / PEAK_BF16_TFLOPS
        r["fwd_hbm_frac"] = fwd_bytes / (r["fwd_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS
        r["bwd_hbm_frac"] = bwd_bytes / (r["bwd_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS
        out[name] = r
        del x, ws
    return out


def bench_bias(fa, torch, w, x, ws, steps):
    """The same forward and backward with an additive bias [1, H, N, N] in the
    input dtype (one score matrix per head, shared over the batch)."""
    from exact_attention_118_amd import synth

    bias = synth.make_bias(w.B, w.H, w.Nq, w.Nk, w.dtype, seed=11, device="cuda", per_batch=False)
    r = _time_fwd_bwd(fa, torch, w, x["Q"], x["K"], x["V"], x["dO"], ws, steps, bias=bias)
    r["bias_shape"] = list(bias.shape)
    r["bias_GB"] = bias.numel() * bias.element_size() / 1e9
    return r


def bench_window(fa, torch, w, x, ws, steps, window=1024):
    """A block-sparse bias: keys more than `window` before the diagonal get
    -inf ([1, 1, N, N] bf16), with and without its tile map (the map's own
    build time reported apart)."""
    i = torch.arange(w.Nq, device="cuda")[:, None] + (w.Nk - w.Nq)
    j = torch.arange(w.Nk, device="cuda")[None, :]
    b = torch.zeros((w.Nq, w.Nk), dtype=torch.float32, device="cuda")
    b[(i - j) > window] = float("-inf")
    bias = b.to(w.dtype).view(1, 1, w.Nq, w.Nk)
    del b, i, j
    tmap = fa.fa_bias_tile_map(bias, w.B, w.H, w.Nq, w.Nk)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fa.fa_bias_tile_map(bias, w.B, w.H, w.Nq, w.Nk, tile_map=tmap)
    e1.record()
    torch.cuda.synchronize()
    out = {"window": window, "map_ms": e0.elapsed_time(e1) / steps,
           "map_bytes": int(tmap.numel()),
           "map_active_frac": float(tmap.float().mean())}
    args = (fa, torch, w, x["Q"], x["K"], x["V"], x["dO"], ws, steps)
    out["with_map"] = _time_fwd_bwd(*args, bias=bias, tile_map=tmap)
    out["without_map"] = _time_fwd_bwd(*args, bias=bias)
    return out


def bench_dropout(fa, torch, w, x, ws, steps, p=0.1):
    """The same forward and backward with dropout p on the probabilities
    (Philox mask drawn in the kernels, forward and backward)."""
    r = _time_fwd_bwd(fa, torch, w, x["Q"], x["K"], x["V"], x["dO"], ws, steps, dropout_p=p)
    r["dropout_p"] = p
    return r


class PowerSampler:
    """Board power and shader clock sampled through amdsmi in a background
    thread; windows of samples are attributed to the probe running then.  Does
    nothing (and reports None) where amdsmi or its device is unavailable."""

    def __init__(self, period_s=0.004, start=True):
        import threading
        self.samples, self.ok, self.note, self.period_s = [], False, None, period_s
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self.h = handles[0]
            try:
                import torch
                bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
                for h in handles:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        self.h = h
            except Exception:
                pass
            self.amdsmi = amdsmi
            self._read()
            self.ok = True
            self.note = f"{len(handles)} device(s) listed by amdsmi"
        except Exception as e:  # no amdsmi, no device access
            self.note = f"amdsmi unavailable: {type(e).__name__}: {e}"
        self.stop = threading.Event()
        self.thread = None
        if start:
            self.start()

    def start(self):
        import threading
        if self.ok and self.thread is None:
            self.thread = threading.Thread(target=self._run, args=(self.period_s,), daemon=True)
            self.thread.start()

    def _read(self):
        a = self.amdsmi
        p = a.amdsmi_get_power_info(self.h)
        c = a.amdsmi_get_clock_info(self.h, a.AmdSmiClkType.GFX)
        watts = p.get("current_socket_power", p.get("average_socket_power"))
        return float(watts), float(c.get("clk")), p.get("power_limit")

    def _run(self, period_s):
        while not self.stop.is_set():
            try:
                w, mhz, lim = self._read()
                self.samples.append((time.perf_counter(), w, mhz, lim))
            except Exception:
                pass
            time.sleep(period_s)

    def window(self, t0, t1):
        xs = [s for s in self.samples if t0 <= s[0] <= t1]
        if not xs:
            return {"power_W": None, "gfx_clock_MHz": None, "samples": 0}
        return {"power_W": sum(s[1] for s in xs) / len(xs),
                "gfx_clock_MHz": sum(s[2] for s in xs) / len(xs),
                "power_limit": xs[-1][3], "samples": len(xs)}

    def close(self):
        self.stop.set()


def run_probes(seconds):
    """Machine probes (libfa_probe.so) and the attention kernels, each run in a
    loop for `seconds` while board power and shader clock are sampled:
    MFMA loops with constant or random operands, with 1 KB of LDS reads and/or
    one exponential and four FMAs per MFMA; the forward, dK/dV and dQ kernels
    on the long-sequence workload; fp32 atomic adds against plain stores in the
    pattern of an MFMA result tile.  Prints one JSON line."""
    import ctypes

    import torch

    import exact_attention_118_amd as fa
    from exact_attention_118_amd import synth

    plib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_118_amd", "libfa_probe.so"))
    plib.fa_probe_mfma.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2
    plib.fa_probe_adds.argtypes = [ctypes.c_int, ctypes.c_void_p] + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    fa.load_library()
    sampler = PowerSampler()
    stream = torch.cuda.current_stream()
    results = []

    def timed(name, launch, work, unit):
        for _ in range(2):
            launch()
        torch.cuda.synchronize()
        evs = []
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds or len(evs) < 3:
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record()
            launch()
            e[1].record()
            evs.append(e)
            if len(evs) % 8 == 0:
                evs[-1][1].synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        med = ms[len(ms) // 2]
        r = {"probe": name, "launches": len(evs), "median_ms": med, unit: work / (med * 1e-3)}
        r.update(sampler.window(t0 + 0.25 * (t1 - t0), t1))
        log(f"{name:44s} {med * 1e3:9.1f} us  {r[unit]:.4g} {unit}  "
            f"power {r['power_W']} W  clock {r['gfx_clock_MHz']} MHz")
        results.append(r)

    blocks, iters = 256, 512
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    mfma_flops = blocks * 8 * iters * 32 * 32768.0
    # one second of the first probe, untimed: amdsmi's power average lags, and
    # the chip starts from idle
    ts = time.perf_counter()
    while time.perf_counter() - ts < 1.0:
        plib.fa_probe_mfma(0, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                           ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
    for mode, label in ((0, "MFMA, constant operands"), (1, "MFMA, random operands"),
                        (3, "random MFMA + 1 KB LDS reads per MFMA"),
                        (11, "random MFMA + 1 KB transposed LDS reads per MFMA"),
                        (5, "random MFMA + 1 exp + 4 FMA per MFMA"),
                        (7, "random MFMA + LDS reads + exp/FMA"),
                        (39, "random MFMA + 0.5 KB LDS reads + exp/FMA"),
                        (17, "one wave per SIMD: random MFMA"),
                        (23, "one wave per SIMD: random MFMA + LDS reads + exp/FMA"),
                        (55, "one wave per SIMD: random MFMA + 0.5 KB LDS reads + exp/FMA")):
        timed(label, lambda m=mode: plib.fa_probe_mfma(m, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                                       ctypes.c_void_p(stream.cuda_stream)),
              mfma_flops / 1e12, "TFLOP/s")

    w = synth.WORKLOADS["b1h32n8192d128_causal"]
    x = synth.make_inputs(w, seed=0, device="cuda")
    O = torch.empty_like(x["Q"])
    L = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device="cuda")
    g = [torch.empty_like(x["Q"]) for _ in range(3)]
    ws = torch.empty(fa.bwd_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, fa.FA_BF16), dtype=torch.uint8,
                     device="cuda")
    pairs = unmasked_pairs(w.Nq, w.Nk, w.causal) * w.B * w.H
    fa.fa_fwd(x["Q"], x["K"], x["V"], O, L, w.scale, w.causal)
    fa.fa_bwd(x["Q"], x["K"], x["V"], O, L, x["dO"], *g, w.scale, w.causal, workspace=ws,
              stages=fa.FA_BWD_PREPROCESS)
    timed("fwd_kernel (4*d flop per pair)",
          lambda: fa.fa_fwd(x["Q"], x["K"], x["V"], O, L, w.scale, w.causal), 4 * w.d * pairs / 1e12,
          "TFLOP/s")
    sds = stores_ds(fa, w, fa.FA_BF16)
    timed("bwd_dkdv_kernel (8*d flop per pair)",
          lambda: fa.fa_bwd(x["Q"], x["K"], x["V"], O, L, x["dO"], *g, w.scale, w.causal, workspace=ws,
                            stages=fa.FA_BWD_DKDV), 8 * w.d * pairs / 1e12, "TFLOP/s")
    if sds:  # dQ = scale * dS K from the stored dS: one GEMM
        timed("bwd_dq_ds_kernel (2*d flop per pair)",
              lambda: fa.fa_bwd(x["Q"], x["K"], x["V"], O, L, x["dO"], *g, w.scale, w.causal,
                                workspace=ws, stages=fa.FA_BWD_DQ), 2 * w.d * pairs / 1e12, "TFLOP/s")
    else:
        timed("bwd_dq_kernel (6*d flop per pair executed)",
              lambda: fa.fa_bwd(x["Q"], x["K"], x["V"], O, L, x["dO"], *g, w.scale, w.causal,
                                workspace=ws, stages=fa.FA_BWD_DQ), 6 * w.d * pairs / 1e12, "TFLOP/s")
        timed("bwd_fused_kernel (14*d flop per pair executed)",
              lambda: fa.fa_bwd(x["Q"], x["K"], x["V"], O, L, x["dO"], *g, w.scale, w.causal,
                                workspace=ws, stages=fa.FA_BWD_DKDV | fa.FA_BWD_DQ),
              14 * w.d * pairs / 1e12, "TFLOP/s")
    del x, O, L, g, ws

    nrb, ablocks, aiters = 8192, 2048, 16  # a 128 MiB buffer
    buf = torch.zeros(nrb * 32 * 128, dtype=torch.float32, device="cuda")
    adds = ablocks * aiters * 4096
    for atomic, label in ((0, "fp32 stores, MFMA-tile pattern"), (1, "fp32 atomic adds (device scope)")):
        buf.zero_()
        timed(label, lambda a=atomic: plib.fa_probe_adds(a, ctypes.c_void_p(buf.data_ptr()), nrb, ablocks,
                                                         aiters, ctypes.c_void_p(stream.cuda_stream)),
              adds / 1e9, "G values/s")
        if atomic:
            # every add of 1.0 landed: each element's count stays far below 2^24
            launches = results[-1]["launches"] + 2
            results[-1]["sum_exact"] = bool(buf.double().sum().item() == float(launches) * adds)
    sampler.close()
    print(json.dumps({"probes": results, "power_sampling": sampler.note, "seconds_per_probe": seconds}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="b1h32n8192d128_causal")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="heads of the workload the float64 oracle is timed on (0 = skip)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-shaped forward")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the forward and backward of the other bf16 workloads")
    ap.add_argument("--no-fp16", action="store_true", help="skip the fp16 forward and backward")
    ap.add_argument("--no-bias", action="store_true",
                    help="skip the forward and backward with an additive bias")
    ap.add_argument("--no-dropout", action="store_true",
                    help="skip the forward and backward with dropout")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many "
                         "MiB (reference point for HBM byte counters under rocprofv3 --pmc)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 counter runs and exit")
    ap.add_argument("--probes", type=float, default=0.0, metavar="SECONDS",
                    help="run the machine probes and the attention kernels, each for SECONDS, "
                         "sampling board power and clock, print one JSON line and exit")
    args = ap.parse_args()
    if args.probes > 0:
        run_probes(args.probes)
        return

    if args.write_traffic:
        write_traffic(*args.write_traffic, copy_mib=args.copy_calibration_mib or 1024)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(attention heads shard across GPUs with no communication, so the per-GPU "
              "figure is the one-GPU figure)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_118_amd as fa
    from exact_attention_118_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load_library()
    w = synth.WORKLOADS[args.workload]
    log(f"workload {w}")
    x = synth.make_inputs(w, seed=0, device="cuda")
    Q, K, V, dO = x["Q"], x["K"], x["V"], x["dO"]
    O = torch.empty_like(Q)
    L = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device="cuda")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    ws = torch.empty(fa.bwd_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, fa.FA_BF16),
                     dtype=torch.uint8, device="cuda")
    sds = stores_ds(fa, w, fa.FA_BF16)
    log(f"backward path: {'stored dS' if sds else 'recomputed dQ'}")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(Q, K, V, O, L, w.scale, w.causal)
        if ev is not None:
            ev[1].record()
        fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws,
                  stages=fa.FA_BWD_PREPROCESS)
        if ev is not None:
            ev[2].record()
        if sds:
            # as fa_bwd runs them: dK/dV (storing dS), then dQ from dS
            fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws,
                      stages=fa.FA_BWD_DKDV)
            if ev is not None:
                ev[3].record()
            fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws,
                      stages=fa.FA_BWD_DQ)
        else:
            # dK/dV and dQ: one launch (bwd_fused_kernel), as fa_bwd runs them
            fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws,
                      stages=fa.FA_BWD_DKDV | fa.FA_BWD_DQ)
            if ev is not None:
                ev[3].record()
        if ev is not None:
            ev[4].record()

    sampler = PowerSampler(start=False)  # amdsmi set up now; it samples after the timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(evs[k])
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    ms_per_step = start.elapsed_time(end) / args.steps

    # Board power and GFX clock (amdsmi) while the same step repeats for about
    # 2.5 s after the timed steps: amdsmi's readings trail the chip by up to a
    # second, far longer than the timed steps last, so only the last 60% of
    # that window counts.  Gives the fraction of the peak at the clock the
    # chip actually ran.
    clock = {"note": sampler.note}
    if sampler.ok:
        sampler.start()
        reps = max(1, int(2.5e3 / ms_per_step))
        c0 = time.perf_counter()
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        c1 = time.perf_counter()
        clock = sampler.window(c0 + 0.4 * (c1 - c0), c1)
        clock["window_s"] = 0.6 * (c1 - c0)
    sampler.close()
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f})")

    def mean_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in evs) / len(evs)

    fwd_ms, pre_ms, main_ms = mean_ms(0, 1), mean_ms(1, 2), mean_ms(2, 4)
    kv_ms, q_ms = mean_ms(2, 3), mean_ms(3, 4)  # stored dS: the dK/dV and dQ launches
    bwd_ms = pre_ms + main_ms
    pairs = unmasked_pairs(w.Nq, w.Nk, w.causal) * w.B * w.H
    fwd_flops, bwd_flops = 4 * w.d * pairs, 10 * w.d * pairs
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12

    # The dK/dV and dQ stages, each launched alone (outside the timed steps):
    # how the backward's time splits between them (the halves of the fused
    # launch where dQ is recomputed).
    def alone(stages, reps=5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws, stages=stages)
        e0.record()
        for _ in range(reps):
            fa.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, w.scale, w.causal, workspace=ws,
                      stages=stages)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    dkdv_ms, dq_ms = alone(fa.FA_BWD_DKDV), alone(fa.FA_BWD_DQ)

    # Algorithmic flops per launch: the forward's 2 GEMMs; the S, dP, dV and
    # dK GEMMs of the dK/dV kernel (8*d per pair) and the dQ GEMM (2*d per
    # pair), in two launches with stored dS, else in one fused launch whose
    # dQ workgroups also recompute S and dP (4*d per pair, not algorithmic).
    csrc = os.path.join(ROOT, "exact_attention_118_amd", "csrc")
    src_b = os.path.join(csrc, "fa_bwd.hip")
    kernels = {"fwd_kernel": {"ms": fwd_ms, "flops": fwd_flops,
                              "source": os.path.join(csrc, "fa_fwd.hip")}}
    if sds:
        kernels["bwd_dkdv_kernel"] = {"ms": kv_ms, "flops": 8 * w.d * pairs, "source": src_b}
        kernels["bwd_dq_ds_kernel"] = {"ms": q_ms, "flops": 2 * w.d * pairs, "source": src_b}
    else:
        kernels["bwd_fused_kernel"] = {"ms": main_ms, "flops": 10 * w.d * pairs, "source": src_b}
    dom_name = max(kernels, key=lambda k: kernels[k]["ms"])
    dom = kernels[dom_name]
    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dom_name, dom["source"]),
                "kernel": dom_name, "kernel_ms": dom["ms"]}
    mhz = clock.get("gfx_clock_MHz")
    if mhz:
        # the same peak scaled to the mean GFX clock amdsmi reported over the timed steps
        roofline["frac_at_measured_clock"] = achieved / (PEAK_BF16_TFLOPS * mhz / 2400.0)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.Nq, "d": w.d,
                   "causal": w.causal, "qk_mult": w.qk_mult, "pass": "fwd+bwd"},
        "roofline": roofline,
        "clock": clock,
        "fwd": {"ms": fwd_ms, "TFLOP/s": fwd_flops / (fwd_ms * 1e-3) / 1e12,
                "mfma_frac": fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "bwd": {"ms": bwd_ms, "TFLOP/s": bwd_flops / (bwd_ms * 1e-3) / 1e12,
                "mfma_frac": bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "path": "stored dS" if sds else "recomputed dQ",
                "preprocess_ms": pre_ms, "dkdv_dq_ms": main_ms,
                **({"dkdv_ms": kv_ms, "dq_ms": q_ms} if sds else {}),
                "alone": {"dkdv_ms": dkdv_ms, "dq_ms": dq_ms,
                          "dkdv_TFLOP/s": 8 * w.d * pairs / (dkdv_ms * 1e-3) / 1e12},
                "executed_mfma_frac": (10 if sds else 14) * w.d * pairs / (bwd_ms * 1e-3) / 1e12
                / PEAK_BF16_TFLOPS},
    }
    del dQ, dK, dV
    if not args.no_configs:
        log("other bf16 workloads")
        out["configs"] = bench_other_configs(fa, torch, steps=10)
    if not args.no_fp16:
        log("fp16 inputs, same workload")
        out["fp16"] = bench_fp16(fa, torch, w, x, ws, steps=max(3, args.steps // 2))
    if not args.no_bias:
        log("additive bias [1, H, N, N], same workload")
        out["bias"] = bench_bias(fa, torch, w, x, ws, steps=max(3, args.steps // 2))
    if not args.no_bias:
        log("block-sparse bias (1024-key window) with and without its tile map")
        out["window_bias"] = bench_window(fa, torch, w, x, ws, steps=max(3, args.steps // 2))
    if not args.no_dropout:
        log("dropout p = 0.1, same workload")
        out["dropout"] = bench_dropout(fa, torch, w, x, ws, steps=max(3, args.steps // 2))
    del ws
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")
        del src, dst
    if not args.no_decode:
        log("decode-shaped forward")
        out["decode"] = bench_decode(fa, torch, steps=10)
        log("a few query rows: key splits against the tiled path")
        out["rows_split"] = bench_rows_split(fa, torch, steps=10)
    if args.cpu_heads > 0:
        log(f"float64 oracle on {args.cpu_heads} heads")
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_heads)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
