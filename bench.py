"""Benchmark: causal attention forward TFLOP/s at B=1, H=32, N=8192, D=128, fp16.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

A step is one attn_fwd call (the whole hot path) over the workload, with
inputs resident in HBM.  W untimed steps (continued until at least 0.3 s of
launches have run, past the part's power-management transient after idle),
then K steps timed between two device synchronisations;
value = 2*B*H*N^2*D / (seconds per step) / 1e12.
The FLOP count is the FA page's causal count (section 1 of "CUDA
FlashAttention: from online softmax to long-sequence IO limits").

One JSON line goes to stdout.  Besides the contract fields it carries:
  roofline      achieved TFLOP/s of the attention kernel (events on the
                launch stream around the timed region) against the MI355X dense
                fp16 MFMA peak, and the HBM traffic rocprofv3 measured for the
                same kernel (profiles/attn_fwd_C4_traffic.txt) when that
                measurement was taken on the current kernel source;
  cpu_baseline  the FP64 oracle timed on this host's cores on a bounded
                sample of the same workload (every s-th query row);
  parity_sample max-abs error of the GPU output on those sampled rows;
  clock         GFX clock and socket power (amdsmi) during a ~2.5 s
                sustained run of the same launch after the timed steps, the
                TFLOP/s of that run, and the achieved rate as a fraction of
                the MFMA peak at that clock;
  extra         the other configurations (C1, C2, C3, C5 attention; G1
                grouped-query attention; S1 without and with the key split;
                D1..D32 paged grouped-query decode at 1K..32K tokens; C4 and
                C5 backward;
                R1, R2 row softmax), timed as the median of 7 group means of
                back-to-back launches (FA page, section 8 method); C1, C2,
                C3, C5, R1 and R2 also carry the FP64 oracle's parity on every
                output element and its own timing beside the GPU's.
Runs on one GPU only; --gpus above 1 exits with a message.

    python bench.py --ceiling

prints instead the sustained rate, GFX clock and socket power of the
matrix-core ceiling probe (libosc_ceiling.so: MFMAs alone, with one LDS
fragment read each, and with the softmax's per-score VALU work added) and of
the C4 attention forward, each run back to back for a few seconds in the same
process: under sustained MFMA load the firmware sets the clock by power and
activity, so these are the rates the part sustains for each instruction mix.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6      # MI355X dense fp16/bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "online_softmax_causal_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_C4_traffic.txt")
COPY_BYTES = 1 << 30          # calibration copy: 1 GiB read + 1 GiB written
WARMUP_MIN_S = 0.3            # warm-up runs at least this long (see main)


def kernel_source_hash(names=("attn_fwd.hip", "mfma_tile.hpp", "online_merge.hpp")) -> str:
    """Short SHA-256 of kernel sources (by default the attention kernel's)."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "online_softmax_causal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if it is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


GRAPH_BELOW_MS = 0.2


def time_groups(fn, stream, groups=7, min_ms=2.0, info=None):
    """Median (and min) over 7 groups of the mean time of R back-to-back calls (ms).

    Calls shorter than GRAPH_BELOW_MS are also captured R at a time into a HIP
    graph (torch.cuda.CUDAGraph) and replayed: the median of those per-call
    times is then the result, since a Python loop of calls that short times
    the host, not the GPU.  `info` (a dict) receives both figures."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-6) * 1e3
    reps = max(5, int(min_ms / one) + 1)

    def run_groups(body, per):
        means = []
        for _ in range(groups):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            body()
            b.record(stream)
            b.synchronize()
            means.append(a.elapsed_time(b) / per)
        means.sort()
        return means[len(means) // 2], means[0]

    def loop():
        for _ in range(reps):
            fn()

    med, mn = run_groups(loop, reps)
    if info is not None:
        info["ms_eager"] = round(med, 5)
    if med < GRAPH_BELOW_MS:
        r = max(10, min(reps, 200))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(r):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        med, mn = run_groups(g.replay, r)
        if info is not None:
            info["ms_graph"] = round(med, 5)
            info["timing"] = "HIP graph of %d calls, replayed" % r
        del g
    return med, mn


def extra_configs(dev, with_oracle=True):
    import torch
    import online_softmax_causal_amd as osc
    import workloads
    out = {}
    oracle_cfgs = ("C1", "C2", "C3", "C5") if with_oracle else ()
    stream = torch.cuda.current_stream()
    for name in ("C1", "C2", "C3", "C5", "F1K", "F2K", "F4K"):
        w = workloads.ATTN[name] if name in workloads.ATTN else workloads.SWEEP[name]
        q, k, v = (t.to(dev) for t in workloads.workload_inputs(w))
        o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        fn = lambda: osc.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.D, w.causal, w.dtype)
        info = {}
        med, mn = time_groups(fn, stream, info=info)
        tf = w.flops / (med * 1e-3) / 1e12
        out[name] = {"workload": w.describe(), "ms": round(med, 5), "ms_min": round(mn, 5),
                     "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4)}
        out[name].update(info)
        if name in oracle_cfgs:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            fn()
            torch.cuda.synchronize()
            base, parity = oracle_full(w, [t.cpu() for t in (q, k, v)],
                                       (o.cpu().double().numpy(), lse.cpu().double().numpy()))
            out[name]["parity"] = parity
            out[name]["cpu_baseline"] = base
        del q, k, v, o, lse
    # Grouped-query attention (K/V heads shared by groups of query heads).
    w = workloads.GQA["G1"]
    q, k, v = (t.to(dev) for t in workloads.workload_inputs(w))
    o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    fn = lambda: osc.attn_fwd_gqa(q, k, v, o, lse, w.B, w.H, w.Hkv, w.N, w.D, w.causal, w.dtype)
    med, mn = time_groups(fn, stream)
    tf = w.flops / (med * 1e-3) / 1e12
    out["G1"] = {"workload": w.describe(), "entry": "attn_fwd_gqa", "ms": round(med, 5),
                 "ms_min": round(mn, 5), "tflops": round(tf, 2),
                 "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4)}
    del q, k, v, o, lse
    # Long sequence, few heads: plain launch against the automatic key split
    # (both kernels, attention and merge, inside the timed region).
    w = workloads.SPLITKV["S1"]
    q, k, v = (t.to(dev) for t in workloads.workload_inputs(w))
    o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    need = osc.attn_fwd_splitkv_workspace(w.B, w.H, w.N, w.D, w.causal, 0)
    ws = torch.empty((max(need, 16) // 4,), dtype=torch.float32, device=dev)
    for entry, fn in (
            ("attn_fwd", lambda: osc.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.D, w.causal,
                                              w.dtype)),
            ("attn_fwd_splitkv", lambda: osc.attn_fwd_splitkv(q, k, v, o, lse, w.B, w.H, w.H, w.N,
                                                              w.D, w.causal, w.dtype, 0, ws,
                                                              need))):
        med, mn = time_groups(fn, stream)
        tf = w.flops / (med * 1e-3) / 1e12
        out["S1 " + entry] = {"workload": w.describe(), "entry": entry, "ms": round(med, 5),
                              "ms_min": round(mn, 5), "tflops": round(tf, 2),
                              "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4),
                              "workspace_bytes": need if entry != "attn_fwd" else 0}
    del q, k, v, o, lse, ws
    # Backward of the headline workload (and of C5): algorithmic FLOP 2.5x the
    # forward's (5 BHN^2D causal, 10 BHN^2D non-causal: the five N x N x D
    # products dQ, dK, dV, dP and S); all three kernels inside the timed region.
    for name in ("C4", "C5"):
        w = workloads.ATTN[name]
        q, k, v, do = (t.to(dev) for t in workloads.bwd_inputs(w.B, w.H, w.N, w.D, w.dtype, w.seed,
                                                               w.sigma_qk, w.sigma_v))
        o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        osc.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.D, w.causal, w.dtype)
        dq, dk, dv = (torch.empty_like(o) for _ in range(3))
        need = osc.attn_bwd_workspace(w.B, w.H, w.N)
        ws = torch.empty((need // 4,), dtype=torch.float32, device=dev)
        fn = lambda: osc.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, w.B, w.H, w.N, w.D, w.causal,
                                  w.dtype, ws, need)
        med, mn = time_groups(fn, stream)
        tf = 2.5 * w.flops / (med * 1e-3) / 1e12
        out[name + " bwd"] = {"workload": w.describe().replace("fwd", "bwd"), "entry": "attn_bwd",
                              "ms": round(med, 5), "ms_min": round(mn, 5), "tflops": round(tf, 2),
                              "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4)}
        del q, k, v, do, o, lse, dq, dk, dv, ws
    # Backward with grouped K/V heads (G1): same algorithmic FLOP as the
    # per-query-head backward (dK, dV of a shared head sum over its group).
    w = workloads.GQA["G1"]
    q, k, v, do = (t.to(dev) for t in workloads.bwd_gqa_inputs(w.B, w.H, w.Hkv, w.N, w.D, w.dtype,
                                                               w.seed))
    o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    osc.attn_fwd_gqa(q, k, v, o, lse, w.B, w.H, w.Hkv, w.N, w.D, w.causal, w.dtype)
    dq = torch.empty_like(o)
    dk, dv = (torch.empty((w.B, w.Hkv, w.N, w.D), dtype=torch.float32, device=dev) for _ in range(2))
    need = osc.attn_bwd_workspace(w.B, w.H, w.N)
    ws = torch.empty((need // 4,), dtype=torch.float32, device=dev)
    fn = lambda: osc.attn_bwd_gqa(q, k, v, o, lse, do, dq, dk, dv, w.B, w.H, w.Hkv, w.N, w.D,
                                  w.causal, w.dtype, ws, need)
    med, mn = time_groups(fn, stream)
    tf = 2.5 * w.flops / (med * 1e-3) / 1e12
    out["G1 bwd"] = {"workload": w.describe().replace("fwd", "bwd"), "entry": "attn_bwd_gqa",
                     "ms": round(med, 5), "ms_min": round(mn, 5), "tflops": round(tf, 2),
                     "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4)}
    del q, k, v, do, o, lse, dq, dk, dv, ws
    # Paged grouped-query decode (KV page, section 8 shapes), automatic split;
    # attention kernel and merge inside the timed region.  HBM-bound: GB/s of
    # algorithmic bytes (K and V of every cached token once, q, o, lse).
    for name, w in workloads.DECODE.items():
        q, cache, bt, ln = (t.to(dev) for t in workloads.decode_workload_inputs(w))
        o = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
        need = osc.paged_decode_workspace(w.B, w.Hq, w.Hkv, w.D, w.page_size, w.max_pages, 0)
        ws = torch.empty((max(need, 16) // 4,), dtype=torch.float32, device=dev)
        fn = lambda: osc.paged_decode(q, cache, bt, ln, o, lse, w.B, w.Hq, w.Hkv, w.D,
                                      w.page_size, w.num_pages, w.max_pages, w.dtype, 0, ws, need)
        info = {}
        med, mn = time_groups(fn, stream, info=info)
        gbs = w.bytes / (med * 1e-3) / 1e9
        out[name] = {"workload": w.describe(), "entry": "paged_decode", "ms": round(med, 5),
                     "ms_min": round(mn, 5), "gbs": round(gbs, 1),
                     "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "workspace_bytes": need}
        out[name].update(info)
        del q, cache, bt, ln, o, lse, ws
    for name in ("R1", "R2"):
        w = workloads.SOFTMAX[name]
        x = workloads.softmax_inputs(w.M, w.N, seed=w.seed, last=w.last).to(dev)
        y = torch.empty_like(x)
        fn = lambda: osc.row_softmax(x, y, w.M, w.N)
        info = {}
        med, mn = time_groups(fn, stream, info=info)
        gbs = w.bytes / (med * 1e-3) / 1e9
        out[name] = {"workload": w.describe(), "ms": round(med, 5), "ms_min": round(mn, 5),
                     "gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
        out[name].update(info)
        if with_oracle:
            y.fill_(float("nan"))
            fn()
            torch.cuda.synchronize()
            base, parity = oracle_full(w, [x.cpu()], (y.cpu().double().numpy(),))
            out[name]["parity"] = parity
            out[name]["cpu_baseline"] = base
        del x, y
    return out


def host_info():
    """Host cores and CPU model (the oracle runs on at most 16 threads, the
    CPU share a GPU of this machine is given)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"host_cores": os.cpu_count(), "affinity_cores": affinity, "cpu_model": model}


def oracle_full(w, inputs, gpu_out):
    """Run the FP64 oracle on a whole workload: its time, throughput and the
    max-abs error of the GPU output on every element."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    if hasattr(w, "M"):   # row softmax
        (x,) = inputs
        y_ref = oracle.row_softmax(x, nthreads=threads)
        secs = time.perf_counter() - t0
        (y,) = gpu_out
        parity = {"elements": int(y_ref.size), "max_abs_y": float(np.abs(y - y_ref).max())}
        base = {"value": round(w.bytes / secs / 1e9, 4), "unit": "GB/s", "seconds": round(secs, 3)}
    else:
        q, k, v = inputs
        if w.Hkv is not None:
            o_ref, lse_ref = oracle.attn_fwd_gqa(q, k, v, w.causal, nthreads=threads)
        else:
            o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, nthreads=threads)
        secs = time.perf_counter() - t0
        o, lse = gpu_out
        parity = {"rows": int(lse_ref.size), "max_abs_o": float(np.abs(o - o_ref).max()),
                  "max_abs_lse": float(np.abs(lse - lse_ref).max())}
        base = {"value": round(w.flops / secs / 1e12, 6), "unit": "TFLOP/s", "seconds": round(secs, 3)}
    base.update({"cores": threads, "kind": "oracle", "sample": "whole workload"})
    return base, parity


def measure_clock(step, flops, seconds=2.5):
    """Run `step` back to back for `seconds`, sampling the GFX clock and the
    socket power with amdsmi; averages over the last 60% of the run.  Returns
    None if amdsmi is not usable."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
        amdsmi.amdsmi_get_gpu_metrics_info(handle)
    except Exception:
        return None
    samples, stop = [], [False]

    def sample():
        while not stop[0]:
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
                samples.append((time.perf_counter(), sum(clks) / len(clks) if clks else None,
                                m.get("current_socket_power")))
            except Exception:
                pass
            time.sleep(0.05)

    th = threading.Thread(target=sample)
    th.start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    e1.record()
    e1.synchronize()
    stop[0] = True
    th.join()
    ms = e0.elapsed_time(e1) / n
    late = [x for x in samples if x[0] > t0 + 0.4 * seconds and x[1] is not None]
    if not late:
        return None
    mhz = sum(x[1] for x in late) / len(late)
    watts = [x[2] for x in late if isinstance(x[2], (int, float))]
    tflops = flops / (ms * 1e-3) / 1e12
    # MFMA peak at the measured clock: 256 CU x 4096 FLOP per clock.
    peak_at_clock = 256 * 4096 * mhz * 1e6 / 1e12
    return {"clock_mhz": round(mhz, 1), "power_w": round(sum(watts) / len(watts), 1) if watts else None,
            "sustained_ms": round(ms, 5), "sustained_tflops": round(tflops, 2),
            "peak_at_clock_tflops": round(peak_at_clock, 1),
            "frac_of_peak_at_clock": round(tflops / peak_at_clock, 4),
            "launches": n, "samples": len(late),
            "source": "amdsmi current_gfxclks (mean over 8 XCDs) and current_socket_power"}


def cpu_baseline(w, q, k, v, o_gpu, lse_gpu, target_s=15.0):
    """Time the FP64 oracle on every s-th query row of the workload.

    A calibration run on a small sample fixes s so the timed sample takes
    about target_s seconds.  FLOP of a sample are counted row by row with the
    same convention as the metric: a causal row i costs 4*(i+1)*D.
    """
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    qd, kd, vd = oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)
    total_rows = w.B * w.H * w.N

    def row_flops(rows):
        i = np.asarray(rows) % w.N
        keys = (i + 1) if w.causal else np.full_like(i, w.N)
        return float((4.0 * keys * w.D).sum())

    def run(stride):
        rows = np.arange(stride // 2, total_rows, stride, dtype=np.int64)
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attn_rows(qd, kd, vd, w.causal, rows, nthreads=threads)
        return rows, time.perf_counter() - t0, o_ref, lse_ref

    stride = 1024
    rows, secs, _, _ = run(stride)
    rate = row_flops(rows) / secs
    want = rate * target_s
    stride = int(max(1, min(total_rows, round(row_flops(range(total_rows)) / want))))
    rows, secs, o_ref, lse_ref = run(stride)
    flops = row_flops(rows)
    o_rows = o_gpu.reshape(-1, w.D)[rows]
    lse_rows = lse_gpu.reshape(-1)[rows]
    parity = {"rows": int(len(rows)),
              "max_abs_o": float(np.abs(o_rows - o_ref).max()),
              "max_abs_lse": float(np.abs(lse_rows - lse_ref).max())}
    base = {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", **host_info(),
            "sample": "%d of %d query rows (every %d-th flat row of %s), %.3g FLOP in %.1f s, "
                      "FP64 three-stage oracle" % (len(rows), total_rows, stride, w.describe(),
                                                   flops, secs)}
    return base, parity


def _launcher(name, dev):
    """A closure launching workload `name` (C1-C5, F*, G1 attention; R1, R2 row
    softmax) on resident inputs, and the kernel-name test that picks its
    dispatches out of a profile."""
    import torch
    import online_softmax_causal_amd as osc
    import workloads
    if name in workloads.SOFTMAX:
        w = workloads.SOFTMAX[name]
        x = workloads.softmax_inputs(w.M, w.N, seed=w.seed, last=w.last).to(dev)
        y = torch.empty_like(x)
        return w, (lambda: osc.row_softmax(x, y, w.M, w.N)), (lambda n: "softmax" in n)
    w = workloads.ATTN.get(name) or workloads.SWEEP.get(name) or workloads.GQA.get(name)
    q, k, v = (t.to(dev) for t in workloads.workload_inputs(w))
    o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    hkv = w.H if w.Hkv is None else w.Hkv
    return w, (lambda: osc.attn_fwd_gqa(q, k, v, o, lse, w.B, w.H, hkv, w.N, w.D, w.causal,
                                        w.dtype)), is_fwd_kernel


def profile_pass(name="C4"):
    """The program rocprofv3 wraps for the counter passes: 3 launches of
    workload `name`, then 3 plain device copies of COPY_BYTES (torch's copy
    kernel) whose HBM traffic is known (read COPY_BYTES, write COPY_BYTES)."""
    import torch
    dev = torch.device("cuda:0")
    _, fn, _ = _launcher(name, dev)
    for _ in range(3):
        fn()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profile pass done:", name, flush=True)


def profile_launches(name, launches=20):
    """Launch workload `name` `launches` times (the rocprofv3 kernel-trace target)."""
    import torch
    dev = torch.device("cuda:0")
    w, fn, _ = _launcher(name, dev)
    for _ in range(launches):
        fn()
    torch.cuda.synchronize()
    print("launches:", launches, w.describe(), flush=True)


def profile_decode(launches=30):
    """Launch the 32K-context paged decode `launches` times (for rocprofv3)."""
    import torch
    import online_softmax_causal_amd as osc
    import workloads
    dev = torch.device("cuda:0")
    w = workloads.DECODE["D32"]
    q, cache, bt, ln = (t.to(dev) for t in workloads.decode_workload_inputs(w))
    o = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    need = osc.paged_decode_workspace(w.B, w.Hq, w.Hkv, w.D, w.page_size, w.max_pages, 0)
    ws = torch.empty((max(need, 16) // 4,), dtype=torch.float32, device=dev)
    for _ in range(launches):
        osc.paged_decode(q, cache, bt, ln, o, lse, w.B, w.Hq, w.Hkv, w.D, w.page_size,
                         w.num_pages, w.max_pages, w.dtype, 0, ws, need)
    torch.cuda.synchronize()
    print("decode launches:", launches, w.describe(), "algorithmic bytes per launch", w.bytes)


def profile_bwd(launches=10):
    """One forward, then `launches` backward calls of the headline workload (for rocprofv3)."""
    import torch
    import online_softmax_causal_amd as osc
    import workloads
    dev = torch.device("cuda:0")
    w = workloads.ATTN["C4"]
    q, k, v, do = (t.to(dev) for t in workloads.bwd_inputs(w.B, w.H, w.N, w.D, w.dtype, w.seed))
    o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    osc.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.D, w.causal, w.dtype)
    dq, dk, dv = (torch.empty_like(o) for _ in range(3))
    need = osc.attn_bwd_workspace(w.B, w.H, w.N)
    ws = torch.empty((need // 4,), dtype=torch.float32, device=dev)
    for _ in range(launches):
        osc.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, w.B, w.H, w.N, w.D, w.causal, w.dtype, ws,
                     need)
    torch.cuda.synchronize()
    print("backward launches:", launches, w.describe().replace("fwd", "bwd"),
          "algorithmic FLOP per launch", 2.5 * w.flops)


def ceiling(seconds=3.0, pairs=2000):
    """Sustained TFLOP/s, clock and power of the ceiling probe's seven mixes,
    of attn_fwd on C4 and C5 and attn_bwd on C4, the LDS read probe, then the
    HBM probes beside row_softmax (R2) and paged_decode (D32), one after the
    other in this process."""
    import ctypes
    import torch
    import online_softmax_causal_amd as osc
    import workloads
    path = os.path.join(ROOT, "online_softmax_causal_amd", "libosc_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit("%s is missing: run python -m online_softmax_causal_amd.build" % path)
    lib = ctypes.CDLL(path)
    lib.osc_ceiling_src_bytes.restype = ctypes.c_int64
    lib.osc_ceiling_mfma_per_wg_iter.restype = ctypes.c_int
    lib.osc_ceiling_mfma_per_wg_iter.argtypes = [ctypes.c_int]
    lib.osc_ceiling_launch.restype = ctypes.c_int
    lib.osc_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(7)
    n16 = lib.osc_ceiling_src_bytes() // 2
    src = (torch.rand(n16, generator=gen) * 4.0 - 2.0).to(torch.float16).to(dev)
    grid = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(grid * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    mixes = ((0, "MFMA only (v_mfma_f32_32x32x16_f16, random fp16 operands)"),
             (1, "MFMA + one 1 KiB LDS fragment read per MFMA per wave"),
             (2, "MFMA + LDS read + fma, exp2, add, 1/2 fp16 pack per MFMA"),
             (3, "MFMA + LDS read + 2 x (fma, exp2, add), 1 fp16 pack per MFMA"),
             (4, "mix 2 at one wave per SIMD"),
             (5, "mix 2 at one wave per SIMD, each LDS fragment feeding two MFMAs"),
             (6, "mix 2 in phases: a step's 16 MFMAs, then its 16 values (two waves per SIMD)"))
    rows = []
    for mix, desc in mixes:
        flops = float(grid) * lib.osc_ceiling_mfma_per_wg_iter(mix) * pairs * 32768.0
        def step(mix=mix):
            e = lib.osc_ceiling_launch(mix, src.data_ptr(), out.data_ptr(), grid, pairs, stream)
            if e != 0:
                raise RuntimeError("ceiling probe launch failed: %d" % e)
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        rows.append((desc, measure_clock(step, flops, seconds)))
    for name in ("C4", "C5"):
        w = workloads.ATTN[name]
        q, k, v = (t.to(dev) for t in workloads.workload_inputs(w))
        o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def attn(w=w, q=q, k=k, v=v, o=o, lse=lse):
            osc.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.D, w.causal, w.dtype)
        for _ in range(20):
            attn()
        torch.cuda.synchronize()
        rows.append(("attn_fwd " + w.describe(), measure_clock(attn, w.flops, seconds)))
        del q, k, v, o, lse
    # C4 backward: algorithmic FLOP (five products, 2.5x the forward's).
    w = workloads.ATTN["C4"]
    q, k, v, do = (t.to(dev) for t in workloads.bwd_inputs(w.B, w.H, w.N, w.D, w.dtype, w.seed))
    o = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    osc.attn_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.D, w.causal, w.dtype)
    grads = [torch.empty_like(o) for _ in range(3)]
    need = osc.attn_bwd_workspace(w.B, w.H, w.N)
    ws = torch.empty((need // 4,), dtype=torch.float32, device=dev)

    def bwd():
        osc.attn_bwd(q, k, v, o, lse, do, *grads, w.B, w.H, w.N, w.D, w.causal, w.dtype, ws, need)
    for _ in range(3):
        bwd()
    torch.cuda.synchronize()
    rows.append(("attn_bwd " + w.describe().replace("fwd", "bwd") + " (algorithmic FLOP)",
                 measure_clock(bwd, 2.5 * w.flops, seconds)))
    del q, k, v, do, o, lse, grads, ws

    # LDS: fragment reads alone, 16 KiB per wave and iteration; bytes per
    # clock per CU at the sampled clock.
    lib.osc_lds_read_launch.restype = ctypes.c_int
    lib.osc_lds_read_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lout = torch.empty(grid * 512, dtype=torch.int32, device=dev)
    lds_rows = []
    for tr, waves, desc in ((0, 8, "ds_read_b128 rows, two waves per SIMD"),
                            (0, 4, "ds_read_b128 rows, one wave per SIMD"),
                            (1, 8, "ds_read_b64_tr_b16 pairs (V^T fragments), two waves per SIMD"),
                            (1, 4, "ds_read_b64_tr_b16 pairs (V^T fragments), one wave per SIMD")):
        iters = 4000

        def lread(tr=tr, waves=waves, iters=iters):
            e = lib.osc_lds_read_launch(tr, waves, src.data_ptr(), lout.data_ptr(), grid, iters, stream)
            if e != 0:
                raise RuntimeError("LDS probe launch failed: %d" % e)
        for _ in range(5):
            lread()
        torch.cuda.synchronize()
        lds_rows.append((desc, measure_clock(lread, float(grid) * waves * iters * 16384.0, seconds)))
    del lout

    # HBM: streaming read and copy of 1 GiB, then the row softmax (R2) and the
    # 32K-token paged decode (D32), each timed the same way (bytes per second).
    lib.osc_hbm_read_launch.restype = ctypes.c_int
    lib.osc_hbm_read_launch.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    lib.osc_hbm_copy_launch.restype = ctypes.c_int
    lib.osc_hbm_copy_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_void_p]
    nbytes = 1 << 30
    hsrc = torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device=dev)
    hdst = torch.empty_like(hsrc)
    hout = torch.empty(grid * 4 * 256, dtype=torch.int32, device=dev)
    hbm_rows = []

    def hread():  # 4 workgroups per CU
        e = lib.osc_hbm_read_launch(hsrc.data_ptr(), nbytes, hout.data_ptr(), grid * 4, stream)
        if e != 0:
            raise RuntimeError("HBM read probe launch failed: %d" % e)

    def hcopy():  # 2 workgroups per CU
        e = lib.osc_hbm_copy_launch(hsrc.data_ptr(), hdst.data_ptr(), nbytes, grid * 2, stream)
        if e != 0:
            raise RuntimeError("HBM copy probe launch failed: %d" % e)
    for desc, fn, moved in (("streaming read, 16-byte non-temporal loads (1 GiB)", hread, nbytes),
                            ("streaming copy, 16-byte non-temporal loads and stores (1 GiB each way)",
                             hcopy, 2 * nbytes)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        hbm_rows.append((desc, measure_clock(fn, moved, seconds)))
    del hsrc, hdst, hout
    sw = workloads.SOFTMAX["R2"]
    x = workloads.softmax_inputs(sw.M, sw.N, seed=sw.seed, last=sw.last).to(dev)
    y = torch.empty_like(x)

    def smax():
        osc.row_softmax(x, y, sw.M, sw.N)
    for _ in range(5):
        smax()
    torch.cuda.synchronize()
    hbm_rows.append((sw.describe() + " (read + write)", measure_clock(smax, 8.0 * sw.M * sw.N, seconds)))
    del x, y
    dw = workloads.DECODE["D32"]
    dq, cache, bt, ln = (t.to(dev) for t in workloads.decode_workload_inputs(dw))
    do_ = torch.empty((dw.B, dw.Hq, dw.D), dtype=torch.float32, device=dev)
    dl = torch.empty((dw.B, dw.Hq), dtype=torch.float32, device=dev)
    dneed = osc.paged_decode_workspace(dw.B, dw.Hq, dw.Hkv, dw.D, dw.page_size, dw.max_pages, 0)
    dws = torch.empty((max(dneed, 16) // 4,), dtype=torch.float32, device=dev)

    def dec():
        osc.paged_decode(dq, cache, bt, ln, do_, dl, dw.B, dw.Hq, dw.Hkv, dw.D, dw.page_size,
                         dw.num_pages, dw.max_pages, dw.dtype, 0, dws, dneed)
    for _ in range(5):
        dec()
    torch.cuda.synchronize()
    hbm_rows.append((dw.describe() + " (reads)", measure_clock(dec, float(dw.bytes), seconds)))
    print("sustained matrix-core rate per instruction mix: %.1f s back-to-back runs, amdsmi sampling"
          % seconds)
    print("probe grid %d workgroups x 8 waves (4 for mixes 4 and 5), %d iterations of 32 MFMAs per wave per launch"
          % (grid, pairs))
    print("")
    print("workload | TFLOP/s | % of 2516.6 | GFX MHz | W | % of peak at that clock")
    for desc, c in rows:
        if c is None:
            print("%s | (amdsmi unavailable)" % desc)
            continue
        print("%s | %.1f | %.1f | %.0f | %.0f | %.1f" % (
            desc, c["sustained_tflops"], 100.0 * c["sustained_tflops"] / PEAK_F16_TFLOPS, c["clock_mhz"],
            c["power_w"] or float("nan"), 100.0 * c["frac_of_peak_at_clock"]))
    print("")
    print("LDS fragment reads alone | B per clock per CU | GFX MHz | W")
    for desc, c in lds_rows:
        if c is None:
            print("%s | (amdsmi unavailable)" % desc)
            continue
        bpc = c["sustained_tflops"] * 1e12 / (256 * c["clock_mhz"] * 1e6)
        print("%s | %.0f | %.0f | %.0f" % (desc, bpc, c["clock_mhz"], c["power_w"] or 0))
    print("")
    print("workload | TB/s | % of 8 TB/s | GFX MHz | W")
    for desc, c in hbm_rows:
        if c is None:
            print("%s | (amdsmi unavailable)" % desc)
            continue
        print("%s | %.2f | %.1f | %.0f | %.0f" % (
            desc, c["sustained_tflops"], 100.0 * c["sustained_tflops"] / (PEAK_HBM_GBS / 1000.0),
            c["clock_mhz"], c["power_w"] or float("nan")))
    print("")
    print("sources_sha256_16: ceiling.hip %s, attn_fwd.hip+mfma_tile.hpp+online_merge.hpp %s, "
          "row_softmax.hip %s, decode.hip %s"
          % (kernel_source_hash(("ceiling.hip",)), kernel_source_hash(),
             kernel_source_hash(("row_softmax.hip",)), kernel_source_hash(("decode.hip", "decode_short.hip", "decode_kernel.hpp"))))


def _pmc_rows(path):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % path)
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter, match):
    vals = {}
    for r in rows:
        if r.get("Counter_Name") == counter and match(r.get("Kernel_Name", "")):
            vals.setdefault(r.get("Dispatch_Id"), 0.0)
            vals[r.get("Dispatch_Id")] += float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=lambda x: int(x))]


def is_fwd_kernel(name: str) -> bool:
    """The attention forward kernels (8-wave pipeline kernel at D = 128, 8-wave unit kernel at
    D = 64, 4-wave ring kernel, key-split kernel)."""
    return any(k in name for k in ("attn_fwd_pipe_kernel", "attn_fwd_units_kernel", "attn_fwd_kernel",
                                   "attn_fwd_ksplit_kernel"))


def traffic_path(name):
    return TRAFFIC_FILE if name == "C4" else os.path.join(ROOT, "profiles", "%s_%s_traffic.txt" % (
        "row_softmax" if name.startswith("R") else "attn_fwd", name))


def summarize_traffic(fetch_dir, write_dir, cmd_fetch, cmd_write, name="C4"):
    """Write profiles/<kernel>_<name>_traffic.txt from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE) of --profile-pass <name>."""
    import workloads
    from types import SimpleNamespace
    if name in workloads.SOFTMAX:
        w = workloads.SOFTMAX[name]
        is_k = lambda n: "softmax" in n
        compulsory = w.bytes
        what = "row_softmax, " + w.describe()
        srcs = ("row_softmax.hip", "online_merge.hpp")
    else:
        w = workloads.ATTN.get(name) or workloads.SWEEP.get(name) or workloads.GQA.get(name)
        is_k = is_fwd_kernel
        hkv = w.H if w.Hkv is None else w.Hkv
        compulsory = (w.B * w.H + 2 * w.B * hkv) * w.N * w.D * 2 + w.B * w.H * w.N * (w.D + 1) * 4
        what = "attention forward, " + w.describe()
        srcs = ("attn_fwd.hip", "mfma_tile.hpp", "online_merge.hpp")
    is_copy = lambda n: not is_k(n)
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    a_fetch = _per_dispatch(fr, "FETCH_SIZE", is_k)
    c_fetch = _per_dispatch(fr, "FETCH_SIZE", is_copy)
    a_write = _per_dispatch(wr, "WRITE_SIZE", is_k)
    c_write = _per_dispatch(wr, "WRITE_SIZE", is_copy)
    # steady-state launches: skip the first of each kind
    mean = lambda xs: sum(xs[1:]) / max(1, len(xs) - 1) if len(xs) > 1 else xs[0]
    kib_c_fetch, kib_c_write = mean(c_fetch[-3:]), mean(c_write[-3:])
    f_scale = COPY_BYTES / (kib_c_fetch * 1024.0)
    w_scale = COPY_BYTES / (kib_c_write * 1024.0)
    a_read = mean(a_fetch) * 1024.0 * f_scale
    a_written = mean(a_write) * 1024.0 * w_scale
    text = "\n".join([
        "%s: HBM traffic per launch (rocprofv3 --pmc)" % what,
        "",
        "commands (from the repository root, TMPDIR=/tmp):",
        "  " + cmd_fetch,
        "  " + cmd_write,
        "  python bench.py --summarize-traffic <fetch_dir> <write_dir> --cfg %s" % name,
        "",
        "kernel FETCH_SIZE per dispatch (KiB): " + ", ".join("%.0f" % x for x in a_fetch),
        "kernel WRITE_SIZE per dispatch (KiB): " + ", ".join("%.0f" % x for x in a_write),
        "copy kernel (%d bytes read + %d written) FETCH_SIZE (KiB): %s" % (
            COPY_BYTES, COPY_BYTES, ", ".join("%.0f" % x for x in c_fetch)),
        "copy kernel WRITE_SIZE (KiB): " + ", ".join("%.0f" % x for x in c_write),
        "calibration: read scale %.4f, write scale %.4f (known bytes / counter bytes of the copy)" % (
            f_scale, w_scale),
        "",
        "hbm_read_bytes_per_launch: %.6g" % a_read,
        "hbm_write_bytes_per_launch: %.6g" % a_written,
        "hbm_bytes_per_launch: %.6g" % (a_read + a_written),
        "compulsory_bytes (inputs read once, outputs written once): %.6g" % compulsory,
        "traffic / compulsory: %.3f" % ((a_read + a_written) / compulsory),
        "kernel_source_sha256_16: %s" % kernel_source_hash(srcs),
        "",
    ])
    with open(traffic_path(name), "w") as f:
        f.write(text)
    print(text)


def summarize_sq(dirs, out_path, cmds, name="C4"):
    """Write profiles/attn_fwd_<name>_sq_counters.txt from rocprofv3 --pmc SQ
    passes of --profile-pass <name>."""
    import statistics
    import workloads
    w = workloads.ATTN.get(name) or workloads.SWEEP.get(name) or workloads.GQA.get(name)
    vals, kern = {}, set()
    for d in dirs:
        rows = _pmc_rows(d)
        for r in rows:
            if is_fwd_kernel(r["Kernel_Name"]):
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                kern.add(r["Kernel_Name"].split("(")[0][:90])
    med = {k: statistics.median(v) for k, v in vals.items()}
    simds, xcds = 256 * 4, 8
    lines = ["attention forward, %s: SQ counters per dispatch (rocprofv3 --pmc)" % w.describe(),
             "kernel: " + ", ".join(sorted(kern)), "", "commands (from the repository root, TMPDIR=/tmp):"]
    lines += ["  " + c for c in cmds]
    lines += ["", "counter | per dispatch | median"]
    for k in sorted(vals):
        lines.append("%s | %s | %.5g" % (k, ", ".join("%.5g" % x for x in vals[k]), med[k]))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
        cycles = med["GRBM_GUI_ACTIVE"] / xcds
        util = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cycles)
        lines += ["",
                  "GPU cycles per dispatch = GRBM_GUI_ACTIVE / 8 XCDs = %.4g" % cycles,
                  "MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles) = %.3f" % util,
                  "algorithmic FLOP / MFMA busy FLOP = %.3f" % (
                      w.flops / (med["SQ_VALU_MFMA_BUSY_CYCLES"] * 1024.0))]
    if "SQ_INSTS_MFMA" in med and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
        lines.append("busy cycles per MFMA instruction = %.2f (v_mfma_f32_32x32x16: 32)"
                     % (med["SQ_VALU_MFMA_BUSY_CYCLES"] / med["SQ_INSTS_MFMA"]))
    if med.get("SQ_INSTS_MFMA"):
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            if k in med:
                lines.append("%s per MFMA instruction = %.2f" % (k, med[k] / med["SQ_INSTS_MFMA"]))
    lines.append("kernel_source_sha256_16: %s" % kernel_source_hash())
    lines.append("")
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarize_sq_bwd(dirs, out_path, cmds):
    """Write profiles/attn_bwd_C4_sq_counters.txt from rocprofv3 --pmc SQ passes of --profile-bwd."""
    import re
    import statistics
    vals = {}
    for d in dirs:
        for r in _pmc_rows(d):
            m = re.search(r"::(attn_bwd_\w+?)<", r["Kernel_Name"])
            if m:
                vals.setdefault((m.group(1), r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    lines = ["attention backward kernels, causal fp16 B1 H32 N8192 D128: SQ counters per dispatch "
             "(rocprofv3 --pmc)", "", "commands (from the repository root, TMPDIR=/tmp):"]
    lines += ["  " + c for c in cmds]
    simds, xcds = 256 * 4, 8
    for kernel in sorted({k for k, _ in vals}):
        med = {c: statistics.median(v) for (k, c), v in vals.items() if k == kernel}
        lines += ["", "%s: counter | median over %d dispatches" % (
            kernel, len(next(v for (k, _), v in vals.items() if k == kernel)))]
        for c in sorted(med):
            lines.append("  %s | %.5g" % (c, med[c]))
        if "GRBM_GUI_ACTIVE" in med and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            cycles = med["GRBM_GUI_ACTIVE"] / xcds
            lines.append("  MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x %.4g cycles) = %.3f"
                         % (cycles, med["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cycles)))
        if med.get("SQ_INSTS_MFMA"):
            lines.append("  VALU instructions per MFMA = %.2f" % (med["SQ_INSTS_VALU"] / med["SQ_INSTS_MFMA"]))
    lines.append("sources_sha256_16: bwd.hip %s" % kernel_source_hash(("bwd.hip",)))
    lines.append("")
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarize_trace(trace_dir, out_path, cmd, last):
    """Write a kernel-duration summary from a rocprofv3 --kernel-trace --stats csv run.

    Reports rocprofv3's own per-kernel statistics and, for the attention
    kernel, the mean over the last `last` launches (the timed steps).
    """
    import csv
    import glob
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit("no kernel_stats.csv / kernel_trace.csv under %s" % trace_dir)
    lines = ["rocprofv3 kernel statistics", "", "command (from the repository root, TMPDIR=/tmp):",
             "  " + cmd, "", "kernel | calls | average us | min us | max us | share %"]
    with open(stats[0]) as f:
        for r in csv.DictReader(f):
            lines.append("%s | %s | %.2f | %.2f | %.2f | %s" % (
                r["Name"][:110], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, r["Percentage"]))
    durs = {}
    with open(trace[0]) as f:
        for r in csv.DictReader(f):
            durs.setdefault(r["Kernel_Name"], []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    lines.append("")
    for name, d in durs.items():
        if is_fwd_kernel(name) or any(k in name for k in ("softmax", "paged_decode", "splitkv_merge",
                                                          "attn_bwd")):
            d.sort()
            tail = [x[1] for x in d[-last:]]
            lines.append("%s: mean of the last %d launches (the timed steps) %.2f us" % (
                name[:110], len(tail), sum(tail) / len(tail) / 1e3))
    # Hashes of the sources of the kernels in this trace.
    groups = ((is_fwd_kernel, ("attn_fwd.hip", "mfma_tile.hpp", "online_merge.hpp")),
              (lambda n: "splitkv_merge" in n, ("splitkv.hip", "online_merge.hpp")),
              (lambda n: "paged_decode" in n, ("decode.hip", "decode_short.hip", "decode_kernel.hpp", "mfma_tile.hpp", "online_merge.hpp")),
              (lambda n: "softmax" in n, ("row_softmax.hip", "online_merge.hpp")),
              (lambda n: "attn_bwd" in n, ("bwd.hip", "mfma_tile.hpp", "online_merge.hpp")))
    parts = ["%s %s" % ("+".join(srcs), kernel_source_hash(srcs))
             for match, srcs in groups if any(match(n) for n in durs)]
    lines.append("sources_sha256_16: " + ", ".join(parts))
    lines.append("")
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the sustained amdsmi clock run")
    ap.add_argument("--profile-pass", nargs="?", const="C4", default=None, metavar="CFG",
                    help="run the fixed launch sequence the counter passes profile (default C4)")
    ap.add_argument("--profile-launches", metavar="CFG",
                    help="only launch workload CFG 20 times (the kernel-trace target)")
    ap.add_argument("--cfg", default="C4", help="workload the --summarize-* options describe")
    ap.add_argument("--profile-decode", action="store_true",
                    help="only launch the 32K-context paged decode 30 times (for rocprofv3)")
    ap.add_argument("--profile-bwd", action="store_true",
                    help="only run the headline workload's backward 10 times (for rocprofv3)")
    ap.add_argument("--ceiling", action="store_true",
                    help="print the MFMA rate the power limit allows per instruction mix, and C4's")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT"))
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR")
    ap.add_argument("--summarize-sq-bwd", nargs="+", metavar="DIR")
    ap.add_argument("--trace-last", type=int, default=20)
    ap.add_argument("--cmd", default="")
    ap.add_argument("--cmd-fetch", default="")
    ap.add_argument("--cmd-write", default="")
    args = ap.parse_args()
    if args.summarize_sq:
        summarize_sq(args.summarize_sq,
                     os.path.join(ROOT, "profiles", "attn_fwd_%s_sq_counters.txt" % args.cfg),
                     args.cmd.split(" ;; "), args.cfg)
        return
    if args.summarize_sq_bwd:
        summarize_sq_bwd(args.summarize_sq_bwd,
                         os.path.join(ROOT, "profiles", "attn_bwd_C4_sq_counters.txt"),
                         args.cmd.split(" ;; "))
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.cmd, args.trace_last)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1],
                          args.cmd_fetch, args.cmd_write, args.cfg)
        return
    if args.profile_pass:
        profile_pass(args.profile_pass)
        return
    if args.profile_launches:
        profile_launches(args.profile_launches)
        return
    if args.profile_decode:
        profile_decode()
        return
    if args.profile_bwd:
        profile_bwd()
        return
    if args.ceiling:
        ceiling()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import online_softmax_causal_amd as osc
    import workloads

    osc.load()
    dev = torch.device("cuda:0")
    w = workloads.ATTN["C4"]
    q, k, v = workloads.workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full((w.B, w.H, w.N, w.D), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        osc.attn_fwd(qd, kd, vd, o, lse, w.B, w.H, w.N, w.D, w.causal, w.dtype, stream)

    # Warm-up: the W requested steps, continued until at least
    # WARMUP_MIN_S of launches have run.  On this part the first tens of
    # milliseconds of work after an idle period run through a power-management
    # transient (launch times of the same kernel go 0.52 -> 0.70 -> 0.51 ms
    # over the first ~50 launches); a few warm-up launches would time that
    # transient instead of the kernel.
    t_warm = time.perf_counter()
    warm_run = 0
    while warm_run < args.warmup or time.perf_counter() - t_warm < WARMUP_MIN_S:
        for _ in range(10 if warm_run >= args.warmup else 1):
            step()
            warm_run += 1
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_warm
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (kernel_ms * 1e-3) / 1e12
    o_host = o.cpu().double().numpy()
    lse_host = lse.cpu().double().numpy()
    clock = measure_clock(step, w.flops) if not args.no_clock else None

    traffic = measured_traffic()
    line = {
        "metric": "causal attn fwd TFLOP/s (2BHN²D) at H=32,D=128,N=8192; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"launches": warm_run, "seconds": round(warm_s, 3),
                       "rule": "the W requested steps, continued until >= %.1f s of launches" % WARMUP_MIN_S},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.describe(), "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "causal": w.causal, "inputs": "Q,K,V iid N(0,1) rounded to fp16, seed %d" % w.seed,
                   "output": "O fp32 [B,H,N,D], LSE fp32 [B,H,N]"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(kernel_ms, 5),
                     "kernel": "attn_fwd_pipe_kernel<f16, D=128, causal>",
                     "kernel_source_sha256_16": kernel_source_hash()},
        "clock": clock,
    }
    if not args.no_cpu:
        base, parity = cpu_baseline(w, q, k, v, o_host, lse_host)
        line["cpu_baseline"] = base
        line["parity_sample"] = parity
    if not args.no_extra:
        line["extra"] = extra_configs(dev, with_oracle=not args.no_cpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
