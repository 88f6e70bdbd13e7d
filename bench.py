"""Benchmark of the hybrid paged GQA attention hot path on one MI355X.

Headline workload (the largest configuration that fits one GPU): the 60-layer decode sweep of
a Gemma-4-31B-shaped stack, five local layers then one global layer, ten times, ending on a
global layer. 16 rows at 32768 tokens of context; local layers: head_dim 256, 16 KV heads,
1024-token window (only window pages backed), 512-token splits; global layers: head_dim 512,
4 KV heads, V read from the K cache (K=V), 1024-token splits; 32 query heads, pages of 16
tokens, globally shuffled page tables, bf16 N(0,1) pools filled on the device. One step = the
60 back-to-back gattn_decode calls (split kernels and logsumexp combines) with every input
resident in HBM (about 34 GB of pools).

Prints one JSON line. value = decode KV GB/s over the timed steps: KV bytes = sum over layers,
rows and KV heads of visible keys * head_dim * 2 B * (1 with K=V, else 2). The other
configurations (tiny decode, the 32-row global decode, the 64-row local decode, the mixed
prefill + decode step of both families, the 65536-token row, FP8 pools, the 12B geometry, KV
append) are sub-records of the same line, with the fp64 oracle timed on the host's cores for each.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "decode attn KV GB/s (% HBM peak); prefill attn TFLOP/s (% bf16 MFMA peak)"
SWEEP_GLOBAL_KERNEL = "decode_split_kernel<512, true, 1, 32768>"
CFG2_KERNEL = "decode_split_kernel<512, false, 1, 32768>"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="only the 60-layer sweep (profiling runs of its kernels)")
    p.add_argument("--only", choices=("prefill", "kv_append"),
                   help="run only this sub-measurement and print it (counter runs of its kernels)")
    p.add_argument("--calib-copy", action="store_true",
                   help="run only a 1 GiB device copy (counter calibration for FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def kernel_source_digest():
    """Digest of the decode path's code (comments and blank lines dropped, so that a change of
    wording does not invalidate the committed counters)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("decode.hip", "common.h", "combine.hip"):
        with open(os.path.join(ROOT, "global_paged_gqa_amd", "csrc", f)) as fh:
            src = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in src.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code.strip():
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(digest, key):
    """HBM bytes per launch of one kernel (``key``, e.g. ``sweep_global``) from the committed counter
    summary, if it was taken on the current decode source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != digest:
        return None
    try:
        return float(vals[f"{key}_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def shader_clock_mhz():
    """The current shader clock level each GPU's driver reports (sysfs pp_dpm_sclk, the level marked
    '*'), in MHz, or None where the file is not readable."""
    import glob
    import re
    clocks = []
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if "*" in line:
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    if m:
                        clocks.append(int(m.group(1)))
        except OSError:
            continue
    return clocks or None


def calib_copy():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": 4 * n, "calib_copy_bytes_written": 4 * n, "launches": 5}))


def oracle_rate(batches, work, unit, min_s, what):
    """Time the fp64 oracle (``oracle.attend_batch``) on host batches, repeating the set until
    ``min_s`` seconds have passed; ``work`` is the algorithmic bytes or flops of one pass."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        for b, rows in batches:
            oracle.attend_batch(b, rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_s or reps >= 50:
            break
    scale = 1e9 if unit == "GB/s" else 1e9
    return {"value": round(work * reps / el / scale, 3), "unit": unit, "cores": oracle.threads(), "kind": "oracle",
            "seconds": round(el, 2), "passes": reps,
            "sample": f"{what}; fp64 two-pass softmax over contiguous K/V, OpenMP over (query, head)"}


def prefill_measure(torch, devio, workloads, traffic, flush, batches, iters=10):
    """The mixed step of each family: its 4 prefill chunks alone (TFLOP/s), its 60 decode rows
    alone (GB/s) and the whole step, gattn_prefill then gattn_decode on one stream. Every timed
    run follows a MALL flush, outside the events."""
    out = {}

    def timed(fn):
        ts = []
        for _ in range(iters):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return median(ts)

    for fam in ("global", "local"):
        pre, dec = workloads.cfg4_mixed(fam)
        batches[f"cfg4_{fam}"] = (pre, dec)
        d = devio.DeviceBatch(pre)
        dd = devio.DeviceBatch(dec)
        # warm-up: the first launches of a kernel run at a lower clock and miss its code caches
        for _ in range(10):
            d.prefill()
            dd.decode(512)
        torch.cuda.synchronize()
        s = pre.spec
        flops = traffic.prefill_flops(s.is_global, s.window, s.num_q_heads, s.head_dim, pre.ctx_lens, pre.q_lens)
        kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, dec.ctx_lens)
        t = timed(d.prefill)
        td = timed(lambda: dd.decode(512))
        tstep = timed(lambda: (d.prefill(), dd.decode(512)))
        # the same step as a single launch: one gattn_prefill over the prefill rows and the q_len-1 decode rows
        dm = devio.DeviceBatch(workloads.concat_batches(pre, dec))
        for _ in range(3):
            dm.prefill()
        tone = timed(dm.prefill)
        del dm
        tf = flops / t / 1e12
        out[fam] = {"tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                    "ms": round(t * 1e3, 4), "flops": flops,
                    "decode_rows_us": round(td * 1e6, 2), "decode_rows_kv_bytes": kv,
                    "decode_rows_gbs": round(kv / td / 1e9, 1),
                    "step_ms": round(tstep * 1e3, 4), "single_launch_step_ms": round(tone * 1e3, 4),
                    "workload": f"{fam}: 4 chunks x 2048 queries, priors {(pre.ctx_lens - pre.q_lens).tolist()}; "
                                f"60 decode rows, contexts ~U{{1..8192}}, split 512"}
        del d, dd
    return out


def append_measure(torch, devio, workloads, stream, flush, iters=20):
    """gattn_kv_append of one mixed step's new tokens (the 4 x 2048 prefill chunks and the 60 decode
    tokens, all 64 rows in one call) for each 31B family: GB/s of algorithmic bytes, every new K and
    V element read once and written once; each timed run after a MALL flush. Beside it, a plain
    device copy of the same bytes under the same flush (one torch copy of K and V, stacked, into a
    contiguous buffer): the practical ceiling of a transfer of this size."""
    import numpy as np
    out = {}
    for fam in ("global", "local"):
        pre, dec = workloads.cfg4_mixed(fam)
        b = workloads.concat_batches(pre, dec)
        s = b.spec
        d = devio.DeviceBatch(b)
        n_new = b.q_lens.astype(np.int32)
        cu = devio.dev(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32))
        T, mx = int(n_new.sum()), int(n_new.max())
        kvn = torch.randn(2, T, s.num_kv_heads, s.head_dim, device="cuda").to(torch.bfloat16).view(torch.int16)
        kn, vn = kvn[0], kvn[1]
        nbytes = kn.numel() * 2 * 2 * 2  # K and V, read and written

        def call():
            devio.nat.gattn_kv_append(d.layer, kn, vn, d.k_pool, d.v_pool, d.num_pages, d.page_table, d.pt_stride,
                                      cu, d.ctx_lens, b.B, mx, None)
        ckv = torch.empty_like(kvn)

        def copy():  # one launch over K and V (stacked), as the append is one launch
            ckv.copy_(kvn)
        for _ in range(5):
            call()
            copy()
        t = median(event_times(torch, stream, call, iters, flush))
        tc = median(event_times(torch, stream, copy, iters, flush))
        out[fam] = {"tokens": T, "rows": b.B, "bytes": nbytes, "us": round(t * 1e6, 2),
                    "gbs": round(nbytes / t / 1e9, 1), "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                    "plain_copy_us": round(tc * 1e6, 2), "plain_copy_gbs": round(nbytes / tc / 1e9, 1)}
        del ckv
        if fam == "local":  # the same tokens into E4M3 pools: 2 bytes read and 1 written per element
            k8 = torch.zeros(d.k_pool.shape, dtype=torch.uint8, device="cuda")
            v8 = torch.zeros(d.k_pool.shape, dtype=torch.uint8, device="cuda")
            nbytes8 = kn.numel() * (2 + 1) * 2

            def call8():
                devio.nat.gattn_kv_append_fp8(d.layer, kn, vn, k8, v8, workloads.FP8_K_SCALE, workloads.FP8_V_SCALE,
                                              d.num_pages, d.page_table, d.pt_stride, cu, d.ctx_lens, b.B, mx, None)
            for _ in range(5):
                call8()
            t8 = median(event_times(torch, stream, call8, iters, flush))
            out["local_fp8"] = {"bytes": nbytes8, "us": round(t8 * 1e6, 2), "gbs": round(nbytes8 / t8 / 1e9, 1)}
            del k8, v8
        del d, kn, vn, kvn
        torch.cuda.empty_cache()
    out["workload"] = ("gattn_kv_append of the mixed step's 8252 new tokens per family (4 prefill chunks of 2048 and "
                       "60 decode tokens, one call over the 64 rows) into the 31B pools")
    return out


class MallFlush:
    """Evicts the 256 MB MALL and the L2s by reading a 1 GiB buffer (a sum into one float), outside
    the timed events. Reading leaves clean lines behind: a 1 GiB write would leave up to 256 MB of
    dirty lines whose write-back the next, timed, kernel would pay for."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.out = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        self.torch.sum(self.buf, 0, out=self.out)


def event_times(torch, stream, fn, n, flush=None):
    """Per-call durations (s) of ``fn`` from HIP events recorded on ``stream``; with ``flush`` (a
    MallFlush), the caches are flushed before each call, outside the events."""
    ts = []
    for _ in range(n):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        if flush is not None:
            torch.cuda.synchronize()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in ts]


def median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def local_decode_measure(torch, devio, workloads, traffic, stream, flush, steps=50):
    """The local-family decode workload (batch 64, hd 256, 16 KV heads, window 1024, contexts
    ~U{512..32768}, window pages only, split 512), pools filled on the device."""
    lay = workloads.paged_layout(workloads.LOCAL_31B, workloads.ragged((3, 0), 512, 32768, 64), (3, 0))
    d = devio.DeviceLayout(lay, workloads.fill_normal_bf16_device)
    s = lay.spec
    kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, lay.ctx_lens)
    for _ in range(5):
        d.decode(512)
    t = median(event_times(torch, stream, lambda: d.decode(512), steps))
    tf = median(event_times(torch, stream, lambda: d.decode(512), 10, flush))
    out = {"workload": "local decode: batch 64, 32 q heads, 16 KV heads, hd 256, window 1024, contexts "
                       "~U{512..32768}, split 512", "kv_bytes": kv, "us": round(t * 1e6, 2),
           "gbs": round(kv / t / 1e9, 1), "frac": round(kv / t / 1e9 / HBM_PEAK_GBS, 4),
           "mall_flushed_gbs": round(kv / tf / 1e9, 1)}
    del d
    # the same rows over an FP8 (E4M3) pool: half the bytes per visible key
    d8 = devio.DeviceLayout(lay, workloads.fill_e4m3_device, fp8=(workloads.FP8_K_SCALE, workloads.FP8_V_SCALE))
    kv8 = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, lay.ctx_lens, 1)
    for _ in range(5):
        d8.decode(512)
    t8 = median(event_times(torch, stream, lambda: d8.decode(512), steps))
    tf8 = median(event_times(torch, stream, lambda: d8.decode(512), 10, flush))
    out["fp8"] = {"kv_bytes": kv8, "us": round(t8 * 1e6, 2), "gbs": round(kv8 / t8 / 1e9, 1),
                  "frac": round(kv8 / t8 / 1e9 / HBM_PEAK_GBS, 4), "mall_flushed_us": round(tf8 * 1e6, 2),
                  "mall_flushed_gbs": round(kv8 / tf8 / 1e9, 1), "speedup_vs_bf16": round(t / t8, 3)}
    return out


def global_fp8_measure(torch, devio, workloads, traffic, stream, flush, steps=50):
    """The measured global decode batch (32 rows, contexts ~U{1..8192}, split 512) over E4M3 pools,
    pools filled on the device; GB/s of FP8 bytes and the speed-up over the same rows in bf16."""
    L = workloads.ragged((2, 0), 1, 8192, 32)
    lay = workloads.paged_layout(workloads.GLOBAL_31B, L, (2, 0))
    s = lay.spec
    out = {}
    for name, fp8 in (("bf16", None), ("fp8", (workloads.FP8_K_SCALE, workloads.FP8_V_SCALE))):
        if fp8 is None:
            d = devio.DeviceLayout(lay, workloads.fill_normal_bf16_device)
        else:
            d = devio.DeviceLayout(lay, workloads.fill_e4m3_device, fp8=fp8)
        kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, L,
                                     2 if fp8 is None else 1)
        for _ in range(5):
            d.decode(512)
        t = median(event_times(torch, stream, lambda: d.decode(512), steps))
        out[name] = {"kv_bytes": kv, "us": round(t * 1e6, 2), "gbs": round(kv / t / 1e9, 1)}
        del d
    out["speedup"] = round(out["bf16"]["us"] / out["fp8"]["us"], 3)
    out["workload"] = "global decode: batch 32, hd 512, 4 KV heads, contexts ~U{1..8192}, split 512; bf16 vs E4M3 pools"
    return out


def gemma12b_measure(torch, devio, workloads, traffic, stream, flush, steps=50):
    """The 12B geometry: global decode (batch 32, 16 q heads over one KV head, hd 512, contexts
    ~U{1..8192}, split 512) as KV GB/s, and the 12B mixed step's prefill rows of both families as
    TFLOP/s; every timed run after a MALL flush."""
    b = workloads.cfg6_12b_global_decode()
    s = b.spec
    kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, b.ctx_lens)
    d = devio.DeviceBatch(b)
    for _ in range(10):
        d.decode(512)
    t = median(event_times(torch, stream, lambda: d.decode(512), steps, flush))
    out = {"global_decode": {"workload": "12B global decode: batch 32, 16 q heads, 1 KV head, hd 512, contexts "
                                         "~U{1..8192}, split 512", "kv_bytes": kv, "us": round(t * 1e6, 2),
                             "gbs": round(kv / t / 1e9, 1), "frac": round(kv / t / 1e9 / HBM_PEAK_GBS, 4)}}
    del d
    for fam in ("global", "local"):
        pre, _ = workloads.cfg6_12b_mixed(fam)
        dp = devio.DeviceBatch(pre)
        s = pre.spec
        flops = traffic.prefill_flops(s.is_global, s.window, s.num_q_heads, s.head_dim, pre.ctx_lens, pre.q_lens)
        for _ in range(10):
            dp.prefill()
        tp = median(event_times(torch, stream, dp.prefill, 10, flush))
        out[f"{fam}_prefill"] = {"workload": f"12B {fam} prefill: 4 chunks x 2048 queries, priors "
                                             f"{(pre.ctx_lens - pre.q_lens).tolist()}", "flops": flops, "ms": round(tp * 1e3, 4),
                                 "tflops": round(flops / tp / 1e12, 2),
                                 "frac_of_bf16_peak": round(flops / tp / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        del dp
    return out


def build_sweep(torch, devio, workloads, traffic):
    """The 60 layers of the decode sweep resident on the device (pools filled there), sharing one
    workspace; returns (layers [(family, DeviceLayout)], layouts, KV bytes total and per family)."""
    nat = devio.nat
    n = workloads.SWEEP_LAYERS
    layers, lays, kv_total, kv_fam = [], [], 0, {"local": 0, "global": 0}
    for l in range(n):
        fam = "global" if nat.gattn_layer_family(l, n) == nat.GLOBAL else "local"
        lay = workloads.sweep_layer(l, fam)
        lays.append(lay)
        s = lay.spec
        kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, lay.ctx_lens)
        kv_total += kv
        kv_fam[fam] += kv
        layers.append((fam, devio.DeviceLayout(lay, workloads.fill_normal_bf16_device)))
    ws_bytes = max(d.workspace_bytes(workloads.SWEEP_SPLIT[f]) for f, d in layers)
    ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device="cuda")
    for _, d in layers:
        d.workspace, d.ws_bytes = ws, ws_bytes
    return layers, lays, kv_total, kv_fam


def combine_time(torch, nat, d, split, stream, n=50):
    """Mean duration of the logsumexp combine alone on the partials a DeviceLayout's last decode left in
    its workspace (to separate the split kernel's own duration from the whole call): n combines back to
    back between one pair of events, so that the events' own latency is not charged to each of them."""
    lay, s = d.lay, d.lay.spec
    ns = d.workspace_bytes(split) // (4 * (s.head_dim + 1) * lay.B * s.num_q_heads)
    n_o = lay.B * s.num_q_heads * ns * s.head_dim
    o_part, lse_part = d.workspace[:n_o], d.workspace[n_o:n_o + lay.B * s.num_q_heads * ns]
    nat.gattn_combine(lay.B, s.num_q_heads, s.head_dim, ns, o_part, lse_part, d.out, d.lse, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        nat.gattn_combine(lay.B, s.num_q_heads, s.head_dim, ns, o_part, lse_part, d.out, d.lse, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / n


def sweep_extras(torch, devio, workloads, traffic, stream, layers, lays, kv_total, kv_fam, t_sweep, reps=10):
    """Per-family layer times, the sweep captured in a HIP graph, and the sweep over FP8 pools."""
    out = {}
    # per-layer call times over five passes of the 60 layers; per family the median call (a single
    # pass can catch a host-side stall between an event and its call)
    evs = []
    for _ in range(5):
        for fam, d in layers:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            d.decode(workloads.SWEEP_SPLIT[fam])
            e1.record(stream)
            evs.append((fam, e0, e1))
    torch.cuda.synchronize()
    per = {"local": [], "global": []}
    for fam, e0, e1 in evs:
        per[fam].append(e0.elapsed_time(e1) * 1e-3)
    for fam in ("local", "global"):
        t_layer = median(per[fam])
        n_layers = 50 if fam == "local" else 10
        out[f"{fam}_layers_gbs"] = round(kv_fam[fam] / (t_layer * n_layers) / 1e9, 1)
        out[f"{fam}_layer_us"] = round(t_layer * 1e6, 2)

    def sweep():
        for fam, d in layers:
            d.decode(workloads.SWEEP_SPLIT[fam])
    # the same 60 calls captured once in a HIP graph and replayed (no launch gaps between layers)
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sweep()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            sweep()
        graph.replay()
        torch.cuda.synchronize()
        tg = median(event_times(torch, stream, graph.replay, reps))
        out["graph_ms"] = round(tg * 1e3, 4)
        out["graph_gbs"] = round(kv_total / tg / 1e9, 1)
        del graph
    except Exception as e:  # report, never hide
        out["graph_error"] = str(e)[:200]
    # the same sweep with the 50 local layers' K/V in FP8 (E4M3) pools (gattn_decode_fp8kv), then every layer
    try:
        ws = layers[0][1].workspace
        layers8 = []
        for (fam, d), lay in zip(layers, lays):
            if fam == "local":
                d = devio.DeviceLayout(lay, workloads.fill_e4m3_device, workspace=ws,
                                       fp8=(workloads.FP8_K_SCALE, workloads.FP8_V_SCALE))
            layers8.append((fam, d))

        def sweep8():
            for fam, d in layers8:
                d.decode(workloads.SWEEP_SPLIT[fam])
        sweep8()
        torch.cuda.synchronize()
        t8 = median(event_times(torch, stream, sweep8, reps))
        kv8 = kv_fam["global"] + kv_fam["local"] // 2
        out["fp8_local"] = {"kv_bytes": kv8, "ms": round(t8 * 1e3, 4), "gbs": round(kv8 / t8 / 1e9, 1),
                            "speedup_vs_bf16": round(t_sweep / t8, 3)}
        layers.clear()  # the bf16 local pools are not used again: drop them before the FP8 global pools
        all8 = []
        for (fam, d), lay in zip(layers8, lays):
            if fam == "global":
                d = devio.DeviceLayout(lay, workloads.fill_e4m3_device, workspace=ws,
                                       fp8=(workloads.FP8_K_SCALE, workloads.FP8_K_SCALE))
            all8.append((fam, d))
        layers8 = all8
        sweep8()
        torch.cuda.synchronize()
        ta = median(event_times(torch, stream, sweep8, reps))
        out["fp8_all"] = {"kv_bytes": kv_total // 2, "ms": round(ta * 1e3, 4),
                          "gbs": round(kv_total // 2 / ta / 1e9, 1), "speedup_vs_bf16": round(t_sweep / ta, 3)}
        del layers8, all8
    except Exception as e:  # report, never hide
        out["fp8_error"] = str(e)[:200]
    return out


def long_measure(torch, devio, workloads, traffic, stream, flush):
    """The single 65536-token global decode row (K=V, split 1024)."""
    lay = workloads.long_global_decode(rows=())
    d = devio.DeviceLayout(lay, workloads.fill_normal_bf16_device)
    s = lay.spec
    kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, lay.ctx_lens)
    for _ in range(5):
        d.decode(1024)
    tl = median(event_times(torch, stream, lambda: d.decode(1024), 50))
    tlf = median(event_times(torch, stream, lambda: d.decode(1024), 10, flush))
    tc = combine_time(torch, devio.nat, d, 1024, stream)
    return {"workload": "one 65536-token global decode row, K=V, split 1024", "kv_bytes": kv,
            "us": round(tl * 1e6, 2), "gbs": round(kv / tl / 1e9, 1), "frac": round(kv / tl / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_gbs": round(kv / (tl - tc) / 1e9, 1), "combine_us": round(tc * 1e6, 2),
            "mall_flushed_us": round(tlf * 1e6, 2), "mall_flushed_gbs": round(kv / tlf / 1e9, 1)}


def cfg2_measure(torch, devio, workloads, traffic, stream, flush, digest, steps=200):
    """The 32-row global decode batch (32 q heads, 4 KV heads, hd 512, contexts ~U{1..8192}, split 512):
    whole call, split kernel alone (call minus the combine's own time) and after a MALL flush."""
    batch = workloads.cfg2_global_decode()
    s = batch.spec
    kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, batch.ctx_lens)
    d = devio.DeviceBatch(batch)
    for _ in range(20):
        d.decode(512)
    torch.cuda.synchronize()
    t = median(event_times(torch, stream, lambda: d.decode(512), steps))
    tf = median(event_times(torch, stream, lambda: d.decode(512), 20, flush))
    nat = devio.nat
    ns = nat.gattn_decode_workspace_bytes(d.layer, batch.B, int(batch.ctx_lens.max()), 512) // (
        4 * (s.head_dim + 1) * batch.B * s.num_q_heads)
    n_o = batch.B * s.num_q_heads * ns * s.head_dim
    # the merge alone, back to back between one pair of events (see combine_time)
    nat.gattn_combine(batch.B, s.num_q_heads, s.head_dim, ns, d.workspace[:n_o], d.workspace[n_o:], d.out, d.lse,
                      stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(50):
        nat.gattn_combine(batch.B, s.num_q_heads, s.head_dim, ns, d.workspace[:n_o], d.workspace[n_o:], d.out, d.lse,
                          stream)
    e1.record(stream)
    torch.cuda.synchronize()
    tc = e0.elapsed_time(e1) * 1e-3 / 50
    # the same call replayed from the decode graph bucket set (buckets 8, 16, 32; the batch fills bucket 32)
    max_ctx = int(batch.ctx_lens.max())
    h = nat.gattn_decode_graphs_create(d.layer, d.q, d.k_pool, d.v_pool, d.num_pages, d.page_table, d.pt_stride,
                                       d.ctx_lens, max_ctx, 512, d.workspace, d.ws_bytes, d.out, d.lse, [8, 16, 32])
    try:
        for _ in range(10):
            nat.gattn_decode_graphs_launch(h, batch.B, stream)
        tg = median(event_times(torch, stream, lambda: nat.gattn_decode_graphs_launch(h, batch.B, stream), steps))
    finally:
        torch.cuda.synchronize()
        nat.gattn_decode_graphs_destroy(h)
    return batch, {"workload": "global decode: batch 32, 32 q heads, 4 KV heads, head_dim 512, contexts "
                               "~U{1..8192}, split 512", "kv_bytes": kv, "us": round(t * 1e6, 2),
                   "gbs": round(kv / t / 1e9, 1), "frac": round(kv / t / 1e9 / HBM_PEAK_GBS, 4),
                   "kernel": CFG2_KERNEL, "kernel_us": round((t - tc) * 1e6, 2),
                   "kernel_gbs": round(kv / (t - tc) / 1e9, 1), "combine_us": round(tc * 1e6, 2),
                   "traffic": measured_traffic(digest, "cfg2"),
                   "mall_flushed_gbs": round(kv / tf / 1e9, 1), "mall_flushed_frac": round(kv / tf / 1e9 / HBM_PEAK_GBS, 4),
                   "graph_bucket_us": round(tg * 1e6, 2), "graph_bucket_gbs": round(kv / tg / 1e9, 1)}


def cpu_baselines(workloads, traffic, batches):
    """The fp64 oracle on each configuration's rows (or a stated sample of them), timed on the host's
    cores, as the same algorithmic GB/s or GFLOP/s the GPU figures use."""
    out = {}
    b1 = workloads.cfg1_tiny_decode()
    s = b1.spec
    kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, b1.ctx_lens)
    out["tiny_decode"] = oracle_rate([(b1, None)], kv, "GB/s", 2.0, "the whole tiny decode (1 row, L 1025)")
    b2 = batches.get("cfg2") or workloads.cfg2_global_decode()
    s = b2.spec
    kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, b2.ctx_lens)
    out["global_decode"] = oracle_rate([(b2, None)], kv, "GB/s", 4.0, "the whole 32-row global decode batch")
    b3 = workloads.cfg3_local_decode()
    s = b3.spec
    kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, b3.ctx_lens)
    out["local_decode"] = oracle_rate([(b3, None)], kv, "GB/s", 4.0, "the whole 64-row local decode batch")
    for fam in ("global", "local"):
        pre, dec = batches.get(f"cfg4_{fam}") or workloads.cfg4_mixed(fam)
        s = pre.spec
        r = int(pre.ctx_lens.argmin())  # the row with the shortest prior (least oracle time)
        fl = traffic.prefill_flops(s.is_global, s.window, s.num_q_heads, s.head_dim, pre.ctx_lens[[r]],
                                   pre.q_lens[[r]])
        rec = oracle_rate([(pre, [r])], fl, "GFLOP/s", 1.0,
                          f"{fam} mixed step: prefill row {r} (2048 queries after a prior of "
                          f"{int(pre.ctx_lens[r] - pre.q_lens[r])})")
        kv = traffic.decode_kv_bytes(s.is_global, s.window, s.num_kv_heads, s.head_dim, s.kv_shared, dec.ctx_lens)
        rec["decode_rows"] = oracle_rate([(dec, None)], kv, "GB/s", 2.0, f"{fam} mixed step: its 60 decode rows")
        out[f"mixed_{fam}"] = rec
    # the sweep: sampled rows of one global and one local layer, weighted as in the sweep (10 : 50)
    g = workloads.sweep_layer(5, "global", rows=(0, 1))
    l0 = workloads.sweep_layer(0, "local", rows=tuple(range(workloads.SWEEP_B)))
    kv_g = traffic.decode_kv_bytes(True, 0, 4, 512, True, g.host.ctx_lens)
    kv_l = traffic.decode_kv_bytes(False, 1024, 16, 256, False, l0.host.ctx_lens)
    out["sweep"] = oracle_rate([(g.host, None)] + [(l0.host, None)] * 5, kv_g + 5 * kv_l, "GB/s", 8.0,
                               "sampled sweep rows: rows 0-1 of global layer 5 (K=V, 32768 tokens) once and all 16 "
                               "rows of local layer 0 five times (the sweep's 10 : 50 layer mix)")
    lg = workloads.long_global_decode(rows=(0,))
    kv = traffic.decode_kv_bytes(True, 0, 4, 512, True, lg.host.ctx_lens)
    out["long_decode"] = oracle_rate([(lg.host, None)], kv, "GB/s", 2.0, "the whole 65536-token row")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU "
              "path: rows shard across GPUs with no attention-side communication.", file=sys.stderr)
        sys.exit(2)
    cpu_model = host_cpu_model()
    import torch
    if args.calib_copy:
        calib_copy()
        return

    import __graft_entry__
    __graft_entry__.ensure_built()
    import workloads
    from global_paged_gqa_amd import devio, traffic

    stream = torch.cuda.current_stream()
    digest = kernel_source_digest()
    if args.only:
        flush = MallFlush(torch)
        if args.only == "prefill":
            sub = prefill_measure(torch, devio, workloads, traffic, flush, {})
        else:
            sub = append_measure(torch, devio, workloads, stream, flush)
        print(json.dumps({"only": args.only, args.only: sub}), flush=True)
        return
    layers, lays, kv_total, kv_fam = build_sweep(torch, devio, workloads, traffic)

    def sweep(global_events=None):
        for fam, d in layers:
            if global_events is not None and fam == "global":
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                d.decode(workloads.SWEEP_SPLIT[fam])
                e1.record(stream)
                global_events.append((e0, e1))
            else:
                d.decode(workloads.SWEEP_SPLIT[fam])

    for _ in range(args.warmup):
        sweep()
    torch.cuda.synchronize()
    # timed region: exactly `steps` sweeps back to back; events around every global-layer call (the
    # dominant kernel) on the library's stream
    gev = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        sweep(gev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = shader_clock_mhz()
    t_sweep = wall / args.steps
    value = kv_total / t_sweep / 1e9
    g_call = sum(a.elapsed_time(b) for a, b in gev) * 1e-3 / len(gev)
    gd = [d for fam, d in layers if fam == "global"][-1]
    g_comb = combine_time(torch, devio.nat, gd, workloads.SWEEP_SPLIT["global"], stream)
    g_kernel = g_call - g_comb
    kv_glayer = kv_fam["global"] // 10
    achieved = kv_glayer / g_kernel / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_sweep * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "60-layer decode sweep (LLLLLG x10, last layer global), 16 rows x 32768 tokens, "
                               "32 q heads; local: hd 256, 16 KV heads, window 1024, split 512; global: hd 512, "
                               "4 KV heads, K=V, split 1024; page 16, shuffled pages, bf16 N(0,1) pools",
                   "layers": workloads.SWEEP_LAYERS, "batch": workloads.SWEEP_B, "context": workloads.SWEEP_L,
                   "kv_bytes_per_step": kv_total, "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": SWEEP_GLOBAL_KERNEL, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(digest, "sweep_global"),
                     "bytes_per_launch": kv_glayer, "kernel_us": round(g_kernel * 1e6, 2),
                     "call_us": round(g_call * 1e6, 2), "combine_us": round(g_comb * 1e6, 2),
                     "kernel_source_digest": digest},
        "host": {"cpu_model": cpu_model, "shader_clock_mhz_after_timed_region": clock},
    }
    sw = {}
    if not args.headline_only:
        try:
            sw = sweep_extras(torch, devio, workloads, traffic, stream, layers, lays, kv_total, kv_fam, t_sweep)
        except Exception as e:  # report, never hide
            sw = {"error": str(e)[:300]}
    result["sweep"] = dict(sw, kv_bytes=kv_total, ms=round(t_sweep * 1e3, 4), gbs=round(value, 1))
    layers = lays = gd = None
    torch.cuda.empty_cache()
    if args.headline_only:
        print(json.dumps(result), flush=True)
        return

    flush = MallFlush(torch)
    batches = {}
    for name, fn in (("long_decode", lambda: long_measure(torch, devio, workloads, traffic, stream, flush)),
                     ("local_decode", lambda: local_decode_measure(torch, devio, workloads, traffic, stream, flush)),
                     ("global_decode_fp8", lambda: global_fp8_measure(torch, devio, workloads, traffic, stream,
                                                                      flush)),
                     ("gemma12b", lambda: gemma12b_measure(torch, devio, workloads, traffic, stream, flush))):
        try:
            result[name] = fn()
        except Exception as e:  # report, never hide
            result[name] = {"error": str(e)[:300]}
        torch.cuda.empty_cache()
    try:
        batches["cfg2"], result["global_decode"] = cfg2_measure(torch, devio, workloads, traffic, stream, flush,
                                                                digest)
    except Exception as e:  # report, never hide
        result["global_decode"] = {"error": str(e)[:300]}
    if not args.no_prefill:
        try:
            result["prefill"] = prefill_measure(torch, devio, workloads, traffic, flush, batches)
        except Exception as e:  # report, never hide
            result["prefill"] = {"error": str(e)[:200]}
    try:
        result["kv_append"] = append_measure(torch, devio, workloads, stream, flush)
    except Exception as e:  # report, never hide
        result["kv_append"] = {"error": str(e)[:200]}
    if not args.no_cpu_baseline:
        base = cpu_baselines(workloads, traffic, batches)
        result["cpu_baseline"] = dict(base["sweep"], host_cpu=cpu_model)
        result["cpu_baselines"] = base
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
