#!/usr/bin/env python3
"""Absorbed MLA decode on one MI355X: KV-tokens/s and achieved HBM GB/s.

A step is one decode step of the whole hot path over every layer of the
workload, through libmla_kv.so's fused decode step in its three launches:
(1) every sequence's new token is stored, its k_pe turned by RoPE at its
position and quantized, while the turned query is absorbed through W_UK;
(2) split-KV partial attention over the quantized cache, the new token
included; (3) merge of the splits and W_UV projection.

Default workload: DeepSeek-V2-Lite-shaped, 27 layers, 16 heads, batch 64,
ragged lengths uniform in [1024, 16384], INT8 latent + INT8 k_pe cache. The
INT4 workload (1 layer, batch 32, 16 heads, 32768 tokens, asymmetric INT4)
is measured in the same run and reported under "int4".

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, published
METRIC = "absorbed MLA decode KV-tokens/s and achieved HBM GB/s (% peak), INT8 & INT4"
KERNEL_SRC = os.path.join(ROOT, "mla_latent_kv_cache_amd", "csrc", "mla_kv.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def row_bytes(fmt):
    from mla_latent_kv_cache_amd.cache import row_bytes as rb
    return rb(fmt)


# ----------------------------------------------------------------- GPU side

class Runner:
    """Holds one workload's cache, weights, queries and the ctypes calls of a step."""

    def __init__(self, wid, extra_steps, fmt=None, layers=None, page_size=0):
        import dataclasses
        import torch
        from mla_latent_kv_cache_amd import LatentCache, _lib
        from mla_latent_kv_cache_amd import workloads as W
        self.torch = torch
        self.W = W
        self.wid = wid
        w = W.WORKLOADS[wid]
        if fmt is not None or layers is not None:  # the same inputs in another cache format / depth
            fmt, layers = fmt or w.fmt, layers or w.layers
            shape = w.name.split("_", 2)[2]  # e.g. b64_h16_ragged1024-16384
            w = dataclasses.replace(w, fmt=fmt, layers=layers, name=f"{fmt}_l{layers}_{shape}")
        if page_size:
            w = dataclasses.replace(w, name=f"{w.name}_paged{page_size}")
        self.w = w
        self.lens0 = W.lengths(wid)
        ragged = isinstance(w.seq, tuple)
        cap = int(self.lens0.max()) + w.append + extra_steps
        cap = (cap + 15) // 16 * 16
        dev = torch.device("cuda:0")
        t0 = time.time()
        if page_size:
            # pages of page_size tokens, handed to the sequences in a shuffled order
            cap = (cap + page_size - 1) // page_size * page_size
            blocks = cap // page_size
            perm = np.random.default_rng(7).permutation(w.batch * blocks)
            table = perm.reshape(w.batch, blocks).astype(np.int32)
            self.cache = cache = LatentCache(w.fmt, w.layers, w.batch, cap, device=dev, page_size=page_size,
                                             num_pages=w.batch * blocks, block_table=table)
        else:
            self.cache = cache = LatentCache(w.fmt, w.layers, w.batch, cap, device=dev)
        # The prefill goes through mla_cache_append, one call per layer, each timed
        # with a pair of HIP events (the synthetic inputs are made outside them).
        lens_dev = torch.tensor(self.lens0, dtype=torch.int32, device=dev) if ragged else None
        stream = torch.cuda.current_stream()
        self.prefill_ms, self.prefill_tokens = 0.0, 0
        for layer in range(w.layers):
            ckv, kpe = W.latent_batch(wid, layer, int(self.lens0.max()), device=dev,
                                      counts=self.lens0 if ragged else None)
            T = ckv.shape[1]
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _lib.check(_lib.lib().mla_cache_append(ctypes.byref(cache.struct), layer, ctypes.c_void_p(ckv.data_ptr()),
                                                   ctypes.c_void_p(kpe.data_ptr()), T,
                                                   ctypes.c_void_p(lens_dev.data_ptr()) if ragged else None,
                                                   ctypes.c_void_p(stream.cuda_stream)), "prefill append")
            e1.record(stream)
            cache._lens[layer] += self.lens0 if ragged else T
            e1.synchronize()
            self.prefill_ms += e0.elapsed_time(e1)
            self.prefill_tokens += int(self.lens0.sum()) if ragged else w.batch * T
            del ckv, kpe
        torch.cuda.synchronize()
        log(f"{w.name}: prefilled {int(self.lens0.sum()) * w.layers} tokens "
            f"({cache.bytes() / 1e9:.2f} GB of cache planes) in {time.time() - t0:.1f}s")
        self.H = w.heads
        self.splits = w.num_splits
        self.q = [W.queries(wid, layer, dev) for layer in range(w.layers)]
        self.wts = [W.weights(wid, layer, dev) for layer in range(w.layers)]
        steps_new = [W.latent_batch(wid, layer, extra_steps, device=dev, kind="step")
                     for layer in range(w.layers)]
        self.new = [[(steps_new[l][0][:, i:i + 1].contiguous(), steps_new[l][1][:, i:i + 1].contiguous())
                     for l in range(w.layers)] for i in range(extra_steps)]
        self.ws = cache.workspace(self.H, self.splits)
        from mla_latent_kv_cache_amd import rope_tables
        self.rope = rope_tables(cap + 1, device=dev)  # positions 0 .. capacity
        self.out = torch.empty((w.batch, self.H, 128), dtype=torch.float32, device=dev)
        self.lib = _lib.lib()
        self.check = _lib.check
        self.stream = torch.cuda.current_stream()
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)
        self.cref = ctypes.byref(cache.struct)
        self.scale = ctypes.c_float(W.SOFTMAX_SCALE)
        vp = lambda t: ctypes.c_void_p(t.data_ptr())
        self.args_q = [(vp(qn), vp(qp)) for qn, qp in self.q]
        self.args_w = [(vp(wuk), vp(wuv)) for wuk, wuv in self.wts]
        self.args_new = [[(vp(c), vp(k)) for c, k in step] for step in self.new]
        self.ws_p, self.ws_n = vp(self.ws), ctypes.c_size_t(self.ws.numel())
        self.rope_p = (vp(self.rope[0]), vp(self.rope[1]), self.rope[0].shape[0])
        self.out_p = vp(self.out)
        self.steps_done = 0
        self.ns = cache.auto_splits(self.H) if self.splits == 0 else self.splits

    def step(self, events=None):
        """One decode step over every layer. events: list to append (start, end) pairs
        recorded around each partial-attention launch."""
        L = self.lib
        i = self.steps_done
        cos_p, sin_p, rows = self.rope_p
        for layer in range(self.w.layers):
            c, k = self.args_new[i][layer]
            qn, qp = self.args_q[layer]
            wuk, wuv = self.args_w[layer]
            st = L.mla_decode_step_begin(self.cref, layer, c, k, qn, qp, cos_p, sin_p, rows, wuk, self.H,
                                         self.scale, self.splits, self.ws_p, self.ws_n, self.sp)
            if st:
                self.check(st, "step_begin")
            if events is not None:
                e0 = self.torch.cuda.Event(enable_timing=True)
                e1 = self.torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
            st = L.mla_decode_partial(self.cref, layer, self.H, self.splits, self.ws_p, self.ws_n, self.sp)
            if st:
                self.check(st, "partial")
            if events is not None:
                e1.record(self.stream)
                events.append((e0, e1, layer))
            st = L.mla_decode_combine(self.cref, wuv, self.H, self.splits, self.ws_p, self.ws_n,
                                      self.out_p, self.sp)
            if st:
                self.check(st, "combine")
        self.cache._lens += 1  # host mirror: one token per sequence per layer
        self.steps_done += 1

    def kv_tokens(self, step_index):
        """Tokens attended in the given step (1-based count of appended tokens)."""
        return int(self.w.layers * (self.lens0 + step_index).sum())

    def layer_tokens(self, step_index):
        return int((self.lens0 + step_index).sum())

    def algorithmic_bytes(self, step_index):
        """Bytes the method must move in one step (per-token cache rows, the
        weights, the queries, the output and the appended rows)."""
        w = self.w
        cache = self.kv_tokens(step_index) * row_bytes(w.fmt)
        weights = w.layers * 2 * w.heads * 128 * 512 * 2
        queries = w.layers * w.batch * w.heads * 192 * 2
        output = w.layers * w.batch * w.heads * 128 * 4
        append = w.layers * w.batch * (1152 + row_bytes(w.fmt))
        return cache + weights + queries + output + append


def append_result(what, tokens, ms, fmt):
    """Appended tokens/s and GB/s: each token reads its bf16 row (1024 + 128 B)
    and writes its cache row."""
    per_token = 1152 + row_bytes(fmt)
    return {"workload": what, "tokens": tokens, "value": tokens / (ms / 1e3), "unit": "appended tokens/s",
            "gb_per_s": tokens * per_token / (ms / 1e3) / 1e9, "bytes_per_token": per_token, "ms": ms}


def measure_append64(reps=50):
    """The decode-time append of the INT8 workload of 8 sequences: 64 new tokens
    per sequence in one mla_cache_append call, repeated into fresh rows; each
    call timed with HIP events."""
    import torch
    from mla_latent_kv_cache_amd import LatentCache, _lib
    from mla_latent_kv_cache_amd import workloads as W
    wid = 1
    w = W.WORKLOADS[wid]
    dev = torch.device("cuda:0")
    T = w.append
    cache = LatentCache(w.fmt, 1, w.batch, T * (reps + 5), device=dev)
    ckv, kpe = W.latent_batch(wid, 0, T, device=dev, kind="append")
    stream = torch.cuda.current_stream()
    L = _lib.lib()
    ms = []
    for i in range(reps + 5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        _lib.check(L.mla_cache_append(ctypes.byref(cache.struct), 0, ctypes.c_void_p(ckv.data_ptr()),
                                      ctypes.c_void_p(kpe.data_ptr()), T, None,
                                      ctypes.c_void_p(stream.cuda_stream)), "append")
        e1.record(stream)
        cache._lens[0] += T
        if i >= 5:
            ms.append((e0, e1))
    torch.cuda.synchronize()
    total = sum(a.elapsed_time(b) for a, b in ms)
    res = append_result(f"{w.fmt} B{w.batch} T{T} per call", reps * w.batch * T, total, w.fmt)
    res["us_per_call"] = total / reps * 1e3
    return res


def measure(wid, steps, warmup, fmt=None, layers=None, page_size=0):
    """W untimed steps, then the K timed steps (value, ms_per_step), then K more
    steps with a pair of HIP events around every partial-attention launch (its
    average duration, for the roofline). The timed steps carry no per-launch
    events: an event recorded between two launches holds the next launch back
    by some 4-5 us, which is measurement overhead, not decode work."""
    import torch
    r = Runner(wid, 2 * steps + warmup, fmt, layers, page_size)
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    log(f"{r.w.name}: warmup done ({warmup} steps); timing {steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(r.stream)
    for _ in range(steps):
        r.step()
    t_end.record(r.stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end)
    first = warmup + 1
    kv = sum(r.kv_tokens(first + i) for i in range(steps))
    algo = sum(r.algorithmic_bytes(first + i) for i in range(steps))
    # the partial kernel's launches, timed one by one on the stream they run on
    events = []
    for _ in range(steps):
        r.step(events)
    torch.cuda.synchronize()
    part_ms = [e0.elapsed_time(e1) for e0, e1, _ in events]
    # algorithmic bytes of each partial launch: the cache rows it attends
    first_ev = warmup + steps + 1
    part_bytes = []
    for i in range(steps):
        per_launch = r.layer_tokens(first_ev + i) * row_bytes(r.w.fmt)
        part_bytes += [per_launch] * r.w.layers
    avg_ms = float(np.mean(part_ms))
    avg_bytes = float(np.mean(part_bytes))
    res = {
        "workload": r.w.name, "fmt": r.w.fmt, "layers": r.w.layers, "batch": r.w.batch,
        "heads": r.w.heads, "num_splits": r.ns, "steps": steps, "warmup": warmup, "ms_per_step": ms / steps,
        "kv_tokens_per_step": kv / steps, "value": kv / (ms / 1e3),
        "gb_per_s": algo / (ms / 1e3) / 1e9,
        "partial_avg_us": avg_ms * 1e3, "partial_bytes_per_launch": avg_bytes,
        "partial_gb_per_s": avg_bytes / (avg_ms / 1e3) / 1e9,
        "partial_launches": len(part_ms),
    }
    res["hbm_frac"] = res["gb_per_s"] / HBM_PEAK_GBS
    res["prefill"] = append_result(r.w.name + " prefill", r.prefill_tokens, r.prefill_ms, r.w.fmt)
    log(f"{r.w.name}: {res['ms_per_step']:.3f} ms/step, {res['value'] / 1e9:.2f} G KV-tokens/s, "
        f"{res['gb_per_s']:.0f} GB/s step ({100 * res['hbm_frac']:.1f}% of 8 TB/s); partial kernel "
        f"{res['partial_avg_us']:.1f} us/launch, {res['partial_gb_per_s']:.0f} GB/s")
    del r
    torch.cuda.empty_cache()
    return res


def stored_traffic(name):
    """Counter-measured HBM bytes per partial launch, from profiles/, if the
    kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_partial_{name}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sha():
        return None
    return float(t.group(1))


def roofline(res):
    return {
        "bound": "hbm", "achieved": round(res["partial_gb_per_s"], 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(res["partial_gb_per_s"] / HBM_PEAK_GBS, 4),
        "traffic": stored_traffic(res["workload"]),
        "kernel": "split16_kernel (mla_decode_partial)",
        "per_launch_bytes": res["partial_bytes_per_launch"],
        "avg_launch_us": round(res["partial_avg_us"], 2),
        "launches_timed": res["partial_launches"],
    }


# ----------------------------------------------------------------- CPU side

def cpu_baseline(wid, seconds):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    workload: the sequences of layer 0, one fused decode step each (dequantize
    the cache rows; turn, quantize and append the new token; absorbed decode
    with the turned query in float64), in passes over the layer until about
    `seconds` of oracle time. Building the synthetic rows and quantizing the
    cached prefix is done once and not timed: on the GPU that cache is
    resident before the timed region."""
    from mla_latent_kv_cache_amd import workloads as W
    from oracle import quant as Q
    from oracle import rope as R
    w = W.WORKLOADS[wid]
    lens = W.lengths(wid)
    cos, sin = R.rope_tables(int(lens.max()) + 1)
    wuk, wuv = (t.float().numpy() for t in W.weights(wid, 0, "cpu"))
    qn, qp = (t.float().numpy() for t in W.queries(wid, 0, "cpu"))
    prepared = []
    for b in range(w.batch):
        c, k = W.latent_rows(wid, 0, b, int(lens[b]), "cpu")
        nc, nk = W.latent_rows(wid, 0, b, 1, "cpu", kind="step")
        prepared.append((Q.quantize_rows(c.float().numpy(), k.float().numpy(), w.fmt),
                         nc.float().numpy()[0], nk.float().numpy()[0]))
    tokens, elapsed, seqs, passes = 0, 0.0, 0, 0
    while elapsed < seconds:
        passes += 1
        for b, (planes, nc, nk) in enumerate(prepared):
            if elapsed >= seconds:
                break
            t0 = time.perf_counter()
            ch, kh = Q.dequantize_rows(planes, w.fmt)
            R.decode_step(ch, kh, int(lens[b]), int(lens[b]) + 1, nc, nk, qn[b], qp[b], wuk, wuv,
                          W.SOFTMAX_SCALE, w.fmt, cos, sin)
            elapsed += time.perf_counter() - t0
            tokens += int(lens[b]) + 1
            seqs += 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = None
    cores = len(os.sched_getaffinity(0))
    return {
        "value": tokens / elapsed, "unit": "KV-tokens/s",
        "cores": threads if threads else cores, "kind": "oracle",
        "sample": f"{seqs} sequence-steps in {passes} pass(es) over the {w.batch} sequences of layer 0 of "
                  f"{w.name} ({tokens} KV tokens), one fused decode step each: oracle RoPE, quantize and "
                  f"append of the new token, fp64 dequantize and absorbed decode; {elapsed:.1f}s of oracle "
                  f"time on {cores} host cores visible, BLAS threads {threads}",
    }


PMC_COPY_BYTES = 1 << 30  # the calibration copy: 1 GiB read, 1 GiB written


def pmc_run(wid):
    """Launches for counter collection (no timing): one step's partial-attention
    launches of the workload, then a plain device copy of PMC_COPY_BYTES twice.
    Run under `rocprofv3 --pmc FETCH_SIZE` and again under `--pmc WRITE_SIZE`."""
    import torch
    r = Runner(wid, 2)
    r.step()
    torch.cuda.synchronize()
    L = r.lib
    for layer in range(r.w.layers):
        qn, qp = r.args_q[layer]
        wuk, _ = r.args_w[layer]
        r.check(L.mla_decode_absorb(r.cref, qn, qp, wuk, r.H, r.scale, r.splits, r.ws_p, r.ws_n, r.sp), "absorb")
        r.check(L.mla_decode_partial(r.cref, layer, r.H, r.splits, r.ws_p, r.ws_n, r.sp), "partial")
    torch.cuda.synchronize()
    a = torch.ones(PMC_COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"pmc run: {r.w.layers} partial launches of {r.w.name}, 2 copies of {PMC_COPY_BYTES} bytes")


def _pmc_means(csv_path, counter):
    """Mean counter value (KiB) per dispatch for the partial kernel and the copy."""
    import csv
    vals = {"partial": {}, "copy": {}}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            kind = "partial" if "split16_kernel" in name else \
                "copy" if "copyBuffer" in name or "copy" in name.lower() else None
            if kind is None:
                continue
            d = vals[kind]
            d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    out = {}
    for kind, d in vals.items():
        v = sorted(d.values())
        if kind == "copy":  # the two large copies are the largest copy dispatches
            v = v[-2:]
        out[kind] = (float(np.mean(v)) if v else None, len(d))
    return out


def summarize_stats(wid, stats_csv, out_path, steps, warmup):
    """Write the profiles/ table of this library's kernels from a rocprofv3
    --kernel-trace --stats run of this script (its run_kernel_stats.csv)."""
    import csv
    from mla_latent_kv_cache_amd import workloads as W
    w = W.WORKLOADS[wid]
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            if "at::" in name or "rocclr" in name:
                continue  # torch kernels building the synthetic inputs, runtime copies
            m = re.search(r"(\w+_kernel)(?:<(\d)((?:, ?(?:true|false))*)>|I?L?i?(\d)E)?", name)
            flags = re.findall(r"true|false", m.group(3) or "") if m else []
            short = (m.group(1) + (f"<{m.group(2) or m.group(4)}>" if (m.group(2) or m.group(4)) else "")
                     + "".join(f" {tag}" for tag, f in zip(("paged", "sliced"), flags) if f == "true")) \
                if m else name[:40]
            rows.append((short, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6))
    rows.sort(key=lambda x: -x[5])
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 bench.py "
           f"--steps {steps} --warmup {warmup} --cpu-seconds 0 --int4-workload -1 --no-formats --workload {wid}")
    lines = [
        f"# rocprofv3 kernel statistics, {w.name}: {warmup} warmup + {steps} timed decode steps (every layer)",
        "# Commands (repository root, one MI355X):",
        f"#   {cmd}",
        f"#   python3 bench.py --summarize-stats <dir>/run_kernel_stats.csv --workload {wid} "
        f"--steps {steps} --warmup {warmup}",
        "# Rows: this library's kernels (the torch kernels that build the synthetic inputs are omitted).",
        "# append_kernel<f> is the prefill (one call per layer) and the benchmark's decode-time append of",
        "# 8 x 64 tokens (55 short calls). A decode step runs, per layer, step_kernel<f>",
        "# (mla_decode_step_begin: store the new token with its k_pe turned, absorb the turned query),",
        "# split16_kernel<f> (mla_decode_partial, 16 heads) and reduce_kernel (mla_decode_combine).",
        "# <f>: 0 bf16, 1 INT8, 2 INT4, 3 INT8 latent + bf16 k_pe, 4 INT4 latent + INT4 k_pe.",
        f"{'kernel':28s}{'calls':>7s}{'avg_us':>11s}{'min_us':>11s}{'max_us':>11s}{'total_ms':>11s}",
    ]
    for r in rows:
        lines.append(f"{r[0]:28s}{r[1]:7d}{r[2]:11.2f}{r[3]:11.2f}{r[4]:11.2f}{r[5]:11.3f}")
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {out_path}")


def summarize_pmc(wid, fetch_csv, write_csv, out_path):
    """Write the profiles/ summary that roofline() reads: HBM bytes per partial
    launch from FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter
    reads for the calibration copy of known size."""
    from mla_latent_kv_cache_amd import workloads as W
    w = W.WORKLOADS[wid]
    fe = _pmc_means(fetch_csv, "FETCH_SIZE")
    wr = _pmc_means(write_csv, "WRITE_SIZE")
    f_fetch = PMC_COPY_BYTES / (fe["copy"][0] * 1024.0)
    f_write = PMC_COPY_BYTES / (wr["copy"][0] * 1024.0)
    hbm = fe["partial"][0] * 1024.0 * f_fetch + wr["partial"][0] * 1024.0 * f_write
    lens = W.lengths(wid)
    algo = float(np.sum(lens + 1)) * row_bytes(w.fmt)  # the cache rows one launch attends
    text = f"""# HBM traffic of the partial-attention kernel, {w.name}
# Commands (from the repository root, on one MI355X; each pass is its own run):
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_fetch> -o run -- python3 bench.py --pmc-run --workload {wid}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_write> -o run -- python3 bench.py --pmc-run --workload {wid}
#   python3 bench.py --summarize-pmc <dir_fetch>/run_counter_collection.csv <dir_write>/run_counter_collection.csv --workload {wid}
# Calibration: a device copy of {PMC_COPY_BYTES} bytes reads FETCH_SIZE {fe['copy'][0]:.1f} KiB and
# WRITE_SIZE {wr['copy'][0]:.1f} KiB per dispatch; the partial kernel's counters are scaled by
# bytes/(KiB*1024) of the copy.
workload: {w.name}
partial_dispatches: {fe['partial'][1]}
fetch_kib_per_launch: {fe['partial'][0]:.1f}
write_kib_per_launch: {wr['partial'][0]:.1f}
copy_fetch_factor: {f_fetch:.4f}
copy_write_factor: {f_write:.4f}
algorithmic_bytes_per_launch: {algo:.0f}
hbm_bytes_per_launch: {hbm:.0f}
traffic_over_algorithmic: {hbm / algo:.3f}
kernel_source_sha256_16: {kernel_sha()}
"""
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write(text)
    log(f"wrote {out_path}: {hbm:.0f} HBM bytes per launch ({hbm / algo:.3f} x algorithmic)")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, help="index into workloads.WORKLOADS")
    ap.add_argument("--int4-workload", type=int, default=2, help="-1 to skip")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="0 to skip the CPU baseline")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the one-layer runs of the INT8_KBF16 and INT4_KINT4 formats and the paged layout")
    ap.add_argument("--pmc-run", action="store_true",
                    help="only issue the launches that the HBM counter summary is taken from")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="write profiles/kernel_stats_<workload>.txt from a rocprofv3 --stats run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/pmc_partial_<workload>.txt from two rocprofv3 counter runs")
    args = ap.parse_args()
    if args.summarize_stats:
        from mla_latent_kv_cache_amd import workloads as W
        name = W.WORKLOADS[args.workload].name
        summarize_stats(args.workload, args.summarize_stats,
                        os.path.join(ROOT, "profiles", f"kernel_stats_{name}.txt"), args.steps, args.warmup)
        return
    if args.summarize_pmc:
        from mla_latent_kv_cache_amd import workloads as W
        name = W.WORKLOADS[args.workload].name
        summarize_pmc(args.workload, args.summarize_pmc[0], args.summarize_pmc[1],
                      os.path.join(ROOT, "profiles", f"pmc_partial_{name}.txt"))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path here is single-GPU "
              "(see DESIGN.md for how it would shard). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    from mla_latent_kv_cache_amd import workloads as W
    if args.pmc_run:
        pmc_run(args.workload)
        return

    main_res = measure(args.workload, args.steps, args.warmup)
    # The one-layer runs below issue one partial launch per step where the
    # main run issues one per layer: they take that many times the steps and
    # warmup steps, so that they warm up and time as many launches. (With
    # the main run's step counts they time a few milliseconds just after a
    # new cache is filled, some 15% below their steady rate.)
    per_layer = W.WORKLOADS[args.workload].layers
    sub_steps, sub_warmup = args.steps * per_layer, args.warmup * per_layer
    keys = ("workload", "value", "ms_per_step", "gb_per_s", "hbm_frac", "kv_tokens_per_step", "num_splits",
            "steps", "warmup")
    int4 = None
    if args.int4_workload >= 0:
        r4 = measure(args.int4_workload, sub_steps, sub_warmup)
        int4 = {k: r4[k] for k in keys}
        int4["unit"] = "KV-tokens/s"
        int4["roofline"] = roofline(r4)
    formats = None
    if not args.no_formats:
        # the other two cache formats, on one layer of the same inputs: INT8
        # latent with bf16 k_pe on the ragged INT8 workload, INT4 with INT4
        # k_pe on the INT4 workload
        formats = {}
        for fmt, wid in (("int8_kbf16", args.workload), ("int4_kint4", max(args.int4_workload, 0))):
            rf = measure(wid, sub_steps, sub_warmup, fmt=fmt, layers=1)
            formats[fmt] = {k: rf[k] for k in keys}
            formats[fmt]["unit"] = "KV-tokens/s"
            formats[fmt]["roofline"] = roofline(rf)
        # the paged layout: one layer of the ragged INT8 inputs in 64-token pages, shuffled
        rp = measure(args.workload, sub_steps, sub_warmup, layers=1, page_size=64)
        formats["int8_paged64"] = {k: rp[k] for k in keys}
        formats["int8_paged64"]["unit"] = "KV-tokens/s"
        formats["int8_paged64"]["roofline"] = roofline(rp)
    # The wide-head workload (128 heads, INT4, 131072 tokens per sequence, 64 splits): bound by the matrix
    # units, not HBM, so its partial kernel is reported against the fp16 MFMA peak as well (not a headline line).
    wide = None
    if not args.no_formats:
        rw = measure(4, sub_steps, sub_warmup)
        tokens = rw["partial_bytes_per_launch"] / row_bytes(rw["fmt"])
        flops = tokens * rw["heads"] * 2 * (576 + 512)  # algorithmic score and value work per launch
        tflops = flops / (rw["partial_avg_us"] / 1e6) / 1e12
        wide = {k: rw[k] for k in keys}
        wide["unit"] = "KV-tokens/s"
        wide["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                            "flop_per_launch": flops, "avg_launch_us": round(rw["partial_avg_us"], 2),
                            "kernel": "split16_kernel (mla_decode_partial), 8 head slices"}
        wide["hbm_roofline"] = roofline(rw)
    append = {"prefill_" + main_res["fmt"]: main_res["prefill"], "decode_append_int8": measure_append64()}
    if args.int4_workload >= 0:
        append["prefill_int4"] = r4["prefill"]
    cpu = None
    if args.cpu_seconds > 0:
        log("timing the oracle on the host cores")
        cpu = cpu_baseline(args.workload, args.cpu_seconds)
    w = W.WORKLOADS[args.workload]
    line = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "cache_format": w.fmt, "layers": w.layers, "batch": w.batch,
            "heads": w.heads, "kv_lora_rank": 512, "rope_dim": 64, "seq_lens": "uniform [1024, 16384]"
            if isinstance(w.seq, tuple) else w.seq, "num_splits": main_res["num_splits"],
            "kv_tokens_per_step": main_res["kv_tokens_per_step"], "parallelism": "single GPU",
        },
        "gb_per_s": main_res["gb_per_s"],
        "hbm_frac": main_res["hbm_frac"],
        "roofline": roofline(main_res),
        "cpu_baseline": cpu,
        "int4": int4,
        "formats": formats,
        "wide_heads": wide,
        "append": append,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
