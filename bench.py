#!/usr/bin/env python3
"""Absorbed MLA decode on one MI355X: KV-tokens/s and achieved HBM GB/s.

A step is one decode step of the whole hot path over every layer of the
workload, through libmla_kv.so's fused decode step: (1) every sequence's new
token is stored, its k_pe turned by RoPE at its position and quantized, while
the turned query is absorbed through W_UK; (2) split-KV partial attention over
the quantized cache, the new token included; (3) merge of the splits and W_UV
projection. The 27 layers of the headline workload are independent, so one
step is one layer-range call over all of them (three launches); the same step
as 27 one-layer calls (81 launches) is reported beside it.

Default workload: DeepSeek-V2-Lite-shaped, 27 layers, 16 heads, batch 64,
ragged lengths uniform in [1024, 16384], INT8 latent + INT8 k_pe cache. The
INT4 workload (1 layer, batch 32, 16 heads, 32768 tokens, asymmetric INT4) is
measured in the same run and reported under "int4"; the other cache formats,
the paged layout and the 128-head workload under "formats" and "wide_heads";
the two small workloads (bf16 B1 S256, INT8 B8 S4096 with its 64-token
append) as microseconds per decode call under "latency".

One-layer runs: before each timed iteration (outside the timed events) a
1 GiB buffer is read through the library's stream-read aid, so that the
256 MB last-level cache holds none of the layer (a read, so no dirty lines
are written back inside the timed launch), and the sequence lengths are
reset, so every iteration attends exactly the named length plus the step's
own token. The same run measures the achievable HBM read rate
("hbm_ceiling") and matrix-unit rate ("mfma_ceiling") with the library's
measurement aids, and times the oracle on the host cores ("cpu_baseline").

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
FLUSH_BYTES = 1 << 30  # written between timed one-layer iterations (the MALL is 256 MB)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def row_bytes(fmt):
    from mla_latent_kv_cache_amd.cache import row_bytes as rb
    return rb(fmt)


def pct(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"p10": float(np.percentile(xs, 10)), "median": float(np.median(xs)),
            "p90": float(np.percentile(xs, 90)), "mean": float(xs.mean()), "n": int(xs.size)}


# ----------------------------------------------------------------- GPU side

class Flusher:
    """Reads a 1 GiB device buffer (mla_stream_read) on the stream, so that the
    next launch finds none of its inputs in the last-level cache. A read, not a
    write: written lines would be dirty in the cache and their write-back would
    land inside the next timed launch."""

    def __init__(self, torch):
        from mla_latent_kv_cache_amd import _lib
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.empty(4096, dtype=torch.int32, device="cuda")
        self.lib = _lib
        self.torch = torch

    def __call__(self):
        st = self.torch.cuda.current_stream()
        self.lib.check(self.lib.lib().mla_stream_read(ctypes.c_void_p(self.buf.data_ptr()), FLUSH_BYTES,
                                                      ctypes.c_void_p(self.sink.data_ptr()), 4096, 0,
                                                      ctypes.c_void_p(st.cuda_stream)), "flush")


class Runner:
    """One workload's cache, weights, queries and the ctypes calls of a step."""

    def __init__(self, wid, extra_steps, fmt=None, layers=None, page_size=0, splits=None):
        import dataclasses
        import torch
        from mla_latent_kv_cache_amd import LatentCache, _lib, rope_tables
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
        self.seq_lens0 = cache.seq_lens.clone()
        log(f"{w.name}: prefilled {int(self.lens0.sum()) * w.layers} tokens "
            f"({cache.bytes() / 1e9:.2f} GB of cache planes) in {time.time() - t0:.1f}s")
        self.H = w.heads
        self.splits = w.num_splits if splits is None else splits
        L = w.layers
        q = [W.queries(wid, layer, dev) for layer in range(L)]
        wts = [W.weights(wid, layer, dev) for layer in range(L)]
        # layer-stacked arguments of the layer-range calls; one-layer views of them
        self.qn = torch.stack([a for a, _ in q]).contiguous()
        self.qp = torch.stack([b for _, b in q]).contiguous()
        self.wuk = torch.stack([a for a, _ in wts]).contiguous()
        self.wuv = torch.stack([b for _, b in wts]).contiguous()
        del q, wts
        steps_new = [W.latent_batch(wid, layer, extra_steps, device=dev, kind="step") for layer in range(L)]
        self.c_new = torch.stack([c for c, _ in steps_new], dim=1).contiguous()  # [B, L, steps, 512] -> below
        self.k_new = torch.stack([k for _, k in steps_new], dim=1).contiguous()
        del steps_new
        # [steps][L][B][row]
        self.c_new = self.c_new.permute(2, 1, 0, 3).contiguous()
        self.k_new = self.k_new.permute(2, 1, 0, 3).contiguous()
        self.rope = rope_tables(cap + 1, device=dev)  # positions 0 .. capacity
        self.out = torch.empty((L, w.batch, self.H, 128), dtype=torch.float32, device=dev)
        self.lib = _lib.lib()
        self.check = _lib.check
        self.stream = torch.cuda.current_stream()
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)
        self.cref = ctypes.byref(cache.struct)
        self.scale = ctypes.c_float(W.SOFTMAX_SCALE)
        self.ws = cache.workspace_layers(L, self.H, self.splits)
        self.ws1 = cache.workspace(self.H, self.splits)
        self.ws_p, self.ws_n = ctypes.c_void_p(self.ws.data_ptr()), ctypes.c_size_t(self.ws.numel())
        self.ws1_p, self.ws1_n = ctypes.c_void_p(self.ws1.data_ptr()), ctypes.c_size_t(self.ws1.numel())
        self.rope_p = (ctypes.c_void_p(self.rope[0].data_ptr()), ctypes.c_void_p(self.rope[1].data_ptr()),
                       self.rope[0].shape[0])
        self.steps_done = 0
        self.ns = cache.auto_splits_layers(L, self.H) if self.splits == 0 else self.splits
        self.ns1 = cache.auto_splits(self.H) if self.splits == 0 else self.splits
        self.extra = extra_steps

    def _p(self, t):
        return ctypes.c_void_p(t.data_ptr())

    def step(self, events=None):
        """One decode step over every layer as one layer-range call, phase by
        phase. events: list to append (start, end) pairs recorded around the
        partial-attention launch."""
        L, i = self.lib, self.steps_done % self.extra
        n = self.w.layers
        cos_p, sin_p, rows = self.rope_p
        p = self._p
        st = L.mla_decode_step_begin_layers(self.cref, 0, n, p(self.c_new[i]), p(self.k_new[i]), p(self.qn),
                                            p(self.qp), cos_p, sin_p, rows, p(self.wuk), self.H, self.scale,
                                            self.splits, self.ws_p, self.ws_n, self.sp)
        if st:
            self.check(st, "step_begin_layers")
        if events is not None:
            e0 = self.torch.cuda.Event(enable_timing=True)
            e1 = self.torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
        st = L.mla_decode_partial_layers(self.cref, 0, n, self.H, self.splits, self.ws_p, self.ws_n, self.sp)
        if st:
            self.check(st, "partial_layers")
        if events is not None:
            e1.record(self.stream)
            events.append((e0, e1))
        st = L.mla_decode_combine_layers(self.cref, n, p(self.wuv), self.H, self.splits, self.ws_p, self.ws_n,
                                         p(self.out), self.sp)
        if st:
            self.check(st, "combine_layers")
        self.cache._lens = np.minimum(self.cache._lens + 1, self.cache.capacity)
        self.steps_done += 1

    def step_per_layer(self):
        """The same step as one-layer calls (three launches per layer)."""
        L, i = self.lib, self.steps_done % self.extra
        cos_p, sin_p, rows = self.rope_p
        p = self._p
        for layer in range(self.w.layers):
            st = L.mla_decode_step(self.cref, layer, p(self.c_new[i, layer]), p(self.k_new[i, layer]),
                                   p(self.qn[layer]), p(self.qp[layer]), cos_p, sin_p, rows, p(self.wuk[layer]),
                                   p(self.wuv[layer]), self.H, self.scale, self.splits, self.ws1_p, self.ws1_n,
                                   p(self.out[layer]), self.sp)
            if st:
                self.check(st, "step")
        self.cache._lens = np.minimum(self.cache._lens + 1, self.cache.capacity)
        self.steps_done += 1

    def reset_lengths(self):
        """Back to the prefilled lengths (a device copy on the stream, and the
        binding's host mirror)."""
        self.cache.seq_lens.copy_(self.seq_lens0)
        self.cache._lens[:] = np.broadcast_to(self.lens0, self.cache._lens.shape)

    def kv_tokens(self, attended_extra):
        """Tokens attended by one step when each sequence holds its prefill
        plus `attended_extra` tokens (the step's own token included)."""
        return int(self.w.layers * (self.lens0 + attended_extra).sum())

    def algorithmic_bytes(self, attended_extra):
        """Bytes the method must move in one step (per-token cache rows, the
        weights, the queries, the output and the appended rows)."""
        w = self.w
        cache = self.kv_tokens(attended_extra) * row_bytes(w.fmt)
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


def measure_stack(wid, steps, warmup, per_layer=True, splits=None):
    """The multi-layer workload: W untimed steps; K timed steps (one event
    between consecutive steps: value, ms_per_step and its spread); K steps
    with events around each partial-attention launch (its average duration,
    for the roofline); K steps as one-layer calls (81 launches each)."""
    import torch
    r = Runner(wid, 3 * steps + warmup + 1, layers=None, splits=splits)
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    log(f"{r.w.name}: warmup done ({warmup} steps); timing {steps} steps")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    first = r.steps_done + 1  # tokens held beyond the prefill during the first timed step
    ev[0].record(r.stream)
    for k in range(steps):
        r.step()
        ev[k + 1].record(r.stream)
    torch.cuda.synchronize()
    per_step = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
    ms = ev[0].elapsed_time(ev[steps])
    kv = sum(r.kv_tokens(first + i) for i in range(steps))
    algo = sum(r.algorithmic_bytes(first + i) for i in range(steps))
    # the partial kernel's launches, timed one by one on the stream they run on
    events = []
    first_ev = r.steps_done + 1
    for _ in range(steps):
        r.step(events)
    torch.cuda.synchronize()
    part_ms = [e0.elapsed_time(e1) for e0, e1 in events]
    part_bytes = [r.kv_tokens(first_ev + i) * row_bytes(r.w.fmt) for i in range(steps)]
    # the same steps as one-layer calls
    ms_pl, kv_pl = float("nan"), 0
    if per_layer:
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        first_pl = r.steps_done + 1
        t0.record(r.stream)
        for _ in range(steps):
            r.step_per_layer()
        t1.record(r.stream)
        torch.cuda.synchronize()
        ms_pl = t0.elapsed_time(t1)
        kv_pl = sum(r.kv_tokens(first_pl + i) for i in range(steps))
    avg_ms = float(np.mean(part_ms))
    avg_bytes = float(np.mean(part_bytes))
    res = {
        "workload": r.w.name, "fmt": r.w.fmt, "layers": r.w.layers, "batch": r.w.batch, "heads": r.w.heads,
        "num_splits": r.ns, "steps": steps, "warmup": warmup, "ms_per_step": ms / steps,
        "ms_per_step_spread": pct(per_step), "kv_tokens_per_step": kv / steps, "value": kv / (ms / 1e3),
        "gb_per_s": algo / (ms / 1e3) / 1e9,
        "partial_avg_us": avg_ms * 1e3, "partial_spread_us": pct(np.asarray(part_ms) * 1e3),
        "partial_bytes_per_launch": avg_bytes, "partial_gb_per_s": avg_bytes / (avg_ms / 1e3) / 1e9,
        "partial_launches": len(part_ms),
        "per_layer_calls": {"ms_per_step": ms_pl / steps, "value": kv_pl / (ms_pl / 1e3),
                            "launches_per_step": 3 * r.w.layers, "num_splits": r.ns1},
    }
    res["hbm_frac"] = res["gb_per_s"] / HBM_PEAK_GBS
    res["prefill"] = append_result(r.w.name + " prefill", r.prefill_tokens, r.prefill_ms, r.w.fmt)
    log(f"{r.w.name}: {res['ms_per_step']:.3f} ms/step (one call; {ms_pl / steps:.3f} as one-layer calls), "
        f"{res['value'] / 1e9:.2f} G KV-tokens/s, {res['gb_per_s']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% of "
        f"8 TB/s); partial kernel {res['partial_avg_us']:.1f} us/launch, {res['partial_gb_per_s']:.0f} GB/s")
    del r
    torch.cuda.empty_cache()
    return res


def measure_layer(wid, iters, warmup, flusher, fmt=None, page_size=0):
    """A one-layer workload: per iteration, outside the timed events, the
    lengths are reset to the prefill and the last-level cache is flushed;
    then one fused decode step (three launches) between events. A second set
    of iterations times the partial-attention launch alone."""
    import torch
    r = Runner(wid, 2, fmt=fmt, layers=1, page_size=page_size)
    assert r.w.layers == 1

    def run(n, part_events=None, step_events=None):
        for _ in range(n):
            r.reset_lengths()
            flusher()
            if step_events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(r.stream)
            r.step(part_events)
            if step_events is not None:
                e1.record(r.stream)
                step_events.append((e0, e1))
    run(warmup)
    torch.cuda.synchronize()
    steps_ev, part_ev = [], []
    run(iters, step_events=steps_ev)
    run(iters, part_events=part_ev)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in steps_ev])
    part_ms = np.array([a.elapsed_time(b) for a, b in part_ev])
    kv = r.kv_tokens(1)  # every iteration attends the prefill plus its own token
    algo = r.algorithmic_bytes(1)
    part_bytes = kv * row_bytes(r.w.fmt)
    med, pmed = float(np.median(step_ms)), float(np.median(part_ms))
    res = {
        "workload": r.w.name, "fmt": r.w.fmt, "layers": 1, "batch": r.w.batch, "heads": r.w.heads,
        "num_splits": r.ns, "iterations": iters, "warmup": warmup, "ms_per_step": med,
        "ms_per_step_spread": pct(step_ms), "kv_tokens_per_step": kv,
        "attended_tokens_per_sequence": float(np.mean(r.lens0 + 1)), "value": kv / (med / 1e3),
        "gb_per_s": algo / (med / 1e3) / 1e9,
        "partial_avg_us": float(part_ms.mean()) * 1e3, "partial_spread_us": pct(part_ms * 1e3),
        "partial_bytes_per_launch": float(part_bytes),
        "partial_gb_per_s": part_bytes / (float(part_ms.mean()) / 1e3) / 1e9,
        "partial_median_gb_per_s": part_bytes / (pmed / 1e3) / 1e9,
        "partial_launches": int(part_ms.size), "llc_flushed": True,
    }
    res["hbm_frac"] = res["gb_per_s"] / HBM_PEAK_GBS
    res["prefill"] = append_result(r.w.name + " prefill", r.prefill_tokens, r.prefill_ms, r.w.fmt)
    log(f"{r.w.name}: {med * 1e3:.1f} us/step (median), {res['value'] / 1e9:.2f} G KV-tokens/s; partial kernel "
        f"{res['partial_avg_us']:.1f} us/launch, {res['partial_gb_per_s']:.0f} GB/s")
    del r
    torch.cuda.empty_cache()
    return res


def measure_latency(wid, iters, flusher):
    """Microseconds per mla_decode_attn call of a small workload on its
    prefilled cache (no append), the last-level cache flushed before each
    call; for the INT8 B8 S4096 workload also the 64-token append (one
    mla_cache_append call) and the decode over the 4160 tokens after it."""
    import torch
    from mla_latent_kv_cache_amd import LatentCache
    from mla_latent_kv_cache_amd import workloads as W
    w = W.WORKLOADS[wid]
    lens = W.lengths(wid)
    cache = LatentCache(w.fmt, 1, w.batch, W.capacity(wid), device="cuda")
    ckv, kpe = W.latent_batch(wid, 0, int(lens.max()), device="cuda")
    cache.append(0, ckv, kpe)
    del ckv, kpe
    qn, qp = W.queries(wid, 0, "cuda")
    wuk, wuv = W.weights(wid, 0, "cuda")
    ws = cache.workspace(w.heads, w.num_splits)
    out = torch.empty((w.batch, w.heads, 128), dtype=torch.float32, device="cuda")

    def decode_us(n):
        evs = []
        for k in range(n + 5):
            flusher()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits, out=out, workspace=ws)
            e1.record()
            if k >= 5:
                evs.append((e0, e1))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs]) * 1e3

    res = {}
    us = decode_us(iters)
    res[w.name] = {"us_per_call": pct(us), "kv_tokens": int(lens.sum()), "calls": int(us.size),
                   "gb_per_s_median": (int(lens.sum()) * row_bytes(w.fmt) + 2 * w.heads * 128 * 512 * 2)
                   / (np.median(us) / 1e6) / 1e9, "llc_flushed": True}
    log(f"{w.name}: decode call {np.median(us):.1f} us (median, p10 {np.percentile(us, 10):.1f}, "
        f"p90 {np.percentile(us, 90):.1f})")
    if w.append:
        new = W.latent_batch(wid, 0, w.append, device="cuda", kind="append")
        evs = []
        for k in range(iters + 5):  # the append into rows 4096..4159, lengths restored each time
            cache.seq_lens.fill_(int(lens[0]))
            flusher()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            cache.append(0, *new)
            cache._lens[0] -= w.append
            e1.record()
            if k >= 5:
                evs.append((e0, e1))
        torch.cuda.synchronize()
        app = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
        cache._lens[0] += w.append  # the last append stays
        us2 = decode_us(iters)
        n2 = int(lens.sum()) + w.batch * w.append
        res[f"{w.name}_append{w.append}"] = {
            "append_us_per_call": pct(app), "appended_tokens": w.batch * w.append,
            "decode_after_append": {"us_per_call": pct(us2), "kv_tokens": n2, "calls": int(us2.size)},
            "llc_flushed": True}
        log(f"{w.name}: append of {w.append} tokens per sequence {np.median(app):.1f} us, decode over "
            f"{int(lens[0]) + w.append} tokens {np.median(us2):.1f} us (medians)")
    del cache
    torch.cuda.empty_cache()
    return res


def measure_stream_read(nbytes=4 << 30, iters=20):
    """Achievable HBM read rate: mla_stream_read (non-temporal loads, as the
    partial kernel's latent loads) over a 4 GiB buffer, for a few grid sizes;
    the best median."""
    import torch
    from mla_latent_kv_cache_amd import _lib
    L = _lib.lib()
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    stream = torch.cuda.current_stream()
    best = None
    rows = {}
    for grid in (1024, 2048, 4096, 8192, 16384):
        sink = torch.empty(grid, dtype=torch.int32, device="cuda")
        ms = []
        for k in range(iters + 3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _lib.check(L.mla_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                         grid, 1, ctypes.c_void_p(stream.cuda_stream)), "stream_read")
            e1.record(stream)
            if k >= 3:
                ms.append((e0, e1))
        torch.cuda.synchronize()
        med = float(np.median([a.elapsed_time(b) for a, b in ms]))
        gbs = nbytes / (med / 1e3) / 1e9
        rows[grid] = round(gbs, 1)
        if best is None or gbs > best[0]:
            best = (gbs, grid)
    del buf
    torch.cuda.empty_cache()
    log(f"stream read: {best[0]:.0f} GB/s ({100 * best[0] / HBM_PEAK_GBS:.1f}% of 8 TB/s) at {best[1]} workgroups")
    return {"gb_per_s": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4), "bytes": nbytes,
            "workgroups": best[1], "by_workgroups": rows, "kernel": "stream_read_kernel (mla_stream_read)"}


def measure_mfma_rate(iters=4000, reps=5):
    """Achievable fp16 matrix-unit rate: mla_mfma_rate with four waves per
    SIMD (4 workgroups of 256 threads per CU); the best of a few launches."""
    import torch
    from mla_latent_kv_cache_amd import _lib
    L = _lib.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 4 * cus
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    best = 0.0
    for k in range(reps + 2):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        _lib.check(L.mla_mfma_rate(ctypes.c_void_p(sink.data_ptr()), wgs, iters, ctypes.c_void_p(stream.cuda_stream)),
                   "mfma_rate")
        e1.record(stream)
        torch.cuda.synchronize()
        if k >= 2:
            flops = wgs * 4 * iters * 8 * 16 * 16 * 32 * 2
            best = max(best, flops / (e0.elapsed_time(e1) / 1e3) / 1e12)
    log(f"matrix units: {best:.0f} TFLOP/s of 16x16x32 fp16 products ({best / MFMA_F16_PEAK_TFLOPS:.3f} of the "
        f"{MFMA_F16_PEAK_TFLOPS:.0f} TFLOP/s peak)")
    return {"tflop_per_s": round(best, 1), "frac_of_peak": round(best / MFMA_F16_PEAK_TFLOPS, 4),
            "workgroups": wgs, "kernel": "mfma_rate_kernel (mla_mfma_rate), 8 independent chains per wave"}


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


def roofline(res, ceiling=None):
    """The partial kernel against the published HBM peak (and, where given,
    against the stream-read rate measured in the same run)."""
    extra = {}
    if ceiling:
        extra["frac_of_measured_stream_read"] = round(res["partial_gb_per_s"] / ceiling["gb_per_s"], 4)
    return {
        "bound": "hbm", "achieved": round(res["partial_gb_per_s"], 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(res["partial_gb_per_s"] / HBM_PEAK_GBS, 4), **extra,
        "traffic": stored_traffic(res["workload"]),
        "kernel": "%s (mla_decode_partial%s)" % (
            "wide_kernel" if res["heads"] > 16 and not res["fmt"].startswith("int4") else "split16_kernel",
            "_layers" if res["layers"] > 1 else ""),
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


def pmc_run(wid, fmt=None, layers=None, page_size=0):
    """Launches for counter collection (no timing): the workload's partial-
    attention launch (all its layers in one layer-range call), then a plain
    device copy of PMC_COPY_BYTES twice. Run under `rocprofv3 --pmc
    FETCH_SIZE` and again under `--pmc WRITE_SIZE`."""
    import torch
    r = Runner(wid, 2, fmt=fmt, layers=layers, page_size=page_size)
    r.step()
    torch.cuda.synchronize()
    r.reset_lengths()
    r.step()
    torch.cuda.synchronize()
    a = torch.ones(PMC_COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"pmc run: 2 steps of {r.w.name} (one partial launch each), 2 copies of {PMC_COPY_BYTES} bytes")
    return r.w.name


def _pmc_means(csv_path, counter):
    """Mean counter value (KiB) per dispatch for the partial kernel and the copy."""
    import csv
    vals = {"partial": {}, "copy": {}}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            kind = "partial" if "split16_kernel" in name or "wide_kernel" in name else \
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


def workload_name(wid, fmt=None, layers=None, page_size=0):
    from mla_latent_kv_cache_amd import workloads as W
    w = W.WORKLOADS[wid]
    name = w.name
    if fmt is not None or layers is not None:
        fmt, layers = fmt or w.fmt, layers or w.layers
        name = f"{fmt}_l{layers}_{w.name.split('_', 2)[2]}"
    if page_size:
        name = f"{name}_paged{page_size}"
    return name


def summarize_stats(name, stats_csv, out_path, cmd):
    """Write the profiles/ table of this library's kernels from a rocprofv3
    --kernel-trace --stats run of this script (its run_kernel_stats.csv)."""
    import csv
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            kname = r["Name"]
            if "at::" in kname or "rocclr" in kname:
                continue  # torch kernels building the synthetic inputs, runtime copies
            m = re.search(r"(\w+_kernel)(?:<(\d+)((?:, ?(?:true|false))*)>|I?L?i?(\d+)E)?", kname)
            flags = re.findall(r"true|false", m.group(3) or "") if m else []
            short = (m.group(1) + (f"<{m.group(2) or m.group(4)}>" if (m.group(2) or m.group(4)) else "")
                     + "".join(f" {tag}" for tag, f in zip(("paged", "sliced"), flags) if f == "true")) \
                if m else kname[:40]
            rows.append((short, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6))
    rows.sort(key=lambda x: -x[5])
    lines = [
        f"# rocprofv3 kernel statistics, {name}",
        "# Command (repository root, one MI355X):",
        f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 bench.py {cmd}",
        f"#   python3 bench.py --summarize-stats <dir>/run_kernel_stats.csv --stats-name {name} "
        f"--stats-cmd '{cmd}'",
        "# Rows: this library's kernels (the torch kernels that build the synthetic inputs are omitted).",
        "# step_kernel<f>: mla_decode_step_begin[_layers] (store the new tokens with k_pe turned, absorb",
        "# the turned queries); split16_kernel<f>: the partial attention, 16 heads per workgroup (sliced:",
        "# one workgroup per 16-head slice); wide_kernel<f>: the partial attention, 32 heads per workgroup;",
        "# combine_kernel<R>: the merge of the partial records and the W_UV projection, R sequences per",
        "# workgroup (reduce_kernel: 4, reduce1_kernel: one, for smaller grids); append_kernel<f>: the",
        "# prefill; stream_read_kernel: the read of a 1 GiB buffer that evicts the last-level cache between",
        "# one-layer runs (not part of the decode).",
        "# <f>: 0 bf16, 1 INT8, 2 INT4, 3 INT8 latent + bf16 k_pe, 4 INT4 latent + INT4 k_pe.",
        f"{'kernel':32s}{'calls':>7s}{'avg_us':>11s}{'min_us':>11s}{'max_us':>11s}{'total_ms':>11s}",
    ]
    for r in rows:
        lines.append(f"{r[0]:32s}{r[1]:7d}{r[2]:11.2f}{r[3]:11.2f}{r[4]:11.2f}{r[5]:11.3f}")
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {out_path}")


def summarize_pmc(wid, fmt, layers, page_size, fetch_csv, write_csv, out_path):
    """Write the profiles/ summary that roofline() reads: HBM bytes per partial
    launch from FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter
    reads for the calibration copy of known size."""
    from mla_latent_kv_cache_amd import workloads as W
    w = W.WORKLOADS[wid]
    name = workload_name(wid, fmt, layers, page_size)
    fmt_eff = fmt or w.fmt
    n_layers = layers or w.layers
    fe = _pmc_means(fetch_csv, "FETCH_SIZE")
    wr = _pmc_means(write_csv, "WRITE_SIZE")
    f_fetch = PMC_COPY_BYTES / (fe["copy"][0] * 1024.0)
    f_write = PMC_COPY_BYTES / (wr["copy"][0] * 1024.0)
    hbm = fe["partial"][0] * 1024.0 * f_fetch + wr["partial"][0] * 1024.0 * f_write
    lens = W.lengths(wid)
    algo = float(np.sum(lens + 1)) * n_layers * row_bytes(fmt_eff)  # the cache rows one launch attends
    args = f"--workload {wid}" + (f" --fmt {fmt}" if fmt else "") + (f" --layers {layers}" if layers else "") + \
        (f" --page-size {page_size}" if page_size else "")
    text = f"""# HBM traffic of the partial-attention kernel, {name}
# Commands (from the repository root, on one MI355X; each pass is its own run):
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_fetch> -o run -- python3 bench.py --pmc-run {args}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_write> -o run -- python3 bench.py --pmc-run {args}
#   python3 bench.py --summarize-pmc <dir_fetch>/run_counter_collection.csv <dir_write>/run_counter_collection.csv {args}
# Calibration: a device copy of {PMC_COPY_BYTES} bytes reads FETCH_SIZE {fe['copy'][0]:.1f} KiB and
# WRITE_SIZE {wr['copy'][0]:.1f} KiB per dispatch; the partial kernel's counters are scaled by
# bytes/(KiB*1024) of the copy.
workload: {name}
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
    # the GPU's clocks take some ten 2 ms steps to settle after the prefill
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--iters", type=int, default=100, help="timed iterations of each one-layer run")
    ap.add_argument("--workload", type=int, default=3, help="index into workloads.WORKLOADS")
    ap.add_argument("--int4-workload", type=int, default=2, help="-1 to skip")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="0 to skip the CPU baseline")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the one-layer runs of the other formats, the paged layout and the 128-head workload")
    ap.add_argument("--no-latency", action="store_true", help="skip the small workloads' per-call latency")
    ap.add_argument("--only", choices=["stack", "layer"], help="profiling runs: only the stack or one layer")
    ap.add_argument("--no-per-layer", action="store_true", help="(with --only stack) skip the one-layer calls")
    ap.add_argument("--splits", type=int, help="(with --only stack) the split count instead of the workload's")
    ap.add_argument("--fmt", help="(with --only layer / --pmc-run) another cache format for the workload")
    ap.add_argument("--layers", type=int, help="(with --pmc-run) layers of the workload to use")
    ap.add_argument("--page-size", type=int, default=0, help="(with --only layer / --pmc-run) paged layout")
    ap.add_argument("--pmc-run", action="store_true",
                    help="only issue the launches that the HBM counter summary is taken from")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="write profiles/kernel_stats_<name>.txt from a rocprofv3 --stats run")
    ap.add_argument("--stats-name", help="workload name for --summarize-stats")
    ap.add_argument("--stats-cmd", default="", help="the bench.py arguments of the profiled run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/pmc_partial_<name>.txt from two rocprofv3 counter runs")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.stats_name, args.summarize_stats,
                        os.path.join(ROOT, "profiles", f"kernel_stats_{args.stats_name}.txt"), args.stats_cmd)
        return
    if args.summarize_pmc:
        name = workload_name(args.workload, args.fmt, args.layers, args.page_size)
        summarize_pmc(args.workload, args.fmt, args.layers, args.page_size, args.summarize_pmc[0],
                      args.summarize_pmc[1], os.path.join(ROOT, "profiles", f"pmc_partial_{name}.txt"))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path here runs on a single GPU. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    from mla_latent_kv_cache_amd import workloads as W
    if args.pmc_run:
        pmc_run(args.workload, args.fmt, args.layers, args.page_size)
        return
    if args.only == "stack":
        measure_stack(args.workload, args.steps, args.warmup, per_layer=not args.no_per_layer, splits=args.splits)
        return
    if args.only == "layer":
        measure_layer(args.workload, args.iters, args.warmup, Flusher(torch), fmt=args.fmt,
                      page_size=args.page_size)
        return

    ceiling = measure_stream_read()
    mfma_ceiling = measure_mfma_rate()
    main_res = measure_stack(args.workload, args.steps, args.warmup)
    flusher = Flusher(torch)
    keys = ("workload", "value", "ms_per_step", "ms_per_step_spread", "gb_per_s", "hbm_frac", "kv_tokens_per_step",
            "attended_tokens_per_sequence", "num_splits", "iterations", "warmup", "llc_flushed")
    int4 = None
    if args.int4_workload >= 0:
        r4 = measure_layer(args.int4_workload, args.iters, args.warmup, flusher)
        int4 = {k: r4[k] for k in keys if k in r4}
        int4["unit"] = "KV-tokens/s"
        int4["roofline"] = roofline(r4, ceiling)
    formats = None
    wide = None
    if not args.no_formats:
        # the other two cache formats, on one layer of the same inputs: INT8
        # latent with bf16 k_pe on the ragged INT8 workload, INT4 with INT4
        # k_pe on the INT4 workload; the ragged INT8 layer in shuffled 64-token pages
        formats = {}
        for key, wid, fmt, ps in (("int8_kbf16", args.workload, "int8_kbf16", 0),
                                  ("int4_kint4", max(args.int4_workload, 0), "int4_kint4", 0),
                                  ("int8_paged64", args.workload, None, 64)):
            rf = measure_layer(wid, args.iters, args.warmup, flusher, fmt=fmt, page_size=ps)
            formats[key] = {k: rf[k] for k in keys if k in rf}
            formats[key]["unit"] = "KV-tokens/s"
            formats[key]["roofline"] = roofline(rf, ceiling)
        # The wide-head workload (128 heads, INT4, 131072 tokens per sequence, 64 splits): bound by the
        # matrix units, not HBM, so its partial kernel is reported against the fp16 MFMA peak as well.
        # The same inputs in the INT8 format run the 32-head kernel (wide_int8).
        for key, fmt, kern in (("wide", None, "split16_kernel (mla_decode_partial), 8 head slices"),
                               ("wide_int8", "int8", "wide_kernel (mla_decode_partial), 4 slices of 32 heads")):
            rw = measure_layer(4, max(20, args.iters // 4), args.warmup, flusher, fmt=fmt)
            tokens = rw["partial_bytes_per_launch"] / row_bytes(rw["fmt"])
            flops = tokens * rw["heads"] * 2 * (576 + 512)  # algorithmic score and value work per launch
            tflops = flops / (rw["partial_avg_us"] / 1e6) / 1e12
            rec = {k: rw[k] for k in keys if k in rw}
            rec["unit"] = "KV-tokens/s"
            rec["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                               "frac_of_measured_mfma_rate": round(tflops / mfma_ceiling["tflop_per_s"], 4),
                               "flop_per_launch": flops, "avg_launch_us": round(rw["partial_avg_us"], 2),
                               "kernel": kern}
            rec["hbm_roofline"] = roofline(rw)
            if key == "wide":
                wide = rec
            else:
                wide["int8"] = rec
    latency = None
    if not args.no_latency:
        latency = {}
        for wid in (0, 1):
            latency.update(measure_latency(wid, args.iters, flusher))
    append = {"prefill_" + main_res["fmt"]: main_res["prefill"]}
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
        "ms_per_step_spread": main_res["ms_per_step_spread"],
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
            "call": "mla_decode_step_layers over the 27 layers (3 launches per step)",
        },
        "gb_per_s": main_res["gb_per_s"],
        "hbm_frac": main_res["hbm_frac"],
        "per_layer_calls": main_res["per_layer_calls"],
        "roofline": roofline(main_res, ceiling),
        "hbm_ceiling": ceiling,
        "mfma_ceiling": mfma_ceiling,
        "cpu_baseline": cpu,
        "int4": int4,
        "formats": formats,
        "wide_heads": wide,
        "latency": latency,
        "append": append,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
