"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from mla_latent_kv_cache_amd import LatentCache
from mla_latent_kv_cache_amd import workloads as W
from oracle import attention as A
from oracle import quant as Q

# The attention tolerance: |gpu - oracle| <= 2e-3 + 1e-2 |oracle|, elementwise.
TOL_ABS = 2e-3
TOL_REL = 1e-2


def f32(t):
    return t.detach().float().cpu().numpy()


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = TOL_ABS + TOL_REL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {got[i]:.6g} oracle {ref[i]:.6g}")
    return float(err.max())


def oracle_planes(ckv, kpe, fmt):
    """The oracle's quantization of bf16 rows (torch tensors on any device)."""
    return Q.quantize_rows(f32(ckv), f32(kpe), fmt)


def _same_bits(a, b, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if b.dtype == np.float16:
        b = b.view(np.uint16)
    if a.dtype == np.float32:
        a = a.view(np.uint32)
    if b.dtype == np.float32:
        b = b.view(np.uint32)
    diff = np.argwhere(a != b.astype(a.dtype))
    if len(diff):
        i = tuple(diff[0])
        raise AssertionError(f"{what}: {len(diff)} differ, first at {i}: gpu {a[i]:#x} oracle {b[i]:#x}")


def assert_planes_equal(got, ref, fmt, what=""):
    """Bit-exact comparison of GPU cache planes with the oracle's (every plane
    the format has; bf16 planes compared as their fp32 widening)."""
    assert set(got) == set(ref), (sorted(got), sorted(ref))
    for key in ref:
        g = got[key]
        g = g.float().numpy() if g.dtype == torch.bfloat16 else g.numpy()
        _same_bits(g, ref[key], f"{what}: {fmt} {key}")


def oracle_decode(ckv, kpe, fmt, q_nope, q_pe, w_uk, w_uv, scale=W.SOFTMAX_SCALE):
    """Oracle output [H,128] for one sequence given its bf16 rows."""
    ch, kh = Q.dequantize_rows(oracle_planes(ckv, kpe, fmt), fmt)
    return A.decode_absorbed(f32(q_nope), f32(q_pe), f32(w_uk), f32(w_uv), ch, kh, scale)


def random_rows(n, seed, dist="outlier", device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    c = torch.randn((n, 512), generator=g, device=device)
    if dist == "skew":
        c = c.abs() * 1.5 - 0.5
    if dist in ("outlier", "skew"):
        c[:, [3, 100, 257, 511]] *= 20
    k = torch.randn((n, 64), generator=g, device=device)
    return c.to(torch.bfloat16), k.to(torch.bfloat16)


def random_problem(fmt, B, H, lens, seed, cap=None, device="cuda"):
    """A filled cache plus queries and weights; returns (cache, rows, q_nope, q_pe, w_uk, w_uv)."""
    lens = [int(x) for x in lens]
    cap = cap or max(max(lens), 1)
    cache = LatentCache(fmt, 1, B, cap, device=device)
    n = max(max(lens), 1)
    ckv = torch.zeros((B, n, 512), dtype=torch.bfloat16, device=device)
    kpe = torch.zeros((B, n, 64), dtype=torch.bfloat16, device=device)
    rows = []
    for b in range(B):
        c, k = random_rows(n, seed * 101 + b, "skew" if fmt.startswith("int4") else "outlier", device)
        ckv[b], kpe[b] = c, k
        rows.append((c[:lens[b]], k[:lens[b]]))
    cache.append(0, ckv, kpe, n_new=lens)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q_nope = torch.randn((B, H, 128), generator=g, device=device).to(torch.bfloat16)
    q_pe = torch.randn((B, H, 64), generator=g, device=device).to(torch.bfloat16)
    w_uk = (torch.randn((H, 128, 512), generator=g, device=device) / 512 ** 0.5).to(torch.bfloat16)
    w_uv = (torch.randn((H, 512, 128), generator=g, device=device) / 512 ** 0.5).to(torch.bfloat16)
    return cache, rows, q_nope, q_pe, w_uk, w_uv


def build_workload(wid, device="cuda", fmt=None):
    """Prefill the cache of a named workload through mla_cache_append (fmt:
    the same inputs stored in another cache format)."""
    w = W.WORKLOADS[wid]
    lens = W.lengths(wid)
    cache = LatentCache(fmt or w.fmt, w.layers, w.batch, W.capacity(wid), device=device)
    ragged = isinstance(w.seq, tuple)
    for layer in range(w.layers):
        ckv, kpe = W.latent_batch(wid, layer, int(lens.max()), device=device,
                                  counts=lens if ragged else None)
        cache.append(layer, ckv, kpe, n_new=lens if ragged else None)
        del ckv, kpe
    torch.cuda.synchronize()
    return cache, lens


def oracle_threads():
    """Host threads for oracle work that runs beside a GPU test (numpy releases
    the interpreter lock in its array loops and in BLAS)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_oracle_jobs(jobs, threads=None, window=None):
    """Run oracle jobs on a thread pool and yield (key, result) in submission
    order. `jobs` yields (key, fn, args); the producer side (which may make GPU
    tensors and copy them to the host) runs on the calling thread, at most
    `window` jobs ahead of the results consumed."""
    threads = threads or oracle_threads()
    window = window or 2 * threads
    pending = []
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for key, fn, args in jobs:
            pending.append((key, pool.submit(fn, *args)))
            while len(pending) >= window:
                k, fut = pending.pop(0)
                yield k, fut.result()
        for k, fut in pending:
            yield k, fut.result()


def oracle_decode_np(ckv, kpe, fmt, q_nope, q_pe, w_uk, w_uv, scale=W.SOFTMAX_SCALE):
    """oracle_decode on host float32 arrays (thread-pool friendly: no torch)."""
    ch, kh = Q.dequantize_rows(Q.quantize_rows(ckv, kpe, fmt), fmt)
    return A.decode_absorbed(q_nope, q_pe, w_uk, w_uv, ch, kh, scale)


def stacked_problem(fmt, L, B, H, lens, seed, cap, page_size=0, table=None, dist=None):
    """lens [L][B]; returns (cache, rows[l][b], q_nope [L,B,H,128], q_pe, w_uk [L,...], w_uv).
    dist: the latent distribution (default: skewed for INT4 latents, outlier
    channels otherwise)."""
    kw = {}
    if page_size:
        kw = dict(page_size=page_size, num_pages=table.numel() + 3, block_table=table)
    cache = LatentCache(fmt, L, B, cap, device="cuda", **kw)
    rows = []
    n = max(1, max(max(r) for r in lens))
    for l in range(L):
        ckv = torch.zeros((B, n, 512), dtype=torch.bfloat16, device="cuda")
        kpe = torch.zeros((B, n, 64), dtype=torch.bfloat16, device="cuda")
        rl = []
        for b in range(B):
            c, k = random_rows(n, seed * 1009 + l * 101 + b, dist or ("skew" if fmt.startswith("int4") else "outlier"))
            ckv[b], kpe[b] = c, k
            rl.append((c[:lens[l][b]], k[:lens[l][b]]))
        cache.append(l, ckv, kpe, n_new=lens[l])
        rows.append(rl)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    qn = torch.randn((L, B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    qp = torch.randn((L, B, H, 64), generator=g, device="cuda").to(torch.bfloat16)
    wuk = (torch.randn((L, H, 128, 512), generator=g, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
    wuv = (torch.randn((L, H, 512, 128), generator=g, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
    return cache, rows, qn, qp, wuk, wuv
