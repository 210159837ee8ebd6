"""The five named workloads at their full sizes: caches prefilled through
mla_cache_append, codes checked bit-exactly on sampled rows, and the decode
output of every sequence (of layers 0, 13 and 26 for the 27-layer stack)
checked against the fp64 oracle one by one."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import LatentCache
from mla_latent_kv_cache_amd import workloads as W

from gpu_util import (assert_close, assert_planes_equal, build_workload, f32, oracle_decode_np,
                      oracle_planes, run_oracle_jobs)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def rows_of(wid, layer, b, n):
    return W.latent_rows(wid, layer, b, n, device="cuda")


def check_sequences(wid, cache, layer, samples, out, q_nope, q_pe, w_uk, w_uv, extra=None, fmt=None):
    """Every sampled sequence's output against the fp64 oracle, one by one
    (the oracle work runs on a host thread pool)."""
    w = W.WORKLOADS[wid]
    fmt = fmt or w.fmt
    lens = cache.lengths(layer)
    qn, qp, wk, wv = f32(q_nope), f32(q_pe), f32(w_uk), f32(w_uv)
    out_h = f32(out)

    def jobs():
        for b in samples:
            c, k = rows_of(wid, layer, b, int(W.lengths(wid)[b]))
            if extra is not None:
                c = torch.cat([c, extra[0][b]])
                k = torch.cat([k, extra[1][b]])
            assert c.shape[0] == lens[b]
            yield b, oracle_decode_np, (f32(c), f32(k), fmt, qn[b], qp[b], wk, wv)

    worst = 0.0
    for b, ref in run_oracle_jobs(jobs()):
        worst = max(worst, assert_close(out_h[b], ref, f"{w.name} layer {layer} seq {b}"))
    print(f"  {w.name} layer {layer}: {len(samples)} sequences, max abs err {worst:.2e}", flush=True)


def check_codes(wid, cache, layer, b, nrows=None):
    w = W.WORKLOADS[wid]
    n = int(W.lengths(wid)[b])
    c, k = rows_of(wid, layer, b, n)
    got = cache.planes(layer, b)
    if nrows is not None:  # a sample of rows spread over the sequence
        idx = np.unique(np.linspace(0, n - 1, nrows).astype(int))
        got = {key: v[idx] for key, v in got.items()}
        c, k = c[idx], k[idx]
    assert_planes_equal(got, oracle_planes(c, k, w.fmt), w.fmt, f"{w.name} layer {layer} seq {b}")


def test_workload0_bf16_full():
    wid = 0
    cache, lens = build_workload(wid)
    check_codes(wid, cache, 0, 0)
    qn, qp = W.queries(wid, 0, "cuda")
    wuk, wuv = W.weights(wid, 0, "cuda")
    out = cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=W.WORKLOADS[wid].num_splits)
    torch.cuda.synchronize()
    check_sequences(wid, cache, 0, range(1), out, qn, qp, wuk, wuv)


def test_workload1_int8_append64_full():
    wid = 1
    w = W.WORKLOADS[wid]
    cache, lens = build_workload(wid)
    for b in (0, 7):
        check_codes(wid, cache, 0, b)
    qn, qp = W.queries(wid, 0, "cuda")
    wuk, wuv = W.weights(wid, 0, "cuda")
    out = cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits)
    torch.cuda.synchronize()
    check_sequences(wid, cache, 0, range(w.batch), out, qn, qp, wuk, wuv)
    # quantize-on-append of 64 tokens per sequence, then decode over 4160
    new = W.latent_batch(wid, 0, w.append, device="cuda", kind="append")
    cache.append(0, *new)
    out = cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits)
    torch.cuda.synchronize()
    assert cache.lengths(0).tolist() == [4096 + 64] * w.batch
    check_sequences(wid, cache, 0, range(w.batch), out, qn, qp, wuk, wuv, extra=new)
    got = cache.planes(0, 3)
    tail = {key: v[4096:] for key, v in got.items()}
    assert_planes_equal(tail, oracle_planes(new[0][3], new[1][3], "int8"), "int8", "appended rows")


def test_workload2_int4_full():
    wid = 2
    w = W.WORKLOADS[wid]
    cache, lens = build_workload(wid)
    check_codes(wid, cache, 0, 0)
    check_codes(wid, cache, 0, 31, nrows=2000)
    qn, qp = W.queries(wid, 0, "cuda")
    wuk, wuv = W.weights(wid, 0, "cuda")
    out = cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    check_sequences(wid, cache, 0, range(w.batch), out, qn, qp, wuk, wuv)


def test_workload3_int8_full_stack_ragged():
    wid = 3
    w = W.WORKLOADS[wid]
    cache, lens = build_workload(wid)
    assert cache.lengths().shape == (27, 64)
    assert (cache.lengths() == lens[None]).all()
    samples = {layer: range(w.batch) for layer in (0, 13, 26)}
    code_seq = {0: 0, 13: int(np.argmax(lens)), 26: int(np.argmin(lens))}
    wuk_all, wuv_all, q_all, outs = {}, {}, {}, {}
    for layer in range(w.layers):
        qn, qp = W.queries(wid, layer, "cuda")
        wuk, wuv = W.weights(wid, layer, "cuda")
        outs[layer] = cache.decode(layer, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits)
        if layer in samples:
            q_all[layer], wuk_all[layer], wuv_all[layer] = (qn, qp), wuk, wuv
    torch.cuda.synchronize()
    for layer in range(w.layers):
        assert torch.isfinite(outs[layer]).all(), layer
    for layer, bs in samples.items():
        check_codes(wid, cache, layer, code_seq[layer], nrows=500)
        qn, qp = q_all[layer]
        check_sequences(wid, cache, layer, bs, outs[layer], qn, qp, wuk_all[layer], wuv_all[layer])


def test_workload4_int4_wide_heads_64_splits_full():
    wid = 4
    w = W.WORKLOADS[wid]
    cache, lens = build_workload(wid)
    check_codes(wid, cache, 0, 5, nrows=3000)
    qn, qp = W.queries(wid, 0, "cuda")
    wuk, wuv = W.weights(wid, 0, "cuda")
    out = cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    check_sequences(wid, cache, 0, range(w.batch), out, qn, qp, wuk, wuv)


def test_workload4_inputs_int8_32_head_kernel_full():
    """The 128-head inputs stored as INT8 (the layer the benchmark times on the
    32-head kernel), 64 splits: every sequence against the oracle."""
    wid = 4
    w = W.WORKLOADS[wid]
    cache, lens = build_workload(wid, fmt="int8")
    qn, qp = W.queries(wid, 0, "cuda")
    wuk, wuv = W.weights(wid, 0, "cuda")
    out = cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    check_sequences(wid, cache, 0, range(w.batch), out, qn, qp, wuk, wuv, fmt="int8")


def test_workload3_int8_one_layer_paged64():
    """One layer of the ragged INT8 inputs in 64-token pages handed out in a
    shuffled order (the benchmark's paged run): sampled codes bit-exact through
    the block table, every sequence's output against the oracle."""
    wid, ps = 3, 64
    w = W.WORKLOADS[wid]
    lens = W.lengths(wid)
    cap = (W.capacity(wid) + ps - 1) // ps * ps
    blocks = cap // ps
    table = np.random.default_rng(7).permutation(w.batch * blocks).reshape(w.batch, blocks).astype(np.int32)
    cache = LatentCache(w.fmt, 1, w.batch, cap, device="cuda", page_size=ps, num_pages=w.batch * blocks,
                        block_table=table)
    ckv, kpe = W.latent_batch(wid, 0, int(lens.max()), device="cuda", counts=lens)
    cache.append(0, ckv, kpe, n_new=lens)
    del ckv, kpe
    qn, qp = W.queries(wid, 0, "cuda")
    wuk, wuv = W.weights(wid, 0, "cuda")
    out = cache.decode(0, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, num_splits=w.num_splits)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    longest, shortest = int(np.argmax(lens)), int(np.argmin(lens))
    check_codes(wid, cache, 0, longest, nrows=700)
    check_sequences(wid, cache, 0, range(w.batch), out, qn, qp, wuk, wuv)
