"""The fused decode step at the shapes the benchmark times, against
oracle.rope.decode_step for every sequence: one layer of the 27-layer INT8
stack (batch 64, 16 heads, ragged lengths in [1024, 16384]) and the 128-head
INT4 workload (batch 16, 131072 cached tokens, 64 splits). Stored rows are
compared bit for bit, lengths must advance by one, outputs must be within
the attention tolerance."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import LatentCache
from mla_latent_kv_cache_amd import workloads as W
from oracle import quant as Q
from oracle import rope as R

from gpu_util import assert_close, assert_planes_equal, f32, run_oracle_jobs

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def run_full_step(wid, layer, steps=2):
    w = W.WORKLOADS[wid]
    lens = W.lengths(wid)
    ragged = isinstance(w.seq, tuple)
    cap = (int(lens.max()) + steps + 15) // 16 * 16
    cache = LatentCache(w.fmt, 1, w.batch, cap, device="cuda")
    ckv, kpe = W.latent_batch(wid, layer, int(lens.max()), device="cuda", counts=lens if ragged else None)
    cache.append(0, ckv, kpe, n_new=lens if ragged else None)
    del ckv, kpe
    qn, qp = W.queries(wid, layer, "cuda")
    wuk, wuv = W.weights(wid, layer, "cuda")
    cos, sin = R.rope_tables(cap + 1)  # the oracle's tables on both sides
    rope = (torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda())
    new_c, new_k = W.latent_batch(wid, layer, steps, device="cuda", kind="step")
    ws = cache.workspace(w.heads, w.num_splits)
    outs = []
    for i in range(steps):
        o = cache.decode_step(0, new_c[:, i].contiguous(), new_k[:, i].contiguous(), qn, qp, wuk, wuv,
                              W.SOFTMAX_SCALE, rope=rope, num_splits=w.num_splits, workspace=ws)
        outs.append(f32(o))
    torch.cuda.synchronize()
    assert cache.seq_lens[0].tolist() == (lens + steps).tolist()
    qn_h, qp_h, wk, wv = f32(qn), f32(qp), f32(wuk), f32(wuv)
    nc, nk = f32(new_c), f32(new_k)
    # step i: the oracle attends the prefix plus the first i new tokens, which
    # it stores itself; checked for the last step, with every stored row
    last = steps - 1

    def jobs():
        for b in range(w.batch):
            c, k = W.latent_rows(wid, layer, b, int(lens[b]), device="cuda")
            c, k = f32(c), f32(k)
            yield b, oracle_rows_then_step, (c, k, w.fmt, int(lens[b]), cap, nc[b], nk[b], qn_h[b], qp_h[b], wk,
                                              wv, cos, sin, last)

    worst = 0.0
    for b, (rows, out) in run_oracle_jobs(jobs()):
        got = cache.planes(0, b)
        for i, planes in enumerate(rows):
            assert_planes_equal({key: v[int(lens[b]) + i:int(lens[b]) + i + 1] for key, v in got.items()},
                                {key: v[None] for key, v in planes.items()}, w.fmt,
                                f"{w.name} seq {b} stored row {i}")
        worst = max(worst, assert_close(outs[last][b], out, f"{w.name} step {last} seq {b} (len {lens[b]})"))
    print(f"  {w.name}: fused step, {w.batch} sequences, max abs err {worst:.2e}", flush=True)


def oracle_rows_then_step(c, k, fmt, length, cap, nc, nk, qn, qp, wk, wv, cos, sin, last):
    """The oracle's steps 0..last of one sequence: each stores its (turned)
    token; returns the stored rows' planes and the last step's output."""
    ch, kh = Q.dequantize_rows(Q.quantize_rows(c, k, fmt), fmt)
    rows = []
    out = None
    for i in range(last + 1):
        planes, n, out = R.decode_step(ch, kh, length + i, cap, nc[i], nk[i], qn, qp, wk, wv, W.SOFTMAX_SCALE,
                                       fmt, cos, sin)
        rows.append(planes)
        c_hat, k_hat = Q.dequantize_rows({key: v[None] for key, v in planes.items()}, fmt)
        ch, kh = np.concatenate([ch, c_hat]), np.concatenate([kh, k_hat])
    return rows, out


def test_fused_step_int8_stack_layer_full():
    run_full_step(3, 0)


def test_fused_step_int8_stack_last_layer_full():
    run_full_step(3, 26, steps=1)


def test_fused_step_int4_128_heads_full():
    run_full_step(4, 0)
