"""Seeded random fused decode steps with angle tables against
oracle.rope.decode_step: format, head count, batch, lengths (empty, full and
anything between), capacity and split count are drawn per case; every
output and the new lengths are checked, and the stored row of every sequence
that had room bit for bit. Each case is reproducible from its index."""

import numpy as np
import pytest
import torch

from oracle import rope as R

from gpu_util import assert_close, assert_planes_equal, f32, random_problem
from test_gpu_step import TAU, new_tokens, oracle_rows, tables

pytestmark = pytest.mark.gpu
FORMATS = ["bf16", "int8", "int4", "int8_kbf16", "int4_kint4"]


def draw_case(k):
    rng = np.random.default_rng(5000 + k)
    fmt = FORMATS[k % len(FORMATS)]
    heads = int(rng.choice([16, 32, 64, 128], p=[0.4, 0.2, 0.2, 0.2]))
    B = int(rng.integers(1, 8))
    cap = int(rng.choice([64, 160, 320]))
    lens = rng.integers(0, cap + 1, size=B)
    lens[rng.random(B) < 0.15] = cap
    lens[rng.random(B) < 0.15] = 0
    splits = int(rng.choice([0, 1, 2, 5, 13]))
    return fmt, heads, B, cap, [int(x) for x in lens], splits


@pytest.mark.parametrize("k", range(30))
def test_random_step_against_oracle(k):
    fmt, heads, B, cap, lens, splits = draw_case(k)
    what = f"case {k}: {fmt} H{heads} B{B} cap {cap} splits {splits} lens {lens}"
    print(what, flush=True)
    cache, rows, qn, qp, wuk, wuv = random_problem(fmt, B, heads, lens, seed=6000 + k, cap=cap)
    ckv_new, kpe_new, qn, qp = new_tokens(B, heads, 7000 + k, fmt)
    cos, sin, rope = tables(cap + 1)
    before = oracle_rows(rows, fmt)
    out = cache.decode_step(0, ckv_new, kpe_new, qn, qp, wuk, wuv, TAU, rope=rope, num_splits=splits)
    torch.cuda.synchronize()
    out_h = f32(out)
    for b in range(B):
        planes, n, ref = R.decode_step(before[b][0], before[b][1], lens[b], cap, f32(ckv_new[b]), f32(kpe_new[b]),
                                       f32(qn[b]), f32(qp[b]), f32(wuk), f32(wuv), TAU, fmt, cos, sin)
        assert n == int(cache.seq_lens[0, b]), f"{what} seq {b}: length"
        assert_close(out_h[b], ref, f"{what} seq {b} (len {lens[b]})")
        if planes is not None:
            got = {key: v[-1:] for key, v in cache.planes(0, b).items()}
            assert_planes_equal(got, {key: v[None] for key, v in planes.items()}, fmt, f"{what} seq {b} stored row")
