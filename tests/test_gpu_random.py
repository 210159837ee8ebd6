"""Seeded random decode problems against the fp64 oracle: format, head count,
batch, ragged lengths (empty, one token, tile edges, several hundred tokens),
split count, layer count and layout (contiguous, or pages of 32-128 tokens
handed out in a shuffled order) are drawn per case, and every output of every
layer is checked. Each case is reproducible from its index."""

import numpy as np
import pytest
import torch

from gpu_util import assert_close, f32, oracle_decode_np, run_oracle_jobs, stacked_problem

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)
FORMATS = ["bf16", "int8", "int4", "int8_kbf16", "int4_kint4"]
EDGES = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129]


def draw_case(k):
    rng = np.random.default_rng(1000 + k)
    fmt = FORMATS[k % len(FORMATS)]
    heads = int(rng.choice([16, 32, 64, 128], p=[0.4, 0.2, 0.2, 0.2]))
    L = int(rng.integers(1, 4))
    B = int(rng.integers(1, 7))
    page = int(rng.choice([0, 0, 32, 64, 128]))
    cap = int(rng.choice([160, 320, 704]))
    if page:
        cap = (cap + page - 1) // page * page
    lens = np.where(rng.random((L, B)) < 0.4, rng.choice(EDGES, size=(L, B)),
                    rng.integers(0, cap + 1, size=(L, B)))
    lens = np.minimum(lens, cap).tolist()
    splits = int(rng.choice([0, 1, 2, 3, 5, 8, 13]))
    return fmt, heads, L, B, page, cap, lens, splits


@pytest.mark.parametrize("k", range(30))
def test_random_problem_against_oracle(k):
    fmt, heads, L, B, page, cap, lens, splits = draw_case(k)
    table = None
    if page:
        blocks = cap // page
        # a shuffled pool of B * blocks + 3 pages (stacked_problem's num_pages)
        perm = np.random.default_rng(2000 + k).permutation(B * blocks + 3)[: B * blocks]
        table = torch.tensor(perm.reshape(B, blocks), dtype=torch.int32)
    cache, rows, qn, qp, wuk, wuv = stacked_problem(fmt, L, B, heads, lens, seed=3000 + k, cap=cap, page_size=page,
                                                    table=table)
    what = f"case {k}: {fmt} H{heads} L{L} B{B} page {page} cap {cap} splits {splits}"
    print(what, flush=True)
    if L == 1:
        out = cache.decode(0, qn[0], qp[0], wuk[0], wuv[0], TAU, num_splits=splits)[None]
    else:
        out = cache.decode_layers(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
    torch.cuda.synchronize()
    out_h, qn_h, qp_h, wk_h, wv_h = f32(out), f32(qn), f32(qp), f32(wuk), f32(wuv)

    def jobs():
        for l in range(L):
            for b in range(B):
                c, kk = rows[l][b]
                yield (l, b), oracle_decode_np, (f32(c), f32(kk), fmt, qn_h[l, b], qp_h[l, b], wk_h[l], wv_h[l], TAU)

    for (l, b), ref in run_oracle_jobs(jobs()):
        assert_close(out_h[l, b], ref, f"{what} layer {l} seq {b} (len {lens[l][b]})")
        if lens[l][b] == 0:
            assert not out_h[l, b].any()
