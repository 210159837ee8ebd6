"""Absorbed decode on the GPU against the fp64 oracle, on small problems that
still span several tiles and splits and have ragged tails."""

import numpy as np
import pytest
import torch

from gpu_util import assert_close, f32, oracle_decode, random_problem
from mla_latent_kv_cache_amd import LatentCache

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def check_all(cache, rows, q_nope, q_pe, w_uk, w_uv, out, fmt, what):
    for b, (c, k) in enumerate(rows):
        ref = oracle_decode(c, k, fmt, q_nope[b], q_pe[b], w_uk, w_uv, TAU)
        assert_close(f32(out[b]), ref, f"{what} seq {b} (len {c.shape[0]})")


@pytest.mark.parametrize("fmt", ["bf16", "int8", "int4", "int8_kbf16", "int4_kint4"])
@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_decode_formats_and_heads(fmt, heads):
    lens = [1, 17, 600, 0]
    cache, rows, qn, qp, wuk, wuv = random_problem(fmt, 4, heads, lens, seed=heads + len(fmt))
    for splits in (1, 3, 0):
        out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        torch.cuda.synchronize()
        check_all(cache, rows, qn, qp, wuk, wuv, out, fmt, f"{fmt} H{heads} splits {splits}")
        assert not out[3].any()  # empty sequence -> zeros


@pytest.mark.parametrize("fmt", ["int8", "int4", "int8_kbf16", "int4_kint4"])
def test_tile_and_split_boundaries(fmt):
    lens = [15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257]
    cache, rows, qn, qp, wuk, wuv = random_problem(fmt, len(lens), 16, lens, seed=5, cap=272)
    for splits in (1, 2, 4, 17):
        out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        torch.cuda.synchronize()
        check_all(cache, rows, qn, qp, wuk, wuv, out, fmt, f"{fmt} splits {splits}")


@pytest.mark.parametrize("fmt,heads", [("int8", 16), ("int4", 16), ("int8", 32)])
def test_dispatch_order_ties_and_large_batch(fmt, heads):
    # The balanced plan scans the lengths 256 at a time and cuts the batch's
    # tiles into equal runs: many tied lengths, and a batch past 256 (two
    # passes of the scan), at 16 heads and at 32 (two head slices), both
    # against the oracle.
    rng = np.random.default_rng(7)
    tied = rng.choice([0, 5, 33, 96, 129], size=40).tolist()
    large = rng.integers(0, 70, size=260).tolist()
    for lens, seed in ((tied, 51), (large, 52)):
        cache, rows, qn, qp, wuk, wuv = random_problem(fmt, len(lens), heads, lens, seed=seed)
        for splits in (0, 3):
            out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
            torch.cuda.synchronize()
            check_all(cache, rows, qn, qp, wuk, wuv, out, fmt, f"B{len(lens)} H{heads} splits {splits}")


def test_split_count_invariance_and_determinism():
    lens = [3000, 1234]
    cache, rows, qn, qp, wuk, wuv = random_problem("int8", 2, 16, lens, seed=9)
    outs = {}
    for splits in (1, 2, 7, 64, 188, 0):
        o1 = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        o2 = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"splits {splits}: two runs differ"
        check_all(cache, rows, qn, qp, wuk, wuv, o1, "int8", f"splits {splits}")
        outs[splits] = f32(o1)
    base = outs[1]
    for s, o in outs.items():
        assert np.max(np.abs(o - base)) <= 1e-3 * (1 + np.abs(base).max()), s


def test_workspace_contents_do_not_matter():
    cache, rows, qn, qp, wuk, wuv = random_problem("int4", 3, 16, [100, 700, 5], seed=13)
    ws = cache.workspace(16, 5)
    ws.fill_(0xFF)  # NaN patterns everywhere
    out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=5, workspace=ws)
    ws.zero_()
    out2 = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    check_all(cache, rows, qn, qp, wuk, wuv, out, "int4", "garbage workspace")


def test_decode_sees_appended_tokens():
    # decode after an append attends to the new rows too
    cache, rows, qn, qp, wuk, wuv = random_problem("int8", 2, 16, [40, 40], seed=21, cap=48)
    from gpu_util import random_rows
    c, k = random_rows(8, 999)
    cache.append(0, torch.stack([c, c]).contiguous(), torch.stack([k, k]).contiguous())
    out = cache.decode(0, qn, qp, wuk, wuv, TAU)
    torch.cuda.synchronize()
    rows2 = [(torch.cat([rc, c]), torch.cat([rk, k])) for rc, rk in rows]
    check_all(cache, rows2, qn, qp, wuk, wuv, out, "int8", "after append")


def test_extreme_scores_stay_finite():
    # large query norms give large score gaps; the online softmax must not overflow
    cache, rows, qn, qp, wuk, wuv = random_problem("int8", 2, 16, [500, 70], seed=31)
    qn = (qn.float() * 4).to(torch.bfloat16)
    qp = (qp.float() * 4).to(torch.bfloat16)
    out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=3)
    torch.cuda.synchronize()
    check_all(cache, rows, qn, qp, wuk, wuv, out, "int8", "large scores")


def test_three_phases_equal_one_call():
    cache, rows, qn, qp, wuk, wuv = random_problem("int4", 3, 32, [333, 18, 1000], seed=41)
    ws = cache.workspace(32, 6)
    ref = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=6, workspace=ws)
    ws2 = cache.workspace(32, 6)
    cache.decode_absorb(qn, qp, wuk, TAU, ws2, num_splits=6)
    cache.decode_partial(0, 32, ws2, num_splits=6)
    out = cache.decode_combine(wuv, ws2, num_splits=6)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_balanced_plan_runs(fmt):
    # 16 heads: W = splits * B workgroups each take an equal run of the batch's
    # 32-token tiles, and a run may cover the end of one sequence and the start
    # of the next. Runs over many short and empty sequences; more workgroups
    # than tiles (idle workgroups); every workgroup on one long sequence among
    # empty ones (one record per workgroup for it); and a batch of 300, whose
    # lengths are scanned in two passes of 256.
    rng = np.random.default_rng(11)
    cases = [
        ([0, 1, 0, 0, 31, 33, 0, 2, 64, 0, 5, 700, 0, 0, 17], (1, 2, 5, 40, 0)),
        ([0] * 10 + [2000] + [0] * 5, (1, 3, 0)),
        ((rng.integers(0, 41, size=300) * (rng.random(300) > 0.2)).tolist(), (1, 2, 0)),
    ]
    for n, (lens, split_list) in enumerate(cases):
        cache, rows, qn, qp, wuk, wuv = random_problem(fmt, len(lens), 16, lens, seed=60 + n)
        for splits in split_list:
            out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
            torch.cuda.synchronize()
            check_all(cache, rows, qn, qp, wuk, wuv, out, fmt, f"case {n} B{len(lens)} splits {splits}")
            for b, L in enumerate(lens):
                if L == 0:
                    assert not out[b].any(), f"case {n} splits {splits}: empty sequence {b} not zero"


def test_auto_split_rule_16_heads():
    # 16 heads, num_splits = 0: floor(3 * CUs / batch) workgroups per sequence
    # on average (three resident per CU), at most ceil(capacity / 128) (4 tiles
    # each for full sequences) or, for a capacity under 32 tiles, at most
    # min(8, its tiles), at least 1
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for B, cap in ((1, 256), (1, 320), (1, 31), (1, 1000), (1, 1100), (8, 4160), (32, 2048), (64, 4096),
                   (300, 64), (1000, 64)):
        cache = LatentCache("int8", 1, B, cap, device=torch.device("cuda"))
        tiles = -(-cap // 32)
        by_len = -(-tiles // 4)
        if by_len < 8:
            by_len = min(tiles, 8)
        want = max(1, min(3 * cus // B, by_len))
        assert cache.auto_splits(16) == want, (B, cap)


@pytest.mark.parametrize("heads", [16, 32, 128])
@pytest.mark.parametrize("fmt", ["int8", "int4", "int8_kbf16", "int4_kint4"])
def test_short_sequences_with_outlier_channels(fmt, heads):
    # Short sequences concentrate the softmax on a few tokens, and the x20
    # outlier channels put latent values near 100: the value product must take
    # the dequantized latent without fp16 rounding (2^-11 of 100 per element
    # would show in outputs that cancel after W_UV)
    lens = [5, 29, 60, 100, 200, 3]
    for seed in (71, 72, 73):
        cache, rows, qn, qp, wuk, wuv = random_problem(fmt, len(lens), heads, lens, seed=seed + heads)
        out = cache.decode(0, qn, qp, wuk, wuv, TAU)
        torch.cuda.synchronize()
        check_all(cache, rows, qn, qp, wuk, wuv, out, fmt, f"{fmt} H{heads} seed {seed}")


@pytest.mark.parametrize("fmt", ["int4", "int4_kint4", "int8", "int8_kbf16"])
def test_groups_at_the_edge_of_the_fp16_domain(fmt):
    # The decode path multiplies codes by scales in fp16 (include/mla_kv.h,
    # domain of the decode path). Groups at the edge of that domain: INT4
    # latents with a 16-channel range of 65280 (scale 4352, 15 s = 65280) and
    # INT8 latents at +-65024 (scale 512, 127 s = 65024). Such tokens give
    # scores in the thousands, so the softmax concentrates on one of them and
    # the INT4 weights multiply the largest scales (p s with p <= 1).
    lens = [3, 40, 97, 130]
    B, H = len(lens), 16
    cache = LatentCache(fmt, 1, B, max(lens), device=torch.device("cuda"))
    from gpu_util import random_rows
    rows = []
    ckv = torch.zeros((B, max(lens), 512), dtype=torch.bfloat16, device="cuda")
    kpe = torch.zeros((B, max(lens), 64), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(5)
    for b, n in enumerate(lens):
        c, k = random_rows(n, 500 + b, "skew" if fmt.startswith("int4") else "outlier")
        c = c.float()
        # a few tokens with one group at the edge, spread over the tiles
        for t in rng.choice(n, size=min(n, 4), replace=False):
            g = int(rng.integers(0, 32))
            if fmt.startswith("int4"):
                vals = torch.linspace(-32640.0, 32640.0, 16)[torch.from_numpy(rng.permutation(16))]
            else:
                vals = torch.from_numpy(rng.choice([-65024.0, 65024.0], size=16)).float()
            c[t, 16 * g:16 * g + 16] = vals.to(c.device)
        c = c.to(torch.bfloat16)
        ckv[b, :n], kpe[b, :n] = c, k
        rows.append((c, k))
    cache.append(0, ckv, kpe, n_new=lens)
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    qn = torch.randn((B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    qp = torch.randn((B, H, 64), generator=g, device="cuda").to(torch.bfloat16)
    wuk = (torch.randn((H, 128, 512), generator=g, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
    wuv = (torch.randn((H, 512, 128), generator=g, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
    # the scales really are at the edge
    from gpu_util import oracle_planes
    sc = np.concatenate([oracle_planes(c, k, fmt)["scale"][:, :32].astype(np.float64).ravel() for c, k in rows])
    assert sc.max() == (4352.0 if fmt.startswith("int4") else 512.0)
    for splits in (1, 0):
        out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        torch.cuda.synchronize()
        check_all(cache, rows, qn, qp, wuk, wuv, out, fmt, f"{fmt} edge groups splits {splits}")


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_small_grid_merge_across_rounds_of_records(fmt):
    # 16 heads x 3 sequences: at most 256 (head, sequence) pairs, so the merge
    # runs one sequence per block, eight waves taking six records each per
    # round of loads (48 a round). Split counts on both sides of 48 records per
    # sequence, several rounds, and an empty sequence among full ones.
    lens = [4000, 0, 2900]
    cache, rows, qn, qp, wuk, wuv = random_problem(fmt, len(lens), 16, lens, seed=77, cap=4096)
    ws = cache.workspace(16, 120)
    for splits in (40, 47, 48, 49, 60, 97, 120):
        out = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        check_all(cache, rows, qn, qp, wuk, wuv, out, fmt, f"{fmt} splits {splits}")
        assert not out[1].any()  # empty sequence -> zeros
