"""The fused decode step on the GPU (RoPE on the new token, append, attend
over L+1) against oracle.rope.decode_step: stored rows bit-exact, lengths
advanced, outputs within the attention tolerance."""

import numpy as np
import pytest
import torch

from oracle import quant as Q
from oracle import rope as R

from gpu_util import assert_close, assert_planes_equal, f32, oracle_planes, random_problem, random_rows

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def new_tokens(B, H, seed, fmt):
    ckv = torch.empty((B, 512), dtype=torch.bfloat16, device="cuda")
    kpe = torch.empty((B, 64), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        c, k = random_rows(1, seed * 31 + b, "skew" if fmt.startswith("int4") else "outlier")
        ckv[b], kpe[b] = c[0], k[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    qn = torch.randn((B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    qp = (torch.randn((B, H, 64), generator=g, device="cuda") * 2).to(torch.bfloat16)
    return ckv, kpe, qn, qp


def oracle_rows(rows, fmt):
    """Dequantized oracle rows of each sequence's cached bf16 tokens."""
    out = []
    for c, k in rows:
        if c.shape[0] == 0:
            out.append((np.zeros((0, 512)), np.zeros((0, 64))))
        else:
            out.append(Q.dequantize_rows(oracle_planes(c, k, fmt), fmt))
    return out


def tables(rows_needed):
    cos, sin = R.rope_tables(rows_needed)
    return cos, sin, (torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda())


@pytest.mark.parametrize("fmt", ["bf16", "int8", "int4", "int8_kbf16", "int4_kint4"])
@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_step_with_rope_against_oracle(fmt, heads):
    cap = 320
    lens = [0, 1, 37, 319, 320]  # the last sequence is full: nothing is stored
    B = len(lens)
    cache, rows, qn, qp, wuk, wuv = random_problem(fmt, B, heads, lens, seed=61 + heads, cap=cap)
    ckv_new, kpe_new, qn, qp = new_tokens(B, heads, 62 + heads, fmt)
    cos, sin, rope = tables(cap + 1)
    before = oracle_rows(rows, fmt)
    for splits in (0, 3):
        c2, rows2, _, _, _, _ = random_problem(fmt, B, heads, lens, seed=61 + heads, cap=cap)
        out = c2.decode_step(0, ckv_new, kpe_new, qn, qp, wuk, wuv, TAU, rope=rope, num_splits=splits)
        torch.cuda.synchronize()
        assert c2.seq_lens[0].tolist() == [1, 2, 38, 320, 320]
        for b in range(B):
            planes, n, ref = R.decode_step(before[b][0], before[b][1], lens[b], cap, f32(ckv_new[b]),
                                           f32(kpe_new[b]), f32(qn[b]), f32(qp[b]), f32(wuk), f32(wuv), TAU,
                                           fmt, cos, sin)
            assert n == int(c2.seq_lens[0, b])
            assert_close(f32(out[b]), ref, f"{fmt} H{heads} splits {splits} seq {b} (len {lens[b]})")
            if planes is not None:
                got = {k: v[-1:] for k, v in c2.planes(0, b).items()}
                assert_planes_equal(got, {k: v[None] for k, v in planes.items()}, fmt,
                                    f"{fmt} seq {b} stored row")


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_step_without_rope_is_append_then_decode(fmt):
    lens = [5, 130, 64]
    B, H = len(lens), 16
    a, _, qn, qp, wuk, wuv = random_problem(fmt, B, H, lens, seed=71, cap=200)
    b_, _, _, _, _, _ = random_problem(fmt, B, H, lens, seed=71, cap=200)
    ckv_new, kpe_new, qn, qp = new_tokens(B, H, 72, fmt)
    out_step = a.decode_step(0, ckv_new, kpe_new, qn, qp, wuk, wuv, TAU, rope=None)
    b_.append(0, ckv_new[:, None].contiguous(), kpe_new[:, None].contiguous())
    out_ref = b_.decode(0, qn, qp, wuk, wuv, TAU)
    torch.cuda.synchronize()
    assert torch.equal(a.seq_lens, b_.seq_lens)
    assert torch.equal(out_step, out_ref)
    for s in range(B):
        pa, pb = a.planes(0, s), b_.planes(0, s)
        for k in pa:
            assert torch.equal(pa[k], pb[k]), (s, k)


def test_consecutive_steps_turn_by_each_position():
    fmt, H, cap = "int8", 16, 64
    lens = [0, 9, 40]
    B = len(lens)
    cache, rows, _, _, wuk, wuv = random_problem(fmt, B, H, lens, seed=81, cap=cap)
    cos, sin, rope = tables(cap + 1)
    cur = oracle_rows(rows, fmt)
    L = list(lens)
    for step in range(3):
        ckv_new, kpe_new, qn, qp = new_tokens(B, H, 90 + step, fmt)
        out = cache.decode_step(0, ckv_new, kpe_new, qn, qp, wuk, wuv, TAU, rope=rope)
        torch.cuda.synchronize()
        for b in range(B):
            planes, n, ref = R.decode_step(cur[b][0], cur[b][1], L[b], cap, f32(ckv_new[b]), f32(kpe_new[b]),
                                           f32(qn[b]), f32(qp[b]), f32(wuk), f32(wuv), TAU, fmt, cos, sin)
            assert_close(f32(out[b]), ref, f"step {step} seq {b}")
            c_hat, k_hat = Q.dequantize_rows({k: v[None] for k, v in planes.items()}, fmt)
            cur[b] = (np.concatenate([cur[b][0], c_hat]), np.concatenate([cur[b][1], k_hat]))
            L[b] = n
    assert cache.seq_lens[0].tolist() == [3, 12, 43]


def test_step_phases_equal_one_call():
    fmt, H = "int4", 16
    lens = [300, 2, 77]
    B = len(lens)
    a, _, qn, qp, wuk, wuv = random_problem(fmt, B, H, lens, seed=101, cap=400)
    b_, _, _, _, _, _ = random_problem(fmt, B, H, lens, seed=101, cap=400)
    ckv_new, kpe_new, qn, qp = new_tokens(B, H, 102, fmt)
    _, _, rope = tables(401)
    ws = a.workspace(H, 5)
    ref = a.decode_step(0, ckv_new, kpe_new, qn, qp, wuk, wuv, TAU, rope=rope, num_splits=5, workspace=ws)
    ws2 = b_.workspace(H, 5)
    b_.decode_step_begin(0, ckv_new, kpe_new, qn, qp, wuk, TAU, ws2, rope=rope, num_splits=5)
    b_.decode_partial(0, H, ws2, num_splits=5)
    out = b_.decode_combine(wuv, ws2, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(a.seq_lens, b_.seq_lens)


@pytest.mark.parametrize("fmt,heads", [("int8", 16), ("int4", 16), ("int8", 128), ("int4_kint4", 64)])
def test_step_two_absorb_batch_tiles(fmt, heads):
    # more than 64 sequences: the step's absorption runs in two batch tiles of
    # 64 rows (the second one partial), and 100 store blocks follow them
    rng = np.random.default_rng(heads)
    lens = rng.integers(0, 90, size=100).tolist()
    lens[0], lens[-1] = 0, 96  # an empty and a full sequence
    cap = 96
    B = len(lens)
    cache, rows, _, _, wuk, wuv = random_problem(fmt, B, heads, lens, seed=201 + heads, cap=cap)
    ckv_new, kpe_new, qn, qp = new_tokens(B, heads, 202 + heads, fmt)
    cos, sin, rope = tables(cap + 1)
    before = oracle_rows(rows, fmt)
    out = cache.decode_step(0, ckv_new, kpe_new, qn, qp, wuk, wuv, TAU, rope=rope)
    torch.cuda.synchronize()
    assert cache.seq_lens[0].tolist() == [min(n + 1, cap) for n in lens]
    out_h, qn_h, qp_h, wk, wv = f32(out), f32(qn), f32(qp), f32(wuk), f32(wuv)
    cn, kn = f32(ckv_new), f32(kpe_new)
    for b in range(B):
        planes, n, ref = R.decode_step(before[b][0], before[b][1], lens[b], cap, cn[b], kn[b], qn_h[b], qp_h[b],
                                       wk, wv, TAU, fmt, cos, sin)
        assert_close(out_h[b], ref, f"{fmt} H{heads} B{B} seq {b} (len {lens[b]})")
        if planes is not None:
            got = {k: v[-1:] for k, v in cache.planes(0, b).items()}
            assert_planes_equal(got, {k: v[None] for k, v in planes.items()}, fmt, f"{fmt} seq {b} stored row")


def test_library_rope_tables_match_the_oracle_tables():
    # mla_rope_tables (the tables the benchmark's decode step uses) against the
    # oracle's, for positions up to the longest workload (131072 tokens and a
    # few steps). Both evaluate cos and sin in fp64 and round to fp32, but
    # theta_i = 10000^(-2i/64) comes from two fp64 pow routines (numpy's and
    # the C library's) that can differ in the last bit; times a position near
    # 131072 that moves an angle by ~1e-11, so entries agree to within one
    # fp32 rounding of the value (2^-24) plus that, not bit for bit.
    from mla_latent_kv_cache_amd import rope_tables
    rows = 131072 + 64
    cos, sin = rope_tables(rows)
    torch.cuda.synchronize()
    rc, rs = R.rope_tables(rows)
    for got, ref, name in ((f32(cos), rc, "cos"), (f32(sin), rs, "sin")):
        assert got.shape == ref.shape
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert err.max() <= 2.0 ** -24 + 1e-9, f"{name}: max abs difference {err.max():.3g}"
        frac = float((err != 0).mean())
        print(f"  rope {name}: {frac:.2e} of entries differ, max {err.max():.2e}", flush=True)
        assert frac < 1e-3
