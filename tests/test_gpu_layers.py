"""Several layers in one call (mla_decode_attn_layers, mla_decode_step_layers)
against the oracle, layer by layer: ragged lengths that differ per layer, so
the balanced plan's runs cross from one layer's sequences into the next
layer's; the contiguous and paged layouts; and the 27-layer INT8 stack at full
size through the fused step, the call the benchmark times."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import LatentCache
from mla_latent_kv_cache_amd import workloads as W
from oracle import quant as Q
from oracle import rope as R

from gpu_util import (assert_close, assert_planes_equal, f32, oracle_decode, oracle_decode_np, oracle_planes,
                      random_rows, run_oracle_jobs, stacked_problem)

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


@pytest.mark.parametrize("fmt", ["bf16", "int8", "int4", "int8_kbf16", "int4_kint4"])
@pytest.mark.parametrize("heads", [16, 128])
def test_decode_layers_against_oracle(fmt, heads):
    L, B, cap = 4, 5, 300
    rng = np.random.default_rng(heads + len(fmt))
    lens = rng.integers(0, cap + 1, size=(L, B)).tolist()
    lens[1][2] = 0
    lens[2] = [0] * B  # a layer with no tokens at all
    cache, rows, qn, qp, wuk, wuv = stacked_problem(fmt, L, B, heads, lens, seed=7 + heads, cap=cap)
    for layer0, n in ((0, L), (1, 2), (3, 1)):
        sl = slice(layer0, layer0 + n)
        args = (qn[sl].contiguous(), qp[sl].contiguous(), wuk[sl].contiguous(), wuv[sl].contiguous())
        for splits in (0, 1, 3):
            out = cache.decode_layers(layer0, *args, TAU, num_splits=splits)
            torch.cuda.synchronize()
            for i in range(n):
                l = layer0 + i
                for b in range(B):
                    c, k = rows[l][b]
                    ref = oracle_decode(c, k, fmt, qn[l, b], qp[l, b], wuk[l], wuv[l], TAU)
                    assert_close(f32(out[i, b]), ref, f"{fmt} H{heads} layers {layer0}+{n} splits {splits} "
                                                      f"layer {l} seq {b} (len {lens[l][b]})")
                    if lens[l][b] == 0:
                        assert not out[i, b].any()
        # one layer through the layer-range call is the one-layer call, bit for bit
        one = cache.decode(layer0, qn[layer0], qp[layer0], wuk[layer0], wuv[layer0], TAU, num_splits=3)
        many = cache.decode_layers(layer0, qn[layer0:layer0 + 1].contiguous(), qp[layer0:layer0 + 1].contiguous(),
                                   wuk[layer0:layer0 + 1].contiguous(), wuv[layer0:layer0 + 1].contiguous(), TAU,
                                   num_splits=3)
        torch.cuda.synchronize()
        assert torch.equal(one, many[0])


@pytest.mark.parametrize("fmt,heads,L,B", [("int8", 128, 4, 20), ("int4", 16, 22, 36), ("bf16", 64, 8, 17)])
def test_sixteen_sequence_combine_against_oracle(fmt, heads, L, B):
    """Layer ranges large enough for the merge that serves 16 sequences per
    block (heads x ceil(B / 16) x layers >= 1024 blocks), with B not a multiple
    of 16 (rows past the batch in the last block) and empty sequences. The
    latents carry no outlier channels: with them, short INT8 sequences reach
    the limit of the fp16 value operand (one element of 1.3 M at 1.15x the
    tolerance here, from the partial kernel, the same through either merge),
    which test_gpu_decode's short-sequence test covers at its own sizes."""
    assert heads * ((B + 15) // 16) * L >= 1024
    cap = 64
    rng = np.random.default_rng(B + L)
    lens = rng.integers(0, cap + 1, size=(L, B)).tolist()
    lens[0][B - 1] = 0
    lens[L - 1] = [0] * (B // 2) + lens[L - 1][B // 2:]
    cache, rows, qn, qp, wuk, wuv = stacked_problem(fmt, L, B, heads, lens, seed=31 + heads, cap=cap, dist="normal")
    out = cache.decode_layers(0, qn, qp, wuk, wuv, TAU, num_splits=2)
    torch.cuda.synchronize()
    qn_h, qp_h, wk_h, wv_h = f32(qn), f32(qp), f32(wuk), f32(wuv)
    out_h = f32(out)

    def jobs():
        for l in range(L):
            for b in range(B):
                c, k = rows[l][b]
                yield (l, b), oracle_decode_np, (f32(c), f32(k), fmt, qn_h[l, b], qp_h[l, b], wk_h[l], wv_h[l], TAU)

    for (l, b), ref in run_oracle_jobs(jobs()):
        assert_close(out_h[l, b], ref, f"{fmt} H{heads} layer {l} seq {b} (len {lens[l][b]})")
        if lens[l][b] == 0:
            assert not out_h[l, b].any()


@pytest.mark.parametrize("fmt,heads", [("int8", 16), ("int4", 32), ("int4_kint4", 128)])
def test_paged_decode_layers_equals_contiguous(fmt, heads):
    L, B, cap, ps = 3, 4, 256, 64
    blocks = cap // ps
    rng = np.random.default_rng(3)
    lens = rng.integers(0, cap + 1, size=(L, B)).tolist()
    perm = np.random.default_rng(4).permutation(B * blocks + 3)[: B * blocks]
    table = torch.tensor(perm.reshape(B, blocks), dtype=torch.int32)
    flat, rows, qn, qp, wuk, wuv = stacked_problem(fmt, L, B, heads, lens, seed=17, cap=cap)
    paged, _, _, _, _, _ = stacked_problem(fmt, L, B, heads, lens, seed=17, cap=cap, page_size=ps, table=table)
    for splits in (0, 2):
        o1 = flat.decode_layers(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        o2 = paged.decode_layers(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), splits
    for l in range(L):
        for b in range(B):
            c, k = rows[l][b]
            assert_close(f32(o2[l, b]), oracle_decode(c, k, fmt, qn[l, b], qp[l, b], wuk[l], wuv[l], TAU),
                         f"paged layer {l} seq {b}")


@pytest.mark.parametrize("fmt,heads,page_size", [("int8", 16, 0), ("int4", 64, 0), ("int8", 32, 32)])
def test_step_layers_against_oracle(fmt, heads, page_size):
    L, B, cap = 3, 6, 128
    rng = np.random.default_rng(heads)
    lens = rng.integers(0, cap, size=(L, B)).tolist()
    lens[0][0], lens[2][5] = 0, cap  # an empty and a full sequence
    table = None
    if page_size:
        blocks = cap // page_size
        table = torch.tensor(np.random.default_rng(8).permutation(B * blocks).reshape(B, blocks), dtype=torch.int32)
    cache, rows, qn, qp, wuk, wuv = stacked_problem(fmt, L, B, heads, lens, seed=27, cap=cap,
                                                    page_size=page_size, table=table)
    g = torch.Generator(device="cuda")
    g.manual_seed(28)
    c_new = torch.randn((L, B, 512), generator=g, device="cuda").to(torch.bfloat16)
    k_new = torch.randn((L, B, 64), generator=g, device="cuda").to(torch.bfloat16)
    cos, sin = R.rope_tables(cap + 1)
    rope = (torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda())
    out = cache.decode_step_layers(0, c_new, k_new, qn, qp, wuk, wuv, TAU, rope=rope)
    torch.cuda.synchronize()
    assert cache.seq_lens.tolist() == [[min(n + 1, cap) for n in r] for r in lens]
    for l in range(L):
        for b in range(B):
            c, k = rows[l][b]
            if lens[l][b]:
                ch, kh = Q.dequantize_rows(oracle_planes(c, k, fmt), fmt)
            else:
                ch, kh = np.zeros((0, 512)), np.zeros((0, 64))
            planes, n, ref = R.decode_step(ch, kh, lens[l][b], cap, f32(c_new[l, b]), f32(k_new[l, b]),
                                           f32(qn[l, b]), f32(qp[l, b]), f32(wuk[l]), f32(wuv[l]), TAU, fmt,
                                           cos, sin)
            assert_close(f32(out[l, b]), ref, f"{fmt} H{heads} step layer {l} seq {b} (len {lens[l][b]})")
            if planes is not None:
                got = {key: v[-1:] for key, v in cache.planes(l, b).items()}
                assert_planes_equal(got, {key: v[None] for key, v in planes.items()}, fmt,
                                    f"layer {l} seq {b} stored row")


@pytest.mark.timeout(900)
def test_step_layers_int8_27_layer_stack_full():
    """The benchmark's timed call: the fused step of all 27 layers of the
    ragged INT8 stack (batch 64, 16 heads) in one set of launches; every
    sequence of layers 0, 13 and 26 against the oracle, and their stored rows
    bit for bit."""
    wid = 3
    w = W.WORKLOADS[wid]
    lens = W.lengths(wid)
    cap = (int(lens.max()) + 1 + 15) // 16 * 16
    cache = LatentCache(w.fmt, w.layers, w.batch, cap, device="cuda")
    for layer in range(w.layers):
        ckv, kpe = W.latent_batch(wid, layer, int(lens.max()), device="cuda", counts=lens)
        cache.append(layer, ckv, kpe, n_new=lens)
        del ckv, kpe
    q = [W.queries(wid, l, "cuda") for l in range(w.layers)]
    wts = [W.weights(wid, l, "cuda") for l in range(w.layers)]
    qn = torch.stack([a for a, _ in q]).contiguous()
    qp = torch.stack([b for _, b in q]).contiguous()
    wuk = torch.stack([a for a, _ in wts]).contiguous()
    wuv = torch.stack([b for _, b in wts]).contiguous()
    del q, wts
    news = [W.latent_batch(wid, l, 1, device="cuda", kind="step") for l in range(w.layers)]
    c_new = torch.stack([c[:, 0] for c, _ in news]).contiguous()
    k_new = torch.stack([k[:, 0] for _, k in news]).contiguous()
    cos, sin = R.rope_tables(cap + 1)
    rope = (torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda())
    out = cache.decode_step_layers(0, c_new, k_new, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, rope=rope)
    torch.cuda.synchronize()
    assert (cache.seq_lens.cpu().numpy() == lens[None] + 1).all()
    assert torch.isfinite(out).all()
    for layer in (0, 13, 26):
        qn_h, qp_h, wk, wv = f32(qn[layer]), f32(qp[layer]), f32(wuk[layer]), f32(wuv[layer])
        cn, kn = f32(c_new[layer]), f32(k_new[layer])

        def jobs():
            for b in range(w.batch):
                c, k = W.latent_rows(wid, layer, b, int(lens[b]), device="cuda")
                yield b, step_job, (f32(c), f32(k), w.fmt, int(lens[b]), cap, cn[b], kn[b], qn_h[b], qp_h[b], wk,
                                    wv, cos, sin)

        worst = 0.0
        out_h = f32(out[layer])
        for b, (planes, ref) in run_oracle_jobs(jobs()):
            worst = max(worst, assert_close(out_h[b], ref, f"27-layer step layer {layer} seq {b}"))
            got = {key: v[-1:] for key, v in cache.planes(layer, b).items()}
            assert_planes_equal(got, {key: v[None] for key, v in planes.items()}, w.fmt,
                                f"layer {layer} seq {b} stored row")
        print(f"  27-layer fused step, layer {layer}: 64 sequences, max abs err {worst:.2e}", flush=True)


def step_job(c, k, fmt, length, cap, cn, kn, qn, qp, wk, wv, cos, sin):
    ch, kh = Q.dequantize_rows(Q.quantize_rows(c, k, fmt), fmt)
    planes, _, out = R.decode_step(ch, kh, length, cap, cn, kn, qn, qp, wk, wv, W.SOFTMAX_SCALE, fmt, cos, sin)
    return planes, out
