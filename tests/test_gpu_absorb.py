"""The absorbed query records against fp64, entry by entry. mla_decode_absorb
writes, for each (sequence, head), tau log2(e) q_nope W_UK (512 channels) and
tau log2(e) q_pe (64) as fp16 hi + lo pairs, and the 32 latent-group sums of
the first part. The records lead the workspace, [batch][heads][1216] fp16: the
576 hi, the 576 lo, the 32 sum hi, the 32 sum lo (the library's layout, read
here as a white-box check). The first launch of the fused step writes the same
records (its RoPE part unturned when no angle tables are given)."""

import numpy as np
import pytest
import torch

from gpu_util import f32, random_problem

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)
QS = TAU * np.log2(np.e)
REC = 1216


def records(ws, B, H):
    n = B * H * REC
    return ws[: 2 * n].view(torch.float16).float().cpu().numpy().astype(np.float64).reshape(B, H, REC)


def check_records(rec, qn, qp, wuk, what):
    """hi + lo against the fp64 value: the MFMA's fp32 accumulation of the 128
    bf16 products (exact in fp32) and the fp16 rounding of lo allow a few fp32
    ulps of the sum of |terms|; a pair whose lo belongs to another hi is off by
    an fp16 ulp of hi (2^-11 relative) and fails by far."""
    q = f32(qn).astype(np.float64)          # [B, H, 128]
    w = f32(wuk).astype(np.float64)         # [H, 128, 512]
    exact = np.einsum("bhd,hdc->bhc", q, w) * QS
    scale = np.einsum("bhd,hdc->bhc", np.abs(q), np.abs(w)) * QS
    got = rec[..., :512] + rec[..., 576:576 + 512]
    err = np.abs(got - exact)
    bound = 2.0 ** -17 * scale + 1e-7  # 128 fp32 additions at worst
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} latent entries off; worst at "
                           f"{np.unravel_index(np.argmax(err / bound), err.shape)} ({(err / bound).max():.1f} x bound)")
    # |lo| at most half an fp16 ulp of hi (plus the subnormal floor): the pair is a split of one value
    hi = rec[..., :512]
    ulp = np.maximum(np.abs(hi) * 2.0 ** -10, 2.0 ** -24)
    assert (np.abs(rec[..., 576:576 + 512]) <= 0.5 * ulp * (1 + 2 ** -10) + 2.0 ** -25).all(), what
    return exact


@pytest.mark.parametrize("B,H", [(5, 16), (5, 128), (64, 16), (70, 32)])
def test_absorbed_records_against_fp64(B, H):
    cache, rows, qn, qp, wuk, wuv = random_problem("int8", B, H, [3] * B, seed=7 * B + H)
    ws = cache.workspace(H, 1)
    ws.fill_(0xFF)  # entries never written read as NaN
    cache.decode_absorb(qn, qp, wuk, TAU, ws, num_splits=1)
    torch.cuda.synchronize()
    rec = records(ws, B, H)
    exact = check_records(rec, qn, qp, wuk, f"B{B} H{H}")
    # the RoPE part: the bf16 query times the scale, split the same way
    pe = f32(qp).astype(np.float64) * QS
    got = rec[..., 512:576] + rec[..., 576 + 512:1152]
    assert (np.abs(got - pe) <= 2.0 ** -22 * np.abs(pe) + 2.0 ** -25).all(), f"B{B} H{H}: q_pe part"
    # group sums: 16 consecutive channels each, hi + lo against fp64 (fp32 additions of the 16 values)
    sums = exact.reshape(B, H, 32, 16).sum(-1)
    gsum = rec[..., 1152:1184] + rec[..., 1184:1216]
    sscale = np.abs(exact).reshape(B, H, 32, 16).sum(-1)
    assert (np.abs(gsum - sums) <= 2.0 ** -19 * sscale + 1e-7).all(), f"B{B} H{H}: group sums"


def test_step_records_latent_part_equals_absorb():
    B, H = 9, 32
    cache, rows, qn, qp, wuk, wuv = random_problem("int8", B, H, [40] * B, seed=99, cap=64)
    ws = cache.workspace(H, 1)
    cache.decode_absorb(qn, qp, wuk, TAU, ws, num_splits=1)
    torch.cuda.synchronize()
    ref = records(ws, B, H)
    ws2 = cache.workspace(H, 1)
    c_new = torch.zeros((B, 512), dtype=torch.bfloat16, device="cuda")
    k_new = torch.zeros((B, 64), dtype=torch.bfloat16, device="cuda")
    cache.decode_step_begin(0, c_new, k_new, qn, qp, wuk, TAU, ws2, num_splits=1)
    torch.cuda.synchronize()
    got = records(ws2, B, H)
    # without angle tables the step's RoPE part is the scaled q_pe, as in the absorption
    assert np.array_equal(got, ref)
