"""Pins for oracle.quant: hand-derived cases, brute force, error bounds,
special cases, and the reduction to the tutorial's per-tensor INT8 snippet."""

import numpy as np
import pytest
import torch

from oracle import quant as Q


def bf16(a):
    """Round fp32 values to bf16 (RNE) and widen back to fp32, exactly."""
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- hand cases

@pytest.mark.parametrize("case", ["int8_pow2_scale", "int8_rounded_scale"])
def test_int8_hand_cases(golden, case):
    g = golden("quant_hand.json")[case]
    x = np.array(g["x"], dtype=np.float32)
    assert np.array_equal(bf16(x), x)  # every value is exactly a bf16
    q, s = Q.quantize_sym_int8(x, 16)
    assert q.tolist() == g["codes"]
    assert s.shape == (1,) and int(s.view(np.uint16)[0]) == g["scale_bits"]


def test_int8_hand_case_inside_a_row(golden):
    # the group sits at channels 48..63 of a 512-wide latent row: group index 3
    g = golden("quant_hand.json")["int8_pow2_scale"]
    row = np.zeros(512, np.float32)
    row[48:64] = g["x"]
    q, s = Q.quantize_sym_int8(row, 16)
    assert q[48:64].tolist() == g["codes"]
    assert not q[:48].any() and not q[64:].any()
    assert int(s.view(np.uint16)[3]) == g["scale_bits"]
    assert np.count_nonzero(s.view(np.uint16)) == 1


def test_kpe_hand_case(golden):
    g = golden("quant_hand.json")["kpe_int8_group8"]
    kpe = np.zeros(64, np.float32)
    kpe[8:16] = g["x"]
    planes = Q.quantize_rows(np.zeros(512, np.float32), kpe, "int8")
    assert planes["kpe"][8:16].tolist() == g["codes"]
    bits = planes["scale"].view(np.uint16)
    assert bits.shape == (40,)
    assert int(bits[32 + 1]) == g["scale_bits"]  # k_pe group 1 follows the 32 latent scales
    assert np.count_nonzero(bits) == 1


def test_int4_hand_case(golden):
    g = golden("quant_hand.json")["int4_asym"]
    x = np.array(g["x"], np.float32)
    q, s, z = Q.quantize_asym_int4(x, 16)
    assert q.tolist() == g["codes"]
    assert int(s.view(np.uint16)[0]) == g["scale_bits"]
    assert int(z.view(np.uint16)[0]) == g["zero_bits"]
    assert Q.pack_nibbles(q).tolist() == g["packed"]
    assert Q.unpack_nibbles(np.array(g["packed"], np.uint8)).tolist() == g["codes"]


def test_int4_hand_case_in_row_planes(golden):
    g = golden("quant_hand.json")["int4_asym"]
    row = np.zeros(512, np.float32)
    row[16:32] = g["x"]  # latent group 1
    p = Q.quantize_rows(row, np.zeros(64, np.float32), "int4")
    assert p["ckv"].shape == (256,) and p["ckv"].dtype == np.uint8
    assert p["ckv"][8:16].tolist() == g["packed"]
    assert int(p["scale"].view(np.uint16)[1]) == g["scale_bits"]
    assert int(p["zero"].view(np.uint16)[1]) == g["zero_bits"]
    assert p["zero"].shape == (32,) and p["scale"].shape == (40,)


# ------------------------------------------------------- brute-force optimality

def test_int8_codes_are_nearest_given_scale():
    x = bf16(rng(1).standard_normal((200, 16)).astype(np.float32) * 3)
    q, s = Q.quantize_sym_int8(x, 16)
    sf = np.repeat(s.astype(np.float64), 16, axis=-1)  # [200, 16]
    cand = np.arange(-127, 128, dtype=np.float64)
    err_all = np.abs(x.astype(np.float64)[..., None] - cand * sf[..., None])  # [200,16,255]
    best = err_all.min(axis=-1)
    mine = np.abs(x - q.astype(np.float64) * sf)
    assert np.all(mine <= best + 1e-12)
    # and the stored scale is the fp16 nearest to max|x| / 127
    a = np.abs(x).max(axis=-1, keepdims=True).astype(np.float64) / 127
    d = np.abs(s.astype(np.float64) - a)
    up = np.nextafter(s, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(s, np.float16(-np.inf)).astype(np.float64)
    assert np.all(d <= np.abs(up - a)) and np.all(d <= np.abs(dn - a))


def test_int4_codes_are_nearest_given_scale_and_zero():
    x = bf16(np.abs(rng(2).standard_normal((200, 16))) * 1.5 - 0.5)
    q, s, z = Q.quantize_asym_int4(x, 16)
    sf = np.repeat(s.astype(np.float64), 16, axis=-1)
    zf = np.repeat(z.astype(np.float64), 16, axis=-1)
    cand = np.arange(16, dtype=np.float64)
    best = np.abs(x.astype(np.float64)[..., None] - (cand * sf[..., None] + zf[..., None])).min(-1)
    mine = np.abs(x - (q * sf + zf))
    assert np.all(mine <= best + 1e-12)
    # the zero-point is the largest fp16 not above the group minimum
    mn = x.min(axis=-1, keepdims=True)
    assert np.all(z.astype(np.float32) <= mn)
    assert np.all(np.nextafter(z, np.float16(np.inf)).astype(np.float32) > mn)


# ------------------------------------------------------------- error bounds

def _normal_scale_rows(s):
    return (s.astype(np.float32) >= 2.0 ** -14).all(axis=-1)


def test_int8_error_bound_half_scale():
    x = bf16(rng(3).standard_normal((500, 512)) * np.where(rng(4).random(512) < 0.01, 20, 1))
    q, s = Q.quantize_sym_int8(x, 16)
    xh = Q.dequantize_sym_int8(q, s, 16)
    bound = np.repeat(s.astype(np.float64), 16, axis=-1) * 0.5 * (1 + 2.0 ** -10)
    ok = np.repeat(_normal_scale_rows(s)[:, None], 512, axis=1)
    assert ok.all()
    assert np.all(np.abs(x - xh) <= bound)


def test_int4_error_bound_half_scale():
    x = bf16(np.abs(rng(5).standard_normal((500, 512))) * 1.5 - 0.5)
    q, s, z = Q.quantize_asym_int4(x, 16)
    xh = Q.dequantize_asym_int4(q, s, z, 16)
    assert _normal_scale_rows(s).all()
    bound = np.repeat(s.astype(np.float64), 16, axis=-1) * 0.5 * (1 + 2.0 ** -10)
    assert np.all(np.abs(x - xh) <= bound)


def test_rows_roundtrip_error_bound():
    c = bf16(rng(6).standard_normal((64, 512)))
    k = bf16(rng(7).standard_normal((64, 64)))
    for fmt in ("int8", "int4"):
        p = Q.quantize_rows(c, k, fmt)
        ch, kh = Q.dequantize_rows(p, fmt)
        s = p["scale"].astype(np.float64)
        assert np.all(np.abs(ch - c) <= np.repeat(s[:, :32], 16, -1) * 0.5 * (1 + 2.0 ** -10))
        assert np.all(np.abs(kh - k) <= np.repeat(s[:, 32:], 8, -1) * 0.5 * (1 + 2.0 ** -10))
    p = Q.quantize_rows(c, k, "bf16")
    ch, kh = Q.dequantize_rows(p, "bf16")
    assert np.array_equal(ch, c) and np.array_equal(kh, k)


# ------------------------------------------------------------- idempotence

def test_int8_idempotent_on_dequantized_values():
    x = bf16(rng(8).standard_normal((300, 16)))
    q, s = Q.quantize_sym_int8(x, 16)
    assert (np.abs(q).max(axis=-1) == 127).all()
    xh = Q.dequantize_sym_int8(q, s, 16).astype(np.float32)  # exact in fp32
    q2, s2 = Q.quantize_sym_int8(xh, 16)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint16), s2.view(np.uint16))


def test_int4_idempotent_on_dequantized_values():
    x = bf16(rng(9).standard_normal((300, 16)))
    q, s, z = Q.quantize_asym_int4(x, 16)
    xh = Q.dequantize_asym_int4(q, s, z, 16)
    sel = (q.min(-1) == 0) & (q.max(-1) == 15) & np.all(xh.astype(np.float32) == xh, axis=-1)
    assert sel.sum() > 100
    q2, s2, z2 = Q.quantize_asym_int4(xh[sel].astype(np.float32), 16)
    assert np.array_equal(q[sel], q2)
    assert np.array_equal(s[sel].view(np.uint16), s2.view(np.uint16))
    assert np.array_equal(z[sel].view(np.uint16), z2.view(np.uint16))


# ------------------------------------------------------------- special cases

def test_all_zero_group():
    q, s = Q.quantize_sym_int8(np.zeros(16, np.float32), 16)
    assert not q.any() and float(s[0]) == 0.0
    q, s, z = Q.quantize_asym_int4(np.zeros(16, np.float32), 16)
    assert not q.any() and float(s[0]) == 0.0 and float(z[0]) == 0.0


def test_single_nonzero_value():
    for v in (0.3, -7.25, 1e-3, 123.0):
        x = np.zeros(16, np.float32)
        x[5] = bf16([v])[0]
        q, s = Q.quantize_sym_int8(x, 16)
        assert q[5] == (127 if v > 0 else -127)
        assert np.count_nonzero(q) == 1
        assert s[0] == np.float16(np.float32(abs(x[5])) / np.float32(127))


def test_constant_int4_group_is_exact():
    for v in (0.75, -3.5, 2.0 ** -3):
        x = np.full(16, v, np.float32)
        q, s, z = Q.quantize_asym_int4(x, 16)
        assert float(s[0]) == 0.0 and not q.any()
        assert Q.dequantize_asym_int4(q, s, z, 16).tolist() == [v] * 16


def test_saturating_scale_and_zero():
    x = np.zeros(16, np.float32)
    x[0] = 1.0e7  # max|x|/127 = 78740 > 65504
    q, s = Q.quantize_sym_int8(x, 16)
    assert float(s[0]) == 65504.0 and q[0] == 127
    x = np.full(16, -70000.0, np.float32)
    x[1] = 0.0
    q, s, z = Q.quantize_asym_int4(x, 16)
    assert float(z[0]) == -65504.0


def test_negative_tie_and_negative_zero():
    x = np.zeros(16, np.float32)
    x[0] = 127.0 / 128  # scale 2^-7
    x[1] = -2.0 ** -8   # -0.5 -> rne -> -0 -> code 0
    x[2] = -0.0
    q, s = Q.quantize_sym_int8(x, 16)
    assert q[1] == 0 and q[2] == 0


# -------------------------------------------- reduction to the tutorial snippet

def test_reduces_to_per_tensor_snippet():
    # The tutorial's per-tensor INT8: scale = max|x| / 127, codes = (x/scale).round().
    # With one group over the whole tensor and the scale kept in fp32, the
    # oracle must give exactly what torch gives for that snippet.
    x = torch.randn(4096, generator=torch.Generator().manual_seed(11)) * 2
    scale = x.abs().max() / 127
    ref = (x / scale).round().to(torch.int8).numpy()
    q, s = Q.quantize_sym_int8(x.numpy(), x.numel(), fp16_scale=False)
    assert np.float32(s[0]) == np.float32(scale.item())
    assert np.array_equal(q, ref)


def test_per_group_beats_per_tensor_on_outliers():
    # The report's ordering (section 3.2): with outlier channels, per-channel-
    # block INT8 error is far below per-tensor INT8 error. Direction only.
    r = rng(12)
    x = bf16(r.standard_normal((256, 512)))
    x[:, r.choice(512, 4, replace=False)] *= 20
    q, s = Q.quantize_sym_int8(x, 16)
    e_grp = np.abs(Q.dequantize_sym_int8(q, s, 16) - x).mean()
    qt, st = Q.quantize_sym_int8(x.reshape(-1), x.size)
    e_ten = np.abs(Q.dequantize_sym_int8(qt, st, x.size).reshape(x.shape) - x).mean()
    assert e_grp * 5 < e_ten


def test_asym_int4_beats_sym_int4_on_skewed_latent():
    # The report's ordering (section 3.2): asymmetric INT4 beats symmetric INT4
    # on an asymmetric latent. Symmetric INT4 here is the same recipe with 7.
    x = bf16(np.abs(rng(13).standard_normal((256, 512))) * 1.5 - 0.5)
    q, s, z = Q.quantize_asym_int4(x, 16)
    e_asym = np.abs(Q.dequantize_asym_int4(q, s, z, 16) - x).mean()
    xg = x.reshape(256, 32, 16)
    s7 = np.abs(xg).max(-1, keepdims=True) / 7
    e_sym = np.abs(np.clip(np.rint(xg / s7), -7, 7) * s7 - xg).mean()
    assert e_asym < e_sym


def test_int4_zero_point_rounds_down(golden):
    g = golden("quant_hand.json")["int4_zero_round_down"]
    x = np.array(g["x"], np.float32)
    assert x[0] == np.float32(-65 * 2.0 ** -26) and np.array_equal(bf16(x), x)
    q, s, z = Q.quantize_asym_int4(x, 16)
    assert int(z.view(np.uint16)[0]) == g["zero_bits"]
    # the scale here is an fp16 subnormal, where the s/2 error bound does not hold
    assert float(s[0]) < 2.0 ** -14


def test_zero_point_of_negative_zero_is_positive_zero():
    x = np.array([-0.0] + [0.0] * 15, np.float32)
    q, s, z = Q.quantize_asym_int4(x, 16)
    assert int(z.view(np.uint16)[0]) == 0
    x = np.array([-0.0] + [1.0] * 15, np.float32)
    q, s, z = Q.quantize_asym_int4(x, 16)
    assert int(z.view(np.uint16)[0]) == 0


def test_zero_scale_is_positive_zero():
    # groups of signed zeros: neither the scale nor the zero-point may carry a sign
    for vals in ([-0.0] * 16, [0.0, -0.0] * 8, [-0.0] * 15 + [0.0]):
        q, s, z = Q.quantize_asym_int4(np.array(vals, np.float32), 16)
        assert int(s.view(np.uint16)[0]) == 0 and int(z.view(np.uint16)[0]) == 0
        assert not q.any()


# ------------------------------------------------ the formats of the next rows

def test_sym_int4_hand_case():
    # max|x| = 1.75 -> s = 1.75 / 7 = 0.25 exactly; x / s = 7, -2, 0.5, 1.5,
    # -4, 2.5, -3.5, 0 -> nearest, ties to even: 7, -2, 0, 2, -4, 2, -4, 0
    x = np.array([1.75, -0.5, 0.125, 0.375, -1.0, 0.625, -0.875, 0.0], np.float32)
    q, s = Q.quantize_sym_int4(x, 8)
    assert s.dtype == np.float16 and float(s[0]) == 0.25
    assert q.tolist() == [7, -2, 0, 2, -4, 2, -4, 0]
    # nibbles are code + 8 (15, 6, 8, 10, 4, 10, 4, 8), the even channel low
    packed = Q.pack_sym_int4(q)
    assert packed.tolist() == [(15 | (6 << 4)), (8 | (10 << 4)), (4 | (10 << 4)), (4 | (8 << 4))]
    assert Q.unpack_sym_int4(packed).tolist() == q.tolist()


def test_sym_int4_bounds_and_extremes():
    x = bf16(rng(21).standard_normal((300, 64)) * 3)
    q, s = Q.quantize_sym_int4(x, 8)
    assert q.min() >= -7 and q.max() <= 7
    xh = Q.dequantize_sym_int8(q, s, 8)
    sg = np.repeat(s.astype(np.float64), 8, axis=-1)
    assert np.all(np.abs(xh - x) <= sg / 2 + 1e-12 * np.abs(x))
    # the element of largest magnitude of each group maps to +-7
    xg, qg = x.reshape(300, 8, 8), q.reshape(300, 8, 8)
    i = np.abs(xg).argmax(-1)
    top = np.take_along_axis(qg, i[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 7)
    q0, s0 = Q.quantize_sym_int4(np.zeros(8, np.float32), 8)
    assert not q0.any() and float(s0[0]) == 0.0


@pytest.mark.parametrize("fmt", ["int8_kbf16", "int4_kint4"])
def test_new_formats_compose_the_existing_quantizers(fmt):
    r = rng(22)
    c = bf16(r.standard_normal((5, 512)) * 4)
    k = bf16(r.standard_normal((5, 64)))
    p = Q.quantize_rows(c, k, fmt)
    ch, kh = Q.dequantize_rows(p, fmt)
    if fmt == "int8_kbf16":
        ref = Q.quantize_rows(c, k, "int8")
        assert np.array_equal(p["ckv"], ref["ckv"]) and np.array_equal(p["scale"], ref["scale"][:, :32])
        assert np.array_equal(kh, k.astype(np.float64))  # k_pe kept exactly
        assert p["scale"].shape == (5, 32)
    else:
        ref = Q.quantize_rows(c, k, "int4")
        for key in ("ckv", "zero"):
            assert np.array_equal(p[key], ref[key])
        assert np.array_equal(p["scale"][:, :32], ref["scale"][:, :32])
        assert p["kpe"].shape == (5, 32) and p["kpe"].dtype == np.uint8
        kq, ks = Q.quantize_sym_int4(k, 8)
        assert np.array_equal(p["scale"][:, 32:], ks)
        assert np.allclose(kh, Q.dequantize_sym_int8(kq, ks, 8), rtol=0, atol=0)
