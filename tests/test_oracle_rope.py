"""Pins for oracle.rope: closed forms of the angle table, the invariants that
define a rotary embedding (norm, relative position, composition, pair
locality), the bf16 rounding against torch, and the fused step's special
cases (empty sequence, full sequence, position-free self score)."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import quant as Q
from oracle import rope as R


def f64_tables(max_pos):
    a = R.rope_angles(max_pos)
    return np.cos(a), np.sin(a)


def test_angle_closed_forms():
    a = R.rope_angles(1001)
    assert a.shape == (1001, 32)
    assert np.all(a[0] == 0.0)
    # theta_i = 10000^(-2i/64): theta_0 = 1, theta_16 = 1/100, theta_31 = 10^-3.875
    assert a[1, 0] == 1.0
    assert abs(a[1, 16] - 0.01) < 1e-17
    assert abs(a[1, 31] - 1.333521432163324e-4) < 1e-18
    assert abs(a[1000, 31] - 0.1333521432163324) < 1e-15


def test_table_values_and_identity_at_zero():
    cos, sin = R.rope_tables(4)
    assert cos.dtype == np.float32 and sin.dtype == np.float32
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    # cos(1) and sin(1), textbook values
    assert abs(float(cos[1, 0]) - 0.5403023058681398) < 6e-8
    assert abs(float(sin[1, 0]) - 0.8414709848078965) < 6e-8
    x = np.random.default_rng(0).standard_normal(64).astype(np.float32)
    assert np.array_equal(R.rotate_f32(x, cos[0], sin[0]), x)


def test_turn_direction_and_pair_locality():
    cos, sin = f64_tables(3)
    e0 = np.zeros(64)
    e0[0] = 1.0
    y = R.rotate_f64(e0, cos[1], sin[1])
    # (1, 0) turns counter-clockwise to (cos 1, sin 1); nothing else moves
    assert abs(y[0] - math.cos(1.0)) < 1e-15 and abs(y[1] - math.sin(1.0)) < 1e-15
    assert np.all(y[2:] == 0.0)
    e5 = np.zeros(64)
    e5[5] = 1.0  # the odd channel of pair 2
    y = R.rotate_f64(e5, cos[2], sin[2])
    assert np.count_nonzero(y) == 2 and y[4] < 0 and y[5] > 0


def test_norm_preserved_per_pair():
    cos, sin = f64_tables(5000)
    x = np.random.default_rng(1).standard_normal((7, 64))
    for pos in (1, 17, 4999):
        y = R.rotate_f64(x, cos[pos], sin[pos])
        n0 = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
        n1 = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
        assert np.allclose(n0, n1, rtol=1e-13, atol=0)


def test_relative_position_and_composition():
    # <R(m) q, R(n) k> depends on m - n only; R(a) R(b) = R(a + b)
    cos, sin = f64_tables(300)
    r = np.random.default_rng(2)
    q, k = r.standard_normal(64), r.standard_normal(64)
    for m, n in ((5, 2), (250, 13), (77, 77)):
        lhs = R.rotate_f64(q, cos[m], sin[m]) @ R.rotate_f64(k, cos[n], sin[n])
        d = m - n
        rhs = R.rotate_f64(q, cos[d], sin[d]) @ k
        assert abs(lhs - rhs) < 1e-12 * (1 + abs(rhs))
    for a, b in ((3, 4), (100, 199)):
        two = R.rotate_f64(R.rotate_f64(q, cos[a], sin[a]), cos[b], sin[b])
        assert np.allclose(two, R.rotate_f64(q, cos[a + b], sin[a + b]), rtol=0, atol=1e-12)


def test_fp32_turn_within_rounding_of_fp64():
    cos, sin = R.rope_tables(2048)
    x = (np.random.default_rng(3).standard_normal((9, 64)) * 30).astype(np.float32)
    for pos in (1, 1000, 2047):
        y32 = R.rotate_f32(x, cos[pos], sin[pos]).astype(np.float64)
        y64 = R.rotate_f64(x, cos[pos], sin[pos])
        bound = 2 * np.finfo(np.float32).eps * (np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]))
        assert np.all(np.abs(y32[..., 0::2] - y64[..., 0::2]) <= bound)
        assert np.all(np.abs(y32[..., 1::2] - y64[..., 1::2]) <= bound)


def test_bf16_rounding_matches_torch():
    assert R.bf16_rne(np.float32(1.0 + 2.0 ** -8)) == 1.0          # tie to even
    assert R.bf16_rne(np.float32(1.0 + 3 * 2.0 ** -8)) == 1.0 + 2.0 ** -6
    x = (np.random.default_rng(4).standard_normal(10000) * 10.0 ** np.random.default_rng(5).integers(-6, 6, 10000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(R.bf16_rne(x), ref)


def _token(seed, H=4):
    r = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    return dict(ckv_new=bf(r.standard_normal(512)), kpe_new=bf(r.standard_normal(64)),
                q_nope=bf(r.standard_normal((H, 128))), q_pe=bf(r.standard_normal((H, 64))),
                w_uk=bf(r.standard_normal((H, 128, 512)) / 512 ** 0.5),
                w_uv=bf(r.standard_normal((H, 512, 128)) / 512 ** 0.5))


@pytest.mark.parametrize("fmt", Q.FORMATS)
def test_step_on_empty_sequence_is_the_value_projection(fmt):
    # position 0 turns nothing; one token gets all the weight: out = c_hat W_UV[h]
    t = _token(6)
    cos, sin = R.rope_tables(8)
    planes, n, out = R.decode_step(np.zeros((0, 512)), np.zeros((0, 64)), 0, 8, t["ckv_new"], t["kpe_new"],
                                   t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], 0.1, fmt, cos, sin)
    assert n == 1
    c_hat, k_hat = Q.dequantize_rows({k: v[None] for k, v in planes.items()}, fmt)
    assert np.allclose(out, np.einsum("c,hce->he", c_hat[0], t["w_uv"]), rtol=1e-12, atol=1e-12)
    ref = Q.quantize_rows(t["ckv_new"][None], t["kpe_new"][None], fmt)
    for k in planes:
        assert np.array_equal(planes[k], ref[k][0])


def test_step_on_full_sequence_stores_nothing():
    t = _token(7)
    cos, sin = R.rope_tables(4)
    r = np.random.default_rng(8)
    ckv, kpe = r.standard_normal((3, 512)), r.standard_normal((3, 64))
    planes, n, out = R.decode_step(ckv, kpe, 3, 3, t["ckv_new"], t["kpe_new"], t["q_nope"], t["q_pe"],
                                   t["w_uk"], t["w_uv"], 0.1, "int8", cos, sin)
    assert planes is None and n == 3
    q_pe = R.rotate_f64(t["q_pe"], cos[3], sin[3])
    ref = A.decode_absorbed(t["q_nope"], q_pe, t["w_uk"], t["w_uv"], ckv, kpe, 0.1)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_new_token_self_score_is_position_free():
    # q_pe . k_pe of the new token is the same at every position (both turn
    # together); checked through the stored bf16 key in the bf16 format
    t = _token(9, H=2)
    cos, sin = R.rope_tables(5000)
    dots = []
    for pos in (0, 1, 4321):
        kq = R.bf16_rne(R.rotate_f32(t["kpe_new"], cos[pos], sin[pos])).astype(np.float64)
        qq = R.rotate_f64(t["q_pe"], cos[pos], sin[pos])
        dots.append(qq @ kq)
    for d in dots[1:]:
        assert np.allclose(d, dots[0], rtol=2e-2, atol=5e-2)  # bf16 rounding of the key only
