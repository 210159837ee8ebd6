"""Pins for oracle.attention: the toy example's orientation, absorbed equals
naive expanded attention, the expanded path equals torch's SDPA, closed forms
and invariants."""

import numpy as np
import pytest
import torch

from oracle import attention as A

TAU = 1.0 / np.sqrt(192.0)


def tiny(seed, H=3, L=7, dc=16, dn=8, dr=4, dv=8):
    r = np.random.default_rng(seed)
    return dict(
        q_nope=r.standard_normal((H, dn)),
        q_pe=r.standard_normal((H, dr)),
        w_uk=r.standard_normal((H, dn, dc)) / np.sqrt(dc),
        w_uv=r.standard_normal((H, dc, dv)) / np.sqrt(dc),
        ckv=r.standard_normal((L, dc)),
        kpe=r.standard_normal((L, dr)),
    )


def test_toy_example_orientation(golden):
    g = golden("toy_mla.json")
    x = np.array(g["x"], float)
    c = x @ np.array(g["w_down"])
    assert np.allclose(c, g["c_kv"], atol=1e-12)
    # K_1 = C W_1^up with W_1^up [d_c, d_k]; the oracle's W_UK[h] is [d_k, d_c].
    w_up = np.array(g["w_up_k_head1"])
    K, V = A.expand_kv(np.array([g["c_kv"]]), np.zeros((1, 0)), w_up.T[None], np.eye(2)[None])
    assert np.allclose(K[0, 0], g["k_head1"], atol=1e-12)
    assert np.allclose(V[0, 0], g["c_kv"], atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_absorbed_equals_expanded(seed):
    t = tiny(seed, H=1 + seed % 4, L=1 + 2 * seed)
    a = A.decode_absorbed(**t, softmax_scale=TAU)
    e = A.decode_expanded(**t, softmax_scale=TAU)
    assert np.max(np.abs(a - e)) <= 1e-12 * max(1.0, np.max(np.abs(e)))


def test_absorbed_equals_expanded_at_model_dims():
    t = tiny(42, H=2, L=9, dc=512, dn=128, dr=64, dv=128)
    a = A.decode_absorbed(**t, softmax_scale=TAU)
    e = A.decode_expanded(**t, softmax_scale=TAU)
    assert np.max(np.abs(a - e)) <= 1e-12 * max(1.0, np.max(np.abs(e)))


@pytest.mark.parametrize("seed", range(4))
def test_expanded_equals_torch_sdpa(seed):
    t = tiny(100 + seed, H=4, L=9)
    H = t["q_nope"].shape[0]
    # build the expanded K and V with torch from the per-head projections
    c = torch.tensor(t["ckv"])
    wuk = torch.tensor(t["w_uk"])
    wuv = torch.tensor(t["w_uv"])
    k = torch.cat([torch.stack([c @ wuk[h].T for h in range(H)]),
                   torch.tensor(t["kpe"]).expand(H, -1, -1)], dim=-1)  # [H, L, 12]
    v = torch.stack([c @ wuv[h] for h in range(H)])  # [H, L, 8]
    q = torch.cat([torch.tensor(t["q_nope"]), torch.tensor(t["q_pe"])], -1)[:, None]  # [H,1,12]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=TAU)[:, 0].numpy()
    e = A.decode_expanded(**t, softmax_scale=TAU)
    assert np.allclose(e, ref, rtol=1e-12, atol=1e-13)


def test_single_token_returns_its_value():
    t = tiny(7, L=1)
    out = A.decode_absorbed(**t, softmax_scale=TAU)
    ref = np.stack([t["ckv"][0] @ t["w_uv"][h] for h in range(t["w_uv"].shape[0])])
    assert np.allclose(out, ref, atol=1e-13)


def test_unit_latent_selects_a_row_of_w_uv():
    # one token whose latent is e_j: the output is row j of W_UV[h]
    dc, dv = 6, 6
    w_uv = np.arange(dc * dv, dtype=float).reshape(1, dc, dv)
    ckv = np.zeros((1, dc))
    ckv[0, 2] = 1.0
    out = A.decode_absorbed(np.ones((1, 3)), np.ones((1, 2)), np.ones((1, 3, dc)), w_uv,
                            ckv, np.zeros((1, 2)), TAU)
    assert out[0].tolist() == w_uv[0, 2].tolist()


def test_zero_query_gives_mean_value():
    t = tiny(8, L=11)
    t["q_nope"][:] = 0
    t["q_pe"][:] = 0
    out = A.decode_absorbed(**t, softmax_scale=TAU)
    mean_c = t["ckv"].mean(axis=0)
    ref = np.stack([mean_c @ t["w_uv"][h] for h in range(t["w_uv"].shape[0])])
    assert np.allclose(out, ref, atol=1e-13)


def test_identical_tokens_give_that_value():
    t = tiny(9, L=5)
    t["ckv"][:] = t["ckv"][0]
    t["kpe"][:] = t["kpe"][0]
    out = A.decode_absorbed(**t, softmax_scale=TAU)
    ref = np.stack([t["ckv"][0] @ t["w_uv"][h] for h in range(t["w_uv"].shape[0])])
    assert np.allclose(out, ref, atol=1e-13)


def test_linear_in_w_uv_and_token_permutation_invariant():
    t = tiny(10, L=13)
    out = A.decode_absorbed(**t, softmax_scale=TAU)
    t2 = dict(t, w_uv=t["w_uv"] * 2.5)
    assert np.allclose(A.decode_absorbed(**t2, softmax_scale=TAU), 2.5 * out, atol=1e-13)
    perm = np.random.default_rng(0).permutation(13)
    t3 = dict(t, ckv=t["ckv"][perm], kpe=t["kpe"][perm])
    assert np.allclose(A.decode_absorbed(**t3, softmax_scale=TAU), out, atol=1e-13)


def test_rope_term_matters():
    # changing only k_pe changes the output (the q_pe . k_pe term is present)
    t = tiny(11, L=6)
    out = A.decode_absorbed(**t, softmax_scale=TAU)
    t2 = dict(t, kpe=t["kpe"] * -1)
    assert not np.allclose(A.decode_absorbed(**t2, softmax_scale=TAU), out)


def test_empty_sequence_is_zero():
    t = tiny(12, L=0)
    assert not A.decode_absorbed(**t, softmax_scale=TAU).any()
    assert not A.decode_expanded(**t, softmax_scale=TAU).any()


def test_split_merge_algebra():
    # The split-KV merge a GPU kernel uses (per split: m = max s, l = sum e^(s-m),
    # acc = sum e^(s-m) c; merged: M = max m, w = e^(m-M), o = sum w acc / sum w l)
    # reproduces the full softmax. Checked here in float64 against the oracle.
    t = tiny(13, H=2, L=23)
    full = A.decode_absorbed(**t, softmax_scale=TAU)
    q_abs = A.absorb_query(t["q_nope"], t["w_uk"])
    s = TAU * (q_abs @ t["ckv"].T + t["q_pe"] @ t["kpe"].T)
    for bounds in ([0, 23], [0, 5, 23], [0, 1, 2, 3, 23], [0, 7, 7, 14, 23]):
        ms, ls, accs = [], [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            if a == b:
                ms.append(np.full(2, -np.inf)); ls.append(np.zeros(2)); accs.append(np.zeros((2, 16)))
                continue
            m = s[:, a:b].max(1)
            e = np.exp(s[:, a:b] - m[:, None])
            ms.append(m); ls.append(e.sum(1)); accs.append(e @ t["ckv"][a:b])
        M = np.max(ms, axis=0)
        w = [np.where(np.isinf(m), 0.0, np.exp(m - M)) for m in ms]
        o_lat = sum(wi[:, None] * ai for wi, ai in zip(w, accs)) / sum(wi * li for wi, li in zip(w, ls))[:, None]
        out = np.stack([o_lat[h] @ t["w_uv"][h] for h in range(2)])
        assert np.allclose(out, full, atol=1e-13)


def test_decode_batch_uses_each_length():
    t = tiny(14, L=10)
    ckv = np.stack([t["ckv"], t["ckv"][::-1]])
    kpe = np.stack([t["kpe"], t["kpe"][::-1]])
    qn = np.stack([t["q_nope"]] * 2)
    qp = np.stack([t["q_pe"]] * 2)
    out = A.decode_batch(qn, qp, t["w_uk"], t["w_uv"], ckv, kpe, [4, 0], TAU)
    ref0 = A.decode_absorbed(t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], t["ckv"][:4], t["kpe"][:4], TAU)
    assert np.allclose(out[0], ref0) and not out[1].any()
