"""The synthetic quantization-error study reproduces the orderings the pages
report (section 4.2 / 3.2 tables, section 5.1), and its error metric behaves."""

import numpy as np
import pytest

from oracle import study as S


@pytest.fixture(scope="module")
def res():
    return S.run(n_seq=2, length=256)


def test_metric_sanity():
    x = np.random.default_rng(0).standard_normal((5, 16))
    assert np.all(S.rel_errors(x, x) == 0)
    assert np.allclose(S.rel_errors(x, np.zeros_like(x)), 1.0)
    assert np.allclose(S.rel_errors(3 * x, 3 * x + 3 * 0.1 * x), 0.1)
    assert S.rel_errors(np.zeros((1, 4)), np.ones((1, 4)))[0] == 0.0


@pytest.mark.parametrize("dist", ["outlier", "skewed"])
def test_per_block_beats_per_token_beats_per_tensor(res, dist):
    r = res[dist]["reconstruction"]
    assert r["latent int8_b32"][0] * 2 < r["latent int8_token"][0] < r["latent int8_tensor"][0]
    a = res[dist]["attention"]
    assert a["int8_b32 + k_pe int8_b8"][0] < a["int8_token + k_pe int8_b8"][0] < a["int8_tensor + k_pe int8_b8"][0]


@pytest.mark.parametrize("dist", ["outlier", "skewed"])
def test_asymmetric_int4_beats_symmetric(res, dist):
    r = res[dist]["reconstruction"]
    assert r["latent int4a_b32"][0] < 0.8 * r["latent int4s_b32"][0]
    a = res[dist]["attention"]
    assert a["int4a_b32 + k_pe int8_b8"][0] < a["int4s_b32 + k_pe int8_b8"][0]


@pytest.mark.parametrize("dist", ["outlier", "skewed"])
def test_more_blocks_are_more_accurate(res, dist):
    r = res[dist]["reconstruction"]
    for kind in ("int8", "int4a"):
        errs = [r[f"latent {kind}_b{n}"][0] for n in (8, 16, 32, 64)]
        assert all(a > b for a, b in zip(errs, errs[1:])), (kind, errs)


@pytest.mark.parametrize("dist", ["outlier", "skewed"])
def test_kpe_int8_is_stable(res, dist):
    r = res[dist]["reconstruction"]
    assert r["k_pe int8_b8"][0] < r["latent int8_b32"][0]
    assert r["k_pe int8_b8"][0] < r["k_pe int4s_b8"][0]
    # keeping k_pe in bf16 changes the INT8 attention error very little
    a = res[dist]["attention"]
    assert abs(a["int8_b32 + k_pe bf16"][0] - a["int8_b32 + k_pe int8_b8"][0]) < 0.25 * a["int8_b32 + k_pe int8_b8"][0]
