"""mla_decode_attn_static (the entry point that allocates nothing, for
callers that cannot allocate) against mla_decode_attn through the C ABI:
bit-identical outputs on two calls in a row, the second with a smaller
input, and the size limit."""

import ctypes

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import _lib

from gpu_util import random_problem

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def call_static(cache, q_nope, q_pe, w_uk, w_uv, H, splits=0):
    out = torch.full((cache.batch, H, 128), float("nan"), dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = _lib.lib().mla_decode_attn_static(ctypes.byref(cache.struct), 0, p(q_nope), p(q_pe), p(w_uk), p(w_uv), H,
                                           TAU, splits, p(out),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out


@pytest.mark.parametrize("fmt,H", [("int8", 16), ("int4", 128)])
def test_static_equals_workspace_call_twice_then_smaller(fmt, H):
    big = random_problem(fmt, 6, H, [1000, 3, 0, 777, 64, 1500], seed=301, cap=1536)
    small = random_problem(fmt, 2, H, [50, 9], seed=302, cap=64)
    for (cache, rows, qn, qp, wuk, wuv), splits in ((big, 0), (small, 0), (big, 3)):
        ref = cache.decode(0, qn, qp, wuk, wuv, TAU, num_splits=splits)
        st, out = call_static(cache, qn, qp, wuk, wuv, H, splits)
        torch.cuda.synchronize()
        assert st == _lib.MLA_OK, _lib.status_str(st)
        assert torch.equal(out, ref), (fmt, H, cache.batch, splits)


def test_static_rejects_a_workspace_beyond_its_array():
    cache, rows, qn, qp, wuk, wuv = random_problem("int8", 4, 128, [10, 20, 30, 40], seed=303, cap=4096)
    need = cache.workspace_bytes(128, 2048)
    assert need > _lib.STATIC_SCRATCH_BYTES
    st, out = call_static(cache, qn, qp, wuk, wuv, 128, splits=2048)
    torch.cuda.synchronize()
    assert st == _lib.MLA_ERR_WORKSPACE
    assert torch.isnan(out).all()  # nothing was launched
