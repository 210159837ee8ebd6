"""The largest sequence the library takes: a bf16 latent plane of exactly
2^30 bytes per sequence (capacity 2^20 tokens, 1024 bytes a row), two
sequences (the second one's rows start 1 GiB into the plane), one full and one
ragged, decoded against the fp64 oracle; one token more is refused."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import LatentCache, MlaError
from mla_latent_kv_cache_amd import _lib

from gpu_util import assert_close, f32, oracle_decode_np, random_rows, run_oracle_jobs

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
TAU = 1.0 / np.sqrt(192.0)


def test_bf16_sequence_plane_of_one_gib():
    cap, H, B = 1 << 20, 16, 2
    lens = [cap, cap - 37]
    cache = LatentCache("bf16", 1, B, cap, device="cuda")
    rows = []
    for b in range(B):
        c, k = random_rows(lens[b], 700 + b, "normal")
        n = [0] * B
        n[b] = lens[b]
        ckv = torch.zeros((B, lens[b], 512), dtype=torch.bfloat16, device="cuda")
        kpe = torch.zeros((B, lens[b], 64), dtype=torch.bfloat16, device="cuda")
        ckv[b], kpe[b] = c, k
        cache.append(0, ckv, kpe, n_new=n)
        del ckv, kpe
        rows.append((f32(c), f32(k)))
        del c, k
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    qn = torch.randn((B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    qp = torch.randn((B, H, 64), generator=g, device="cuda").to(torch.bfloat16)
    wuk = (torch.randn((H, 128, 512), generator=g, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
    wuv = (torch.randn((H, 512, 128), generator=g, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
    out = cache.decode(0, qn, qp, wuk, wuv, TAU)
    torch.cuda.synchronize()
    assert cache.lengths(0).tolist() == lens
    out_h, qn_h, qp_h, wk, wv = f32(out), f32(qn), f32(qp), f32(wuk), f32(wuv)
    jobs = ((b, oracle_decode_np, (rows[b][0], rows[b][1], "bf16", qn_h[b], qp_h[b], wk, wv, TAU))
            for b in range(B))
    for b, ref in run_oracle_jobs(jobs, threads=2):
        assert_close(out_h[b], ref, f"seq {b} of {lens[b]} tokens")


def test_one_token_past_the_plane_limit_is_refused():
    with pytest.raises(MlaError) as e:
        cache = LatentCache("bf16", 1, 1, (1 << 20) + 16, device="cuda")
        qn = torch.zeros((1, 16, 128), dtype=torch.bfloat16, device="cuda")
        qp = torch.zeros((1, 16, 64), dtype=torch.bfloat16, device="cuda")
        wuk = torch.zeros((16, 128, 512), dtype=torch.bfloat16, device="cuda")
        wuv = torch.zeros((16, 512, 128), dtype=torch.bfloat16, device="cuda")
        cache.decode(0, qn, qp, wuk, wuv, TAU)
    assert e.value.status == _lib.MLA_ERR_UNSUPPORTED
