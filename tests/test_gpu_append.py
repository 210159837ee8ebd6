"""Quantize-on-append on the GPU, bit-exact against the oracle quantizer."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import LatentCache, MlaError
from mla_latent_kv_cache_amd import _lib

from gpu_util import assert_planes_equal, f32, oracle_planes, random_rows

pytestmark = pytest.mark.gpu
FORMATS = ["bf16", "int8", "int4", "int8_kbf16", "int4_kint4"]


@pytest.mark.parametrize("fmt", FORMATS)
def test_append_in_pieces_bit_exact(fmt):
    B, cap = 3, 64
    cache = LatentCache(fmt, 2, B, cap)
    rows = {b: [] for b in range(B)}
    for piece, T in enumerate((20, 17, 1)):
        ckv = torch.empty((B, T, 512), dtype=torch.bfloat16, device="cuda")
        kpe = torch.empty((B, T, 64), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            c, k = random_rows(T, 1000 * piece + b, "skew" if fmt.startswith("int4") else "outlier")
            ckv[b], kpe[b] = c, k
            rows[b].append((c, k))
        cache.append(1, ckv, kpe)
    torch.cuda.synchronize()
    assert cache.seq_lens[1].tolist() == [38] * B and cache.seq_lens[0].tolist() == [0] * B
    for b in range(B):
        c = torch.cat([r[0] for r in rows[b]])
        k = torch.cat([r[1] for r in rows[b]])
        assert_planes_equal(cache.planes(1, b), oracle_planes(c, k, fmt), fmt, f"{fmt} seq {b}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_append_ragged_counts(fmt):
    B, T = 4, 33
    cache = LatentCache(fmt, 1, B, 80)
    ckv = torch.empty((B, T, 512), dtype=torch.bfloat16, device="cuda")
    kpe = torch.empty((B, T, 64), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        ckv[b], kpe[b] = random_rows(T, 77 + b)
    counts = [0, 1, 16, 33]
    cache.append(0, ckv, kpe, n_new=counts)
    cache.append(0, ckv, kpe, n_new=[2, 0, 17, 3])
    torch.cuda.synchronize()
    assert cache.seq_lens[0].tolist() == [2, 1, 33, 36]
    for b, (n1, n2) in enumerate(zip(counts, [2, 0, 17, 3])):
        c = torch.cat([ckv[b, :n1], ckv[b, :n2]])
        k = torch.cat([kpe[b, :n1], kpe[b, :n2]])
        assert_planes_equal(cache.planes(0, b), oracle_planes(c, k, fmt), fmt, f"{fmt} seq {b}")


def edge_rows():
    """Rows whose groups hit the special cases of the quantizers."""
    rows = np.zeros((8, 512), np.float32)
    kp = np.zeros((8, 64), np.float32)
    rows[0] = 0.0                                         # all-zero groups
    rows[1] = 0.75                                        # constant groups
    rows[2, 5] = -7.25                                    # one non-zero value
    rows[3] = np.linspace(-1e-6, 1e-6, 512)               # fp16-subnormal scales / zero-points
    rows[4] = np.where(np.arange(512) % 3 == 0, 1.0e7, -3.0)  # saturating scales
    rows[5] = -0.0                                        # negative zeros
    rows[5, ::7] = 0.0
    rows[5, 17] = -1e-39                                  # an fp32 denormal group minimum
    rows[6] = np.where(np.arange(512) % 2 == 0, -70000.0, 70000.0)  # beyond fp16 range
    rows[7] = (np.arange(512) % 16) * 0.125 - 0.5         # exact ties in INT8 and INT4
    kp[0] = 0.0
    kp[1] = -2.0
    kp[2, 3] = 1e-30
    kp[3] = np.linspace(-3, 3, 64)
    kp[4] = 1.0e6
    kp[7] = (np.arange(64) % 8) * 0.25 - 1.0
    to_bf = lambda a: torch.tensor(a).to(torch.bfloat16)
    return to_bf(rows), to_bf(kp)


@pytest.mark.parametrize("fmt", ["int8", "int4", "int8_kbf16", "int4_kint4"])
def test_append_edge_groups_bit_exact(fmt):
    c, k = edge_rows()
    cache = LatentCache(fmt, 1, 1, 8)
    cache.append(0, c[None].cuda(), k[None].cuda())
    torch.cuda.synchronize()
    assert_planes_equal(cache.planes(0, 0), oracle_planes(c, k, fmt), fmt, "edge rows")


def test_append_capacity_guard_and_noop():
    cache = LatentCache("int8", 1, 2, 10)
    c, k = random_rows(8, 5)
    ckv = torch.stack([c, c]).contiguous()
    kpe = torch.stack([k, k]).contiguous()
    cache.append(0, ckv, kpe)
    with pytest.raises(MlaError) as e:
        cache.append(0, ckv, kpe)
    assert e.value.status == _lib.MLA_ERR_CAPACITY
    cache.append(0, ckv[:, :0].contiguous(), kpe[:, :0].contiguous())  # zero rows: no-op
    torch.cuda.synchronize()
    assert cache.seq_lens[0].tolist() == [8, 8] and cache.lengths(0).tolist() == [8, 8]


@pytest.mark.parametrize("fmt", FORMATS)
def test_get_matches_oracle_dequantization(fmt):
    from oracle import quant as Q
    B, cap = 2, 40
    cache = LatentCache(fmt, 1, B, cap)
    ckv = torch.empty((B, 30, 512), dtype=torch.bfloat16, device="cuda")
    kpe = torch.empty((B, 30, 64), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        ckv[b], kpe[b] = random_rows(30, 300 + b, "skew")
    cache.append(0, ckv, kpe, n_new=[30, 11])
    gc, gk = cache.get(0)
    torch.cuda.synchronize()
    for b, n in enumerate((30, 11)):
        ch, kh = Q.dequantize_rows(oracle_planes(ckv[b, :n], kpe[b, :n], fmt), fmt)
        # the exact dequantized value rounded once to fp32
        assert np.array_equal(f32(gc[b, :n]), ch.astype(np.float32))
        assert np.array_equal(f32(gk[b, :n]), kh.astype(np.float32))
        assert not gc[b, n:].any() and not gk[b, n:].any()
