"""The quantization-error study through the HIP path: for each quantized
cache format, the attention-output error of the GPU decode over the quantized
cache against the GPU decode over a bf16 cache of the same rows equals the
oracle study's (oracle.study.attention_error) for the same quantizers."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import LatentCache
from mla_latent_kv_cache_amd import workloads as W
from oracle import study as S

pytestmark = pytest.mark.gpu

CASES = {  # format: (study input workload, latent method, k_pe method)
    "int8": (1, "int8_b32", "int8_b8"),
    "int8_kbf16": (1, "int8_b32", None),
    "int4": (2, "int4a_b32", "int8_b8"),
    "int4_kint4": (2, "int4a_b32", "int4s_b8"),
}


def gpu_outputs(fmt, seqs, qn, qp, wuk, wuv):
    B, L = len(seqs), seqs[0][0].shape[0]
    cache = LatentCache(fmt, 1, B, L)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    cache.append(0, bf(np.stack([s[0] for s in seqs])), bf(np.stack([s[1] for s in seqs])))
    out = cache.decode(0, bf(qn), bf(qp), bf(wuk), bf(wuv), W.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("fmt", list(CASES))
def test_study_attention_error_through_the_kernels(fmt):
    wid, lm, km = CASES[fmt]
    seqs, qn, qp, wuk, wuv = S.inputs(wid, n_seq=4, length=512)
    ref = gpu_outputs("bf16", seqs, qn, qp, wuk, wuv)
    got = gpu_outputs(fmt, seqs, qn, qp, wuk, wuv)
    e = np.concatenate([S.rel_errors(ref[b], got[b]) for b in range(len(seqs))])
    mean_o, max_o = S.attention_error(seqs, qn, qp, wuk, wuv, W.SOFTMAX_SCALE, lm, km)
    assert abs(e.mean() - mean_o) <= 0.15 * mean_o + 1e-3, (fmt, e.mean(), mean_o)
    assert abs(e.max() - max_o) <= 0.25 * max_o + 2e-3, (fmt, e.max(), max_o)
