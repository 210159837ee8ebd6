"""Seeded synthetic inputs shaped like DeepSeek-V2-Lite MLA decode.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantization, no attention). Both the HIP path and the CPU
oracle consume the bf16 tensors it returns.

Shapes come from the reports ("Absorbed MLA Cache Optimization on
DeepSeek-V2-Lite": 27 layers, 16 heads, kv_lora_rank 512 + rope 64, qk_nope
128, v 128, sections 1.1-1.3). The trained weights and real activations the
reports measured on are not available; these workloads stand in for them:

  weights  W_UK [H,128,512], W_UV [H,512,128] ~ N(0, 1/512)
  queries  q_nope [B,H,128], q_pe [B,H,64] ~ N(0, 1)
  latent   "normal":        c_kv ~ N(0,1)
           "outlier":       c_kv ~ N(0,1), 4 distinct channels per layer x20
           "skew_outlier":  c_kv = |N(0,1)| * 1.5 - 0.5, then the same outliers
  k_pe     ~ N(0, 1)
Every value is drawn in fp32 and rounded to bf16 (round to nearest even).

Each tensor has its own torch.Generator seeded from (workload, layer, kind,
sequence), so any one sequence of any layer can be regenerated alone. The
draws depend on the device the generator runs on (torch's CPU and GPU
generators differ); callers that compare against the oracle copy the same
bf16 tensors to the host rather than regenerating them.
"""

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SOFTMAX_SCALE = 1.0 / math.sqrt(128 + 64)


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str
    layers: int
    batch: int
    heads: int
    seq: object          # int, or (lo, hi) inclusive for ragged lengths
    dist: str
    append: int = 0      # tokens appended per sequence after the prefill
    num_splits: int = 0  # 0 = the library's choice
    notes: str = field(default="", compare=False)


WORKLOADS = (
    Workload("bf16_l1_b1_h16_s256", "bf16", 1, 1, 16, 256, "normal",
             notes="bf16 latent cache, the small correctness case"),
    Workload("int8_l1_b8_h16_s4096", "int8", 1, 8, 16, 4096, "outlier", append=64,
             notes="INT8 latent + INT8 k_pe, quantize-on-append of 64 tokens per sequence"),
    Workload("int4_l1_b32_h16_s32768", "int4", 1, 32, 16, 32768, "skew_outlier",
             notes="asymmetric INT4 latent + INT8 k_pe on a skewed latent"),
    Workload("int8_l27_b64_h16_ragged1024-16384", "int8", 27, 64, 16, (1024, 16384), "outlier",
             notes="DeepSeek-V2-Lite-shaped full stack, ragged lengths, one decode step per layer"),
    Workload("int4_l1_b16_h128_s131072", "int4", 1, 16, 128, 131072, "skew_outlier", num_splits=64,
             notes="wide-head long context, 64 KV splits"),
)

_KINDS = {"weights": 1, "queries": 2, "latent": 3, "append": 4, "step": 5, "outliers": 6, "lengths": 7}


def seed_for(wid, layer, kind, b=0):
    return ((int(wid) * 64 + int(layer)) * 16 + _KINDS[kind]) * (1 << 20) + int(b) + 12345


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, device, seed):
    return torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def lengths(wid):
    """Per-sequence cached lengths (int64 [B]); the same for every layer."""
    w = WORKLOADS[wid]
    if isinstance(w.seq, tuple):
        lo, hi = w.seq
        g = _gen("cpu", seed_for(wid, 0, "lengths"))
        return torch.randint(lo, hi + 1, (w.batch,), generator=g).numpy().astype(np.int64)
    return np.full(w.batch, int(w.seq), dtype=np.int64)


def capacity(wid):
    w = WORKLOADS[wid]
    base = w.seq[1] if isinstance(w.seq, tuple) else int(w.seq)
    return base + w.append + (1 if isinstance(w.seq, tuple) else 0)


def weights(wid, layer, device="cpu"):
    """(W_UK [H,128,512], W_UV [H,512,128]) bf16, ~N(0, 1/512)."""
    H = WORKLOADS[wid].heads
    g = _gen(device, seed_for(wid, layer, "weights"))
    std = 1.0 / math.sqrt(512.0)
    w_uk = (torch.randn((H, 128, 512), generator=g, device=device) * std).to(torch.bfloat16)
    w_uv = (torch.randn((H, 512, 128), generator=g, device=device) * std).to(torch.bfloat16)
    return w_uk, w_uv


def queries(wid, layer, device="cpu", step=0):
    """(q_nope [B,H,128], q_pe [B,H,64]) bf16, ~N(0, 1)."""
    w = WORKLOADS[wid]
    g = _gen(device, seed_for(wid, layer, "queries", step))
    q_nope = torch.randn((w.batch, w.heads, 128), generator=g, device=device).to(torch.bfloat16)
    q_pe = torch.randn((w.batch, w.heads, 64), generator=g, device=device).to(torch.bfloat16)
    return q_nope, q_pe


def outlier_channels(wid, layer):
    """The 4 distinct latent channels scaled x20 in this layer (empty for 'normal')."""
    if WORKLOADS[wid].dist == "normal":
        return torch.empty(0, dtype=torch.long)
    g = _gen("cpu", seed_for(wid, layer, "outliers"))
    return torch.randperm(512, generator=g)[:4]


def latent_rows(wid, layer, b, n, device="cpu", kind="latent"):
    """(c_kv [n,512], k_pe [n,64]) bf16 for sequence b of a layer.

    kind "latent" is the prefilled cache, "append" the appended tokens,
    "step" the token a decode step stores (b may then index the step).
    """
    w = WORKLOADS[wid]
    g = _gen(device, seed_for(wid, layer, kind, b))
    c = torch.randn((n, 512), generator=g, device=device)
    if w.dist == "skew_outlier":
        c = c.abs() * 1.5 - 0.5
    idx = outlier_channels(wid, layer).to(device)
    if idx.numel():
        c[:, idx] *= 20.0
    k = torch.randn((n, 64), generator=g, device=device)
    return c.to(torch.bfloat16), k.to(torch.bfloat16)


def latent_batch(wid, layer, n, device="cpu", kind="latent", counts=None):
    """Stack of latent_rows over the batch, padded to n rows: ([B,n,512], [B,n,64])."""
    w = WORKLOADS[wid]
    ckv = torch.zeros((w.batch, n, 512), dtype=torch.bfloat16, device=device)
    kpe = torch.zeros((w.batch, n, 64), dtype=torch.bfloat16, device=device)
    for b in range(w.batch):
        m = n if counts is None else int(counts[b])
        if m:
            c, k = latent_rows(wid, layer, b, m, device, kind)
            ckv[b, :m] = c
            kpe[b, :m] = k
    return ckv, kpe
