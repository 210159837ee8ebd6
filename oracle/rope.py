"""Oracle of the fused decode step: rotate the new token's RoPE parts, append
it, attend over the grown sequence (numpy only).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline use this module; the HIP library never does.

What the pages fix, and the readings taken where they leave it open:

* "DeepSeek的MLA技术", optimization 2 (adapting RoPE to MLA): the RoPE key is
  rotated by its position after it is produced and is cached already rotated;
  the page calls a rotary-embedding function but never defines it. Reading:
  the rotary embedding as first defined (RoFormer, Su et al. 2021):
  channel pairs (2i, 2i+1), i < 32, turn by the angle pos * theta_i with
  theta_i = base^(-2i/64) and base 10000:
      y[2i]   = x[2i] cos(a_i) - x[2i+1] sin(a_i)
      y[2i+1] = x[2i] sin(a_i) + x[2i+1] cos(a_i),    a_i = pos * theta_i.
  The query's RoPE part turns by the same position, the new token's own.
* "Absorbed MLA Cache Optimization", section 2.1 (store / get): a decode step
  stores the new token's latent and rotated k_pe, then attends over every
  stored token, the new one included. Position = index of the new token in
  its sequence = the sequence length before the append.
* The angles enter as tables (cos, sin; fp32; one row per position), as in
  serving code, so both sides turn by the same numbers. rope_tables builds
  them from the definition above in fp64 and rounds each entry to fp32.
* Rounding (reading): the new k_pe is turned in fp32, every product and every
  sum rounded to fp32 (no fused multiply-add), then rounded to bf16 (nearest
  even), the model's dtype, and appended exactly as an unrotated bf16 input
  would be (oracle.quant). The query is turned in fp64 from the same table.
* A full sequence (length = capacity) stores nothing, keeps its length, and
  its query still turns by the position it would have had (= capacity).
"""

import numpy as np

from oracle import attention as A
from oracle import quant as Q

ROPE_DIM = 64
ROPE_BASE = 10000.0


def rope_angles(max_pos, dim=ROPE_DIM, base=ROPE_BASE):
    """a[pos, i] = pos * base^(-2i/dim), float64, shape [max_pos, dim/2]."""
    i = np.arange(dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / dim)
    return np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]


def rope_tables(max_pos, dim=ROPE_DIM, base=ROPE_BASE):
    """(cos, sin) of rope_angles, each computed in fp64 and rounded to fp32."""
    a = rope_angles(max_pos, dim, base)
    return np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)


def rotate_f32(x, cos_row, sin_row):
    """Turn the pairs of x [..., 64] with one fp32 table row (cos, sin [32]).

    fp32 arithmetic, one rounding per product and per sum, in the order
    written in the module header."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos_row, dtype=np.float32)
    s = np.asarray(sin_row, dtype=np.float32)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = (x0 * c) - (x1 * s)
    y[..., 1::2] = (x0 * s) + (x1 * c)
    return y


def rotate_f64(x, cos_row, sin_row):
    """The same turn in float64 (the table values widened exactly)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos_row, dtype=np.float64)
    s = np.asarray(sin_row, dtype=np.float64)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def bf16_rne(x):
    """Round fp32 values to bf16, nearest even (finite inputs); returned as fp32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def decode_step(ckv_hat, kpe_hat, length, cap, ckv_new, kpe_new, q_nope, q_pe, w_uk, w_uv,
                softmax_scale, fmt, cos, sin):
    """One sequence's fused decode step.

    ckv_hat [L,512], kpe_hat [L,64]: its dequantized cached rows (L = length);
    ckv_new [512], kpe_new [64]: the new token (bf16 values, k_pe not yet
    turned); q_nope [H,128], q_pe [H,64] (q_pe not yet turned); cos, sin: fp32
    tables with at least cap + 1 rows, or None for no rotation.
    Returns (planes of the stored row or None if the sequence was full,
    new length, out [H,128] float64).
    """
    pos = int(length)
    kpe_in = np.asarray(kpe_new, dtype=np.float32)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    if cos is not None:
        kpe_in = bf16_rne(rotate_f32(kpe_in, cos[pos], sin[pos]))
        q_pe = rotate_f64(q_pe, cos[pos], sin[pos])
    planes = None
    ckv_all, kpe_all = np.asarray(ckv_hat, np.float64), np.asarray(kpe_hat, np.float64)
    if pos < cap:
        planes = Q.quantize_rows(np.asarray(ckv_new, np.float32)[None], kpe_in[None], fmt)
        c_hat, k_hat = Q.dequantize_rows(planes, fmt)
        ckv_all = np.concatenate([ckv_all, c_hat], axis=0)
        kpe_all = np.concatenate([kpe_all, k_hat], axis=0)
        planes = {k: v[0] for k, v in planes.items()}
    out = A.decode_absorbed(q_nope, q_pe, w_uk, w_uv, ckv_all, kpe_all, softmax_scale)
    return planes, min(pos + 1, cap), out
