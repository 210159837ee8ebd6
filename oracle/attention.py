"""Oracle for one absorbed-MLA decode step (float64, numpy only).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline use this module; the HIP library never does.

Shapes (one sequence, one layer): H heads; latent d_c = 512; rope 64;
qk_nope 128; v 128; L cached tokens.

  q_nope [H,128], q_pe [H,64]        the new token's query, already rotated
  w_uk   [H,128,512]                 per-head key up-projection, K_nope = W_UK[h] c
  w_uv   [H,512,128]                 per-head value up-projection, V = c W_UV[h]
  ckv    [L,512], kpe [L,64]         dequantized cache rows
  softmax_scale                      multiplies q.k before the softmax

What the pages fix:
* "DeepSeek的MLA技术", MLA mechanism step 2: each head's key and value come
  from the cached latent, K_i = C W_i^upK and V_i = C W_i^upV; the
  MLAttentionWithCache code re-expands every cached token each step, then
  scores = Q_i K_i^T * scale, softmax over the cached tokens, output = p V_i.
  That is decode_expanded below (the naive path).
* "Absorbed MLA Cache Optimization", sections 1.1 and 2.1: the cache holds the
  512-d latent plus the 64-d k_pe (the decoupled RoPE key, shared by all heads)
  and projects at compute time. The key of head h is the concatenation
  [W_UK[h] c_t, k_pe_t] (the 192-d key of section 1.3).
* Absorption (the reading taken): by associativity, q_nope . (W_UK[h] c_t) =
  (q_nope W_UK[h]) . c_t and sum_t p_t (c_t W_UV[h]) = (sum_t p_t c_t) W_UV[h],
  so decode_absorbed computes the same number without expanding any token.
  The two are checked equal in the tests; that pins this reading.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def absorb_query(q_nope, w_uk):
    """q_abs[h, c] = sum_d q_nope[h, d] * W_UK[h, d, c]   ->  [H, 512]."""
    q_nope = _f64(q_nope)
    w_uk = _f64(w_uk)
    return np.einsum("hd,hdc->hc", q_nope, w_uk)


def softmax(scores):
    """Softmax over the last axis: exp(s - max) / sum exp(s - max)."""
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def decode_absorbed(q_nope, q_pe, w_uk, w_uv, ckv, kpe, softmax_scale):
    """Absorbed decode for one sequence: returns out [H, 128] (float64).

    1. q_abs = q_nope W_UK[h]                       (absorb through W_UK)
    2. s[h, t] = scale * (q_abs[h] . c_t + q_pe[h] . k_pe_t)
    3. p = softmax over t
    4. o_lat[h] = sum_t p[h, t] c_t                 (512-d, in latent space)
    5. out[h] = o_lat[h] W_UV[h]                    (project through W_UV)
    An empty sequence (L = 0) gives an all-zero output.
    """
    q_pe = _f64(q_pe)
    w_uv = _f64(w_uv)
    ckv = _f64(ckv)
    kpe = _f64(kpe)
    H = q_pe.shape[0]
    dv = w_uv.shape[-1]
    if ckv.shape[0] == 0:
        return np.zeros((H, dv))
    q_abs = absorb_query(q_nope, w_uk)
    scores = softmax_scale * (q_abs @ ckv.T + q_pe @ kpe.T)  # [H, L]
    p = softmax(scores)
    o_lat = p @ ckv  # [H, 512]
    return np.einsum("hc,hce->he", o_lat, w_uv)


def expand_kv(ckv, kpe, w_uk, w_uv):
    """Naive per-head expansion of every cached token.

    K[h, t] = [W_UK[h] c_t  ||  k_pe_t]   (128 + 64 = 192)
    V[h, t] = c_t W_UV[h]                 (128)
    """
    ckv = _f64(ckv)
    kpe = _f64(kpe)
    w_uk = _f64(w_uk)
    w_uv = _f64(w_uv)
    H = w_uk.shape[0]
    L = ckv.shape[0]
    k_nope = np.einsum("hdc,tc->htd", w_uk, ckv)  # [H, L, 128]
    k_rope = np.broadcast_to(kpe[None], (H, L, kpe.shape[-1]))
    K = np.concatenate([k_nope, k_rope], axis=-1)
    V = np.einsum("tc,hce->hte", ckv, w_uv)  # [H, L, 128]
    return K, V


def decode_expanded(q_nope, q_pe, w_uk, w_uv, ckv, kpe, softmax_scale):
    """Naive expanded decode for one sequence: out [H, 128] (float64).

    Per head: q = [q_nope || q_pe]; s = scale * q K^T; p = softmax(s); out = p V.
    """
    q = np.concatenate([_f64(q_nope), _f64(q_pe)], axis=-1)  # [H, 192]
    H = q.shape[0]
    dv = _f64(w_uv).shape[-1]
    if _f64(ckv).shape[0] == 0:
        return np.zeros((H, dv))
    K, V = expand_kv(ckv, kpe, w_uk, w_uv)
    out = np.empty((H, dv))
    for h in range(H):
        s = softmax_scale * (K[h] @ q[h])  # [L]
        p = softmax(s)
        out[h] = p @ V[h]
    return out


def decode_batch(q_nope, q_pe, w_uk, w_uv, ckv, kpe, lengths, softmax_scale,
                 fn=decode_absorbed):
    """Apply a per-sequence decode to a batch.

    q_nope [B,H,128], q_pe [B,H,64]; ckv [B,cap,512], kpe [B,cap,64] dequantized
    rows (only the first lengths[b] rows of sequence b are attended).
    Returns out [B, H, 128].
    """
    B = len(lengths)
    outs = []
    for b in range(B):
        n = int(lengths[b])
        outs.append(fn(q_nope[b], q_pe[b], w_uk, w_uv, ckv[b][:n], kpe[b][:n], softmax_scale))
    return np.stack(outs)
