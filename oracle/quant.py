"""Oracle quantizers for the latent KV cache (fp32-exact, numpy only).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline use this module; the HIP library never does.

What the pages fix, and the reading taken where they leave it open:

* "Absorbed MLA Cache Optimization on DeepSeek-V2-Lite", section 3.2 / 4.2
  quantization tables: the 512-d latent is quantized per channel block, 32
  blocks, INT8 ("per-channel INT8 (32 blocks)") or asymmetric INT4 ("非对称
  INT4 (32块)"); k_pe is quantized INT8 in 8 blocks. Reading: blocks are
  contiguous channel groups (16 latent channels, 8 k_pe channels), each with
  its own scale per token, since new tokens are quantized as they are stored
  (section 2.1, AbsorbedMLACache.store quantizes compressed_kv on store).
* "DeepSeek的MLA技术", optimization 3 (quantization): the symmetric INT8 step
  is scale = max|x| / 127 and codes = round(x / scale), dequant = codes*scale.
  Reading: the scale is stored as fp16 and the codes are computed by dividing
  by the STORED scale, so dequantization uses exactly the value quantization
  used; round() is round-half-to-even; codes are clamped to [-127, 127].
* INT4 k_pe ("Absorbed MLA Cache Optimization", section 3.2: the 7.6 KB per
  token of the INT4 configuration needs k_pe in 4 bits as well; symmetric, 8
  groups). Reading: the INT8 rule with 7 in place of 127: s = fp16(max|x| / 7),
  codes = clamp(rne(x / s), -7, 7), stored as the nibble code + 8 (1..15),
  the even channel in the low nibble; x_hat = code * s.
* latent INT8 with k_pe kept in bf16 (the report's configuration "B",
  section 3.2 table): latent as INT8 above, k_pe copied.
* Asymmetric INT4 (report section 3.2, "非对称"): reading: a float offset z
  (fp16, the group minimum rounded toward -inf) and an fp16 scale
  s = (max - z) / 15, each stored as +0 when zero; codes = clamp(rne((x - z) / s), 0, 15); x_hat = q*s + z.
  Two codes per byte, the even channel in the low nibble.

Arithmetic: inputs are bf16 values widened to fp32 (exact). Every step below is
one IEEE fp32 operation rounded to nearest even (numpy float32 semantics, no
fused multiply-add), the fp32->fp16 conversion is round-to-nearest-even, and a
scale or zero-point that would overflow fp16 saturates to +-65504. Inputs must
be finite. The dequantizers return float64, in which q*s and q*s+z are exact.
"""

import numpy as np

F32 = np.float32
F16_MAX = 65504.0

LATENT_DIM = 512
ROPE_DIM = 64
GROUP_LATENT = 16
GROUP_ROPE = 8
N_GROUPS_LATENT = LATENT_DIM // GROUP_LATENT  # 32
N_GROUPS_ROPE = ROPE_DIM // GROUP_ROPE  # 8

FORMATS = ("bf16", "int8", "int4", "int8_kbf16", "int4_kint4")


def _f32(x):
    x = np.asarray(x)
    if x.dtype != np.float32:
        x = x.astype(np.float32)
    return x


def fp16_rne(v):
    """fp32 -> fp16, round to nearest even, saturating at +-65504."""
    v = _f32(v)
    h = v.astype(np.float16)
    h = np.where(np.isinf(h), np.copysign(np.float16(F16_MAX), h), h)
    return h.astype(np.float16)


def fp16_round_down(v):
    """fp32 -> fp16, rounded toward -inf (largest fp16 <= v), saturating."""
    v = _f32(v)
    h = v.astype(np.float16)  # nearest even
    h = np.where(np.isposinf(h), np.float16(F16_MAX), h).astype(np.float16)
    too_big = h.astype(np.float32) > v
    h = np.where(too_big, np.nextafter(h, np.float16(-np.inf)), h).astype(np.float16)
    h = np.where(np.isneginf(h), np.float16(-F16_MAX), h).astype(np.float16)
    # a zero-point of zero is stored as +0 (the sign of a zero minimum is not
    # well defined when a group holds both +0 and -0)
    h = np.where(h == 0, np.float16(0.0), h).astype(np.float16)
    return h


def _groups(x, group):
    x = _f32(x)
    n = x.shape[-1]
    if n % group:
        raise ValueError(f"last dim {n} is not a multiple of group {group}")
    return x.reshape(x.shape[:-1] + (n // group, group))


def quantize_sym_int8(x, group, fp16_scale=True):
    """Symmetric INT8 per contiguous channel group.

    Per group: a = max|x|; s = fp16(a / 127); q = clamp(rne(x / s), -127, 127);
    a group whose stored scale is 0 gets all-zero codes.
    Returns (codes int8 [..., n], scales [..., n/group]) where scales are fp16,
    or fp32 when fp16_scale is False (the unrounded scale of the tutorial's
    per-tensor snippet, used to check that this reduces to it).
    """
    xg = _groups(x, group)
    a = np.max(np.abs(xg), axis=-1)
    s32 = a / F32(127.0)
    s = fp16_rne(s32) if fp16_scale else s32
    sf = s.astype(np.float32)[..., None]
    nonzero = sf != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(nonzero, xg / np.where(nonzero, sf, F32(1.0)), F32(0.0))
    q = np.clip(np.rint(r), -127, 127)
    q = np.where(nonzero, q, 0).astype(np.int8)
    return q.reshape(_f32(x).shape), s


def dequantize_sym_int8(codes, scales, group):
    """x_hat = q * s in float64 (exact)."""
    q = np.asarray(codes).astype(np.float64)
    qg = q.reshape(q.shape[:-1] + (q.shape[-1] // group, group))
    return (qg * np.asarray(scales).astype(np.float64)[..., None]).reshape(q.shape)


def quantize_sym_int4(x, group):
    """Symmetric INT4 per contiguous channel group (the k_pe of int4_kint4).

    Per group: a = max|x|; s = fp16(a / 7); q = clamp(rne(x / s), -7, 7); a
    group whose stored scale is 0 gets all-zero codes.
    Returns (codes int8 in -7..7 [..., n], scales fp16 [..., n/group]).
    """
    xg = _groups(x, group)
    a = np.max(np.abs(xg), axis=-1)
    s = fp16_rne(a / F32(7.0))
    sf = s.astype(np.float32)[..., None]
    nonzero = sf != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(nonzero, xg / np.where(nonzero, sf, F32(1.0)), F32(0.0))
    q = np.clip(np.rint(r), -7, 7)
    q = np.where(nonzero, q, 0).astype(np.int8)
    return q.reshape(_f32(x).shape), s


def pack_sym_int4(codes):
    """Codes -7..7 as nibbles code + 8, two per byte, the even channel low."""
    return pack_nibbles((np.asarray(codes).astype(np.int16) + 8).astype(np.uint8))


def unpack_sym_int4(packed):
    return unpack_nibbles(packed).astype(np.int8) - 8


def quantize_asym_int4(x, group):
    """Asymmetric INT4 per contiguous channel group, codes not yet packed.

    Per group: z = fp16 round-down of min x; s = fp16((max x - z) / 15);
    q = clamp(rne((x - z) / s), 0, 15); a group whose stored scale is 0 gets
    all-zero codes (it dequantizes to z).
    Returns (codes uint8 in 0..15 [..., n], scales fp16, zeros fp16 [..., n/group]).
    """
    xg = _groups(x, group)
    mn = np.min(xg, axis=-1)
    mx = np.max(xg, axis=-1)
    z = fp16_round_down(mn)
    zf = z.astype(np.float32)
    s = fp16_rne((mx - zf) / F32(15.0))
    # a zero scale is stored as +0: for a group of zeros of both signs, the
    # sign of max - z would depend on which zero min and max happen to pick
    s = np.where(s == 0, np.float16(0.0), s).astype(np.float16)
    sf = s.astype(np.float32)[..., None]
    nonzero = sf != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(nonzero, (xg - zf[..., None]) / np.where(nonzero, sf, F32(1.0)), F32(0.0))
    q = np.clip(np.rint(r), 0, 15)
    q = np.where(nonzero, q, 0).astype(np.uint8)
    return q.reshape(_f32(x).shape), s, z


def pack_nibbles(codes):
    """Two 4-bit codes per byte: byte k = q[2k] | q[2k+1] << 4."""
    q = np.asarray(codes).astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequantize_asym_int4(codes, scales, zeros, group):
    """x_hat = q * s + z in float64 (exact); codes unpacked (0..15)."""
    q = np.asarray(codes).astype(np.float64)
    qg = q.reshape(q.shape[:-1] + (q.shape[-1] // group, group))
    s = np.asarray(scales).astype(np.float64)[..., None]
    z = np.asarray(zeros).astype(np.float64)[..., None]
    return (qg * s + z).reshape(q.shape)


def quantize_rows(ckv, kpe, fmt):
    """Quantize cache rows exactly as they are laid out in the cache planes.

    ckv: [..., 512] and kpe: [..., 64] bf16 values (given as fp32 or bf16-exact).
    Returns a dict with the planes of one cache row:
      bf16: ckv, kpe unchanged (as float32; the planes hold the same bf16 bits)
      int8: ckv int8 [...,512], kpe int8 [...,64], scale fp16 [...,40]
      int4: ckv uint8 [...,256] packed, kpe int8 [...,64], scale fp16 [...,40],
            zero fp16 [...,32]
    The scale row holds the 32 latent-group scales, then the 8 k_pe-group scales.
    """
    ckv = _f32(ckv)
    kpe = _f32(kpe)
    if fmt == "bf16":
        return {"ckv": ckv, "kpe": kpe}
    if fmt == "int8_kbf16":
        cq, cs = quantize_sym_int8(ckv, GROUP_LATENT)
        return {"ckv": cq, "kpe": kpe, "scale": cs}
    if fmt == "int4_kint4":
        cq, cs, cz = quantize_asym_int4(ckv, GROUP_LATENT)
        kq, ks = quantize_sym_int4(kpe, GROUP_ROPE)
        return {"ckv": pack_nibbles(cq), "kpe": pack_sym_int4(kq),
                "scale": np.concatenate([cs, ks], axis=-1), "zero": cz}
    kq, ks = quantize_sym_int8(kpe, GROUP_ROPE)
    if fmt == "int8":
        cq, cs = quantize_sym_int8(ckv, GROUP_LATENT)
        return {"ckv": cq, "kpe": kq, "scale": np.concatenate([cs, ks], axis=-1)}
    if fmt == "int4":
        cq, cs, cz = quantize_asym_int4(ckv, GROUP_LATENT)
        return {"ckv": pack_nibbles(cq), "kpe": kq,
                "scale": np.concatenate([cs, ks], axis=-1), "zero": cz}
    raise ValueError(f"unknown format {fmt!r}")


def dequantize_rows(planes, fmt):
    """Inverse of quantize_rows, in float64: returns (ckv_hat [...,512], kpe_hat [...,64])."""
    if fmt == "bf16":
        return (np.asarray(planes["ckv"]).astype(np.float64),
                np.asarray(planes["kpe"]).astype(np.float64))
    scale = np.asarray(planes["scale"])
    s_lat = scale[..., :N_GROUPS_LATENT]
    s_rope = scale[..., N_GROUPS_LATENT:]
    if fmt == "int8_kbf16":
        return (dequantize_sym_int8(planes["ckv"], s_lat, GROUP_LATENT),
                np.asarray(planes["kpe"]).astype(np.float64))
    if fmt == "int4_kint4":
        kpe_hat = dequantize_sym_int8(unpack_sym_int4(planes["kpe"]), s_rope, GROUP_ROPE)
        codes = unpack_nibbles(planes["ckv"])
        return dequantize_asym_int4(codes, s_lat, planes["zero"], GROUP_LATENT), kpe_hat
    kpe_hat = dequantize_sym_int8(planes["kpe"], s_rope, GROUP_ROPE)
    if fmt == "int8":
        return dequantize_sym_int8(planes["ckv"], s_lat, GROUP_LATENT), kpe_hat
    if fmt == "int4":
        codes = unpack_nibbles(planes["ckv"])
        return dequantize_asym_int4(codes, s_lat, planes["zero"], GROUP_LATENT), kpe_hat
    raise ValueError(f"unknown format {fmt!r}")
