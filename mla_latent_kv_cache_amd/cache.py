"""Python face of the library: a latent KV cache held in torch device tensors.

torch provides device memory and the current stream; every computation is a
call into libmla_kv.so (see include/mla_kv.h for the operations and the
passages of the pages they follow).
"""

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import FORMATS, MlaCacheStruct, MlaError, check

LATENT = 512
ROPE = 64
NOPE = 128
VDIM = 128
N_SCALES = 40
N_ZEROS = 32


def row_bytes(fmt):
    """Bytes one token occupies in one layer of a cache of this format: the
    planes' row sizes of include/mla_kv.h added up (1152, 656, 464, 704, 432)."""
    lat = {"bf16": LATENT * 2, "int8": LATENT, "int4": LATENT // 2, "int8_kbf16": LATENT, "int4_kint4": LATENT // 2}
    kpe = {"bf16": ROPE * 2, "int8": ROPE, "int4": ROPE, "int8_kbf16": ROPE * 2, "int4_kint4": ROPE // 2}
    scales = {"bf16": 0, "int8_kbf16": N_ZEROS}.get(fmt, N_SCALES)
    zeros = N_ZEROS if fmt in ("int4", "int4_kint4") else 0
    return lat[fmt] + kpe[fmt] + 2 * (scales + zeros)


def rope_tables(rows, base=10000.0, device="cuda", stream=None):
    """RoPE angle tables for decode_step, made by the library's
    mla_rope_tables: (cos, sin), fp32 [rows, 32] on the device, row p holding
    cos / sin of p * base^(-2i/64) for channel pair (2i, 2i+1)."""
    device = torch.device(device)
    cos = torch.empty((int(rows), ROPE // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    check(_lib.lib().mla_rope_tables(_ptr(cos), _ptr(sin), int(rows), float(base), _stream(stream)),
          "mla_rope_tables")
    return cos, sin


def _unblock(t):
    """Latent rows in logical order from the block layout: t [..., R, row]
    (R a multiple of 16) holds, in each 16 rows, chunk c of row i at byte
    (16 c + i) * 16 of the block."""
    shape = t.shape
    row_bytes = shape[-1] * t.element_size()
    u = t.contiguous().view(torch.uint8).reshape(tuple(shape[:-2]) + (shape[-2] // 16, row_bytes // 16, 16, 16))
    u = u.transpose(-3, -2).contiguous()  # [.., blocks, row i, chunk c, 16 B]
    return u.reshape(tuple(shape[:-2]) + (shape[-2], row_bytes)).view(t.dtype).reshape(shape)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


class LatentCache:
    """Per-layer latent cache planes for `batch` sequences of up to `capacity` tokens.

    Layout (see include/mla_kv.h): kpe, scale, zero are [num_layers, batch,
    capacity, row] tensors; ckv is [num_layers, batch, capacity rounded up to
    16, row] with each 16 rows stored as blocks of 16-byte chunks (chunk c of
    row i at byte (16 c + i) * 16 of the block; `planes` undoes this);
    seq_lens is int32 [num_layers, batch].
    A host mirror of the lengths guards capacity before each append.
    """

    def __init__(self, fmt, num_layers, batch, capacity, device="cuda", page_size=0, num_pages=None,
                 block_table=None):
        """page_size > 0 makes the planes pools of num_pages pages of page_size
        tokens per layer; block_table (int32 [batch, capacity // page_size],
        host or device) maps each sequence's token blocks to pages (default:
        sequence b's blocks are pages b * blocks .. in order)."""
        if fmt not in FORMATS:
            raise ValueError(f"format must be one of {list(FORMATS)}")
        self.fmt = fmt
        self.num_layers, self.batch, self.capacity = int(num_layers), int(batch), int(capacity)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.page_size = int(page_size)
        self.block_table = None
        if self.page_size:
            blocks = self.capacity // self.page_size
            self.num_pages = int(num_pages) if num_pages is not None else self.batch * blocks
            if block_table is None:
                block_table = torch.arange(self.batch * blocks, dtype=torch.int32).reshape(self.batch, blocks)
            self.block_table = torch.as_tensor(block_table, dtype=torch.int32).to(self.device).contiguous()
            _need(self.block_table, "block_table", torch.int32, (self.batch, blocks), self.device)
            shape = (self.num_layers, self.num_pages, self.page_size)
        else:
            self.num_pages = 0
            shape = (self.num_layers, self.batch, self.capacity)
        # latent rows in whole 16-row blocks per sequence (pages hold whole blocks)
        lshape = shape if self.page_size else (self.num_layers, self.batch, (self.capacity + 15) // 16 * 16)
        kw = dict(device=self.device)
        lat = {"bf16": "bf16", "int8": "int8", "int4": "int4", "int8_kbf16": "int8", "int4_kint4": "int4"}[fmt]
        kp = {"bf16": "bf16", "int8_kbf16": "bf16", "int4_kint4": "int4"}.get(fmt, "int8")
        if lat == "bf16":
            self.ckv = torch.empty(lshape + (LATENT,), dtype=torch.bfloat16, **kw)
        elif lat == "int8":
            self.ckv = torch.empty(lshape + (LATENT,), dtype=torch.int8, **kw)
        else:
            self.ckv = torch.empty(lshape + (LATENT // 2,), dtype=torch.uint8, **kw)
        if kp == "bf16":
            self.kpe = torch.empty(shape + (ROPE,), dtype=torch.bfloat16, **kw)
        elif kp == "int8":
            self.kpe = torch.empty(shape + (ROPE,), dtype=torch.int8, **kw)
        else:
            self.kpe = torch.empty(shape + (ROPE // 2,), dtype=torch.uint8, **kw)
        n_scales = {"bf16": 0, "int8_kbf16": N_ZEROS}.get(fmt, N_SCALES)  # 0, 32 or 40 per row
        self.scale = torch.empty(shape + (n_scales,), dtype=torch.float16, **kw) if n_scales else None
        self.zero = torch.empty(shape + (N_ZEROS,), dtype=torch.float16, **kw) if lat == "int4" else None
        self.seq_lens = torch.zeros((self.num_layers, self.batch), dtype=torch.int32, **kw)
        self._lens = np.zeros((self.num_layers, self.batch), dtype=np.int64)
        self.struct = MlaCacheStruct(
            FORMATS[fmt], self.num_layers, self.batch, self.capacity, LATENT, ROPE, 16, 8,
            self.ckv.data_ptr(), self.kpe.data_ptr(),
            self.scale.data_ptr() if self.scale is not None else 0,
            self.zero.data_ptr() if self.zero is not None else 0,
            self.seq_lens.data_ptr(), self.page_size, self.num_pages,
            self.block_table.data_ptr() if self.block_table is not None else 0)

    # ------------------------------------------------------------ queries
    def lengths(self, layer=None):
        """Host mirror of seq_lens (the device copy is the one the kernels use)."""
        return self._lens.copy() if layer is None else self._lens[layer].copy()

    def bytes(self):
        """Device bytes of all cache planes."""
        return sum(t.numel() * t.element_size() for t in (self.ckv, self.kpe, self.scale, self.zero)
                   if t is not None)

    def _layer(self, layer):
        if not 0 <= layer < self.num_layers:
            raise IndexError(f"layer {layer} out of range [0, {self.num_layers})")

    # ------------------------------------------------------------- append
    def append(self, layer, ckv_new, kpe_new, n_new=None, stream=None):
        """Quantize and store new tokens: ckv_new bf16 [B,T,512], kpe_new bf16 [B,T,64].

        n_new: optional per-sequence counts (host sequence of ints, <= T).
        """
        self._layer(layer)
        T = ckv_new.shape[1] if ckv_new.dim() == 3 else -1
        _need(ckv_new, "ckv_new", torch.bfloat16, (self.batch, T, LATENT), self.device)
        _need(kpe_new, "kpe_new", torch.bfloat16, (self.batch, T, ROPE), self.device)
        if n_new is None:
            counts = np.full(self.batch, T, dtype=np.int64)
            n_dev = None
        else:
            counts = np.asarray(n_new, dtype=np.int64).reshape(-1)
            if counts.shape != (self.batch,) or (counts < 0).any() or (counts > T).any():
                raise ValueError("n_new must hold batch counts in [0, T]")
            n_dev = torch.tensor(counts, dtype=torch.int32, device=self.device)
        if (self._lens[layer] + counts > self.capacity).any():
            raise MlaError(_lib.MLA_ERR_CAPACITY, "append")
        check(_lib.lib().mla_cache_append(ctypes.byref(self.struct), layer, _ptr(ckv_new), _ptr(kpe_new),
                                          T, _ptr(n_dev), _stream(stream)), "mla_cache_append")
        self._lens[layer] += counts
        self._keep = n_dev  # keep the count tensor alive until the stream has used it

    # ------------------------------------------------------------- decode
    def auto_splits(self, heads):
        n = ctypes.c_int32(0)
        check(_lib.lib().mla_decode_auto_splits(ctypes.byref(self.struct), heads, ctypes.byref(n)),
              "mla_decode_auto_splits")
        return n.value

    def workspace_bytes(self, heads, num_splits=0):
        n = ctypes.c_size_t(0)
        check(_lib.lib().mla_decode_workspace_bytes(ctypes.byref(self.struct), heads, num_splits,
                                                    ctypes.byref(n)), "mla_decode_workspace_bytes")
        return n.value

    def workspace(self, heads, num_splits=0):
        """A device workspace tensor large enough for decode(heads, num_splits)."""
        return torch.empty(self.workspace_bytes(heads, num_splits), dtype=torch.uint8, device=self.device)

    def decode(self, layer, q_nope, q_pe, w_uk, w_uv, softmax_scale, num_splits=0, out=None,
               workspace=None, stream=None):
        """Absorbed decode attention of one layer: returns out fp32 [B, H, 128]."""
        self._layer(layer)
        H = q_nope.shape[1] if q_nope.dim() == 3 else -1
        _need(q_nope, "q_nope", torch.bfloat16, (self.batch, H, NOPE), self.device)
        _need(q_pe, "q_pe", torch.bfloat16, (self.batch, H, ROPE), self.device)
        _need(w_uk, "w_uk", torch.bfloat16, (H, NOPE, LATENT), self.device)
        _need(w_uv, "w_uv", torch.bfloat16, (H, LATENT, VDIM), self.device)
        if out is None:
            out = torch.empty((self.batch, H, VDIM), dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, (self.batch, H, VDIM), self.device)
        if workspace is None:
            workspace = self.workspace(H, num_splits)
        check(_lib.lib().mla_decode_attn(ctypes.byref(self.struct), layer, _ptr(q_nope), _ptr(q_pe),
                                         _ptr(w_uk), _ptr(w_uv), H, float(softmax_scale), num_splits,
                                         _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)),
              "mla_decode_attn")
        return out

    def _step_args(self, layer, ckv_new, kpe_new, q_nope, q_pe, w_uk, rope):
        self._layer(layer)
        H = q_nope.shape[1] if q_nope.dim() == 3 else -1
        _need(ckv_new, "ckv_new", torch.bfloat16, (self.batch, LATENT), self.device)
        _need(kpe_new, "kpe_new", torch.bfloat16, (self.batch, ROPE), self.device)
        _need(q_nope, "q_nope", torch.bfloat16, (self.batch, H, NOPE), self.device)
        _need(q_pe, "q_pe", torch.bfloat16, (self.batch, H, ROPE), self.device)
        _need(w_uk, "w_uk", torch.bfloat16, (H, NOPE, LATENT), self.device)
        cos = sin = None
        rows = 0
        if rope is not None:
            cos, sin = rope
            rows = cos.shape[0] if cos.dim() == 2 else -1
            _need(cos, "rope cos", torch.float32, (rows, ROPE // 2), self.device)
            _need(sin, "rope sin", torch.float32, (rows, ROPE // 2), self.device)
        return H, cos, sin, rows

    def decode_step_begin(self, layer, ckv_new, kpe_new, q_nope, q_pe, w_uk, softmax_scale, workspace,
                          rope=None, num_splits=0, stream=None):
        """Phase 1 of decode_step: store the new tokens and absorb the turned
        queries into the workspace; decode_partial and decode_combine follow."""
        H, cos, sin, rows = self._step_args(layer, ckv_new, kpe_new, q_nope, q_pe, w_uk, rope)
        check(_lib.lib().mla_decode_step_begin(ctypes.byref(self.struct), layer, _ptr(ckv_new), _ptr(kpe_new),
                                               _ptr(q_nope), _ptr(q_pe), _ptr(cos), _ptr(sin), rows, _ptr(w_uk),
                                               H, float(softmax_scale), num_splits, _ptr(workspace),
                                               workspace.numel(), _stream(stream)), "mla_decode_step_begin")
        self._lens[layer] = np.minimum(self._lens[layer] + 1, self.capacity)

    def decode_step(self, layer, ckv_new, kpe_new, q_nope, q_pe, w_uk, w_uv, softmax_scale, rope=None,
                    num_splits=0, out=None, workspace=None, stream=None):
        """Fused decode step of one layer: store one new token per sequence (its
        k_pe turned by RoPE at its position), then attend over every stored
        token. ckv_new bf16 [B,512], kpe_new bf16 [B,64] (not turned); q_pe not
        turned; rope: (cos, sin) fp32 [rows >= capacity + 1, 32] device tensors
        (see rope_tables), or None for no turn. Returns out fp32 [B, H, 128].
        A full sequence stores nothing and keeps its length."""
        H, cos, sin, rows = self._step_args(layer, ckv_new, kpe_new, q_nope, q_pe, w_uk, rope)
        _need(w_uv, "w_uv", torch.bfloat16, (H, LATENT, VDIM), self.device)
        if out is None:
            out = torch.empty((self.batch, H, VDIM), dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, (self.batch, H, VDIM), self.device)
        if workspace is None:
            workspace = self.workspace(H, num_splits)
        check(_lib.lib().mla_decode_step(ctypes.byref(self.struct), layer, _ptr(ckv_new), _ptr(kpe_new),
                                         _ptr(q_nope), _ptr(q_pe), _ptr(cos), _ptr(sin), rows, _ptr(w_uk),
                                         _ptr(w_uv), H, float(softmax_scale), num_splits, _ptr(workspace),
                                         workspace.numel(), _ptr(out), _stream(stream)), "mla_decode_step")
        self._lens[layer] = np.minimum(self._lens[layer] + 1, self.capacity)
        return out

    # ------------------------------------------------- several layers at once
    def auto_splits_layers(self, layer_count, heads):
        n = ctypes.c_int32(0)
        check(_lib.lib().mla_decode_auto_splits_layers(ctypes.byref(self.struct), layer_count, heads,
                                                       ctypes.byref(n)), "mla_decode_auto_splits_layers")
        return n.value

    def workspace_bytes_layers(self, layer_count, heads, num_splits=0):
        n = ctypes.c_size_t(0)
        check(_lib.lib().mla_decode_workspace_bytes_layers(ctypes.byref(self.struct), layer_count, heads,
                                                           num_splits, ctypes.byref(n)),
              "mla_decode_workspace_bytes_layers")
        return n.value

    def workspace_layers(self, layer_count, heads, num_splits=0):
        return torch.empty(self.workspace_bytes_layers(layer_count, heads, num_splits), dtype=torch.uint8,
                           device=self.device)

    def _layers_args(self, layer0, q_nope, q_pe, w_uk, w_uv):
        n = q_nope.shape[0] if q_nope.dim() == 4 else -1
        if not (0 <= layer0 and n >= 1 and layer0 + n <= self.num_layers):
            raise IndexError(f"layers [{layer0}, {layer0 + n}) out of range [0, {self.num_layers})")
        H = q_nope.shape[2]
        _need(q_nope, "q_nope", torch.bfloat16, (n, self.batch, H, NOPE), self.device)
        _need(q_pe, "q_pe", torch.bfloat16, (n, self.batch, H, ROPE), self.device)
        _need(w_uk, "w_uk", torch.bfloat16, (n, H, NOPE, LATENT), self.device)
        _need(w_uv, "w_uv", torch.bfloat16, (n, H, LATENT, VDIM), self.device)
        return n, H

    def decode_layers(self, layer0, q_nope, q_pe, w_uk, w_uv, softmax_scale, num_splits=0, out=None,
                      workspace=None, stream=None):
        """Absorbed decode of layers layer0 .. layer0 + n - 1 in one set of
        launches; every argument is stacked over the n layers (q_nope
        [n,B,H,128], q_pe [n,B,H,64], w_uk [n,H,128,512], w_uv [n,H,512,128]).
        Returns out fp32 [n, B, H, 128]."""
        n, H = self._layers_args(layer0, q_nope, q_pe, w_uk, w_uv)
        if out is None:
            out = torch.empty((n, self.batch, H, VDIM), dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, (n, self.batch, H, VDIM), self.device)
        if workspace is None:
            workspace = self.workspace_layers(n, H, num_splits)
        check(_lib.lib().mla_decode_attn_layers(ctypes.byref(self.struct), layer0, n, _ptr(q_nope), _ptr(q_pe),
                                                _ptr(w_uk), _ptr(w_uv), H, float(softmax_scale), num_splits,
                                                _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)),
              "mla_decode_attn_layers")
        return out

    def decode_step_layers(self, layer0, ckv_new, kpe_new, q_nope, q_pe, w_uk, w_uv, softmax_scale, rope=None,
                           num_splits=0, out=None, workspace=None, stream=None):
        """The fused decode step of layers layer0 .. layer0 + n - 1 in one set
        of launches: ckv_new bf16 [n,B,512], kpe_new bf16 [n,B,64] (not
        turned), the other arguments stacked as for decode_layers. Returns out
        fp32 [n, B, H, 128]."""
        n, H = self._layers_args(layer0, q_nope, q_pe, w_uk, w_uv)
        _need(ckv_new, "ckv_new", torch.bfloat16, (n, self.batch, LATENT), self.device)
        _need(kpe_new, "kpe_new", torch.bfloat16, (n, self.batch, ROPE), self.device)
        cos = sin = None
        rows = 0
        if rope is not None:
            cos, sin = rope
            rows = cos.shape[0] if cos.dim() == 2 else -1
            _need(cos, "rope cos", torch.float32, (rows, ROPE // 2), self.device)
            _need(sin, "rope sin", torch.float32, (rows, ROPE // 2), self.device)
        if out is None:
            out = torch.empty((n, self.batch, H, VDIM), dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, (n, self.batch, H, VDIM), self.device)
        if workspace is None:
            workspace = self.workspace_layers(n, H, num_splits)
        check(_lib.lib().mla_decode_step_layers(ctypes.byref(self.struct), layer0, n, _ptr(ckv_new), _ptr(kpe_new),
                                                _ptr(q_nope), _ptr(q_pe), _ptr(cos), _ptr(sin), rows, _ptr(w_uk),
                                                _ptr(w_uv), H, float(softmax_scale), num_splits, _ptr(workspace),
                                                workspace.numel(), _ptr(out), _stream(stream)),
              "mla_decode_step_layers")
        self._lens[layer0:layer0 + n] = np.minimum(self._lens[layer0:layer0 + n] + 1, self.capacity)
        return out

    # ------------------------------------------------ decode, phase by phase
    def decode_absorb(self, q_nope, q_pe, w_uk, softmax_scale, workspace, num_splits=0, stream=None):
        """Phase 1 of decode: absorbed, scaled queries into the workspace."""
        H = q_nope.shape[1] if q_nope.dim() == 3 else -1
        _need(q_nope, "q_nope", torch.bfloat16, (self.batch, H, NOPE), self.device)
        _need(q_pe, "q_pe", torch.bfloat16, (self.batch, H, ROPE), self.device)
        _need(w_uk, "w_uk", torch.bfloat16, (H, NOPE, LATENT), self.device)
        check(_lib.lib().mla_decode_absorb(ctypes.byref(self.struct), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), H,
                                           float(softmax_scale), num_splits, _ptr(workspace),
                                           workspace.numel(), _stream(stream)), "mla_decode_absorb")

    def decode_partial(self, layer, heads, workspace, num_splits=0, stream=None):
        """Phase 2 of decode: split-KV attention of every (sequence, split)."""
        self._layer(layer)
        check(_lib.lib().mla_decode_partial(ctypes.byref(self.struct), layer, heads, num_splits,
                                            _ptr(workspace), workspace.numel(), _stream(stream)),
              "mla_decode_partial")

    def decode_combine(self, w_uv, workspace, num_splits=0, out=None, stream=None):
        """Phase 3 of decode: merge the splits and project through W_UV."""
        H = w_uv.shape[0]
        _need(w_uv, "w_uv", torch.bfloat16, (H, LATENT, VDIM), self.device)
        if out is None:
            out = torch.empty((self.batch, H, VDIM), dtype=torch.float32, device=self.device)
        _need(out, "out", torch.float32, (self.batch, H, VDIM), self.device)
        check(_lib.lib().mla_decode_combine(ctypes.byref(self.struct), _ptr(w_uv), H, num_splits,
                                            _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)),
              "mla_decode_combine")
        return out

    # ---------------------------------------------------------------- get
    def get(self, layer, stream=None):
        """Dequantized copy of one layer: (ckv fp32 [B,cap,512], kpe fp32 [B,cap,64])."""
        self._layer(layer)
        ckv = torch.empty((self.batch, self.capacity, LATENT), dtype=torch.float32, device=self.device)
        kpe = torch.empty((self.batch, self.capacity, ROPE), dtype=torch.float32, device=self.device)
        check(_lib.lib().mla_cache_get(ctypes.byref(self.struct), layer, _ptr(ckv), _ptr(kpe),
                                       _stream(stream)), "mla_cache_get")
        return ckv, kpe

    def planes(self, layer, b):
        """The raw cache planes of one sequence (first seq_len rows, gathered
        through the block table when paged), as host tensors."""
        n = int(self._lens[layer, b])
        planes = {"ckv": self.ckv, "kpe": self.kpe, "scale": self.scale, "zero": self.zero}
        out = {}
        for key, t in planes.items():
            if t is None:
                continue
            if self.page_size:
                used = self.block_table[b].long()[: (n + self.page_size - 1) // self.page_size]
                rows = t[layer, used]  # [pages, page_size, row]
                if key == "ckv":
                    rows = _unblock(rows)
                out[key] = rows.reshape((-1,) + tuple(t.shape[3:]))[:n].cpu()
            else:
                rows = t[layer, b]
                out[key] = (_unblock(rows[None])[0] if key == "ckv" else rows)[:n].cpu()
        return out
