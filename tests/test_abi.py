"""The C ABI without a GPU: the library loads, exports what include/mla_kv.h
declares, and rejects bad arguments on the host before launching anything.

Device pointers below are fake (never dereferenced): every call here returns
from host-side validation.
"""

import ctypes
import math
import os
import re

import pytest

from mla_latent_kv_cache_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def header_functions():
    src = open(os.path.join(ROOT, "include", "mla_kv.h")).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char \*)\s*\**\s*(mla_\w+)\s*\(", src, re.M)))


def cache_struct(fmt="int8", L=2, B=3, cap=100, **over):
    f = _lib.FORMATS[fmt]
    s = _lib.MlaCacheStruct(f, L, B, cap, 512, 64, 16, 8, FAKE, FAKE + 0x100000,
                            FAKE + 0x200000 if fmt != "bf16" else 0,
                            FAKE + 0x300000 if fmt.startswith("int4") else 0, FAKE + 0x400000)
    for k, v in over.items():
        setattr(s, k, v)
    return s


def test_library_loads_and_exports_every_declared_symbol():
    L = _lib.lib()
    declared = header_functions()
    assert set(declared) == set(_lib.SYMBOLS), declared
    for name in declared:
        assert hasattr(L, name)


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5):
        assert _lib.status_str(st) and _lib.status_str(st) != "unknown status"
    assert _lib.status_str(-99) == "unknown status"


def _ws(s, heads=16, splits=4):
    n = ctypes.c_size_t(0)
    st = _lib.lib().mla_decode_workspace_bytes(ctypes.byref(s), heads, splits, ctypes.byref(n))
    return st, n.value


def test_workspace_size_formula():
    s = cache_struct(B=3)
    st, n = _ws(s, 16, 4)
    assert st == 0

    def a256(v):
        return (v + 255) // 256 * 256
    B, H, ns = 3, 16, 4
    # absorbed queries: per (sequence, head) 576 channels as fp16 hi and lo, plus
    # 32 group sums as hi and lo
    qa = a256(B * H * (2 * 576 + 2 * 32) * 2)
    # the balanced plan's ns * B ranges, one record per (range, sequence) pair
    # a range covers, at most ns * B + B; then the per-sequence table (first
    # record, count) as int32 pairs
    recs = ns * B + B
    expect = qa + 2 * a256(recs * H * 4) + a256(recs * H * 512 * 4) + a256(B * 2 * 4)
    assert n == expect
    # any head count: the same records and table, rows for every head
    st, n = _ws(s, 32, 4)
    assert st == 0
    H = 32
    qa = a256(B * H * (2 * 576 + 2 * 32) * 2)
    assert n == qa + 2 * a256(recs * H * 4) + a256(recs * H * 512 * 4) + a256(B * 2 * 4)


@pytest.mark.parametrize("field,value,status", [
    ("format", 7, _lib.MLA_ERR_INVALID_ARG),
    ("num_layers", 0, _lib.MLA_ERR_INVALID_ARG),
    ("batch", 0, _lib.MLA_ERR_INVALID_ARG),
    ("capacity", 0, _lib.MLA_ERR_INVALID_ARG),
    ("kv_lora_rank", 256, _lib.MLA_ERR_UNSUPPORTED),
    ("rope_dim", 32, _lib.MLA_ERR_UNSUPPORTED),
    ("group_latent", 32, _lib.MLA_ERR_UNSUPPORTED),
    ("group_rope", 16, _lib.MLA_ERR_UNSUPPORTED),
    ("ckv", 0, _lib.MLA_ERR_INVALID_ARG),
    ("seq_lens", 0, _lib.MLA_ERR_INVALID_ARG),
    ("ckv", FAKE + 8, _lib.MLA_ERR_INVALID_ARG),  # not 16-byte aligned
    ("scale", 0, _lib.MLA_ERR_INVALID_ARG),       # quantized format needs scales
    ("zero", FAKE, _lib.MLA_ERR_INVALID_ARG),     # INT8 has no zero-points
])
def test_cache_descriptor_validation(field, value, status):
    s = cache_struct("int8", **{field: value})
    assert _ws(s)[0] == status


def test_format_plane_rules():
    assert _ws(cache_struct("bf16"))[0] == 0
    assert _ws(cache_struct("bf16", scale=FAKE))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int4"))[0] == 0
    assert _ws(cache_struct("int4", zero=0))[0] == _lib.MLA_ERR_INVALID_ARG
    # latent INT8 with bf16 k_pe: scales, no zero-points; INT4 with INT4 k_pe: both
    assert _ws(cache_struct("int8_kbf16"))[0] == 0
    assert _ws(cache_struct("int8_kbf16", scale=0))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int8_kbf16", zero=FAKE))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int4_kint4"))[0] == 0
    assert _ws(cache_struct("int4_kint4", zero=0))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int8", format=5))[0] == _lib.MLA_ERR_INVALID_ARG


def test_paging_rules():
    ok = dict(cap=256, page_size=64, num_pages=10, block_table=FAKE + 0x500000)
    assert _ws(cache_struct("int8", **ok))[0] == 0
    assert _ws(cache_struct("int8", **{**ok, "page_size": 48}))[0] == _lib.MLA_ERR_INVALID_ARG   # not a power of two
    assert _ws(cache_struct("int8", **{**ok, "page_size": 16}))[0] == _lib.MLA_ERR_INVALID_ARG   # under one tile
    assert _ws(cache_struct("int8", **{**ok, "cap": 200}))[0] == _lib.MLA_ERR_INVALID_ARG        # pages do not tile it
    assert _ws(cache_struct("int8", **{**ok, "num_pages": 0}))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int8", **{**ok, "block_table": 0}))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int8", **{**ok, "block_table": FAKE + 2}))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int8", page_size=0, block_table=FAKE))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _ws(cache_struct("int8", page_size=-64))[0] == _lib.MLA_ERR_INVALID_ARG


def test_null_cache_and_outputs():
    L = _lib.lib()
    n = ctypes.c_size_t(0)
    assert L.mla_decode_workspace_bytes(None, 16, 1, ctypes.byref(n)) == _lib.MLA_ERR_INVALID_ARG
    s = cache_struct()
    assert L.mla_decode_workspace_bytes(ctypes.byref(s), 16, 1, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(None, 0, FAKE, FAKE, 1, None, None) == _lib.MLA_ERR_INVALID_ARG


@pytest.mark.parametrize("heads", [0, 8, 17, 48, 96, 256])
def test_unsupported_head_counts(heads):
    assert _ws(cache_struct(), heads=heads)[0] == _lib.MLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("splits", [-1, 4097])
def test_split_count_range(splits):
    assert _ws(cache_struct(), splits=splits)[0] == _lib.MLA_ERR_INVALID_ARG


def _decode(s, layer=0, heads=16, scale=0.07, splits=4, ws=FAKE, ws_bytes=None, q=FAKE, out=FAKE):
    if ws_bytes is None:
        ws_bytes = _ws(s, heads, splits)[1]
    return _lib.lib().mla_decode_attn(ctypes.byref(s), layer, q, FAKE, FAKE, FAKE, heads, scale, splits,
                                      ws, ws_bytes, out, None)


def test_decode_argument_validation_before_launch():
    s = cache_struct()
    assert _decode(s, layer=2) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(s, layer=-1) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(s, heads=24) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(s, scale=math.nan) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(s, scale=math.inf) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(s, q=0) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(s, q=FAKE + 4) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(s, out=0) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(s, ws=0) == _lib.MLA_ERR_WORKSPACE
    assert _decode(s, ws=FAKE + 16) == _lib.MLA_ERR_WORKSPACE  # workspace must be 256-byte aligned
    need = _ws(s, 16, 4)[1]
    assert _decode(s, ws_bytes=need - 1) == _lib.MLA_ERR_WORKSPACE


def _step(s, layer=0, ckv=FAKE, kpe=FAKE, cos=FAKE + 0x500000, sin=FAKE + 0x600000, rows=101, heads=16,
          scale=0.1, splits=4, ws=FAKE + 0x700000, ws_bytes=None, out=FAKE + 0x800000):
    if ws_bytes is None:
        ws_bytes = _ws(s, heads, splits)[1]
    return _lib.lib().mla_decode_step(ctypes.byref(s), layer, ckv, kpe, FAKE, FAKE, cos, sin, rows, FAKE,
                                      FAKE, heads, scale, splits, ws, ws_bytes, out, None)


def test_step_argument_validation_before_launch():
    s = cache_struct(cap=100)
    assert _step(s, layer=2) == _lib.MLA_ERR_INVALID_ARG
    assert _step(s, ckv=0) == _lib.MLA_ERR_INVALID_ARG
    assert _step(s, kpe=FAKE + 8) == _lib.MLA_ERR_INVALID_ARG
    assert _step(s, cos=0) == _lib.MLA_ERR_INVALID_ARG          # one table without the other
    assert _step(s, sin=0) == _lib.MLA_ERR_INVALID_ARG
    assert _step(s, cos=FAKE + 2) == _lib.MLA_ERR_INVALID_ARG   # tables are fp32
    assert _step(s, rows=100) == _lib.MLA_ERR_INVALID_ARG       # rows must reach position = capacity
    assert _step(s, heads=24) == _lib.MLA_ERR_UNSUPPORTED
    assert _step(s, scale=math.nan) == _lib.MLA_ERR_INVALID_ARG
    assert _step(s, out=0) == _lib.MLA_ERR_INVALID_ARG
    assert _step(s, ws=0) == _lib.MLA_ERR_WORKSPACE
    assert _step(s, ws_bytes=_ws(s, 16, 4)[1] - 1) == _lib.MLA_ERR_WORKSPACE


def test_append_argument_validation_before_launch():
    L = _lib.lib()
    s = cache_struct()
    b = ctypes.byref(s)
    assert L.mla_cache_append(b, 5, FAKE, FAKE, 1, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(b, 0, FAKE, FAKE, -1, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(b, 0, 0, FAKE, 1, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(b, 0, FAKE, FAKE + 2, 1, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_cache_append(b, 0, FAKE, FAKE, 1, FAKE + 2, None) == _lib.MLA_ERR_INVALID_ARG
    # zero new tokens is a no-op that launches nothing
    assert L.mla_cache_append(b, 0, 0, 0, 0, None, None) == _lib.MLA_OK


def test_get_argument_validation_before_launch():
    L = _lib.lib()
    s = cache_struct()
    assert L.mla_cache_get(ctypes.byref(s), 2, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_cache_get(ctypes.byref(s), 0, None, None, None) == _lib.MLA_OK


def test_size_limits_before_launch():
    # one sequence's rows of any plane must stay below 2^30 bytes (the kernels
    # address them through 32-bit buffer descriptors)
    L = _lib.lib()
    ok = cache_struct("bf16", cap=(1 << 20))            # 1 Mi tokens x 1024 B
    assert _ws(ok, 16, 4)[0] == _lib.MLA_OK
    big = cache_struct("bf16", cap=(1 << 20) + 1)
    assert _ws(big, 16, 4)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert L.mla_cache_append(ctypes.byref(big), 0, FAKE, FAKE, 1, None, None) == _lib.MLA_ERR_UNSUPPORTED
    assert _ws(cache_struct("int4", cap=(1 << 22)), 16, 4)[0] == _lib.MLA_OK   # 256-byte latent rows
    assert _ws(cache_struct("int4", cap=(1 << 23) + 1), 16, 4)[0] == _lib.MLA_ERR_UNSUPPORTED
    # the partial grid (ranges x head slices) and the plan's tile count are
    # 32-bit: a batch whose tiles or workgroups pass 2^31 - 1 is refused
    huge = cache_struct("int8", B=1 << 20, cap=(1 << 20))
    assert _decode(huge) == _lib.MLA_ERR_UNSUPPORTED
    wide = cache_struct("int8", B=1 << 19, cap=64)
    assert _ws(wide, 128, 4096)[0] == _lib.MLA_OK  # the size alone is fine
    ws = _ws(wide, 128, 4096)[1]
    assert _decode(wide, heads=128, splits=4096, ws_bytes=ws) == _lib.MLA_ERR_UNSUPPORTED


def test_static_decode_validation_and_size_limit_before_any_device_call():
    # mla_decode_attn_static checks its arguments and the size of the
    # workspace it would need against its fixed array before it touches a
    # device (here there is none)
    L = _lib.lib()
    s = cache_struct("int8", B=4, cap=4096)
    big = _ws(s, 128, 2048)[1]
    assert big > _lib.STATIC_SCRATCH_BYTES
    call = lambda st, layer=0, heads=128, splits=2048, out=FAKE: L.mla_decode_attn_static(
        ctypes.byref(st), layer, FAKE, FAKE, FAKE, FAKE, heads, 0.07, splits, out, None)
    assert call(s) == _lib.MLA_ERR_WORKSPACE
    assert call(s, layer=2) == _lib.MLA_ERR_INVALID_ARG
    assert call(s, heads=24) == _lib.MLA_ERR_UNSUPPORTED
    assert call(s, splits=-1) == _lib.MLA_ERR_INVALID_ARG
    assert call(s, out=0) == _lib.MLA_ERR_INVALID_ARG


def test_rope_tables_argument_validation_before_launch():
    L = _lib.lib()
    assert L.mla_rope_tables(0, FAKE, 10, 10000.0, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_rope_tables(FAKE, FAKE + 2, 10, 10000.0, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_rope_tables(FAKE, FAKE, -1, 10000.0, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_rope_tables(FAKE, FAKE, 10, 0.0, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_rope_tables(FAKE, FAKE, 10, math.inf, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_rope_tables(FAKE, FAKE, 0, 10000.0, None) == _lib.MLA_OK  # nothing to launch


def test_measurement_aids_validate_before_launch():
    L = _lib.lib()
    assert L.mla_stream_read(0, 1 << 20, FAKE, 16, 1, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_stream_read(FAKE, 1000, FAKE, 16, 1, None) == _lib.MLA_ERR_INVALID_ARG  # not a multiple of 16
    assert L.mla_stream_read(FAKE, 1 << 20, FAKE, 0, 0, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_stream_read(FAKE, 0, FAKE, 16, 0, None) == _lib.MLA_OK  # nothing to read
    assert L.mla_mfma_rate(0, 16, 10, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_mfma_rate(FAKE + 2, 16, 10, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_mfma_rate(FAKE, 0, 10, None) == _lib.MLA_ERR_INVALID_ARG
    assert L.mla_mfma_rate(FAKE, 16, -1, None) == _lib.MLA_ERR_INVALID_ARG


def test_python_binding_has_no_fallback(monkeypatch, tmp_path):
    # With the library missing the binding raises instead of computing anything.
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()
