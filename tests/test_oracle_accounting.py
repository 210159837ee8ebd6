"""Pins for oracle.accounting: the byte and capacity numbers the pages print."""

import pytest

from oracle import accounting as acc

GIB10 = 10 * acc.GIB


def test_expanded_cache_bytes(golden):
    g = golden("kv_bytes.json")
    assert acc.expanded_bytes_per_layer() == g["expanded_bytes_per_layer"]["value"]
    per_tok = acc.per_token_bytes(acc.expanded_bytes_per_layer())
    assert per_tok == g["expanded_bytes_per_token"]["value"]
    assert round(acc.kib(per_tok), 1) == g["expanded_bytes_per_token"]["kib"]


def test_theoretical_line_as_printed(golden):
    g = golden("kv_bytes.json")["theoretical_elements_per_token"]
    n = (512 + 64 + 128) * acc.N_LAYERS
    assert n == g["value"]
    assert round(acc.kib(n), 1) == g["kib"]
    assert round(acc.compression_ratio(n), 1) == g["ratio"]


@pytest.mark.parametrize("idx", range(5))
def test_format_sizes_ratios_capacity(golden, idx):
    f = golden("kv_bytes.json")["formats"][idx]
    lat_bits, rope_bits = acc.PAYLOAD_FORMATS[f["name"]]
    assert (lat_bits, rope_bits) == (f["latent_bits"], f["rope_bits"])
    per_layer = acc.payload_bytes_per_layer(lat_bits, rope_bits)
    assert per_layer == f["bytes_per_layer"]
    per_tok = acc.per_token_bytes(per_layer)
    assert round(acc.kib(per_tok), 1) == f["kib"]
    assert round(acc.compression_ratio(per_tok), 1) == f["ratio"]
    n = acc.tokens_in(GIB10, per_tok)
    assert abs(n - f["tokens_in_10gb"]) <= f["tokens_rel_tol"] * f["tokens_in_10gb"]


def test_expanded_capacity(golden):
    g = golden("kv_bytes.json")["expanded_tokens_in_10gb"]
    n = acc.tokens_in(GIB10, acc.per_token_bytes(acc.expanded_bytes_per_layer()))
    assert abs(n - g["value"]) <= g["rel_tol"] * g["value"]


def test_mixed_format_capacity_from_its_size(golden):
    g = golden("kv_bytes.json")["mixed_18_2kb_tokens_in_10gb"]
    per_tok = g["kib"] * acc.KIB
    assert round(acc.compression_ratio(per_tok), 1) == g["ratio"]
    n = GIB10 // per_tok
    assert abs(n - g["value"]) <= g["rel_tol"] * g["value"]


def test_unit_reading_is_binary():
    # 690K only comes out with KiB/GiB: the decimal reading gives 643K.
    per_tok = acc.per_token_bytes(576)
    assert acc.tokens_in(GIB10, per_tok) == 690420
    assert 10 * 10 ** 9 // per_tok == 643004


def test_cache_row_bytes_with_metadata():
    assert acc.cache_row_bytes("bf16") == 1152
    assert acc.cache_row_bytes("int8") == 656
    assert acc.cache_row_bytes("int4") == 464
    assert acc.cache_row_bytes("int8_kbf16") == 704
    assert acc.cache_row_bytes("int4_kint4") == 432
    # payloads of the two: 640 and 288 bytes per layer, the report's "B" and
    # headline INT4 configurations
    assert acc.cache_row_bytes("int8_kbf16") - 64 == acc.payload_bytes_per_layer(8, 16)
    assert acc.cache_row_bytes("int4_kint4") - 144 == acc.payload_bytes_per_layer(4, 4)
    # every cache row plane is a whole number of 16-byte vectors
    for nbytes in (512, 256, 64, 128, 80, 64):
        assert nbytes % 16 == 0


def test_package_row_bytes_equal_the_oracle():
    # the binding's own row arithmetic (used by the benchmark) against the oracle's
    from mla_latent_kv_cache_amd.cache import row_bytes
    for fmt in ("bf16", "int8", "int4", "int8_kbf16", "int4_kint4"):
        assert row_bytes(fmt) == acc.cache_row_bytes(fmt), fmt
