"""Per-token KV byte and capacity arithmetic (oracle, pure integers).

Test infrastructure: only tests and the benchmark use this module.

What the pages fix ("Absorbed MLA Cache Optimization on DeepSeek-V2-Lite"):
* section 1.2/1.3: the expanded cache stores per layer a 192-d key
  (nope 128 + rope 64) and a 128-d value for each of 16 heads in bf16, which
  is 10,240 B per layer and 276,480 B = 270 KB over 27 layers;
* section 2.2 / 3.1: the absorbed cache stores 512 + 64 bf16 values,
  1,152 B per layer, 30.4 KB per token;
* section 3.2 / 4.1 / 4.3: INT8 latent + INT8 k_pe 15.2 KB (17.8x), latent8 +
  kpe16 16.9 KB (16x), INT4 + kpe8 8.4 KB (32x), INT4 latent + INT4 k_pe
  7.6 KB (35.6x), and the tokens that fit in 10 GB of KV space.
Reading taken: the pages count code bytes only (no scales), and KB and GB are
KiB and GiB; this is the only reading that reproduces all of their numbers.
The real footprint with the fp16 scales and zero-points of this cache is given
by cache_row_bytes.
"""

N_LAYERS = 27
N_HEADS = 16
QK_NOPE = 128
QK_ROPE = 64
V_DIM = 128
LATENT = 512
KIB = 1024
GIB = 1024 ** 3


def expanded_bytes_per_layer(heads=N_HEADS, nope=QK_NOPE, rope=QK_ROPE, v=V_DIM, elem=2):
    """Expanded K (nope+rope) and V per head, bf16: (192 + 128) * 16 * 2 = 10,240."""
    return (nope + rope + v) * heads * elem


def payload_bytes_per_layer(latent_bits, rope_bits, latent=LATENT, rope=QK_ROPE):
    """Code bytes of one token in one layer: latent and k_pe at the given widths."""
    bits = latent * latent_bits + rope * rope_bits
    assert bits % 8 == 0
    return bits // 8


# The cache formats of the pages, as (latent bits, k_pe bits).
PAYLOAD_FORMATS = {
    "absorbed_bf16": (16, 16),
    "int8": (8, 8),
    "latent8_kpe16": (8, 16),
    "int4_kpe8": (4, 8),
    "int4_kpe4": (4, 4),
}


def per_token_bytes(bytes_per_layer, layers=N_LAYERS):
    return bytes_per_layer * layers


def kib(nbytes):
    return nbytes / KIB


def compression_ratio(bytes_per_token, baseline=None):
    if baseline is None:
        baseline = per_token_bytes(expanded_bytes_per_layer())
    return baseline / bytes_per_token


def tokens_in(space_bytes, bytes_per_token):
    """How many whole tokens fit in the given KV space."""
    return space_bytes // bytes_per_token


def cache_row_bytes(fmt):
    """Bytes one token occupies in one layer of THIS cache, metadata included.

    bf16: 512*2 + 64*2 = 1152
    int8: 512 codes + 64 k_pe codes + 40 fp16 scales (32 latent groups of 16,
          8 k_pe groups of 8) = 656
    int4: 256 packed + 64 k_pe codes + 40 fp16 scales + 32 fp16 zero-points = 464
    int8_kbf16: 512 codes + 64 bf16 k_pe + 32 fp16 latent scales = 704
    int4_kint4: 256 packed + 32 packed k_pe + 40 fp16 scales + 32 fp16 zero-points = 432
    """
    if fmt == "bf16":
        return LATENT * 2 + QK_ROPE * 2
    scales = (LATENT // 16 + QK_ROPE // 8) * 2
    zeros = (LATENT // 16) * 2
    if fmt == "int8":
        return LATENT + QK_ROPE + scales
    if fmt == "int4":
        return LATENT // 2 + QK_ROPE + scales + zeros
    if fmt == "int8_kbf16":
        return LATENT + QK_ROPE * 2 + (LATENT // 16) * 2
    if fmt == "int4_kint4":
        return LATENT // 2 + QK_ROPE // 2 + scales + zeros
    raise ValueError(fmt)
