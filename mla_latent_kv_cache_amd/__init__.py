"""Absorbed MLA decode over a quantized latent KV cache, for MI355X (gfx950).

The compute lives in libmla_kv.so (HIP, built from csrc/mla_kv.hip; C ABI in
include/mla_kv.h). This package marshals arguments to it:

  LatentCache   cache planes in torch device tensors; append / decode /
                decode_step / get
  rope_tables   RoPE angle tables for decode_step
  workloads     seeded synthetic inputs shaped like DeepSeek-V2-Lite
"""

import importlib

__all__ = ["LatentCache", "MlaError", "rope_tables", "workloads"]


def __getattr__(name):
    # Loading the HIP library is deferred until a caller needs it, so that the
    # input generators can be imported on machines without the library.
    if name == "LatentCache":
        return importlib.import_module(".cache", __name__).LatentCache
    if name == "rope_tables":
        return importlib.import_module(".cache", __name__).rope_tables
    if name == "MlaError":
        return importlib.import_module("._lib", __name__).MlaError
    if name == "workloads":
        return importlib.import_module(".workloads", __name__)
    raise AttributeError(name)
