"""libkvq for MI355X (gfx950): decode attention read directly from a low-bit, group-wise,
asymmetrically quantized KV cache.

The compute lives in libkvq.so (hand-written HIP, built by `python -m
bit_kv_cache_pack_amd.build`); `kvq` is its ctypes binding, with the same names as the C
ABI in include/kvq.h and argument marshalling only.
"""
from .kvq import (KVQ_OUT_F16, KVQ_OUT_F32, Format, KVQError, kvq_append_residual,  # noqa: F401
                  kvq_combine, kvq_decode_attention, kvq_quantize_pack, suggest_splits)
