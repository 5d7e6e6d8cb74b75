"""Plain CPU oracle for the fused KV-cache encode/decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library under ``kv_cache_compression_kvc_amd/csrc``.

What it computes (all arithmetic in float64, numpy):

1. sign flip with a seeded +/-1 vector, then the orthonormal Walsh-Hadamard
   transform along head_dim -- the "randomized Hadamard transform" that the
   episode notes of *FastKVComp: checking whether high-throughput KV
   compression pays off* (radioguide.fm) name as the first pipeline stage;
2. per-group asymmetric min/max low-bit quantization -- the second stage
   named there ("only quantization loses information");
3. sub-byte packing of the codes and the blob layout;
4. the matching decode: unpack, dequantize, inverse transform.

The abstract of *Beyond Compression Ratio: High-Throughput KV Compression for
Disaggregated LLM Serving* says the production kernel fuses stages 1 and 2
into one tiled pass with no full-size intermediate; the oracle deliberately
does not fuse anything, so that each step can be checked by eye.

Readings of points the pages leave open (sign generator, Hadamard ordering,
fp16 meta rounding directions, blob layout, paged edges) are listed in the
module docstrings where each is used.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, brute force on tiny inputs, library routines (scipy's
Hadamard, numpy's float16 conversion) or published test vectors under
``tests/golden``.
"""

from .signs import splitmix64_outputs, sign_vector, sign_bits_mask
from .rounding import round_binary, to_fp16, rd16, ru16, rne_bf16, rne_fp16, \
    storage_to_f64, f64_to_storage
from .rht import hadamard, rotate_raw, rotate, unrotate
from .quant import group_meta, code_values, nearest_codes, quantize, pack_codes, unpack_codes, \
    dequantize
from .blob import BlobLayout, blob_layout, encode, decode, EncodeTrace, \
    paged_layout, gather_request, encode_paged, decode_paged, tile_codes, untile_codes, code_offsets

__all__ = [
    "splitmix64_outputs", "sign_vector", "sign_bits_mask",
    "round_binary", "to_fp16", "rd16", "ru16", "rne_bf16", "rne_fp16",
    "storage_to_f64", "f64_to_storage",
    "hadamard", "rotate_raw", "rotate", "unrotate",
    "group_meta", "code_values", "nearest_codes", "quantize", "pack_codes", "unpack_codes",
    "dequantize",
    "BlobLayout", "blob_layout", "encode", "decode", "EncodeTrace",
    "paged_layout", "gather_request", "encode_paged", "decode_paged",
    "tile_codes", "untile_codes", "code_offsets",
]
