"""DF11 (DFloat11) lossless BF16 weight compression for one AMD Instinct MI355X.

Host encoder and gfx950 decoder live in libdf11.so (C ABI: include/df11.h);
this package is its Python binding plus the seeded synthetic workloads.
"""

from .df11 import (DF11Block, DF11BlockBatch, DF11Tensor, HostStream, build_codebook, codebook_arrays, compress,
                   compress_block, decode_table, decompress, decompress_batch, encode, histogram)
from ._lib import Df11Error

__all__ = [
    "DF11Block", "DF11BlockBatch", "DF11Tensor", "Df11Error", "HostStream", "build_codebook", "codebook_arrays",
    "compress", "compress_block", "decode_table", "decompress", "decompress_batch", "encode", "histogram",
]
