"""DF11 (DFloat11) lossless BF16 weight compression for one AMD Instinct MI355X.

Host encoders and gfx950 decoders (DF11 Huffman, the decode fused into a
small-batch matmul, and an rANS exponent coder) live in libdf11.so (C ABI:
include/df11.h); this package is its Python binding, the model-forward helpers
(runtime: blocks decoded before use, projections with the decode fused in,
forwards captured into HIP graphs) and the seeded synthetic workloads.
"""

from .df11 import (DF11Block, DF11BlockBatch, DF11RansTensor, DF11Tensor, HostStream, RansHostStream, build_codebook,
                   codebook_arrays, compress, compress_block, decode_table, decompress, decompress_batch, encode,
                   histogram, linear_batch, rans_compress, rans_encode)
from ._lib import Df11Error

__all__ = [
    "DF11Block", "DF11BlockBatch", "DF11RansTensor", "DF11Tensor", "Df11Error", "HostStream", "RansHostStream",
    "build_codebook", "codebook_arrays", "compress", "compress_block", "decode_table", "decompress",
    "decompress_batch", "encode", "histogram", "linear_batch", "rans_compress", "rans_encode",
]
