"""DF11 (DFloat11) lossless BF16 weight compression for one AMD Instinct MI355X."""
