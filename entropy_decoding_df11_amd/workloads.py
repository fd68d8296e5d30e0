"""Seeded synthetic BF16 weight generators.

This module is shared by the tests, the benchmark and the oracle's test
harness.  It draws random numbers and rounds them to BF16; it contains none of
the DF11 codec (no histogram, no Huffman code, no bit packing, no split or
merge of the BF16 fields).

The pages that describe DF11 measure on trained LLM weights ("DFloat11:
Kompresi inferensi GPU lossless ...", GeekNews, sections "Ruang kompresi yang
tersisa pada exponent BFloat16" and "Hasil evaluasi dan efek nyata").  No
weights are available here, so these generators stand in for them with the
same shapes and with the statistics those sections report: about 40 exponent
values in use, an exponent entropy near 2.6 bits and a rapidly falling
frequency by rank.

Every generator uses ``numpy.random.default_rng(seed)`` (PCG64) and returns a
flat ``numpy.uint16`` array holding BF16 bit patterns in row-major order.
"""

from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Tuple

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 with round-to-nearest-even.

    Returns the 16-bit patterns as ``uint16``.  Inputs must be finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _normal_with_replacements(rng: np.random.Generator, n: int, sigma: float,
                              replacements: List[Tuple[float, float]]) -> np.ndarray:
    """N(0, sigma^2) samples where each (fraction, scale) pair replaces
    round(fraction*n) distinct entries by N(0, scale^2) samples."""
    x = rng.standard_normal(n) * sigma
    counts = [int(round(f * n)) for f, _ in replacements]
    total = sum(counts)
    if total:
        idx = rng.choice(n, total, replace=False)
        start = 0
        for (f, scale), c in zip(replacements, counts):
            x[idx[start:start + c]] = rng.standard_normal(c) * scale
            start += c
    return x


# --------------------------------------------------------------------------
# The five workloads.  Sizes follow the shapes named for each workload.
# --------------------------------------------------------------------------

LLAMA3_8B_BLOCK: List[Tuple[str, Tuple[int, int]]] = [
    ("q_proj", (4096, 4096)),
    ("k_proj", (1024, 4096)),
    ("v_proj", (1024, 4096)),
    ("o_proj", (4096, 4096)),
    ("gate_proj", (14336, 4096)),
    ("up_proj", (14336, 4096)),
    ("down_proj", (4096, 14336)),
]


def gen_single_matrix(seed: int = 0, rows: int = 1024, cols: int = 1024) -> np.ndarray:
    """1024x1024 matrix, N(0, 0.02^2), rounded to BF16."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(rows * cols) * 0.02)


def gen_projection_with_outliers(seed: int = 1, rows: int = 4096, cols: int = 4096) -> np.ndarray:
    """4096x4096 projection: N(0, 0.02^2) with 1e-4 of the entries replaced
    by N(0, 1) outliers and another 1e-4 by N(0, 1e-8) tiny values."""
    rng = np.random.default_rng(seed)
    x = _normal_with_replacements(rng, rows * cols, 0.02, [(1e-4, 1.0), (1e-4, 1e-4)])
    return f32_to_bf16_bits(x)


def gen_student_t(seed: int = 2, rows: int = 14336, cols: int = 4096) -> np.ndarray:
    """14336x4096 MLP up-projection: Student-t(5) scaled by 0.015."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_t(5, rows * cols) * 0.015)


def gen_block(seed: int = 3, shapes: List[Tuple[str, Tuple[int, int]]] = None
              ) -> Tuple[np.ndarray, List[Tuple[str, int, Tuple[int, int]]]]:
    """Llama-3-8B-shaped transformer block: every linear weight is
    N(0, 0.02^2) with 1e-4 of its entries replaced by N(0, 1) outliers.

    Returns the row-major concatenation and a view table of
    (name, element offset, shape).
    """
    shapes = LLAMA3_8B_BLOCK if shapes is None else shapes
    rng = np.random.default_rng(seed)
    parts = []
    views = []
    off = 0
    for name, (r, c) in shapes:
        x = _normal_with_replacements(rng, r * c, 0.02, [(1e-4, 1.0)])
        parts.append(f32_to_bf16_bits(x))
        views.append((name, off, (r, c)))
        off += r * c
    return np.concatenate(parts), views


LM_HEAD_SHAPE = (128256, 4096)


def gen_lm_head(seed: int = 5, shape: Tuple[int, int] = LM_HEAD_SHAPE, rows_per_chunk: int = 8192) -> np.ndarray:
    """LM-head / embedding-sized matrix (128256x4096 for a 128K vocabulary):
    N(0, 0.02^2) with 1e-4 of the entries replaced by N(0, 1) outliers, drawn
    row-chunk by row-chunk (rows_per_chunk rows per draw, in order) so that
    no float64 copy of the whole matrix is held."""
    rows, cols = shape
    rng = np.random.default_rng(seed)
    out = np.empty(rows * cols, dtype=np.uint16)
    for r0 in range(0, rows, rows_per_chunk):
        n = (min(rows, r0 + rows_per_chunk) - r0) * cols
        out[r0 * cols:r0 * cols + n] = f32_to_bf16_bits(_normal_with_replacements(rng, n, 0.02, [(1e-4, 1.0)]))
    return out


STRESS_CENTER = 120
STRESS_RANKS = 40


def stress_rank_exponents(n_ranks: int = STRESS_RANKS, center: int = STRESS_CENTER) -> np.ndarray:
    """Exponent value for each frequency rank: 120, 119, 121, 118, 122, ..."""
    r = np.arange(1, n_ranks + 1)
    step = r // 2
    sign = np.where(r % 2 == 0, -1, 1)
    return (center + sign * step).astype(np.int64)


def stress_rank_probabilities(kind: str = "tuned", n_ranks: int = STRESS_RANKS,
                              s: float = 1.6, head: int = 16, ratio: float = 0.6) -> np.ndarray:
    """Rank probabilities for the stress stream.

    ``literal``: p_r proportional to r^-s over all ranks.
    ``tuned``: that Zipf law for ranks 1..head, then a geometric tail
    p_r = ratio * p_(r-1).  A ratio below 1/phi makes every tail symbol one
    level deeper in the code tree, which yields the long codes the stress
    workload is meant to exercise.
    """
    r = np.arange(1, n_ranks + 1, dtype=np.float64)
    p = r ** (-s)
    if kind == "tuned":
        for i in range(head, n_ranks):
            p[i] = p[i - 1] * ratio
    elif kind != "literal":
        raise ValueError(kind)
    return p / p.sum()


def gen_stress(seed: int = 4, n: int = 1 << 28, kind: str = "tuned") -> np.ndarray:
    """Stress stream: exponents i.i.d. over 40 ranks centred at 120, sign and
    7-bit mantissa uniform.  Values are built as (-1)^s * (1 + m/128) * 2^(e-127),
    which is exact in float32 and therefore in BF16."""
    rng = np.random.default_rng(seed)
    ranks = rng.choice(STRESS_RANKS, n, p=stress_rank_probabilities(kind))
    exps = stress_rank_exponents()[ranks]
    sm = rng.integers(0, 256, n, dtype=np.uint8)
    sign = np.where(sm >= 128, np.float32(-1.0), np.float32(1.0))
    frac = np.float32(1.0) + (sm % 128).astype(np.float32) / np.float32(128.0)
    vals = np.ldexp(frac, (exps - 127).astype(np.int32)).astype(np.float32) * sign
    return f32_to_bf16_bits(vals)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_elements: int
    description: str
    make: Callable[..., np.ndarray]


def _block_only(seed: int = 3) -> np.ndarray:
    return gen_block(seed)[0]


WORKLOADS: Dict[str, Workload] = {
    "single_1024x1024": Workload("single_1024x1024", 1 << 20,
                                 "1024x1024 N(0,0.02^2), seed 0", gen_single_matrix),
    "proj_4096x4096_outliers": Workload("proj_4096x4096_outliers", 1 << 24,
                                        "4096x4096 N(0,0.02^2) + 1e-4 N(0,1) + 1e-4 N(0,1e-8), seed 1",
                                        gen_projection_with_outliers),
    "mlp_14336x4096_t5": Workload("mlp_14336x4096_t5", 14336 * 4096,
                                  "14336x4096 Student-t(5)*0.015, seed 2", gen_student_t),
    "llama3_8b_block": Workload("llama3_8b_block", sum(r * c for _, (r, c) in LLAMA3_8B_BLOCK),
                                "Llama-3-8B block q,k,v,o,gate,up,down, N(0,0.02^2) + 1e-4 N(0,1), "
                                "shared codebook, seed 3", _block_only),
    "lm_head_128256x4096": Workload("lm_head_128256x4096", LM_HEAD_SHAPE[0] * LM_HEAD_SHAPE[1],
                                    "128256x4096 N(0,0.02^2) + 1e-4 N(0,1), row chunks of 8192, seed 5",
                                    gen_lm_head),
    "stress_2p28_zipf": Workload("stress_2p28_zipf", 1 << 28,
                                 "2^28 exponents over 40 ranks (Zipf 1.6 head, 0.6 geometric tail), "
                                 "uniform sign/mantissa, seed 4", gen_stress),
}


def make(name: str) -> np.ndarray:
    """Generate a named workload with its default seed."""
    return WORKLOADS[name].make()
