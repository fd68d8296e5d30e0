"""Index arithmetic of the whole-line decompression of tile-ordered matrices
(csrc/df11_pairs.h, composed as merge_group_pairs composes it), built with
g++ on its own and checked against the MFMA tile order's definition: every
chunk of a group is merged once and stored once, at its row-major place,
from the stage unit its merge wrote, eight lanes to a 128-byte line, and a
line counts as whole exactly when the group holds all its chunks."""

import os
import subprocess
from collections import defaultdict

import numpy as np
import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(REPO, "entropy_decoding_df11_amd", "csrc")


@pytest.fixture(scope="module")
def cli(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("pairs") / "pairs_cli")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", f"-I{CSRC}", os.path.join(REPO, "tests", "cpp", "pairs_cli.cpp"),
                    "-o", exe], check=True)

    def run(cols, c0, n):
        res = subprocess.run([exe], input=f"Q {cols} {c0} {n}\n", capture_output=True, text=True, check=True)
        merges, stores = [], []
        for ln in res.stdout.split("\n"):
            f = ln.split()
            if f and f[0] == "M":
                merges.append(tuple(int(v) for v in f[1:]))
            elif f and f[0] == "S":
                stores.append(tuple(int(v) for v in f[1:]))
        return merges, stores

    return run


def tile_origin(c, cols):
    """Row-major index of the first element of chunk c of a matrix in MFMA
    tile order: 512-element blocks, block b is n-tile b mod 4 of global
    k-step b / 4, global k-step g is k-step g mod (cols / 32) of the 64-row
    panel g / (cols / 32); lane l of a block holds row 16 nt + (l mod 16),
    columns 32 ks + 8 (l / 16) .. + 7."""
    lane, block = c % 64, c // 64
    nt, g = block % 4, block // 4
    panel, ks = divmod(g, cols // 32)
    return (64 * panel + 16 * nt + lane % 16) * cols + 32 * ks + 8 * (lane // 16)


def _check(cli, cols, c0, n):
    merges, stores = cli(cols, c0, n)
    merged = {}
    for p, h, w, lane, c, unit in merges:
        assert c0 <= c < c0 + n and c not in merged
        assert 0 <= unit < 136
        merged[c] = (p, w, unit)
    assert sorted(merged) == list(range(c0, c0 + n))
    # stage units of one wave and pair-round are distinct
    per_stage = defaultdict(set)
    for c, (p, w, unit) in merged.items():
        assert unit not in per_stage[(p, w)]
        per_stage[(p, w)].add(unit)
    stored = {}
    lines = defaultdict(list)
    for p, s, w, lane, c, unit, dst, whole in stores:
        assert c0 <= c < c0 + n and c not in stored
        assert merged[c] == (p, w, unit), (c, merged[c], (p, w, unit))
        assert dst == tile_origin(c, cols), (c, dst, tile_origin(c, cols))
        stored[c] = (dst, whole)
        lines[(p, s, w, lane // 8)].append((lane % 8, dst))
    assert sorted(stored) == sorted(merged)
    for key, items in lines.items():
        # the lanes of one row write consecutive 8-element runs of one 64-element line
        base = items[0][1] - 8 * items[0][0]
        assert base % 64 == 0
        assert all(dst == base + 8 * q for q, dst in items)
    # whole: every chunk of the line (by the definition) lies in the group
    line_of = {}
    first, last = (c0 // 512) * 512, -(-(c0 + n) // 512) * 512
    for c in range(first, last):
        line_of.setdefault(tile_origin(c, cols) // 64, []).append(c)
    for c, (dst, whole) in stored.items():
        chunks = line_of[dst // 64]
        assert len(chunks) == 8
        assert whole == all(c0 <= x < c0 + n for x in chunks), (c, chunks)


@pytest.mark.parametrize("cols", [64, 128, 192, 4096, 14336])
def test_pair_rounds_against_the_tile_order(cli, cols):
    rng = np.random.default_rng(cols)
    total = 64 * 4 * cols // 8  # chunks of a 256-row matrix
    cases = [(0, 0), (0, 1), (0, 512), (511, 2), (512, 1024), (3, 2048), (total - 700, 700)]
    for _ in range(12):
        c0 = int(rng.integers(0, total - 1))
        cases.append((c0, int(rng.integers(0, min(2600, total - c0) + 1))))
    for c0, n in cases:
        _check(cli, cols, c0, n)
