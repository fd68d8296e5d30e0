"""Pins for the CPU oracle (oracle/): checks against what the DF11 pages and the
mathematics fix, never against the oracle itself.

Source: GeekNews, "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan
LLM menjadi 70% ukurannya", sections "Ruang kompresi yang tersisa pada exponent
BFloat16", "Format DFloat11", "Decoding berbasis LUT hierarkis" and "Kernel GPU
2 tahap dan metadata bantu".
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from entropy_decoding_df11_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _entropy(counts):
    p = counts[counts > 0].astype(np.float64)
    p /= p.sum()
    return float(-(p * np.log2(p)).sum())


def _hist_from_weights(weights, symbols=None):
    hist = np.zeros(256, np.uint64)
    symbols = list(range(100, 100 + len(weights))) if symbols is None else symbols
    for s, w in zip(symbols, weights):
        hist[s] = w
    return hist, symbols


# ---------------------------------------------------------------------------
# BF16 fields ("Ruang kompresi ...": 1 sign, 8 exponent, 7 mantissa bits)
# ---------------------------------------------------------------------------

def _page_statistics():
    """The page's stated figures (tests/golden/page_statistics.json, each
    with its section)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_statistics.json")) as f:
        return json.load(f)


def test_split_matches_ieee_bf16_semantics_exhaustively():
    w = np.arange(65536, dtype=np.uint32)
    e_all = (w >> 7) & 0xFF
    keep = e_all < 240
    w = w[keep].astype(np.uint16)
    assert w.size == 61440
    e, sm = oracle.split(w)
    # Value of every pattern as float32 (BF16 is the top half of a float32).
    val = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sign = np.where(sm >= 128, -1.0, 1.0)
    mant = (sm & 0x7F).astype(np.float64)
    ee = e.astype(np.int64)
    normal = sign * np.ldexp(1.0 + mant / 128.0, ee - 127)
    sub = sign * np.ldexp(mant / 128.0, -126)
    expect = np.where(ee == 0, sub, normal)
    assert np.array_equal(val, expect)
    # signed zeros: the sign byte must follow the float sign bit too
    assert np.array_equal(np.signbit(val), sm >= 128)


def test_merge_inverts_split_exhaustively():
    w = np.arange(65536, dtype=np.uint32)
    w = w[((w >> 7) & 0xFF) < 240].astype(np.uint16)
    e, sm = oracle.split(w)
    assert np.array_equal(oracle.merge(e, sm), w)


@pytest.mark.parametrize("bits", [0x7F80, 0xFF80, 0x7FC0, 0x7800, 0xF812])
def test_reserved_exponents_rejected(bits):
    # exponent >= 240: Inf/NaN (255) and |x| >= 2^113; the pages reuse 240..255 as pointers
    lo, hi = _page_statistics()["pointer_values"]["value"]
    assert lo <= (bits >> 7) & 0xFF <= hi
    w = np.array([0x3F80, bits, 0x3F00], np.uint16)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.split(w)
    assert ei.value.code == -2
    with pytest.raises(oracle.OracleError):
        oracle.histogram(w)
    with pytest.raises(oracle.OracleError):
        oracle.encode(w)


def test_largest_usable_exponent_encodes():
    """Exponent 239, just below the pointer range, is an ordinary value."""
    lo, _ = _page_statistics()["pointer_values"]["value"]
    w = np.array([0x3F80, (lo - 1) << 7, 0x8000 | ((lo - 1) << 7) | 0x55, 0x3F00], np.uint16)
    assert np.array_equal(oracle.decode_treewalk(oracle.encode(w)), w)


# ---------------------------------------------------------------------------
# Huffman code lengths ("Format DFloat11")
# ---------------------------------------------------------------------------

def _optimal_cost_bruteforce(weights):
    """Minimum of sum(w_i * l_i) over all complete prefix codes (Kraft sum == 1)."""
    n = len(weights)
    best = None
    for lens in itertools.product(range(1, n), repeat=n):
        if sum(2.0 ** -l for l in lens) != 1.0:
            continue
        cost = sum(w * l for w, l in zip(weights, lens))
        best = cost if best is None else min(best, cost)
    return best


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7])
def test_huffman_cost_matches_bruteforce_optimum(n):
    rng = np.random.default_rng(100 + n)
    for trial in range(6 if n < 7 else 3):
        weights = [int(x) for x in rng.integers(1, 50, n)]
        if trial == 0:
            weights = [1] * n  # all ties
        hist, syms = _hist_from_weights(weights)
        lens = oracle.code_lengths(hist)
        got = sum(w * int(lens[s]) for w, s in zip(weights, syms))
        assert got == _optimal_cost_bruteforce(weights), (weights, [int(lens[s]) for s in syms])


def test_dyadic_weights_give_exact_lengths_and_entropy():
    ks = [1, 2, 3, 4, 5, 6, 7, 7]
    weights = [2 ** (7 - k) for k in ks]  # p_i = 2^-k_i
    hist, syms = _hist_from_weights(weights)
    lens = oracle.code_lengths(hist)
    assert [int(lens[s]) for s in syms] == ks
    total = sum(weights)
    lbar = sum(w * int(lens[s]) for w, s in zip(weights, syms)) / total
    assert lbar == pytest.approx(_entropy(np.array(weights)), abs=1e-12)


@pytest.mark.parametrize("m", [1, 2, 3, 5, 7])
def test_equal_weights_power_of_two(m):
    hist, syms = _hist_from_weights([9] * (2 ** m), symbols=list(range(2 ** m)))
    lens = oracle.code_lengths(hist)
    assert all(int(lens[s]) == m for s in syms)


def _fib(n):
    f = [1, 1]
    while len(f) < n:
        f.append(f[-1] + f[-2])
    return f[:n]


@pytest.mark.parametrize("n", [3, 10, 20, 33])
def test_fibonacci_weights_give_deepest_tree(n):
    hist, syms = _hist_from_weights(_fib(n), symbols=list(range(60, 60 + n)))
    lens = oracle.code_lengths(hist)
    got = sorted((int(lens[s]) for s in syms), reverse=True)
    assert got == sorted(list(range(1, n)) + [n - 1], reverse=True)


def test_code_longer_than_32_bits_rejected():
    hist, _ = _hist_from_weights(_fib(34), symbols=list(range(60, 94)))
    with pytest.raises(oracle.OracleError) as ei:
        oracle.code_lengths(hist)
    assert ei.value.code == -3


def test_single_exponent_gets_phantom_partner():
    hist = np.zeros(256, np.uint64)
    hist[127] = 1000
    lens = oracle.code_lengths(hist)
    assert int(lens[127]) == 1 and int(lens[0]) == 1 and int((lens > 0).sum()) == 2
    empty = oracle.code_lengths(np.zeros(256, np.uint64))
    assert int(empty[0]) == 1 and int(empty[1]) == 1 and int((empty > 0).sum()) == 2
    hist = np.zeros(256, np.uint64)
    hist[0] = 5
    lens = oracle.code_lengths(hist)
    assert int(lens[0]) == 1 and int(lens[1]) == 1


# ---------------------------------------------------------------------------
# Canonical codes and bit packing: the hand example
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "hand_example_abca.json")) as f:
        return json.load(f)


def test_hand_example_codebook_and_packing():
    g = _golden()
    w = np.array([int(h, 16) for h in g["bf16_hex"]], np.uint16)
    # the BF16 patterns are the float values the fixture names
    assert np.array_equal((w.astype(np.uint32) << 16).view(np.float32), np.array(g["values_f32"], np.float32))
    s = oracle.encode(w, n=g["layout"]["bytes_per_thread"], G=g["layout"]["threads_per_group"])
    for e, l in g["code_lengths"].items():
        assert int(s["code_lengths"][int(e)]) == l
    for e, c in g["codes"].items():
        assert int(s["codes"][int(e)]) == c
    assert int((s["code_lengths"] > 0).sum()) == len(g["code_lengths"])
    assert s["total_bits"] == g["total_bits"]
    assert s["enc"][0] == int(g["enc_first_byte_hex"], 16)
    assert not s["enc"][1:].any()
    assert s["n_threads"] == g["n_threads"] and s["n_groups"] == g["n_groups"]
    assert s["gaps"][0] == int(g["gaps_first_byte_hex"], 16)
    assert s["out_pos"].tolist() == g["out_pos"]
    assert s["sm"][:4].tolist() == [int(h, 16) for h in g["sign_mantissa_hex"]]
    assert s["n_luts"] == g["n_luts"]
    for lo, hi, sym in g["root_lut_ranges"]:
        assert np.all(s["luts"][0][lo:hi + 1] == sym)
    assert np.array_equal(oracle.decode_treewalk(s), w)


def _prefix_free(lens, codes):
    items = [(int(l), int(c)) for l, c in zip(lens, codes) if l]
    for (la, ca), (lb, cb) in itertools.permutations(items, 2):
        if la <= lb and (cb >> (lb - la)) == ca:
            return False
    return True


@pytest.mark.parametrize("seed", range(8))
def test_canonical_codes_prefix_free_and_kraft_complete(seed):
    rng = np.random.default_rng(seed)
    n_sym = int(rng.integers(2, 60))
    syms = sorted(rng.choice(240, n_sym, replace=False).tolist())
    weights = [int(x) for x in rng.zipf(1.5, n_sym)]
    hist, _ = _hist_from_weights(weights, syms)
    lens = oracle.code_lengths(hist)
    codes = oracle.canonical_codes(lens)
    assert _prefix_free(lens, codes)
    assert sum(1 << (32 - int(l)) for l in lens if l) == 1 << 32
    # canonical: code values increase with (length, exponent), left-justified
    order = sorted((int(lens[s]), s) for s in range(256) if lens[s])
    just = [int(codes[s]) << (32 - l) for l, s in order]
    assert just == sorted(just) and len(set(just)) == len(just)


# ---------------------------------------------------------------------------
# Hierarchical LUTs ("Decoding berbasis LUT hierarkis")
# ---------------------------------------------------------------------------

def _expected_lut_entry(lens, codes, luts, lut_prefixes, lut_id, x):
    """Brute force from the code table: the code continuing prefix (depth d)
    with the 8 bits of x, or the LUT of the node reached after those 8 bits."""
    d, prefix = lut_prefixes[lut_id]
    path = (prefix << 8) | x  # d + 8 bits
    for s in range(256):
        l = int(lens[s])
        if d < l <= d + 8 and (path >> (d + 8 - l)) == int(codes[s]):
            return s
    for j, (dj, pj) in enumerate(lut_prefixes):
        if dj == d + 8 and pj == path:
            return 256 - j
    return None


def _lut_prefixes(lens, codes):
    nodes = set()
    for s in range(256):
        l = int(lens[s])
        for d in (8, 16, 24):
            if d < l:
                nodes.add((d, int(codes[s]) >> (l - d)))
    return [(0, 0)] + sorted(nodes)


@pytest.mark.parametrize("case", ["single_1024x1024", "fib30", "literal_zipf"])
def test_luts_agree_with_code_table_exhaustively(case):
    if case == "fib30":
        hist, _ = _hist_from_weights(_fib(30), symbols=list(range(90, 120)))
    elif case == "literal_zipf":
        p = workloads.stress_rank_probabilities("literal")
        hist = np.zeros(256, np.uint64)
        hist[workloads.stress_rank_exponents()] = np.round(p * 1e9).astype(np.uint64)
    else:
        hist = oracle.histogram(workloads.make(case))
    cb = oracle.codebook(hist)
    lens, codes, luts = cb["code_lengths"], cb["codes"], cb["luts"]
    prefixes = _lut_prefixes(lens, codes)
    assert luts.shape[0] == len(prefixes) <= 17
    for i in range(luts.shape[0]):
        for x in range(256):
            assert luts[i][x] == _expected_lut_entry(lens, codes, luts, prefixes, i, x), (i, x)
    # pointer values only in 240..255; symbols only used exponents
    sym = luts[luts < 240]
    assert np.all(lens[sym] > 0)


def test_literal_zipf_needs_eight_luts():
    # the pages report k = 4..8 compact LUTs; the literal Zipf(1.6) stress law reaches the upper end
    p = workloads.stress_rank_probabilities("literal")
    hist = np.zeros(256, np.uint64)
    hist[workloads.stress_rank_exponents()] = np.round(p * 1e9).astype(np.uint64)
    cb = oracle.codebook(hist)
    assert cb["n_luts"] == 8 and cb["max_len"] == 10


def test_too_many_luts_rejected():
    # Dyadic weights for 33 codes of 7 bits, 173 of 8 and 34 of 9 (Kraft sum 1,
    # all 240 usable exponents): the 34 nine-bit codes hang in pairs under 17
    # internal nodes at depth 8, one more than the 16 pointer values 240..255.
    weights = [4] * 33 + [2] * 173 + [1] * 34
    hist, _ = _hist_from_weights(weights, symbols=list(range(240)))
    lens = oracle.code_lengths(hist)
    assert sorted(np.bincount(lens[lens > 0])[7:].tolist()) == [33, 34, 173]
    codes = oracle.canonical_codes(lens)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.build_luts(lens, codes)
    assert ei.value.code == -4


# ---------------------------------------------------------------------------
# Gaps and output positions ("Kernel GPU 2 tahap dan metadata bantu")
# ---------------------------------------------------------------------------

def _metadata_bruteforce(w, lens, n, G):
    """Code starts from the cumulative code lengths, then gaps and group offsets
    straight from their definitions."""
    e = (w.astype(np.int64) >> 7) & 0xFF
    l = lens[e].astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(l)])  # last entry: stream end (sentinel start)
    total = int(starts[-1])
    T = -(-total // (8 * n))
    gaps, out_pos = [], []
    for t in range(T):
        s_t = 8 * n * t
        i = int(np.searchsorted(starts, s_t, side="left"))
        gaps.append(int(starts[i]) - s_t)
        if t % G == 0:
            out_pos.append(min(i, len(w)))
    out_pos.append(len(w))
    return gaps, out_pos, total


@pytest.mark.parametrize("seed,n,G,size", [(0, 8, 64, 1), (1, 8, 64, 37), (2, 4, 64, 1000), (3, 8, 128, 5000),
                                          (4, 16, 64, 3000), (5, 5, 64, 777), (6, 8, 256, 20000)])
def test_gaps_and_offsets_match_definition(seed, n, G, size):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size) * rng.choice([0.02, 0.5, 1e-3], size)
    w = workloads.f32_to_bf16_bits(x)
    s = oracle.encode(w, n=n, G=G)
    gaps, out_pos, total = _metadata_bruteforce(w, s["code_lengths"], n, G)
    assert s["total_bits"] == total
    assert oracle.gap_values(s).tolist() == gaps
    assert s["out_pos"].tolist() == out_pos
    counts = oracle.check_metadata(s)
    assert int(counts.sum()) == size


@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers"])
def test_metadata_invariants(workload, name):
    s = oracle.encode(workload(name))
    gaps = oracle.gap_values(s)
    assert gaps[0] == 0
    assert gaps.max() < s["max_len"] <= 32
    assert gaps.max() < 1 << _page_statistics()["gap_bits"]["value"]  # a gap fits its 5-bit field
    op = s["out_pos"].astype(np.int64)
    assert op[0] == 0 and op[-1] == s["n_elements"] and np.all(np.diff(op) >= 0)
    counts = oracle.check_metadata(s)
    assert counts.sum() == s["n_elements"]
    assert counts.max() <= 64


# ---------------------------------------------------------------------------
# Round trips and the pages' aggregate figures
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers"])
def test_lossless_roundtrip_all_decoders(workload, name):
    w = workload(name)
    s = oracle.encode(w)
    assert np.array_equal(oracle.decode_treewalk(s), w)
    assert np.array_equal(oracle.decode_lut(s), w)
    out = np.zeros_like(w)
    oracle.decode_groups_parallel(s, 0, s["n_groups"], out, 4)
    assert np.array_equal(out, w)


@pytest.mark.parametrize("seed", range(6))
def test_roundtrip_random_streams(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 20000))
    kind = seed % 3
    if kind == 0:  # uniform over many exponents
        w = rng.integers(0, 65536, n).astype(np.uint16)
        w = w[((w >> 7) & 0xFF) < 240]
    elif kind == 1:  # deep chain of exponents
        p = np.array(_fib(30)[::-1], np.float64)
        e = rng.choice(np.arange(90, 120), n, p=p / p.sum())
        sm = rng.integers(0, 256, n)
        w = (((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)).astype(np.uint16)
    else:
        w = workloads.f32_to_bf16_bits(rng.standard_t(3, n) * 0.05)
    s = oracle.encode(w, n=int(rng.choice([4, 8, 12])), G=int(rng.choice([64, 256])))
    assert np.array_equal(oracle.decode_treewalk(s), w)
    assert np.array_equal(oracle.decode_lut(s), w)
    oracle.check_metadata(s)


def test_empty_and_single_element():
    s = oracle.encode(np.zeros(0, np.uint16))
    assert s["n_threads"] == 0 and s["n_groups"] == 0 and s["out_pos"].tolist() == [0] and s["total_bits"] == 0
    assert oracle.decode_treewalk(s).size == 0
    w = np.array([0xC0A0], np.uint16)
    s = oracle.encode(w)
    assert s["total_bits"] == 1 and s["n_threads"] == 1 and s["out_pos"].tolist() == [0, 1]
    assert np.array_equal(oracle.decode_treewalk(s), w)
    z = np.zeros(1000, np.uint16)  # one exponent value: phantom partner, 1 bit per weight
    s = oracle.encode(z)
    assert s["total_bits"] == 1000
    assert np.array_equal(oracle.decode_treewalk(s), z)


@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers"])
def test_entropy_bound_kraft_and_size(workload, name):
    w = workload(name)
    s = oracle.encode(w)
    hist = s["hist"].astype(np.float64)
    H = _entropy(hist)
    lens = s["code_lengths"].astype(np.float64)
    lbar = float((hist * lens).sum() / hist.sum())
    # textbook Huffman bound: H <= mean length < H + 1
    assert H <= lbar < H + 1
    assert sum(1 << (32 - int(l)) for l in s["code_lengths"] if l) == 1 << 32
    # size: EncodedExponent + PackedSignMantissa + Gaps + output positions + LUTs + CodeLengths
    n = s["n_elements"]
    size = n + -(-s["total_bits"] // 8) + -(-5 * s["n_threads"] // 8) + 4 * (s["n_groups"] + 1) + 256 * (s["n_luts"] + 1)
    # "Format DFloat11": about 11 bits per weight, about 70% of BF16
    page = _page_statistics()
    assert abs(8 + lbar - page["bits_per_weight"]["value"]) <= 0.5
    assert abs(size / (2 * n) - page["size_fraction"]["value"]) <= 0.06


@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers", "mlp_14336x4096_t5"])
def test_field_entropies_match_pages(workload, name):
    """'Ruang kompresi ...': sign and mantissa entropies are close to their bit
    widths, the exponent carries about 2.6 bits and about 40 values occur."""
    w = workload(name)
    e, sm = oracle.split(w)
    h_sign = _entropy(np.bincount(sm >> 7, minlength=2))
    h_mant = _entropy(np.bincount(sm & 0x7F, minlength=128))
    hist = oracle.histogram(w)
    h_exp = _entropy(hist.astype(np.float64))
    page = _page_statistics()
    assert h_sign > 0.999
    assert h_mant > 6.9
    assert abs(h_exp - page["exponent_entropy_bits"]["value"]) < 0.2
    assert 20 <= int((hist > 0).sum()) <= page["used_exponent_values"]["value"] + 5


def test_block_and_stress_code_lengths_in_pages_range():
    """'Decoding berbasis LUT hierarkis': for LLM weights the longest code is
    about 24-32 bits and 4-8 compact LUTs suffice."""
    page = _page_statistics()
    lo_len, hi_len = page["max_code_length_range"]["value"]
    lo_k, hi_k = page["compact_lut_count_range"]["value"]
    w, _ = workloads.gen_block()
    cb = oracle.codebook(oracle.histogram(w))
    assert lo_len <= cb["max_len"] <= hi_len and lo_k <= cb["n_luts"] <= hi_k
    w = workloads.gen_stress(n=1 << 24)
    cb = oracle.codebook(oracle.histogram(w))
    assert 28 <= cb["max_len"] <= hi_len and lo_k <= cb["n_luts"] <= hi_k
    assert 36 <= int((oracle.histogram(w) > 0).sum()) <= 40  # all 40 ranks occur at the full 2^28 size


# ---------------------------------------------------------------------------
# The pins catch planted mistakes
# ---------------------------------------------------------------------------

def test_planted_mistakes_are_caught(workload):
    w = workload("single_1024x1024")[:50000]
    s = oracle.encode(w)
    # a flipped payload bit changes the decoded weights
    bad = dict(s)
    bad["enc"] = s["enc"].copy()
    bad["enc"][100] ^= 0x10
    try:
        assert not np.array_equal(oracle.decode_treewalk(bad), w)
    except oracle.OracleError:
        pass
    # a wrong gap breaks the metadata re-walk
    bad = dict(s)
    bad["gaps"] = s["gaps"].copy()
    bad["gaps"][3] ^= 0x04
    with pytest.raises(oracle.OracleError):
        oracle.check_metadata(bad)
    # an off-by-one group offset is caught too
    bad = dict(s)
    bad["out_pos"] = s["out_pos"].copy()
    bad["out_pos"][1] += 1
    with pytest.raises(oracle.OracleError):
        oracle.check_metadata(bad)
    # swapping two code lengths of different size breaks optimality
    lens = s["code_lengths"].copy()
    a, b = int(np.argmax(s["hist"])), int(np.argmax(lens))
    lens[a], lens[b] = lens[b], lens[a]
    cost_good = int((s["hist"] * s["code_lengths"].astype(np.uint64)).sum())
    cost_bad = int((s["hist"] * lens.astype(np.uint64)).sum())
    assert cost_bad > cost_good


# ---------------------------------------------------------------------------
# The decompressed matrix in a matmul ("Dekompresi yang disesuaikan untuk
# inferensi GPU"; a GEMM consuming decoded tiles, "Opini Hacker News")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,value", [(0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133), (0x8000, -0.0),
                                        (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127), (0x3E20, 0.15625)])
def test_bf16_values(bits, value):
    got = oracle.bf16_to_f64(np.array([bits], np.uint16))[0]
    assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value)


def _bf16_of_ints(v):
    """BF16 patterns of small integers (|v| < 256 is exact in 8 significant bits)."""
    return workloads.f32_to_bf16_bits(np.asarray(v, np.float32))


def test_linear_one_hot_tokens_pick_columns():
    """A token that is 1 at column c and 0 elsewhere yields column c of W:
    y[t, r] = W[r, c_t] exactly.  A transposed W, or rows and columns swapped
    in the reshape, picks the wrong entries."""
    rng = np.random.default_rng(0)
    out_f, in_f = 37, 24
    w = workloads.f32_to_bf16_bits(rng.standard_normal(out_f * in_f).astype(np.float32) * 0.02)
    s = oracle.encode(w)
    cols = [0, 5, 23, 11]
    x = np.zeros((len(cols), in_f), np.uint16)
    for t, c in enumerate(cols):
        x[t, c] = 0x3F80
    y = oracle.linear(s, x, out_f)
    assert y.shape == (len(cols), out_f)
    wv = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(out_f, in_f)
    for t, c in enumerate(cols):
        assert np.array_equal(y[t], wv[:, c])


def test_linear_small_integers_exact():
    """Integer weights and tokens: every product and partial sum is an
    integer far below 2^53, so y equals the integer dot products exactly,
    computed here with Python integers."""
    rng = np.random.default_rng(1)
    out_f, in_f, T = 9, 40, 3
    wi = rng.integers(-8, 9, (out_f, in_f))
    xi = rng.integers(-5, 6, (T, in_f))
    s = oracle.encode(_bf16_of_ints(wi.ravel()))
    y = oracle.linear(s, _bf16_of_ints(xi), out_f)
    for t in range(T):
        for r in range(out_f):
            assert y[t, r] == sum(int(xi[t, c]) * int(wi[r, c]) for c in range(in_f))


def test_linear_matches_exact_rational_sum():
    """Random BF16 weights and tokens of mixed magnitude: the float64 result
    lies within the float64 summation bound of the exact rational dot
    product (each BF16 value is a dyadic rational, so Fraction is exact)."""
    from fractions import Fraction
    rng = np.random.default_rng(2)
    out_f, in_f, T = 6, 64, 2
    w = workloads.f32_to_bf16_bits((rng.standard_normal(out_f * in_f) * np.exp(rng.uniform(-20, 5, out_f * in_f)))
                                   .astype(np.float32))
    x = workloads.f32_to_bf16_bits(rng.standard_normal(T * in_f).astype(np.float32)).reshape(T, in_f)
    s = oracle.encode(w)
    y = oracle.linear(s, x, out_f)

    def frac(bits):
        return Fraction((np.array([bits], np.uint16).astype(np.uint32) << 16).view(np.float32)[0].item())

    wf = [[frac(w[r * in_f + c]) for c in range(in_f)] for r in range(out_f)]
    xf = [[frac(x[t, c]) for c in range(in_f)] for t in range(T)]
    for t in range(T):
        for r in range(out_f):
            exact = sum(xf[t][c] * wf[r][c] for c in range(in_f))
            mag = sum(abs(xf[t][c] * wf[r][c]) for c in range(in_f))
            assert abs(Fraction(y[t, r]) - exact) <= Fraction(in_f) * Fraction(2) ** -53 * mag


def test_linear_rejects_partial_rows():
    s = oracle.encode(_bf16_of_ints(np.arange(10) % 7))
    with pytest.raises(ValueError):
        oracle.linear(s, np.zeros((1, 3), np.uint16), 3)


# ---------------------------------------------------------------------------
# rANS exponent coder ("Opini Hacker News" names rANS as the SIMD-friendlier
# coder; the format is the plain static rANS of asymmetric numeral systems
# with 16-bit renormalisation, laid out in 64-lane segments)
# ---------------------------------------------------------------------------

def _bf16_of_exponents(exps):
    return (np.asarray(exps, np.uint32) << 7).astype(np.uint16)


def _freq_table(pairs):
    f = np.zeros(256, np.uint32)
    for s, v in pairs.items():
        f[s] = v
    return f


def test_rans_hand_example_state_arithmetic():
    """M = 4 (2 probability bits), f(100) = 3 with c = 0, f(101) = 1 with
    c = 3; one lane, symbols 100, 101, 100 in decode order, so the encoder
    codes them last to first from x = L = 65536:
      100: 65536 = 3 * 21845 + 1   -> 21845 * 4 + 1 + 0 = 87381
      101: 87381 = 1 * 87381 + 0   -> 87381 * 4 + 0 + 3 = 349527
      100: 349527 = 3 * 116509 + 0 -> 116509 * 4 + 0 + 0 = 466036
    No state reaches f * 2^30, so no word is written."""
    freq = _freq_table({100: 3, 101: 1})
    w = _bf16_of_exponents([100, 101, 100])
    s = oracle.rans_encode(w, prob_bits=2, lanes=1, steps=3, freq=freq)
    assert s["states"].tolist() == [466036]
    assert s["words"].size == 0
    assert s["word_offsets"].tolist() == [0, 0]
    assert np.array_equal(oracle.rans_decode(s), w)


def test_rans_hand_example_renormalisation():
    """M = 4096, f(100) = 4095 (c = 0), f(101) = 1 (c = 4095); symbols 101,
    101.  The second-coded 101 (first decoded) finds x = 65536 * 4096 + 4095
    = 0x10000FFF >= 1 * 2^20, so the low 16 bits 0x0FFF = 4095 are written and
    x becomes 0x1000 = 4096; then x = 4096 * 4096 + 4095 = 16781311."""
    freq = _freq_table({100: 4095, 101: 1})
    w = _bf16_of_exponents([101, 101])
    s = oracle.rans_encode(w, prob_bits=12, lanes=1, steps=2, freq=freq)
    assert s["states"].tolist() == [16781311]
    assert s["words"].tolist() == [4095]
    assert np.array_equal(oracle.rans_decode(s), w)


def test_rans_hand_example_lanes_and_word_order():
    """Two lanes, three steps: lane 0 takes positions 0, 2, 4 and lane 1
    positions 1, 3, 5.  M = 4096, f(100) = 2048 (c 0), f(101) = 1 (c 2048),
    f(102) = 2047 (c 2049); positions 0..5 hold 101 101 101 101 100 102.
      lane 0, coding 100, 101, 101:  131072 -> 536872960 -> writes 2048, 33556480
      lane 1, coding 102, 101, 101:  133153 -> 545396736 -> writes 6144, 34088960
    At step 0 both lanes write; the decoder reads lane 0's word first, so the
    stored words are 2048, 6144."""
    freq = _freq_table({100: 2048, 101: 1, 102: 2047})
    w = _bf16_of_exponents([101, 101, 101, 101, 100, 102])
    s = oracle.rans_encode(w, prob_bits=12, lanes=2, steps=3, freq=freq)
    assert s["states"].tolist() == [33556480, 34088960]
    assert s["words"].tolist() == [2048, 6144]
    assert np.array_equal(oracle.rans_decode(s), w)


def test_rans_quantized_frequencies(workload):
    """Frequencies sum to M, every used exponent gets at least 1 and unused
    ones 0, and the quantized code costs within 1% of the entropy."""
    for name in ("single_1024x1024", "proj_4096x4096_outliers"):
        w = workload(name)
        hist = oracle.histogram(w)
        freq = oracle.rans_quantize(hist)
        assert int(freq.sum()) == 4096
        assert np.array_equal(freq > 0, hist > 0)
        used = hist > 0
        cost = float((hist[used] * np.log2(4096.0 / freq[used])).sum()) / w.size
        assert cost <= 1.01 * _entropy(hist)


@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers"])
def test_rans_roundtrip_and_size_bound(workload, name):
    """Lossless, and the words hold what the states shed: coding s takes x to
    within M of x * M / f[s], a word takes 16 bits out of x, and every state
    starts at 2^16, so 16 * words + sum of (log2 x_final - 16) equals the
    information sum of log2(M / f[s]) up to each step's rounding, log2(1 +
    f[s] / x) with x several thousand times f[s] for these streams (the test
    allows 0.5% of the total, plus 16 bits per state)."""
    w = workload(name)[:3_000_000]
    s = oracle.rans_encode(w)
    assert np.array_equal(oracle.rans_decode(s), w)
    e = (w >> 7) & 0xFF
    f = s["freq"][e].astype(np.float64)
    info = float(np.log2(4096.0 / f).sum())
    shed = float((np.log2(s["states"].astype(np.float64)) - 16.0).sum())
    assert abs(16 * s["words"].size + shed - info) <= 0.005 * info + 16 * s["states"].size


def test_rans_single_exponent_needs_no_words():
    """One exponent value: f = M, coding leaves every state at L, no words."""
    w = _bf16_of_exponents(np.full(70000, 120))
    s = oracle.rans_encode(w)
    assert s["words"].size == 0
    assert np.all(s["states"] == 65536)
    assert np.array_equal(oracle.rans_decode(s), w)


def test_rans_ragged_last_segment_and_empty():
    rng = np.random.default_rng(3)
    for n in (0, 1, 63, 64, 65, 32768, 32769, 100_003):
        w = workloads.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * 0.02)
        s = oracle.rans_encode(w)
        assert s["word_offsets"].size == (n + 32767) // 32768 + 1
        assert np.array_equal(oracle.rans_decode(s), w)


def test_rans_planted_mistakes_are_caught(workload):
    w = workload("single_1024x1024")[:200_000]
    s = oracle.rans_encode(w)
    # a changed word breaks the decode or its end check
    bad = dict(s)
    bad["words"] = s["words"].copy()
    bad["words"][10] ^= 0x0100
    try:
        assert not np.array_equal(oracle.rans_decode(bad), w)
    except oracle.OracleError:
        pass
    # a changed start state is caught by the end check (states must return to L)
    bad = dict(s)
    bad["states"] = s["states"].copy()
    bad["states"][5] += 1
    with pytest.raises(oracle.OracleError):
        oracle.rans_decode(bad)
    # swapped word offsets of two segments
    bad = dict(s)
    bad["word_offsets"] = s["word_offsets"].copy()
    bad["word_offsets"][1] += 1
    with pytest.raises(oracle.OracleError):
        oracle.rans_decode(bad)
