"""DF11 oracle: ctypes wrapper around the plain C reference in df11_oracle.c.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import this package.  It shares no code with
the HIP path (entropy_decoding_df11_amd) and imports nothing from it.

The C file follows the GeekNews page "DFloat11: Kompresi inferensi GPU
lossless yang mengecilkan LLM menjadi 70% ukurannya" step by step; see its
header for the sections and the readings of open points.
"""

from __future__ import annotations

import concurrent.futures
import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np

ORACLE_DIR = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(ORACLE_DIR, "df11_oracle.c")
LIB_PATH = os.path.join(ORACLE_DIR, "liboracle_df11.so")

ERRORS = {
    -1: "ORC_E_INVALID_ARG",
    -2: "ORC_E_RESERVED_EXPONENT",
    -3: "ORC_E_CODE_TOO_LONG",
    -4: "ORC_E_TOO_MANY_LUTS",
    -5: "ORC_E_BUFFER_TOO_SMALL",
    -6: "ORC_E_BAD_STREAM",
    -7: "ORC_E_TOO_LARGE",
}
MAX_LUTS = 17


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"oracle {what}: {ERRORS.get(code, code)}")


def build(verbose: bool = False) -> str:
    """Compile df11_oracle.c with gcc into liboracle_df11.so."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", LIB_PATH + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{res.stdout}\n{res.stderr}")
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_LIB = None


def load() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
            build()
        _LIB = ctypes.CDLL(LIB_PATH)
        for fn in ("orc_split", "orc_merge", "orc_histogram", "orc_code_lengths", "orc_canonical_codes",
                   "orc_build_luts", "orc_layout", "orc_encode", "orc_decode_treewalk",
                   "orc_decode_groups_treewalk", "orc_decode_lut", "orc_check_metadata", "orc_rans_quantize",
                   "orc_rans_encode", "orc_rans_decode"):
            getattr(_LIB, fn).restype = ctypes.c_int
        _LIB.orc_total_bits.restype = ctypes.c_uint64
    return _LIB


def _p(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(rc, what)


def split(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    w = np.ascontiguousarray(w, dtype=np.uint16)
    e = np.empty(w.size, np.uint8)
    sm = np.empty(w.size, np.uint8)
    _check(load().orc_split(_p(w), ctypes.c_uint64(w.size), _p(e), _p(sm)), "split")
    return e, sm


def merge(e: np.ndarray, sm: np.ndarray) -> np.ndarray:
    e = np.ascontiguousarray(e, dtype=np.uint8)
    sm = np.ascontiguousarray(sm, dtype=np.uint8)
    w = np.empty(e.size, np.uint16)
    _check(load().orc_merge(_p(e), _p(sm), ctypes.c_uint64(e.size), _p(w)), "merge")
    return w


def histogram(w: np.ndarray, hist: Optional[np.ndarray] = None) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.uint16)
    if hist is None:
        hist = np.zeros(256, np.uint64)
    _check(load().orc_histogram(_p(w), ctypes.c_uint64(w.size), _p(hist)), "histogram")
    return hist


def code_lengths(hist: np.ndarray) -> np.ndarray:
    hist = np.ascontiguousarray(hist, dtype=np.uint64)
    lens = np.zeros(256, np.uint8)
    _check(load().orc_code_lengths(_p(hist), _p(lens)), "code_lengths")
    return lens


def canonical_codes(lens: np.ndarray) -> np.ndarray:
    lens = np.ascontiguousarray(lens, dtype=np.uint8)
    codes = np.zeros(256, np.uint32)
    _check(load().orc_canonical_codes(_p(lens), _p(codes)), "canonical_codes")
    return codes


def build_luts(lens: np.ndarray, codes: np.ndarray) -> np.ndarray:
    lens = np.ascontiguousarray(lens, dtype=np.uint8)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    luts = np.zeros((MAX_LUTS, 256), np.uint8)
    k = ctypes.c_uint32(0)
    _check(load().orc_build_luts(_p(lens), _p(codes), _p(luts), ctypes.byref(k)), "build_luts")
    return luts[: k.value].copy()


def total_bits(lens: np.ndarray, hist: np.ndarray) -> int:
    lens = np.ascontiguousarray(lens, dtype=np.uint8)
    hist = np.ascontiguousarray(hist, dtype=np.uint64)
    return int(load().orc_total_bits(_p(lens), _p(hist)))


def layout(n_elements: int, bits: int, n: int = 8, G: int = 256) -> Dict[str, int]:
    sizes = np.zeros(6, np.uint64)
    _check(load().orc_layout(ctypes.c_uint64(n_elements), ctypes.c_uint64(bits), ctypes.c_uint32(n),
                             ctypes.c_uint32(G), _p(sizes)), "layout")
    keys = ["n_threads", "n_groups", "enc_bytes", "sm_bytes", "gaps_bytes", "out_pos_bytes"]
    return {k: int(v) for k, v in zip(keys, sizes)}


def codebook(hist: np.ndarray) -> Dict[str, np.ndarray]:
    lens = code_lengths(hist)
    codes = canonical_codes(lens)
    luts = build_luts(lens, codes)
    return {"code_lengths": lens, "codes": codes, "luts": luts, "n_luts": luts.shape[0],
            "max_len": int(lens.max())}


def encode(w: np.ndarray, n: int = 8, G: int = 256, cb: Optional[Dict] = None) -> Dict:
    """Encode with the oracle.  Returns the codebook, the padded buffers and
    the header fields."""
    w = np.ascontiguousarray(w, dtype=np.uint16).reshape(-1)
    hist = histogram(w)
    if cb is None:
        cb = codebook(hist)
    bits = total_bits(cb["code_lengths"], hist)
    sz = layout(w.size, bits, n, G)
    enc = np.zeros(sz["enc_bytes"], np.uint8)
    sm = np.zeros(sz["sm_bytes"], np.uint8)
    gaps = np.zeros(sz["gaps_bytes"], np.uint8)
    out_pos = np.zeros(sz["n_groups"] + 1, np.uint32)
    tb = ctypes.c_uint64(0)
    _check(load().orc_encode(_p(w), ctypes.c_uint64(w.size), _p(cb["code_lengths"]), _p(cb["codes"]),
                             ctypes.c_uint32(n), ctypes.c_uint32(G), _p(enc), _p(sm), _p(gaps), _p(out_pos),
                             ctypes.byref(tb)), "encode")
    assert tb.value == bits
    out = dict(cb)
    out.update(sz)
    max_group = int(np.max(np.diff(out_pos.astype(np.int64)))) if sz["n_groups"] else 0
    out.update({"enc": enc, "sm": sm, "gaps": gaps, "out_pos": out_pos, "total_bits": bits,
                "n_elements": w.size, "n": n, "G": G, "hist": hist, "max_group_elems": max_group})
    return out


def decode_treewalk(s: Dict) -> np.ndarray:
    w = np.empty(s["n_elements"], np.uint16)
    _check(load().orc_decode_treewalk(_p(s["code_lengths"]), _p(s["codes"]), _p(s["enc"]),
                                      ctypes.c_uint64(s["total_bits"]), _p(s["sm"]),
                                      ctypes.c_uint64(s["n_elements"]), _p(w)), "decode_treewalk")
    return w


def decode_groups(s: Dict, g0: int, g1: int, out: np.ndarray) -> None:
    """Tree-walk decode of groups [g0, g1) into out (the full-size output)."""
    _check(load().orc_decode_groups_treewalk(
        _p(s["code_lengths"]), _p(s["codes"]), _p(s["enc"]), ctypes.c_uint64(s["total_bits"]), _p(s["gaps"]),
        _p(s["out_pos"]), _p(s["sm"]), ctypes.c_uint32(s["n"]), ctypes.c_uint32(s["G"]),
        ctypes.c_uint64(s["n_threads"]), ctypes.c_uint64(g0), ctypes.c_uint64(g1), _p(out)), "decode_groups")


def decode_groups_parallel(s: Dict, g0: int, g1: int, out: np.ndarray, threads: int) -> None:
    """Groups are independent, so [g0, g1) is split over host threads (ctypes
    releases the GIL during each call)."""
    threads = max(1, threads)
    bounds = np.linspace(g0, g1, threads + 1).astype(np.int64)
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        futs = [ex.submit(decode_groups, s, int(a), int(b), out) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        for f in futs:
            f.result()


def decode_lut(s: Dict) -> np.ndarray:
    luts = np.zeros((MAX_LUTS, 256), np.uint8)
    luts[: s["luts"].shape[0]] = s["luts"]
    w = np.empty(s["n_elements"], np.uint16)
    _check(load().orc_decode_lut(_p(luts), ctypes.c_uint32(s["luts"].shape[0]), _p(s["code_lengths"]),
                                 _p(s["enc"]), ctypes.c_uint64(s["total_bits"]), _p(s["sm"]),
                                 ctypes.c_uint64(s["n_elements"]), _p(w)), "decode_lut")
    return w


def check_metadata(s: Dict) -> np.ndarray:
    """Re-walk every thread's codes; returns the per-thread counts."""
    counts = np.zeros(max(1, s["n_threads"]), np.uint32)
    _check(load().orc_check_metadata(_p(s["code_lengths"]), _p(s["codes"]), _p(s["enc"]),
                                     ctypes.c_uint64(s["total_bits"]), _p(s["gaps"]), _p(s["out_pos"]),
                                     ctypes.c_uint64(s["n_elements"]), ctypes.c_uint32(s["n"]),
                                     ctypes.c_uint32(s["G"]), ctypes.c_uint64(s["n_threads"]), _p(counts)),
           "check_metadata")
    return counts[: s["n_threads"]]


def gap_values(s: Dict) -> np.ndarray:
    """Unpack the 5-bit MSB-first gaps (test helper)."""
    bits = np.unpackbits(s["gaps"])[: 5 * s["n_threads"]].reshape(-1, 5).astype(np.uint32)
    return (bits * np.array([16, 8, 4, 2, 1], np.uint32)).sum(axis=1) if s["n_threads"] else np.zeros(0, np.uint32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Values of BF16 bit patterns: a BF16 is the upper 16 bits of an IEEE
    binary32 word, so widening it to float32 and then float64 is exact."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def linear(s: Dict, x: np.ndarray, out_features: int) -> np.ndarray:
    """y = x W^T in float64, W being the stream decoded (tree walk) and viewed
    as an out_features x in_features row-major matrix, x an n_tokens x
    in_features matrix of BF16 patterns.

    The page's section "Dekompresi yang disesuaikan untuk inferensi GPU" uses
    each decompressed weight matrix in a matrix multiplication; the section
    "Opini Hacker News" suggests decompressing inside the GEMM.  The oracle
    keeps the two steps apart: decode the whole matrix, then one float64
    matmul (each BF16 x BF16 product is exact in float64)."""
    w = decode_treewalk(s)
    if out_features <= 0 or w.size % out_features:
        raise ValueError("the stream does not hold out_features whole rows")
    in_features = w.size // out_features
    wm = bf16_to_f64(w).reshape(out_features, in_features)
    xm = bf16_to_f64(np.asarray(x)).reshape(-1, in_features)
    return xm @ wm.T


# rANS exponent coder (see the rANS section of df11_oracle.c for the format):
# 12-bit probabilities, 64 lanes, 512 steps per segment.
RANS_PROB_BITS = 12
RANS_LANES = 64
RANS_STEPS = 512


def rans_quantize(hist: np.ndarray, prob_bits: int = RANS_PROB_BITS) -> np.ndarray:
    """Frequencies summing to 2^prob_bits for the exponent histogram."""
    hist = np.ascontiguousarray(hist, dtype=np.uint64)
    freq = np.zeros(256, np.uint32)
    _check(load().orc_rans_quantize(_p(hist), ctypes.c_uint32(prob_bits), _p(freq)), "rans_quantize")
    return freq


def rans_encode(w: np.ndarray, prob_bits: int = RANS_PROB_BITS, lanes: int = RANS_LANES, steps: int = RANS_STEPS,
                freq: Optional[np.ndarray] = None) -> Dict:
    """rANS-code the exponents of BF16 words w; sign/mantissa bytes as in DF11."""
    w = np.ascontiguousarray(w, dtype=np.uint16).reshape(-1)
    if freq is None:
        freq = rans_quantize(histogram(w), prob_bits)
    freq = np.ascontiguousarray(freq, dtype=np.uint32)
    seg = lanes * steps
    n_seg = (w.size + seg - 1) // seg
    states = np.zeros(max(n_seg * lanes, 1), np.uint32)
    offsets = np.zeros(n_seg + 1, np.uint64)
    words = np.zeros(max(w.size, 1), np.uint16)
    n_words = ctypes.c_uint64(0)
    sm = np.zeros(max(w.size, 1), np.uint8)
    _check(load().orc_rans_encode(_p(w), ctypes.c_uint64(w.size), ctypes.c_uint32(prob_bits), _p(freq),
                                  ctypes.c_uint32(lanes), ctypes.c_uint32(steps), _p(states), _p(offsets), _p(words),
                                  ctypes.c_uint64(words.size), ctypes.byref(n_words), _p(sm)), "rans_encode")
    return {"freq": freq, "prob_bits": prob_bits, "lanes": lanes, "steps": steps, "n_elements": w.size,
            "states": states[:n_seg * lanes], "word_offsets": offsets, "words": words[:n_words.value].copy(),
            "sm": sm[:w.size]}


def rans_decode(s: Dict) -> np.ndarray:
    w = np.empty(s["n_elements"], np.uint16)
    states = np.ascontiguousarray(s["states"], dtype=np.uint32)
    offsets = np.ascontiguousarray(s["word_offsets"], dtype=np.uint64)
    words = np.ascontiguousarray(s["words"], dtype=np.uint16)
    sm = np.ascontiguousarray(s["sm"], dtype=np.uint8)
    keep = (states if states.size else np.zeros(1, np.uint32), words if words.size else np.zeros(1, np.uint16),
            sm if sm.size else np.zeros(1, np.uint8))
    _check(load().orc_rans_decode(_p(np.ascontiguousarray(s["freq"], dtype=np.uint32)), ctypes.c_uint32(s["prob_bits"]),
                                  ctypes.c_uint32(s["lanes"]), ctypes.c_uint32(s["steps"]), _p(keep[0]), _p(offsets),
                                  _p(keep[1]), _p(keep[2]), ctypes.c_uint64(s["n_elements"]),
                                  _p(w if w.size else np.zeros(1, np.uint16))), "rans_decode")
    return w


def rans_compressed_bytes(s: Dict) -> int:
    """Bytes of the rANS stream: frequencies (2 bytes each), start states,
    word offsets (4 bytes each), words and sign/mantissa bytes."""
    return 2 * 256 + 4 * s["states"].size + 4 * s["word_offsets"].size + 2 * s["words"].size + s["sm"].size
