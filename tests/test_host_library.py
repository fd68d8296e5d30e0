"""Host side of libdf11.so against the oracle, and the C ABI surface.

These run without a GPU: the encoder and codebook builder are host code, and
df11_decompress validates its arguments before any HIP call.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from entropy_decoding_df11_amd import _lib, df11, workloads

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libdf11.so not built")
    return _lib.load()


def _assert_same_stream(host, ref):
    cb = df11.codebook_arrays(host.codebook)
    assert np.array_equal(cb["code_lengths"], ref["code_lengths"])
    assert np.array_equal(cb["codes"], ref["codes"])
    assert np.array_equal(cb["luts"], ref["luts"])
    assert cb["n_luts"] == ref["n_luts"] and cb["max_len"] == ref["max_len"]
    for k in ("enc", "sm", "gaps", "out_pos"):
        assert np.array_equal(getattr(host, k), ref[k]), k
    h = host.header_dict()
    for k in ("n_threads", "n_groups", "enc_bytes", "sm_bytes", "gaps_bytes", "total_bits", "n_elements",
              "max_group_elems"):
        assert h[k] == ref[k], k
    assert h["out_pos_bytes"] == 4 * (ref["n_groups"] + 1)


def test_header_exports_match_library():
    lib = _lib_or_skip()
    with open(os.path.join(REPO, "include", "df11.h")) as f:
        text = f.read()
    declared = sorted(set(re.findall(r"\b(df11_[a-z_]+)\s*\(", text)))
    assert declared == sorted(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.df11_status_str(-3) == b"DF11_E_CODE_TOO_LONG"
    assert lib.df11_status_str(0) == b"DF11_OK"


def test_header_structs_match_binding_sizes():
    # the binding's structs mirror the header: check sizes/offsets with a tiny C probe compiled by gcc
    import subprocess
    import tempfile
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "df11.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(df11_codebook), sizeof(df11_layout), sizeof(df11_header),
         sizeof(df11_device_stream), offsetof(df11_device_stream, enc), offsetof(df11_device_stream, decode_table_bits),
         offsetof(df11_header, max_group_elems), sizeof(df11_rans_header), sizeof(df11_rans_device_stream),
         offsetof(df11_rans_device_stream, table), offsetof(df11_rans_header, prob_bits));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        with open(c, "w") as f:
            f.write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(REPO, "include"), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(_lib.Codebook), ctypes.sizeof(_lib.Layout), ctypes.sizeof(_lib.Header),
            ctypes.sizeof(_lib.DeviceStream), _lib.DeviceStream.enc.offset, _lib.DeviceStream.decode_table_bits.offset,
            _lib.Header.max_group_elems.offset, ctypes.sizeof(_lib.RansHeader), ctypes.sizeof(_lib.RansDeviceStream),
            _lib.RansDeviceStream.table.offset, _lib.RansHeader.prob_bits.offset]
    assert got == want


@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers"])
def test_library_encoder_matches_oracle_bytes(workload, name):
    _lib_or_skip()
    w = workload(name)
    _assert_same_stream(df11.encode(w), oracle.encode(w))


@pytest.mark.parametrize("seed", range(12))
def test_library_encoder_matches_oracle_random(seed):
    _lib_or_skip()
    rng = np.random.default_rng(500 + seed)
    size = int(rng.choice([0, 1, 2, 3, 63, 64, 65, 1000, 4097, 33333]))
    n = int(rng.choice([4, 5, 8, 12, 16]))
    G = int(rng.choice([64, 128, 256]))
    kind = seed % 4
    if kind == 0:
        w = workloads.f32_to_bf16_bits(rng.standard_normal(size) * 0.02)
    elif kind == 1:
        w = rng.integers(0, 65536, size * 2).astype(np.uint16)
        w = w[((w >> 7) & 0xFF) < 240][:size]
    elif kind == 2:
        w = np.full(size, 0x3F80 if seed % 2 else 0x0000, np.uint16)
    else:
        p = np.array([2.0 ** -min(k, 30) for k in range(1, 32)])
        e = rng.choice(np.arange(100, 131), size, p=p / p.sum())
        w = workloads.f32_to_bf16_bits(np.ldexp(1.0, e - 127))
    _assert_same_stream(df11.encode(w, bytes_per_thread=n, threads_per_group=G), oracle.encode(w, n=n, G=G))


@pytest.mark.parametrize("seed", range(40))
def test_library_codebook_matches_oracle_on_random_histograms(seed):
    _lib_or_skip()
    rng = np.random.default_rng(seed)
    hist = np.zeros(256, np.uint64)
    k = int(rng.integers(1, 240))
    syms = rng.choice(240, k, replace=False)
    style = seed % 3
    if style == 0:
        hist[syms] = rng.integers(1, 1000, k)
    elif style == 1:
        hist[syms] = np.round(1e12 * rng.power(0.2, k) ** 8).astype(np.uint64) + 1
    else:
        hist[syms] = rng.zipf(1.3, k).astype(np.uint64)
    try:
        ref = oracle.codebook(hist)
    except oracle.OracleError as e:
        with pytest.raises(_lib.Df11Error) as ei:
            df11.build_codebook(hist)
        assert ei.value.status == e.code
        return
    cb = df11.codebook_arrays(df11.build_codebook(hist))
    for key in ("code_lengths", "codes", "luts", "n_luts", "max_len"):
        assert np.array_equal(cb[key], ref[key]), key


def _fib(n):
    f = [1, 1]
    while len(f) < n:
        f.append(f[-1] + f[-2])
    return f[:n]


def test_library_error_paths():
    _lib_or_skip()
    # reserved exponent
    with pytest.raises(_lib.Df11Error) as ei:
        df11.histogram(np.array([0x3F80, 0x7F80], np.uint16))
    assert ei.value.status == -2
    # code longer than 32 bits
    hist = np.zeros(256, np.uint64)
    hist[60:94] = _fib(34)
    with pytest.raises(_lib.Df11Error) as ei:
        df11.build_codebook(hist)
    assert ei.value.status == -3
    # more than 16 lower LUTs (17 internal nodes at depth 8)
    hist = np.zeros(256, np.uint64)
    hist[:240] = [4] * 33 + [2] * 173 + [1] * 34
    with pytest.raises(_lib.Df11Error) as ei:
        df11.build_codebook(hist)
    assert ei.value.status == -4
    # bad layouts
    w = np.array([0x3F80] * 10, np.uint16)
    for n, G in ((3, 256), (8, 100), (8, 0)):
        with pytest.raises(_lib.Df11Error) as ei:
            df11.encode(w, bytes_per_thread=n, threads_per_group=G)
        assert ei.value.status == -1
    # an exponent missing from the codebook
    cb = df11.build_codebook(df11.histogram(np.array([0x3F80, 0x3F00], np.uint16)))
    with pytest.raises(_lib.Df11Error) as ei:
        df11.encode(np.array([0x4000], np.uint16), codebook=cb)
    assert ei.value.status == -1
    # decode table sizes
    lib = _lib.load()
    assert lib.df11_decode_table_bytes(9) == 0 and lib.df11_decode_table_bytes(13) == 0
    assert lib.df11_decode_table_bytes(12) == 10 << 12
    buf = np.zeros(10, np.uint32)
    assert lib.df11_build_decode_table(ctypes.byref(cb), 12, buf.ctypes.data_as(ctypes.c_void_p), 40) == -5


def _fake_device_stream(host):
    """A device-stream struct whose pointers are never dereferenced (validation only)."""
    s = _lib.DeviceStream()
    s.h = host.header
    addr = 1 << 40
    for name in ("enc", "sm", "gaps", "out_pos", "luts", "code_lengths", "decode_table"):
        setattr(s, name, addr)
        addr += 1 << 32
    s.decode_table_bits = 12
    return s


def test_decompress_validation_runs_before_any_launch():
    lib = _lib_or_skip()
    host = df11.encode(workloads.gen_single_matrix(rows=64, cols=64))
    out = ctypes.c_void_p(1 << 48)
    # null stream struct
    assert lib.df11_decompress(None, out, None) == -1
    s = _fake_device_stream(host)
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.bytes_per_thread = 4
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -1
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.enc_bytes += 16
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -6
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.n_luts = 18
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -6
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.decode_table_bits = 9
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -1
    # without a decode table (the kernel derives it), the width must still be 10..12, or 0
    bad.decode_table = None
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -1
    bad.decode_table_bits = 13
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -1
    bad.decode_table_bits = 0
    bad.h.enc_bytes += 16  # (a later check still fails: nothing is launched)
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -6
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.sm = (1 << 40) + 8  # misaligned
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -1
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.n_elements = 1 << 32
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -7
    bad.h.n_elements = _lib.MAX_ELEMENTS + 1
    assert lib.df11_decompress(ctypes.byref(bad), out, None) == -7
    # output aliasing an input
    assert lib.df11_decompress(ctypes.byref(s), ctypes.c_void_p(s.sm), None) == -1
    # misaligned output
    assert lib.df11_decompress(ctypes.byref(s), ctypes.c_void_p((1 << 48) + 2), None) == -1
    # scratch too small for the block entry point
    assert lib.df11_decompress_block(ctypes.byref(s), out, host.n_elements - 1, None) == -5
    # an empty stream is a valid no-op that launches nothing
    empty = df11.encode(np.zeros(0, np.uint16))
    es = _lib.DeviceStream()
    es.h = empty.header
    assert lib.df11_decompress(ctypes.byref(es), None, None) == 0


def _greedy_window(lens, codes, x, bits, max_syms):
    """The complete codes at the start of a bits-wide window (brute force over the code table)."""
    syms, starts, used = [], [], 0
    while len(syms) < max_syms:
        found = None
        for s in range(256):
            l = int(lens[s])
            if l and used + l <= bits and ((x >> (bits - used - l)) & ((1 << l) - 1)) == int(codes[s]):
                found = (s, l)
                break
        if found is None:
            break
        syms.append(found[0])
        starts.append(used)
        used += found[1]
    return syms, starts, used


@pytest.mark.parametrize("bits", [10, 12])
@pytest.mark.parametrize("case", ["single_1024x1024", "stress"])
def test_decode_table_matches_code_table(workload, bits, case):
    _lib_or_skip()
    w = workload("single_1024x1024") if case == "single_1024x1024" else workloads.gen_stress(n=1 << 20)
    ref = oracle.codebook(oracle.histogram(w))
    cb = df11.build_codebook(df11.histogram(w))
    table = df11.decode_table(cb, bits)
    size = 1 << bits
    assert table.nbytes == 10 * size
    lo, aux = table[0:2 * size:2], table[1:2 * size:2]
    starts_mask = table[2 * size:].view(np.uint16)
    rot = lambda e: ((e >> 1) | (e << 7)) & 0xFF
    for x in range(size):
        syms, starts, used = _greedy_window(ref["code_lengths"], ref["codes"], x, bits, 5)
        a = int(aux[x])
        if not syms:
            # long first code: only the position field moves (by 128), and the
            # code starts at offset 0
            assert int(lo[x]) == 0 and a == 0x80 and int(starts_mask[x]) == 1
            assert ref["luts"][0][x >> (bits - 8)] >= 240
            continue
        assert a & 0xFFFF == (len(syms) << 11) + used
        assert int(starts_mask[x]) == sum(1 << s for s in starts)
        assert a >> 24 == 0
        got = [(int(lo[x]) >> (8 * j)) & 0xFF for j in range(4)] + [(a >> 16) & 0xFF]
        assert got == [rot(s) for s in syms] + [0] * (5 - len(syms))


def test_schedule_words_constant_matches_header():
    import re
    with open(os.path.join(os.path.dirname(__file__), "..", "include", "df11.h")) as f:
        m = re.search(r"#define\s+DF11_SCHEDULE_WORDS\s+(\d+)", f.read())
    assert m and int(m.group(1)) == _lib.SCHEDULE_WORDS


def test_decompress_batch_validation_runs_before_any_launch():
    """Every batch error is found before anything is launched (no GPU here)."""
    lib = _lib_or_skip()
    host = df11.encode(workloads.gen_single_matrix(rows=64, cols=64))
    s = _fake_device_stream(host)
    n = host.header.n_elements

    def call(streams, outs):
        arr = (_lib.DeviceStream * max(len(streams), 1))(*streams)
        ptrs = (ctypes.c_void_p * max(len(outs), 1))(*outs)
        return lib.df11_decompress_batch(arr, len(streams), ptrs, None)

    assert lib.df11_decompress_batch(None, 0, None, None) == 0  # empty batch
    assert lib.df11_decompress_batch(None, 1, None, None) == -1
    # more streams than one launch takes
    assert call([s] * (_lib.MAX_BATCH + 1), [1 << 48] * (_lib.MAX_BATCH + 1)) == -7
    # a stream whose header is inconsistent
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.enc_bytes += 16
    assert call([s, bad], [1 << 48, (1 << 48) + (1 << 32)]) == -6
    # different decode-table widths in one batch
    other = _lib.DeviceStream.from_buffer_copy(s)
    other.decode_table_bits = 11
    assert call([s, other], [1 << 48, (1 << 48) + (1 << 32)]) == -1
    # outputs that overlap each other, or another stream's input
    assert call([s, s], [1 << 48, (1 << 48) + 2 * (n // 2) // 16 * 16]) == -1
    assert call([s, s], [1 << 48, s.enc]) == -1
    # misaligned output
    assert call([s], [(1 << 48) + 8]) == -1
    # the timed entry point validates the same way
    assert lib.df11_decompress_batch_timed(None, 0, None, None, None, None) == 0
    assert lib.df11_decompress_batch_timed(None, 1, None, None, None, None) == -1
    arr = (_lib.DeviceStream * 2)(s, bad)
    ptrs = (ctypes.c_void_p * 2)(1 << 48, (1 << 48) + (1 << 32))
    assert lib.df11_decompress_batch_timed(arr, 2, ptrs, None, None, None) == -6


def test_linear_constants_match_header():
    import re
    with open(os.path.join(os.path.dirname(__file__), "..", "include", "df11.h")) as f:
        text = f.read()
    assert int(re.search(r"#define\s+DF11_LINEAR_MAX_TOKENS\s+(\d+)", text).group(1)) == _lib.LINEAR_MAX_TOKENS
    assert int(re.search(r"#define\s+DF11_LINEAR_MIN_IN_FEATURES\s+(\d+)", text).group(1)) == \
        _lib.LINEAR_MIN_IN_FEATURES


def test_linear_validation_runs_before_any_launch():
    """Every df11_linear argument error is found before anything is launched
    (no GPU here)."""
    lib = _lib_or_skip()
    host = df11.encode(workloads.gen_single_matrix(rows=64, cols=1024))
    s = _fake_device_stream(host)
    x, y = ctypes.c_void_p(1 << 48), ctypes.c_void_p((1 << 48) + (1 << 32))

    def call(st, xp, t, i, o, yp):
        return lib.df11_linear(ctypes.byref(st) if st is not None else None, xp, t, i, o, yp, None)

    assert call(None, x, 1, 1024, 64, y) == -1
    assert call(s, x, 0, 1024, 64, y) == -1                        # no tokens
    assert call(s, x, _lib.LINEAR_MAX_TOKENS + 1, 1024, 64, y) == -1
    assert call(s, x, 1, 1024, 63, y) == -1                        # out * in != N
    assert call(s, x, 1, 256, 256, y) == -1                        # rows shorter than the minimum
    big = _fake_device_stream(df11.encode(workloads.gen_single_matrix(rows=64, cols=1028)))
    assert call(big, x, 1, 1028, 64, y) == -1                      # in_features not a multiple of 8
    assert call(s, ctypes.c_void_p((1 << 48) + 8), 1, 1024, 64, y) == -1   # x misaligned
    assert call(s, x, 1, 1024, 64, ctypes.c_void_p((1 << 48) + (1 << 32) + 2)) == -1  # y misaligned
    assert call(s, x, 2, 1024, 64, ctypes.c_void_p((1 << 48) + 16)) == -1  # y overlaps x
    assert call(s, x, 1, 1024, 64, ctypes.c_void_p(s.sm)) == -1    # y overlaps the stream
    assert call(s, None, 1, 1024, 64, y) == -1
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.enc_bytes += 16
    assert call(bad, x, 1, 1024, 64, y) == -6
    # an empty stream (no rows) launches nothing
    empty = df11.encode(np.zeros(0, np.uint16))
    es = _lib.DeviceStream()
    es.h = empty.header
    assert lib.df11_linear(ctypes.byref(es), None, 1, 1024, 0, None, None) == 0
    # the accumulating entry points validate the same way
    assert lib.df11_linear_acc(ctypes.byref(s), x, 0, 1024, 64, y, None) == -1
    assert lib.df11_linear_acc(ctypes.byref(s), x, 1, 1024, 64, ctypes.c_void_p(s.sm), None) == -1
    assert lib.df11_linear_acc(ctypes.byref(bad), x, 1, 1024, 64, y, None) == -6
    arr = (_lib.DeviceStream * 1)(bad)
    ys = (ctypes.c_void_p * 1)(y)
    rows = np.array([64], np.uint32)
    assert lib.df11_linear_batch_acc(arr, 1, x, 1, 1024, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                     ys, None, None, None) == -6


# ---------------------------------------------------------------------------
# rANS coder: the library's encoder against the oracle's, byte for byte
# ---------------------------------------------------------------------------

def test_rans_constants_match_header():
    import re
    with open(os.path.join(os.path.dirname(__file__), "..", "include", "df11.h")) as f:
        text = f.read()
    for name, val in (("PROB_BITS", _lib.RANS_PROB_BITS), ("LANES", _lib.RANS_LANES), ("STEPS", _lib.RANS_STEPS),
                      ("TABLE_ENTRIES", _lib.RANS_TABLE_ENTRIES)):
        assert int(re.search(r"#define\s+DF11_RANS_%s\s+(\d+)" % name, text).group(1)) == val
    assert oracle.RANS_PROB_BITS == _lib.RANS_PROB_BITS and oracle.RANS_LANES == _lib.RANS_LANES
    assert oracle.RANS_STEPS == _lib.RANS_STEPS


def _rans_equal(w):
    h = df11.rans_encode(w)
    o = oracle.rans_encode(w)
    assert np.array_equal(h.freq, o["freq"])
    assert np.array_equal(h.states, o["states"])
    assert np.array_equal(h.word_offsets, o["word_offsets"].astype(np.uint32))
    assert np.array_equal(h.words, o["words"])
    assert np.array_equal(h.sm, o["sm"])
    assert h.compressed_bytes() == oracle.rans_compressed_bytes(o)
    assert int(h.header.n_words) == o["words"].size
    return h


@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers"])
def test_rans_encoder_matches_oracle_bytes(workload, name):
    w = workload(name)[:5_000_000]
    h = _rans_equal(w)
    assert 8 * h.compressed_bytes() / w.size < 10.75  # below DF11's ~10.8 bits per weight here


@pytest.mark.parametrize("n", [0, 1, 7, 64, 65, 32767, 32768, 32769, 100_003])
def test_rans_encoder_matches_oracle_ragged(n):
    rng = np.random.default_rng(n)
    _rans_equal(workloads.f32_to_bf16_bits(rng.standard_normal(n) * 0.02))


def test_rans_encoder_matches_oracle_special_streams():
    _rans_equal(np.full(70_000, 120 << 7, np.uint16))           # one exponent: no words
    _rans_equal(workloads.gen_stress(seed=4, n=300_000))        # 29-30-bit Huffman codes
    _rans_equal(workloads.gen_stress(seed=4, n=300_000, kind="literal"))


@pytest.mark.parametrize("seed", range(6))
def test_rans_quantize_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    hist = np.zeros(256, np.uint64)
    used = rng.choice(240, size=int(rng.integers(1, 240)), replace=False)
    hist[used] = rng.integers(1, 10 ** int(rng.integers(1, 9)), used.size)
    assert np.array_equal(df11.rans_quantize(hist), oracle.rans_quantize(hist))


def test_rans_slot_table_matches_definition():
    """Entry k: rotated exponent of the slot's symbol, f - 1, k - c."""
    w = workloads.gen_stress(seed=4, n=200_000)
    freq = df11.rans_quantize(df11.histogram(w))
    table = df11.rans_table(freq)
    cum = np.concatenate([[0], np.cumsum(freq)]).astype(np.int64)
    for k in range(0, 4096, 7):
        s = int(np.searchsorted(cum, k, side="right") - 1)
        assert cum[s] <= k < cum[s + 1]
        e = int(table[k])
        assert e & 0xFF == ((s >> 1) | ((s & 1) << 7)) & 0xFF
        assert (e >> 8) & 0xFFF == freq[s] - 1
        assert e >> 20 == k - cum[s]


def test_rans_errors():
    lib = _lib_or_skip()
    hist = np.zeros(256, np.uint64)
    hist[245] = 3
    freq = np.zeros(256, np.uint32)
    assert lib.df11_rans_quantize(hist.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                  freq.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))) == -2
    bad = np.zeros(256, np.uint32)
    bad[100] = 4095  # does not sum to 4096
    table = np.zeros(4096, np.uint32)
    assert lib.df11_rans_build_table(bad.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                     table.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))) == -1


def test_rans_decompress_validation_runs_before_any_launch():
    """Every df11_rans_decompress argument error is found before a launch (no GPU here)."""
    lib = _lib_or_skip()
    host = df11.rans_encode(workloads.gen_single_matrix(rows=64, cols=1024))
    s = _lib.RansDeviceStream()
    s.h = host.header
    addr = 1 << 40
    for name in ("table", "states", "word_offsets", "words", "sm"):
        setattr(s, name, addr)
        addr += 1 << 32
    out = ctypes.c_void_p(1 << 48)

    def call(st, o=out):
        return lib.df11_rans_decompress(ctypes.byref(st), o, None)

    assert lib.df11_rans_decompress(None, out, None) == -1
    for field, val, rc in (("prob_bits", 11, -1), ("lanes", 32, -1), ("steps", 256, -1), ("n_segments", 5, -6)):
        bad = _lib.RansDeviceStream.from_buffer_copy(s)
        setattr(bad.h, field, val)
        assert call(bad) == rc, field
    bad = _lib.RansDeviceStream.from_buffer_copy(s)
    bad.h.n_words = bad.h.n_elements + 1
    assert call(bad) == -6
    bad = _lib.RansDeviceStream.from_buffer_copy(s)
    bad.h.n_elements = 1 << 32
    assert call(bad) == -7
    bad.h.n_elements = _lib.MAX_ELEMENTS + 1
    assert call(bad) == -7
    bad = _lib.RansDeviceStream.from_buffer_copy(s)
    bad.words = (1 << 40) + 8  # not 16-byte aligned
    assert call(bad) == -1
    assert call(s, ctypes.c_void_p((1 << 48) + 8)) == -1       # misaligned output
    assert call(s, ctypes.c_void_p(s.sm)) == -1                # output over the stream
    bad = _lib.RansDeviceStream.from_buffer_copy(s)
    bad.table = None
    assert call(bad) == -1
    empty = _lib.RansDeviceStream()
    empty.h = df11.rans_encode(np.zeros(0, np.uint16)).header
    assert lib.df11_rans_decompress(ctypes.byref(empty), None, None) == 0


def test_linear_batch_validation_runs_before_any_launch():
    lib = _lib_or_skip()
    host = df11.encode(workloads.gen_single_matrix(rows=64, cols=1024))
    s = _fake_device_stream(host)
    x = ctypes.c_void_p(1 << 48)

    def call(streams, out_f, outs, t=1, in_f=1024):
        arr = (_lib.DeviceStream * max(len(streams), 1))(*streams)
        of = np.array(out_f if out_f else [0], np.uint32)
        ptrs = (ctypes.c_void_p * max(len(outs), 1))(*outs)
        return lib.df11_linear_batch(arr, len(streams), x, t, in_f, of.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                     ptrs, None, None, None)

    y0, y1 = (1 << 48) + (1 << 32), (1 << 48) + (2 << 32)
    assert lib.df11_linear_batch(None, 0, x, 1, 1024, None, None, None, None, None) == 0  # empty batch
    assert lib.df11_linear_batch(None, 1, x, 1, 1024, None, None, None, None, None) == -1
    assert call([s] * (_lib.MAX_BATCH + 1), [64] * (_lib.MAX_BATCH + 1), [y0] * (_lib.MAX_BATCH + 1)) == -7
    assert call([s, s], [64, 63], [y0, y1]) == -1               # rows that do not match a stream
    assert call([s, s], [64, 64], [y0, y0 + 64]) == -1          # outputs overlap each other
    assert call([s, s], [64, 64], [y0, s.enc]) == -1            # an output over another stream
    other = _lib.DeviceStream.from_buffer_copy(s)
    other.decode_table_bits = 11
    assert call([s, other], [64, 64], [y0, y1]) == -1           # different table widths
    assert call([s], [64], [y0], t=9) == -1                     # too many tokens


def test_device_check_of_the_binding():
    """The binding's device check: a host tensor is never on a CUDA device
    (decided without a GPU), and tensors match a device of their own type."""
    import torch
    from entropy_decoding_df11_amd.df11 import _on_device
    assert not _on_device(torch.zeros(1), "cuda")
    assert not _on_device(torch.zeros(1), "cuda:0")
    assert _on_device(torch.zeros(1), "cpu")


def test_committed_profiles_match_the_kernel_sources():
    """The rocprofv3 summaries under profiles/ name the sha256 prefix of the
    kernel source they were taken on; the bench line's HBM traffic comes from
    the counter summary only while that prefix matches the current source."""
    import hashlib
    import json

    def prefix(name):
        with open(os.path.join(REPO, "entropy_decoding_df11_amd", "csrc", name), "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]

    with open(os.path.join(REPO, "profiles", "df11_decode_kernel_llama3_8b_block_pmc.json")) as f:
        pmc = json.load(f)
    assert pmc["kernel_source_sha256_16"] == prefix("df11_decode.hip")
    assert 1.0 <= pmc["traffic_over_algorithmic"] < 1.2
    for md, src in (("df11_decode_kernel_llama3_8b_block_counters.md", "df11_decode.hip"),
                    ("df11_rans_decode_kernel_llama3_8b_block_counters.md", "df11_rans_decode.hip")):
        with open(os.path.join(REPO, "profiles", md)) as f:
            assert prefix(src) in f.read(), md


def test_element_limit_of_a_stream():
    """A stream holds at most DF11_MAX_ELEMENTS = 2^32 - 2^16 elements: the
    planner accepts that many (sizes only, no data) and rejects one more,
    and the header mirrors the same limit."""
    lib = _lib_or_skip()
    with open(os.path.join(REPO, "include", "df11.h")) as f:
        m = re.search(r"#define DF11_MAX_ELEMENTS (\d+)ull", f.read())
    assert m and int(m.group(1)) == _lib.MAX_ELEMENTS == (1 << 32) - (1 << 16)
    for n, rc in ((_lib.MAX_ELEMENTS, 0), (_lib.MAX_ELEMENTS + 1, -7), (1 << 32, -7)):
        hist = np.zeros(256, dtype=np.uint64)
        hist[127], hist[126] = n - n // 3, n // 3
        cb = df11.build_codebook(hist)
        h = _lib.Header()
        lay = _lib.Layout(8, 256)
        got = lib.df11_plan(ctypes.byref(cb), hist.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n,
                            ctypes.byref(lay), ctypes.byref(h))
        assert got == rc, n
        if rc == 0:
            assert h.n_elements == n and h.sm_bytes == -(-n // 64) * 64


def _tile_order_reference(w, rows, cols):
    """MFMA tile order from its definition: position (p, ks, nt, l, j) holds
    W[64 p + 16 nt + l % 16][32 ks + 8 (l // 16) + j]; numpy axes
    (p, nt, l % 16, ks, l // 16, j) put in the order (p, ks, nt, l // 16, l % 16, j)."""
    t = w.reshape(rows // 64, 4, 16, cols // 32, 4, 8)
    return np.ascontiguousarray(t.transpose(0, 3, 1, 4, 2, 5)).reshape(-1)


def test_tile_order_matches_its_definition():
    _lib_or_skip()
    rng = np.random.default_rng(3)
    for rows, cols in ((64, 32), (128, 96), (192, 4096), (64, 14336)):
        w = rng.integers(0, 1 << 16, rows * cols, dtype=np.uint16)
        got = df11.tile_order(w, rows, cols)
        assert np.array_equal(got, _tile_order_reference(w, rows, cols)), (rows, cols)
    # spot checks straight from the formula, one element at a time
    rows, cols = 128, 96
    w = np.arange(rows * cols, dtype=np.uint32).astype(np.uint16)
    got = df11.tile_order(w, rows, cols)
    for s in rng.integers(0, rows * cols, 200):
        p, q = divmod(int(s), 64 * cols)
        ks, u = divmod(q, 2048)
        nt, v = divmod(u, 512)
        lane, j = divmod(v, 8)
        r, c = 64 * p + 16 * nt + lane % 16, 32 * ks + 8 * (lane // 16) + j
        assert got[s] == w[r * cols + c]


def test_tile_order_errors():
    lib = _lib_or_skip()
    w = np.zeros(64 * 32, np.uint16)
    out = np.zeros_like(w)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))  # noqa: E731
    assert lib.df11_tile_order(p(w), 64, 32, p(out)) == 0
    assert lib.df11_tile_order(p(w), 32, 64, p(out)) == -1    # rows not a multiple of 64
    assert lib.df11_tile_order(p(w), 64 * 2, 16, p(out)) == -1  # cols not a multiple of 32
    assert lib.df11_tile_order(None, 64, 32, p(out)) == -1
    assert lib.df11_tile_order(p(w), 64, 32, p(w)) == -1      # in place


def test_matmul_validation_runs_before_any_launch():
    lib = _lib_or_skip()
    w = workloads.gen_single_matrix(rows=128, cols=1024)
    host = df11.encode(df11.tile_order(w, 128, 1024))
    s = _fake_device_stream(host)
    s.tile_cols = 1024
    x, y = ctypes.c_void_p(1 << 46), ctypes.c_void_p(1 << 47)

    def call(st, t=4, i=1024, o=128, xp=x, yp=y):
        return lib.df11_matmul(ctypes.byref(st) if st is not None else None, xp, t, i, o, yp, None)

    assert call(None) == -1
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.tile_cols = 0                    # a stream in row order
    assert call(bad) == -1
    bad.tile_cols = 512                  # tile columns that do not match in_features
    assert call(bad) == -1
    bad.tile_cols = 48                   # not a multiple of 32
    assert call(bad) == -1
    assert call(s, t=0) == -1            # no tokens
    assert call(s, i=512, o=256) == -1   # in_features does not match the tile columns
    assert call(s, xp=ctypes.c_void_p((1 << 46) + 8)) == -1  # x not 16-byte aligned
    assert call(s, yp=ctypes.c_void_p(s.sm)) == -1  # y overlaps the stream
    assert call(s, yp=ctypes.c_void_p((1 << 46) + 64)) == -1  # y overlaps x
    assert call(s, t=1 << 26) == -7      # n_tokens * out_features >= 2^32
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.enc_bytes += 16
    assert call(bad) == -6
    # the row-order product takes no tiled stream
    assert lib.df11_linear(ctypes.byref(s), x, 1, 1024, 128, y, None) == -1
    assert lib.df11_matmul_acc(ctypes.byref(s), x, 4, 1024, 64, y, None) == -1
    assert lib.df11_matmul_timed(ctypes.byref(s), x, 0, 1024, 128, y, None, None, None) == -1
    # decompressing a tiled stream checks its shape: N a multiple of 64 * tile_cols
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.tile_cols = 96
    assert lib.df11_decompress(ctypes.byref(bad), ctypes.c_void_p(1 << 48), None) == -1


def test_matmul_batch_validation_runs_before_any_launch():
    lib = _lib_or_skip()
    w = workloads.gen_single_matrix(rows=128, cols=1024)
    host = df11.encode(df11.tile_order(w, 128, 1024))
    s = _fake_device_stream(host)
    s.tile_cols = 1024
    x = 1 << 46

    def call(streams, xs, ys, t=2, ins=None, outs_f=None, acc=0):
        n = len(streams)
        arr = (_lib.DeviceStream * max(n, 1))(*streams)
        xp = (ctypes.c_void_p * max(n, 1))(*xs)
        yp = (ctypes.c_void_p * max(n, 1))(*ys)
        inf = np.array(ins or [1024] * n, np.uint32)
        outf = np.array(outs_f or [128] * n, np.uint32)
        return lib.df11_matmul_batch(arr, n, xp, t, inf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                     outf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), yp, acc, None, None, None)

    assert lib.df11_matmul_batch(None, 0, None, 1, None, None, None, 0, None, None, None) == 0  # empty batch
    assert lib.df11_matmul_batch(None, 1, None, 1, None, None, None, 0, None, None, None) == -1
    y0, y1 = 1 << 47, (1 << 47) + (1 << 20)
    assert call([s] * 17, [x] * 17, [y0 + (i << 20) for i in range(17)]) == -7  # too many streams
    assert call([s, s], [x, x], [y0, y0 + 64]) == -1          # outputs overlap
    assert call([s, s], [x, y1 + 8], [y0, y1]) == -1          # an output overlaps another product's x
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.tile_cols = 0
    assert call([s, bad], [x, x], [y0, y1]) == -1             # one stream in row order: nothing launches
    bad = _lib.DeviceStream.from_buffer_copy(s)
    bad.h.enc_bytes += 16
    assert call([s, bad], [x, x], [y0, y1], acc=1) == -6
