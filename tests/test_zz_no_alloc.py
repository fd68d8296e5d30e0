"""df11_decompress_batch_noalloc, the allocation-free batched decode, through
the C ABI: its output must equal df11_decompress_batch's (and the original
weights) on two calls in a row, the second with a smaller input."""

import ctypes
import sys

import numpy as np
import pytest

from entropy_decoding_df11_amd import _lib, df11, workloads

pytestmark = pytest.mark.gpu


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _u16(t):
    import torch
    return t.detach().reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)


def _call(fn, tensors, outs, st):
    arr = (_lib.DeviceStream * len(tensors))(*[t.device_stream() for t in tensors])
    ptrs = (ctypes.c_void_p * len(tensors))(*[o.data_ptr() for o in outs])
    return fn(arr, len(tensors), ptrs, ctypes.c_void_p(st.cuda_stream))


def test_noalloc_batch_matches_batch_on_two_calls():
    import torch
    assert torch.cuda.is_available()
    lib = _lib.load()
    st = torch.cuda.current_stream()
    rng = np.random.default_rng(7)
    # first call: the Llama-3-8B block with a codebook per weight (seven streams,
    # long enough for the dynamic schedule); second call: three small streams
    flat, views = workloads.gen_block()
    big = [np.ascontiguousarray(flat[o:o + r * c]) for _, o, (r, c) in views]
    small = [workloads.f32_to_bf16_bits(rng.standard_normal(n) * 0.02) for n in (1, 77777, 300001)]
    for call, ws in (("block, 7 streams", big), ("3 small streams", small)):
        _note(f"noalloc batch: {call}")
        ts = [df11.compress(w, shape=(w.size,)) for w in ws]
        ref = [torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16) for w in ws]
        got = [torch.full((w.size,), 0x1234, dtype=torch.int16, device="cuda").view(torch.bfloat16) for w in ws]
        torch.cuda.synchronize()
        assert _call(lib.df11_decompress_batch, ts, ref, st) == 0
        assert _call(lib.df11_decompress_batch_noalloc, ts, got, st) == 0
        torch.cuda.synchronize()
        for w, a, b in zip(ws, ref, got):
            ua, ub = _u16(a), _u16(b)
            assert np.array_equal(ub, ua)
            assert np.array_equal(ub, w)
        del ts, ref, got


def test_noalloc_batch_matches_batch_tile_ordered():
    """Tile-ordered streams (decompressed back to row-major in whole lines)
    through both entry points, two calls in a row, the second smaller."""
    import torch
    assert torch.cuda.is_available()
    lib = _lib.load()
    st = torch.cuda.current_stream()
    rng = np.random.default_rng(8)
    calls = (("3 tiled matrices", [(1024, 4096), (64, 14336), (192, 128)]), ("1 tiled matrix", [(128, 1024)]))
    for call, shapes in calls:
        _note(f"noalloc batch: {call}")
        ws = [workloads.f32_to_bf16_bits(rng.standard_normal(r * c) * 0.02) for r, c in shapes]
        ts = [df11.compress(w, shape=s, layout="mfma_tiles") for w, s in zip(ws, shapes)]
        ref = [torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16) for w in ws]
        got = [torch.full((w.size,), 0x1234, dtype=torch.int16, device="cuda").view(torch.bfloat16) for w in ws]
        torch.cuda.synchronize()
        assert _call(lib.df11_decompress_batch, ts, ref, st) == 0
        assert _call(lib.df11_decompress_batch_noalloc, ts, got, st) == 0
        torch.cuda.synchronize()
        for w, a, b in zip(ws, ref, got):
            assert np.array_equal(_u16(b), _u16(a))
            assert np.array_equal(_u16(b), w)
        del ts, ref, got


def test_noalloc_batch_rejects_too_many_streams():
    import torch
    assert torch.cuda.is_available()
    lib = _lib.load()
    arr = (_lib.DeviceStream * 17)()
    ptrs = (ctypes.c_void_p * 17)()
    assert lib.df11_decompress_batch_noalloc(arr, 17, ptrs, None) == -7
    assert lib.df11_decompress_batch_noalloc(None, 0, None, None) == 0
