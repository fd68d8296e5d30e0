"""Python API over the DF11 C ABI.

Method: "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan LLM menjadi
70% ukurannya" (GeekNews).  Every step of encoding and decoding runs in
libdf11.so; this module only moves arguments.  PyTorch provides device memory
and streams.

    t = compress(weight_bf16_cpu)          # host encode + upload
    w = t.decompress()                     # bf16 tensor on the GPU, bit-exact
    blk = compress_block({"q_proj": q, ...})
    views = blk.decompress()               # one scratch buffer, a view per weight
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple, Union

import numpy as np

from . import _lib

DEFAULT_BYTES_PER_THREAD = 8
DEFAULT_THREADS_PER_GROUP = 256
DEFAULT_DECODE_TABLE_BITS = 11

ArrayLike = Union[np.ndarray, "torch.Tensor"]  # noqa: F821


def _u16(x: ArrayLike) -> np.ndarray:
    """BF16 bit patterns as a contiguous uint16 numpy array (host)."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy input must hold BF16 bit patterns as uint16")
        return np.ascontiguousarray(x).reshape(-1)
    import torch
    if x.dtype != torch.bfloat16:
        raise TypeError(f"expected a bfloat16 tensor, got {x.dtype}")
    return x.detach().to("cpu").contiguous().reshape(-1).view(torch.int16).numpy().view(np.uint16)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def histogram(bf16: ArrayLike, hist: Optional[np.ndarray] = None) -> np.ndarray:
    """Accumulate the exponent histogram (uint64[256]) of BF16 data."""
    w = _u16(bf16)
    if hist is None:
        hist = np.zeros(256, dtype=np.uint64)
    lib = _lib.load()
    _lib.check(lib.df11_histogram(_ptr(w, ctypes.c_uint16), w.size, _ptr(hist, ctypes.c_uint64)), "df11_histogram")
    return hist


def build_codebook(hist: np.ndarray) -> _lib.Codebook:
    hist = np.ascontiguousarray(hist, dtype=np.uint64)
    cb = _lib.Codebook()
    lib = _lib.load()
    _lib.check(lib.df11_build_codebook(_ptr(hist, ctypes.c_uint64), ctypes.byref(cb)), "df11_build_codebook")
    return cb


def codebook_arrays(cb: _lib.Codebook) -> Dict[str, np.ndarray]:
    """Copy a codebook into numpy arrays (code_lengths, codes, luts[n_luts])."""
    return {
        "code_lengths": np.ctypeslib.as_array(cb.code_lengths).copy(),
        "codes": np.ctypeslib.as_array(cb.codes).copy(),
        "luts": np.ctypeslib.as_array(cb.luts).copy()[: cb.n_luts],
        "n_luts": int(cb.n_luts),
        "max_len": int(cb.max_len),
    }


def decode_table(cb: _lib.Codebook, bits: int = DEFAULT_DECODE_TABLE_BITS) -> np.ndarray:
    lib = _lib.load()
    nbytes = lib.df11_decode_table_bytes(bits)
    if nbytes == 0:
        raise ValueError(f"unsupported decode table width {bits}")
    table = np.zeros(nbytes // 4, dtype=np.uint32)
    _lib.check(lib.df11_build_decode_table(ctypes.byref(cb), bits, table.ctypes.data_as(ctypes.c_void_p), nbytes),
               "df11_build_decode_table")
    return table


@dataclasses.dataclass
class HostStream:
    """A DF11 stream in host memory (numpy buffers sized by the header)."""

    header: _lib.Header
    codebook: _lib.Codebook
    enc: np.ndarray
    sm: np.ndarray
    gaps: np.ndarray
    out_pos: np.ndarray

    @property
    def n_elements(self) -> int:
        return int(self.header.n_elements)

    def compressed_bytes(self) -> int:
        """Algorithmic size: EncodedExponent (unpadded) + PackedSignMantissa +
        Gaps (5 bits per thread) + output positions + LUTs + CodeLengths."""
        h = self.header
        return int((h.total_bits + 7) // 8 + h.n_elements + (5 * h.n_threads + 7) // 8 + 4 * (h.n_groups + 1)
                   + 256 * (h.n_luts + 1))

    def header_dict(self) -> Dict[str, int]:
        return {name: int(getattr(self.header, name)) for name, _ in _lib.Header._fields_}


def encode(bf16: ArrayLike, codebook: Optional[_lib.Codebook] = None,
           bytes_per_thread: int = DEFAULT_BYTES_PER_THREAD,
           threads_per_group: int = DEFAULT_THREADS_PER_GROUP) -> HostStream:
    """Encode BF16 data on the host.  With no codebook, one is built from the
    data's own histogram."""
    w = _u16(bf16)
    lib = _lib.load()
    hist = histogram(w)
    if codebook is None:
        codebook = build_codebook(hist)
    lay = _lib.Layout(bytes_per_thread, threads_per_group)
    h = _lib.Header()
    _lib.check(lib.df11_plan(ctypes.byref(codebook), _ptr(hist, ctypes.c_uint64), w.size, ctypes.byref(lay),
                             ctypes.byref(h)), "df11_plan")
    enc = np.empty(h.enc_bytes, dtype=np.uint8)
    sm = np.empty(h.sm_bytes, dtype=np.uint8)
    gaps = np.empty(h.gaps_bytes, dtype=np.uint8)
    out_pos = np.empty(h.n_groups + 1, dtype=np.uint32)
    _lib.check(lib.df11_encode(ctypes.byref(codebook), _ptr(w, ctypes.c_uint16), w.size, ctypes.byref(lay),
                               ctypes.byref(h), _ptr(enc, ctypes.c_uint8), _ptr(sm, ctypes.c_uint8),
                               _ptr(gaps, ctypes.c_uint8), _ptr(out_pos, ctypes.c_uint32)), "df11_encode")
    return HostStream(h, codebook, enc, sm, gaps, out_pos)


class DF11Tensor:
    """A DF11 stream resident in GPU memory, decompressed on demand."""

    def __init__(self, host: HostStream, shape: Sequence[int], device="cuda",
                 decode_table_bits: int = DEFAULT_DECODE_TABLE_BITS, groups_per_workgroup: int = 0,
                 tile_cols: int = 0):
        import torch
        self.host_header = host.header
        self.shape = tuple(int(s) for s in shape)
        self.device = torch.device(device)
        self.decode_table_bits = decode_table_bits

        def up(a: np.ndarray) -> "torch.Tensor":
            b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
            if b.size == 0:
                b = np.zeros(16, dtype=np.uint8)
            return torch.from_numpy(b.copy()).to(self.device)

        arrays = codebook_arrays(host.codebook)
        self._bufs = {
            "enc": up(host.enc),
            "sm": up(host.sm),
            "gaps": up(host.gaps),
            "out_pos": up(host.out_pos),
            "luts": up(arrays["luts"]),
            "code_lengths": up(arrays["code_lengths"]),
            "decode_table": up(decode_table(host.codebook, decode_table_bits)),
        }
        self._compressed_bytes = host.compressed_bytes()
        s = _lib.DeviceStream()
        s.h = host.header
        for name, t in self._bufs.items():
            setattr(s, name, t.data_ptr())
        s.decode_table_bits = decode_table_bits
        s.groups_per_workgroup = groups_per_workgroup
        # A matrix stored in MFMA tile order (df11_tile_order) for matmul():
        # its column count; decompress() writes it back row-major.
        s.tile_cols = tile_cols
        self.tile_cols = tile_cols
        # The kernel's work counter for dynamic load balancing (zero between
        # launches).  Launches of one DF11Tensor must not overlap in time.
        self._schedule = torch.zeros(_lib.SCHEDULE_WORDS, dtype=torch.int32, device=self.device)
        s.schedule = self._schedule.data_ptr()
        self._last_stream = None  # the stream of the latest launch (see _claim)
        self._stream_struct = s
        # The uploads and the counters' zero fill ran on the current stream:
        # finish them, so that a first launch on any stream sees them.
        torch.cuda.current_stream(self.device).synchronize()

    def clone(self) -> "DF11Tensor":
        """The same stream in new device buffers (same bytes, other addresses)
        with work counters of its own."""
        import copy
        import torch
        c = copy.copy(self)
        c._bufs = {name: t.clone() for name, t in self._bufs.items()}
        c._schedule = torch.zeros_like(self._schedule)
        s = _lib.DeviceStream.from_buffer_copy(self._stream_struct)
        for name, t in c._bufs.items():
            setattr(s, name, t.data_ptr())
        if not self._stream_struct.decode_table:  # (launched without the table)
            s.decode_table = None
        if self._stream_struct.schedule:
            s.schedule = c._schedule.data_ptr()
        c._stream_struct = s
        c._last_stream = None
        torch.cuda.current_stream(self.device).synchronize()
        return c

    def use_decode_table(self, on: bool) -> None:
        """Launch with the host-built first-level decode table (default), or
        with the page's arrays alone (no table): every workgroup then derives
        the same table in LDS from the LUTs and CodeLengths."""
        self._stream_struct.decode_table = self._bufs["decode_table"].data_ptr() if on else None

    def set_dynamic_schedule(self, on: bool) -> None:
        """Balance work between workgroups at run time (default) or assign it
        statically."""
        self._stream_struct.schedule = self._schedule.data_ptr() if on else None

    def set_max_workgroups(self, n: int) -> None:
        """Launch at most n workgroups (0: fill the GPU), leaving CUs to
        kernels running concurrently on other streams."""
        self._stream_struct.max_workgroups = n

    def set_groups_per_workgroup(self, gpw: int) -> None:
        """Launch shape: groups decoded together by one workgroup (0 = default, 1, 2, 4)."""
        self._stream_struct.groups_per_workgroup = gpw

    @property
    def n_elements(self) -> int:
        return int(self.host_header.n_elements)

    @property
    def header(self) -> _lib.Header:
        return self.host_header

    def compressed_bytes(self) -> int:
        return self._compressed_bytes

    def device_stream(self) -> _lib.DeviceStream:
        return self._stream_struct

    def _hip_stream(self, stream) -> ctypes.c_void_p:
        import torch
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(st.cuda_stream)

    def _claim(self, stream) -> ctypes.c_void_p:
        """The HIP stream of a launch of this tensor (torch's current stream
        by default), ordered after the tensor's previous launch when that one
        went to another stream: launches of one tensor share its work
        counters, which a launch leaves at zero only when it has finished,
        so they must not overlap in time.  (Under graph capture the graph's
        own dependencies order the launches.)"""
        import torch
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        last = self._last_stream
        if last is not None and last.cuda_stream != st.cuda_stream and not torch.cuda.is_current_stream_capturing():
            st.wait_stream(last)
        self._last_stream = st
        return ctypes.c_void_p(st.cuda_stream)

    def decompress(self, out: Optional["torch.Tensor"] = None, stream=None, events=None) -> "torch.Tensor":  # noqa: F821
        """Decode into out (a new bf16 tensor of the original shape by default),
        enqueued on stream (torch's current stream by default).  events, a pair
        of torch.cuda.Event(enable_timing=True), are recorded at the decode
        kernel's own start and end.  Launches of one DF11Tensor share its
        work counters and must not overlap in time: decode one tensor on one
        stream at a time."""
        import torch
        if out is None:
            out = torch.empty(self.shape, dtype=torch.bfloat16, device=self.device)
        if out.dtype != torch.bfloat16 or out.numel() != self.n_elements or not out.is_contiguous():
            raise ValueError("out must be a contiguous bfloat16 tensor with the stream's element count")
        if not _on_device(out, self.device):
            raise ValueError("out must be on the stream's device")
        self._launch(out, stream, events)
        return out

    def _launch(self, out: "torch.Tensor", stream, events) -> None:  # noqa: F821
        lib = _lib.load()
        st = self._claim(stream)
        if events is None:
            _lib.check(lib.df11_decompress(ctypes.byref(self._stream_struct), ctypes.c_void_p(out.data_ptr()), st),
                       "df11_decompress")
            return
        start, stop = events
        _lib.check(lib.df11_decompress_timed(ctypes.byref(self._stream_struct), ctypes.c_void_p(out.data_ptr()), st,
                                             ctypes.c_void_p(_event_handle(start, st)),
                                             ctypes.c_void_p(_event_handle(stop, st))), "df11_decompress_timed")


    def linear(self, x: "torch.Tensor", out: Optional["torch.Tensor"] = None, stream=None,  # noqa: F821
               events=None, accumulate: bool = False) -> "torch.Tensor":  # noqa: F821
        """y = x W^T with the decode fused into the product (df11_linear): W
        is this tensor as an (out_features, in_features) matrix, x a
        contiguous bfloat16 (n_tokens, in_features) tensor on the same device
        with 1 <= n_tokens <= 8.  Returns out, a float32 (n_tokens,
        out_features) tensor (a new one by default).  events: as for
        decompress, recorded at the fused kernel's own start and end.  With
        accumulate, out (required) receives out + x W^T (df11_linear_acc)."""
        import torch
        if len(self.shape) != 2:
            raise ValueError("linear needs a 2-D weight (out_features, in_features)")
        out_f, in_f = self.shape
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != in_f or not x.is_contiguous():
            raise ValueError("x must be a contiguous bfloat16 (n_tokens, in_features) tensor")
        if not _on_device(x, self.device):
            raise ValueError("x must be on the weight's device")
        n_tokens = x.shape[0]
        if out is None:
            if accumulate:
                raise ValueError("accumulate needs out")
            out = torch.empty((n_tokens, out_f), dtype=torch.float32, device=self.device)
        if out.dtype != torch.float32 or out.shape != (n_tokens, out_f) or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 (n_tokens, out_features) tensor")
        if not _on_device(out, self.device):
            raise ValueError("out must be on the weight's device")
        lib = _lib.load()
        st = self._claim(stream)
        args = (ctypes.byref(self._stream_struct), ctypes.c_void_p(x.data_ptr()), n_tokens, in_f, out_f,
                ctypes.c_void_p(out.data_ptr()), st)
        if accumulate:
            if events is not None:
                raise ValueError("accumulate takes no events")
            _lib.check(lib.df11_linear_acc(*args), "df11_linear_acc")
        elif events is None:
            _lib.check(lib.df11_linear(*args), "df11_linear")
        else:
            start, stop = events
            _lib.check(lib.df11_linear_timed(*args, ctypes.c_void_p(_event_handle(start, st)),
                                             ctypes.c_void_p(_event_handle(stop, st))), "df11_linear_timed")
        return out

    def matmul(self, x: "torch.Tensor", out: Optional["torch.Tensor"] = None, stream=None,  # noqa: F821
               events=None, accumulate: bool = False) -> "torch.Tensor":  # noqa: F821
        """y = x W^T on the matrix cores with the decode fused in (df11_matmul),
        for any number of tokens: W is this tensor, compressed with
        layout="mfma_tiles", as an (out_features, in_features) matrix; x a
        contiguous bfloat16 (n_tokens, in_features) tensor.  Returns out, a
        float32 (n_tokens, out_features) tensor (a new one by default).
        events: as for decompress.  With accumulate, out (required)
        receives out + x W^T (df11_matmul_acc)."""
        import torch
        if len(self.shape) != 2 or not self.tile_cols:
            raise ValueError("matmul needs a 2-D weight compressed with layout='mfma_tiles'")
        out_f, in_f = self.shape
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != in_f or not x.is_contiguous():
            raise ValueError("x must be a contiguous bfloat16 (n_tokens, in_features) tensor")
        if not _on_device(x, self.device):
            raise ValueError("x must be on the weight's device")
        n_tokens = x.shape[0]
        if out is None:
            if accumulate:
                raise ValueError("accumulate needs out")
            out = torch.empty((n_tokens, out_f), dtype=torch.float32, device=self.device)
        if out.dtype != torch.float32 or out.shape != (n_tokens, out_f) or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 (n_tokens, out_features) tensor")
        if not _on_device(out, self.device):
            raise ValueError("out must be on the weight's device")
        lib = _lib.load()
        st = self._claim(stream)
        args = (ctypes.byref(self._stream_struct), ctypes.c_void_p(x.data_ptr()), n_tokens, in_f, out_f,
                ctypes.c_void_p(out.data_ptr()), st)
        if accumulate:
            if events is not None:
                raise ValueError("accumulate takes no events")
            _lib.check(lib.df11_matmul_acc(*args), "df11_matmul_acc")
        elif events is None:
            _lib.check(lib.df11_matmul(*args), "df11_matmul")
        else:
            start, stop = events
            _lib.check(lib.df11_matmul_timed(*args, ctypes.c_void_p(_event_handle(start, st)),
                                             ctypes.c_void_p(_event_handle(stop, st))), "df11_matmul_timed")
        return out


def matmul_batch(tensors: Sequence[DF11Tensor], xs: Sequence["torch.Tensor"], outs=None, stream=None,  # noqa: F821
                 events=None, accumulate: bool = False) -> List["torch.Tensor"]:  # noqa: F821
    """[xs[i] W_i^T for each W_i in tensors] on the matrix cores in one launch
    (df11_matmul_batch): every W_i compressed with layout="mfma_tiles", every
    xs[i] a contiguous bfloat16 (n_tokens, in_features_i) tensor with the
    same n_tokens (the same tensor may serve several weights).  Returns the
    float32 outputs (new tensors by default); events as for
    DF11Tensor.decompress.  With accumulate, each of outs (required)
    receives outs[i] + xs[i] W_i^T."""
    import torch
    if not tensors:
        return []
    if len(tensors) > _lib.MAX_BATCH or len(xs) != len(tensors):
        raise ValueError(f"one x per weight, at most {_lib.MAX_BATCH} weights per launch")
    n_tokens = None
    for t, x in zip(tensors, xs):
        if len(t.shape) != 2 or not t.tile_cols:
            raise ValueError("every weight must be 2-D and compressed with layout='mfma_tiles'")
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != t.shape[1] or not x.is_contiguous():
            raise ValueError("each x must be a contiguous bfloat16 (n_tokens, in_features) tensor")
        if n_tokens is not None and x.shape[0] != n_tokens:
            raise ValueError("every x must have the same number of tokens")
        n_tokens = x.shape[0]
        if not _on_device(x, t.device):
            raise ValueError("every x must be on its weight's device")
    if outs is None:
        if accumulate:
            raise ValueError("accumulate needs outs")
        outs = [torch.empty((n_tokens, t.shape[0]), dtype=torch.float32, device=t.device) for t in tensors]
    for t, y in zip(tensors, outs):
        if y.dtype != torch.float32 or y.shape != (n_tokens, t.shape[0]) or not y.is_contiguous():
            raise ValueError("each output must be a contiguous float32 (n_tokens, out_features) tensor")
        if not _on_device(y, t.device):
            raise ValueError("every output must be on its weight's device")
    lib = _lib.load()
    st = [t._claim(stream) for t in tensors][0]
    n = len(tensors)
    arr = (_lib.DeviceStream * n)(*[t._stream_struct for t in tensors])
    in_f = np.array([t.shape[1] for t in tensors], np.uint32)
    out_f = np.array([t.shape[0] for t in tensors], np.uint32)
    xp = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    yp = (ctypes.c_void_p * n)(*[y.data_ptr() for y in outs])
    ev = (None, None) if events is None else (ctypes.c_void_p(_event_handle(events[0], st)),
                                              ctypes.c_void_p(_event_handle(events[1], st)))
    _lib.check(lib.df11_matmul_batch(arr, n, xp, n_tokens, _ptr(in_f, ctypes.c_uint32), _ptr(out_f, ctypes.c_uint32),
                                     yp, 1 if accumulate else 0, st, *ev), "df11_matmul_batch")
    return outs


def linear_batch(tensors: Sequence[DF11Tensor], x: "torch.Tensor", outs=None, stream=None,  # noqa: F821
                 events=None, accumulate: bool = False) -> List["torch.Tensor"]:  # noqa: F821
    """[x W_i^T for each W_i in tensors] in one launch (df11_linear_batch):
    every W_i is (out_features_i, in_features) with the same in_features, x
    a contiguous bfloat16 (n_tokens, in_features) tensor, 1 <= n_tokens <= 8
    (a block's q, k and v, or gate and up).  Returns the float32 outputs
    (new tensors by default); events as for DF11Tensor.linear.  With
    accumulate, each of outs (required) receives outs[i] + x W_i^T
    (df11_linear_batch_acc)."""
    import torch
    if not tensors:
        return []
    if len(tensors) > _lib.MAX_BATCH:
        raise ValueError(f"at most {_lib.MAX_BATCH} matrices per launch")
    in_f = tensors[0].shape[1] if len(tensors[0].shape) == 2 else -1
    if any(len(t.shape) != 2 or t.shape[1] != in_f for t in tensors):
        raise ValueError("every weight must be 2-D with the same in_features")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != in_f or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 (n_tokens, in_features) tensor")
    if not all(_on_device(x, t.device) for t in tensors):
        raise ValueError("x and every weight must be on the same device")
    n_tokens = x.shape[0]
    if outs is None:
        if accumulate:
            raise ValueError("accumulate needs outs")
        outs = [torch.empty((n_tokens, t.shape[0]), dtype=torch.float32, device=x.device) for t in tensors]
    for t, y in zip(tensors, outs):
        if y.dtype != torch.float32 or y.shape != (n_tokens, t.shape[0]) or not y.is_contiguous():
            raise ValueError("each output must be a contiguous float32 (n_tokens, out_features) tensor")
        if not _on_device(y, x.device):
            raise ValueError("every output must be on the weights' device")
    lib = _lib.load()
    st = [t._claim(stream) for t in tensors][0]
    arr = (_lib.DeviceStream * len(tensors))(*[t._stream_struct for t in tensors])
    out_f = np.array([t.shape[0] for t in tensors], np.uint32)
    ptrs = (ctypes.c_void_p * len(tensors))(*[y.data_ptr() for y in outs])
    ev = (None, None) if events is None else (ctypes.c_void_p(_event_handle(events[0], st)),
                                              ctypes.c_void_p(_event_handle(events[1], st)))
    fn, name = (lib.df11_linear_batch_acc, "df11_linear_batch_acc") if accumulate else \
        (lib.df11_linear_batch, "df11_linear_batch")
    _lib.check(fn(arr, len(tensors), ctypes.c_void_p(x.data_ptr()), n_tokens, in_f, _ptr(out_f, ctypes.c_uint32),
                  ptrs, st, *ev), name)
    return outs


def _on_device(t: "torch.Tensor", device) -> bool:  # noqa: F821
    """Whether tensor t lives on device (an index-less CUDA device means the
    current one)."""
    import torch
    dev = torch.device(device)
    if t.device.type != dev.type:
        return False
    if dev.type != "cuda":
        return True
    here = lambda d: d.index if d.index is not None else torch.cuda.current_device()  # noqa: E731
    return here(t.device) == here(dev)


def _event_handle(ev, stream: ctypes.c_void_p) -> int:
    """The hipEvent_t behind a torch.cuda.Event, created by recording it once
    on the launch stream (the decode launch records it again)."""
    import torch
    if not isinstance(ev, torch.cuda.Event):
        raise TypeError("events must be torch.cuda.Event objects")
    if ev.cuda_event == 0:
        ev.record(torch.cuda.ExternalStream(stream.value) if stream.value else torch.cuda.default_stream())
    return ev.cuda_event


def tile_order(w: ArrayLike, rows: int, cols: int) -> np.ndarray:
    """A rows x cols BF16 matrix (uint16 patterns) reordered into MFMA tile
    order (df11_tile_order)."""
    src = _u16(w)
    if src.size != rows * cols:
        raise ValueError("rows * cols must equal the element count")
    out = np.empty_like(src)
    _lib.check(_lib.load().df11_tile_order(_ptr(src, ctypes.c_uint16), rows, cols, _ptr(out, ctypes.c_uint16)),
               "df11_tile_order")
    return out


def compress(tensor: ArrayLike, shape: Optional[Sequence[int]] = None, device="cuda",
             codebook: Optional[_lib.Codebook] = None,
             decode_table_bits: int = DEFAULT_DECODE_TABLE_BITS, layout: str = "rows") -> DF11Tensor:
    """Encode a BF16 tensor on the host and upload the stream to the GPU.
    layout="rows" keeps the elements in their own order; layout="mfma_tiles"
    (a 2-D weight, rows a multiple of 64, columns of 32) stores them in the
    order the matrix-core product consumes them (DF11Tensor.matmul)."""
    if shape is None:
        shape = tuple(tensor.shape)
    if layout == "rows":
        host = encode(tensor, codebook=codebook)
        return DF11Tensor(host, shape, device=device, decode_table_bits=decode_table_bits)
    if layout != "mfma_tiles":
        raise ValueError("layout must be 'rows' or 'mfma_tiles'")
    if len(shape) != 2:
        raise ValueError("layout='mfma_tiles' needs a 2-D (out_features, in_features) weight")
    rows, cols = (int(v) for v in shape)
    host = encode(tile_order(tensor, rows, cols), codebook=codebook)
    return DF11Tensor(host, shape, device=device, decode_table_bits=decode_table_bits, tile_cols=cols)


def decompress(t: DF11Tensor, out=None, stream=None):
    return t.decompress(out=out, stream=stream)


class DF11Block:
    """Every linear weight of one transformer block as a single DF11 stream
    with a shared codebook, decompressed in one launch into one scratch buffer
    ("Dekompresi per transformer block")."""

    def __init__(self, tensor: DF11Tensor, views: List[Tuple[str, int, Tuple[int, ...]]]):
        self.tensor = tensor
        self.views = views
        self._view_cache = (None, None)  # (scratch tensor, its views)

    @property
    def n_elements(self) -> int:
        return self.tensor.n_elements

    def clone(self) -> "DF11Block":
        """The same block in new device buffers."""
        return DF11Block(self.tensor.clone(), self.views)

    def set_max_workgroups(self, n: int) -> None:
        """Launch at most n workgroups (0: fill the GPU)."""
        self.tensor.set_max_workgroups(n)

    def decompress(self, scratch: Optional["torch.Tensor"] = None, stream=None,
                   events=None) -> Dict[str, "torch.Tensor"]:  # noqa: F821
        """Decode the block into scratch (at least n_elements bf16; a new one
        by default) and return a view per weight.  events: as for
        DF11Tensor.decompress."""
        import torch
        t = self.tensor
        if scratch is None:
            scratch = torch.empty(t.n_elements, dtype=torch.bfloat16, device=t.device)
        if scratch.dtype != torch.bfloat16 or not scratch.is_contiguous():
            raise ValueError("scratch must be a contiguous bfloat16 tensor")
        if not _on_device(scratch, t.device):
            raise ValueError("scratch must be on the stream's device")
        if events is not None:
            if scratch.numel() < t.n_elements:
                raise _lib.Df11Error(-5, "df11_decompress_timed")
            t._launch(scratch, stream, events)
        else:
            lib = _lib.load()
            _lib.check(lib.df11_decompress_block(ctypes.byref(t.device_stream()), ctypes.c_void_p(scratch.data_ptr()),
                                                 scratch.numel(), t._claim(stream)), "df11_decompress_block")
        cached, views = self._view_cache
        if cached is not scratch:  # the views of a scratch buffer are built once
            flat = scratch.reshape(-1)
            views = {name: flat[off:off + int(np.prod(shape))].view(shape) for name, off, shape in self.views}
            self._view_cache = (scratch, views)
        return views


def decompress_batch(tensors: Sequence[DF11Tensor], outs: Sequence["torch.Tensor"], stream=None,  # noqa: F821
                     events=None) -> None:
    """Decode several streams, each with its own codebook, in one launch:
    outs[i] (a contiguous bf16 tensor of tensors[i].n_elements elements)
    receives tensors[i].  All streams must use the same decode-table width.
    events: as for DF11Tensor.decompress, recorded at the batched kernel's
    own start and end (df11_decompress_batch_timed)."""
    import torch
    if len(tensors) != len(outs):
        raise ValueError("one output per stream")
    for t, o in zip(tensors, outs):
        if o.dtype != torch.bfloat16 or o.numel() != t.n_elements or not o.is_contiguous():
            raise ValueError("each out must be a contiguous bfloat16 tensor with its stream's element count")
        if not (_on_device(o, tensors[0].device) and _on_device(o, t.device)):
            raise ValueError("every stream and output must be on one device")
    n = len(tensors)
    arr = (_lib.DeviceStream * max(n, 1))(*[t.device_stream() for t in tensors])
    ptrs = (ctypes.c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
    st = [t._claim(stream) for t in tensors][0] if n else ctypes.c_void_p(0)
    lib = _lib.load()
    if events is None:
        _lib.check(lib.df11_decompress_batch(arr, n, ptrs, st), "df11_decompress_batch")
        return
    _lib.check(lib.df11_decompress_batch_timed(arr, n, ptrs, st, ctypes.c_void_p(_event_handle(events[0], st)),
                                               ctypes.c_void_p(_event_handle(events[1], st))),
               "df11_decompress_batch_timed")


def decompress_batch_noalloc(tensors: Sequence[DF11Tensor], outs: Sequence["torch.Tensor"],  # noqa: F821
                             stream=None) -> None:
    """decompress_batch through df11_decompress_batch_noalloc: the library
    allocates nothing and uses its own fixed work counters, which every call
    on a GPU shares (calls must not overlap in time on one GPU)."""
    import torch
    if len(tensors) != len(outs):
        raise ValueError("one output per stream")
    for t, o in zip(tensors, outs):
        if o.dtype != torch.bfloat16 or o.numel() != t.n_elements or not o.is_contiguous():
            raise ValueError("each out must be a contiguous bfloat16 tensor with its stream's element count")
        if not (_on_device(o, tensors[0].device) and _on_device(o, t.device)):
            raise ValueError("every stream and output must be on one device")
    n = len(tensors)
    arr = (_lib.DeviceStream * max(n, 1))(*[t.device_stream() for t in tensors])
    ptrs = (ctypes.c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
    st = tensors[0]._hip_stream(stream) if n else ctypes.c_void_p(0)
    _lib.check(_lib.load().df11_decompress_batch_noalloc(arr, n, ptrs, st), "df11_decompress_batch_noalloc")


class DF11BlockBatch:
    """Every linear weight of one transformer block as its own DF11 stream
    (a codebook per weight), decoded in one batched launch into one scratch
    buffer ("Dekompresi per transformer block")."""

    def __init__(self, tensors: List[DF11Tensor], views: List[Tuple[str, int, Tuple[int, ...]]], n_elements: int):
        self.tensors = tensors
        self.views = views
        self._n = n_elements
        self._view_cache = (None, None, None)

    @property
    def n_elements(self) -> int:
        """Scratch elements needed (each weight starts on a 16-byte boundary)."""
        return self._n

    def compressed_bytes(self) -> int:
        return sum(t.compressed_bytes() for t in self.tensors)

    def clone(self) -> "DF11BlockBatch":
        """The same streams in new device buffers."""
        return DF11BlockBatch([t.clone() for t in self.tensors], self.views, self._n)

    def set_max_workgroups(self, n: int) -> None:
        """Launch at most n workgroups in total (0: fill the GPU)."""
        for t in self.tensors:
            t.set_max_workgroups(n)

    def decompress(self, scratch: Optional["torch.Tensor"] = None, stream=None,
                   events=None) -> Dict[str, "torch.Tensor"]:  # noqa: F821
        """Decode every weight into scratch (at least n_elements bf16; a new
        one by default) in one launch and return a view per weight.  events:
        as for decompress_batch."""
        import torch
        if scratch is None:
            scratch = torch.empty(self._n, dtype=torch.bfloat16, device=self.tensors[0].device)
        if scratch.dtype != torch.bfloat16 or not scratch.is_contiguous() or scratch.numel() < self._n:
            raise ValueError("scratch must be a contiguous bfloat16 tensor of at least n_elements")
        if not _on_device(scratch, self.tensors[0].device):
            raise ValueError("scratch must be on the streams' device")
        cached, views, outs = self._view_cache
        if cached is not scratch:
            flat = scratch.reshape(-1)
            outs = [flat[off:off + int(np.prod(shape))] for _, off, shape in self.views]
            views = {name: o.view(shape) for (name, _, shape), o in zip(self.views, outs)}
            self._view_cache = (scratch, views, outs)
        decompress_batch(self.tensors, outs, stream=stream, events=events)
        return views


def compress_block(weights: Union[Dict[str, ArrayLike], List[Tuple[str, ArrayLike]]], device="cuda",
                   decode_table_bits: int = DEFAULT_DECODE_TABLE_BITS,
                   codebook: str = "shared", layout: str = "rows") -> Union[DF11Block, DF11BlockBatch]:
    """Encode a block's weights for decompression in one launch.

    codebook="shared": concatenate them row-major in the given order, build
    one codebook from the summed histogram and encode one stream (DF11Block).
    codebook="per_weight": one stream and codebook per weight, decoded by a
    batched launch (DF11BlockBatch, at most 16 weights); with
    layout="mfma_tiles" each weight is stored in the order of the
    matrix-core product (DF11Tensor.matmul, matmul_batch) and still
    decompresses row-major."""
    items = list(weights.items()) if isinstance(weights, dict) else list(weights)
    if layout != "rows" and codebook != "per_weight":
        raise ValueError("layout='mfma_tiles' needs codebook='per_weight'")
    if codebook == "per_weight":
        tensors, views, off = [], [], 0
        for name, w in items:
            shape = tuple(int(s) for s in w.shape)
            tensors.append(compress(_u16(w), shape=shape, device=device, decode_table_bits=decode_table_bits,
                                    layout=layout))
            views.append((name, off, shape))
            off += (int(np.prod(shape)) + 7) // 8 * 8
        return DF11BlockBatch(tensors, views, off)
    if codebook != "shared":
        raise ValueError("codebook must be 'shared' or 'per_weight'")
    parts, views, off = [], [], 0
    for name, w in items:
        shape = tuple(int(s) for s in w.shape)
        flat = _u16(w)
        parts.append(flat)
        views.append((name, off, shape))
        off += flat.size
    data = np.concatenate(parts) if parts else np.zeros(0, dtype=np.uint16)
    t = compress(data, shape=(data.size,), device=device, decode_table_bits=decode_table_bits)
    return DF11Block(t, views)


# ---------------------------------------------------------------------------
# rANS exponent coder (format in include/df11.h): the alternative entropy
# coder that the discussion on the page names as the SIMD-friendlier one.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class RansHostStream:
    """An rANS-coded stream in host memory."""

    header: _lib.RansHeader
    freq: np.ndarray          # 256 uint32 frequencies summing to 2^12
    states: np.ndarray        # n_segments * 64 uint32 start states
    word_offsets: np.ndarray  # n_segments + 1 uint32
    words: np.ndarray         # n_words uint16
    sm: np.ndarray            # N sign/mantissa bytes

    @property
    def n_elements(self) -> int:
        return int(self.header.n_elements)

    def compressed_bytes(self) -> int:
        """Frequencies (2 bytes each) + start states + word offsets + words +
        sign/mantissa bytes."""
        return int(2 * 256 + 4 * self.states.size + 4 * self.word_offsets.size + 2 * self.words.size
                   + self.sm.size)


def rans_quantize(hist: np.ndarray) -> np.ndarray:
    hist = np.ascontiguousarray(hist, dtype=np.uint64)
    freq = np.zeros(256, np.uint32)
    _lib.check(_lib.load().df11_rans_quantize(_ptr(hist, ctypes.c_uint64), _ptr(freq, ctypes.c_uint32)),
               "df11_rans_quantize")
    return freq


def rans_encode(bf16: ArrayLike, freq: Optional[np.ndarray] = None) -> RansHostStream:
    """rANS-encode BF16 data on the host (frequencies from the data's own
    histogram unless given)."""
    w = _u16(bf16)
    lib = _lib.load()
    if freq is None:
        freq = rans_quantize(histogram(w))
    freq = np.ascontiguousarray(freq, dtype=np.uint32)
    seg = _lib.RANS_LANES * _lib.RANS_STEPS
    n_seg = (w.size + seg - 1) // seg
    states = np.empty(max(n_seg * _lib.RANS_LANES, 1), np.uint32)
    offsets = np.empty(n_seg + 1, np.uint32)
    words = np.empty(max(w.size, 1), np.uint16)
    sm = np.empty(max(w.size, 1), np.uint8)
    h = _lib.RansHeader()
    _lib.check(lib.df11_rans_encode(_ptr(freq, ctypes.c_uint32), _ptr(w, ctypes.c_uint16), w.size,
                                    _ptr(states, ctypes.c_uint32), _ptr(offsets, ctypes.c_uint32),
                                    _ptr(words, ctypes.c_uint16), words.size, _ptr(sm, ctypes.c_uint8),
                                    ctypes.byref(h)), "df11_rans_encode")
    return RansHostStream(h, freq, states[:n_seg * _lib.RANS_LANES], offsets, words[:h.n_words].copy(),
                          sm[:w.size])


def rans_table(freq: np.ndarray) -> np.ndarray:
    table = np.empty(_lib.RANS_TABLE_ENTRIES, np.uint32)
    _lib.check(_lib.load().df11_rans_build_table(_ptr(np.ascontiguousarray(freq, dtype=np.uint32), ctypes.c_uint32),
                                                 _ptr(table, ctypes.c_uint32)), "df11_rans_build_table")
    return table


class DF11RansTensor:
    """An rANS-coded stream resident in GPU memory, decompressed on demand."""

    def __init__(self, host: RansHostStream, shape: Sequence[int], device="cuda"):
        import torch
        self.shape = tuple(int(s) for s in shape)
        self.device = torch.device(device)
        self.host_header = host.header
        n = host.n_elements

        def up(a: np.ndarray, size: int) -> "torch.Tensor":
            b = np.zeros(max(size, 16), dtype=np.uint8)
            raw = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
            b[:raw.size] = raw
            return torch.from_numpy(b).to(self.device)

        n_words = int(host.header.n_words)
        slots = (n_words + 7) // 8 * 8 + 8  # the decoder reads words 8 at a time
        self._bufs = {
            # (an empty stream has no frequencies and is never decoded)
            "table": up(rans_table(host.freq) if n else np.zeros(_lib.RANS_TABLE_ENTRIES, np.uint32),
                        4 * _lib.RANS_TABLE_ENTRIES),
            "states": up(host.states, 4 * host.states.size),
            "word_offsets": up(host.word_offsets, 4 * host.word_offsets.size),
            "words": up(host.words, 2 * slots),
            "sm": up(host.sm, (n + 63) // 64 * 64),
        }
        self._compressed_bytes = host.compressed_bytes()
        s = _lib.RansDeviceStream()
        s.h = host.header
        for name, t in self._bufs.items():
            setattr(s, name, t.data_ptr())
        self._stream_struct = s
        # The uploads and the counters' zero fill ran on the current stream:
        # finish them, so that a first launch on any stream sees them.
        torch.cuda.current_stream(self.device).synchronize()

    @property
    def n_elements(self) -> int:
        return int(self.host_header.n_elements)

    @property
    def header(self) -> _lib.RansHeader:
        return self.host_header

    def clone(self) -> "DF11RansTensor":
        """The same stream in new device buffers."""
        import copy
        import torch
        c = copy.copy(self)
        c._bufs = {name: t.clone() for name, t in self._bufs.items()}
        s = _lib.RansDeviceStream.from_buffer_copy(self._stream_struct)
        for name, t in c._bufs.items():
            setattr(s, name, t.data_ptr())
        c._stream_struct = s
        torch.cuda.current_stream(self.device).synchronize()
        return c

    def compressed_bytes(self) -> int:
        return self._compressed_bytes

    def decompress(self, out: Optional["torch.Tensor"] = None, stream=None, events=None) -> "torch.Tensor":  # noqa: F821
        """Decode into out (a new bf16 tensor of the original shape by
        default) on stream (torch's current stream by default); events as
        for DF11Tensor.decompress."""
        import torch
        if out is None:
            out = torch.empty(self.shape, dtype=torch.bfloat16, device=self.device)
        if out.dtype != torch.bfloat16 or out.numel() != self.n_elements or not out.is_contiguous():
            raise ValueError("out must be a contiguous bfloat16 tensor with the stream's element count")
        if not _on_device(out, self.device):
            raise ValueError("out must be on the stream's device")
        lib = _lib.load()
        st = DF11Tensor._hip_stream(self, stream)
        if events is None:
            _lib.check(lib.df11_rans_decompress(ctypes.byref(self._stream_struct), ctypes.c_void_p(out.data_ptr()),
                                                st), "df11_rans_decompress")
        else:
            start, stop = events
            _lib.check(lib.df11_rans_decompress_timed(ctypes.byref(self._stream_struct),
                                                      ctypes.c_void_p(out.data_ptr()), st,
                                                      ctypes.c_void_p(_event_handle(start, st)),
                                                      ctypes.c_void_p(_event_handle(stop, st))),
                       "df11_rans_decompress_timed")
        return out


def rans_compress(tensor: ArrayLike, shape: Optional[Sequence[int]] = None, device="cuda") -> DF11RansTensor:
    """rANS-encode a BF16 tensor on the host and upload the stream."""
    if shape is None:
        shape = tuple(tensor.shape)
    return DF11RansTensor(rans_encode(tensor), shape, device=device)
