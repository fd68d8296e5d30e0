"""ctypes view of the C ABI in include/df11.h (argument marshalling only).

Loading fails loudly when libdf11.so has not been built: there is no fallback
implementation of any step.
"""

from __future__ import annotations

import ctypes
import os

# DF11_LIB_PATH names another build of the same library (the sanitizer build
# of the CPU tests); by default the in-tree libdf11.so.
LIB_PATH = os.environ.get("DF11_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdf11.so")

DF11_OK = 0
STATUS_NAMES = {
    0: "DF11_OK",
    -1: "DF11_E_INVALID_ARG",
    -2: "DF11_E_RESERVED_EXPONENT",
    -3: "DF11_E_CODE_TOO_LONG",
    -4: "DF11_E_TOO_MANY_LUTS",
    -5: "DF11_E_BUFFER_TOO_SMALL",
    -6: "DF11_E_BAD_STREAM",
    -7: "DF11_E_TOO_LARGE",
    -8: "DF11_E_HIP",
}
MAX_LUTS = 17
SCHEDULE_WORDS = 144  # DF11_SCHEDULE_WORDS
MAX_BATCH = 16  # DF11_MAX_BATCH
MAX_ELEMENTS = (1 << 32) - (1 << 16)  # DF11_MAX_ELEMENTS
LINEAR_MAX_TOKENS = 8  # DF11_LINEAR_MAX_TOKENS
LINEAR_MIN_IN_FEATURES = 512  # DF11_LINEAR_MIN_IN_FEATURES
RANS_PROB_BITS = 12  # DF11_RANS_PROB_BITS
RANS_LANES = 64  # DF11_RANS_LANES
RANS_STEPS = 512  # DF11_RANS_STEPS
RANS_TABLE_ENTRIES = 4096  # DF11_RANS_TABLE_ENTRIES

# Every function the header declares; the ABI test checks each is exported.
EXPORTED = [
    "df11_histogram",
    "df11_build_codebook",
    "df11_plan",
    "df11_encode",
    "df11_tile_order",
    "df11_decode_table_bytes",
    "df11_build_decode_table",
    "df11_decompress",
    "df11_decompress_block",
    "df11_decompress_batch",
    "df11_decompress_timed",
    "df11_decompress_batch_timed",
    "df11_decompress_batch_noalloc",
    "df11_matmul",
    "df11_matmul_acc",
    "df11_matmul_timed",
    "df11_matmul_batch",
    "df11_linear",
    "df11_linear_timed",
    "df11_linear_batch",
    "df11_linear_acc",
    "df11_linear_batch_acc",
    "df11_rans_quantize",
    "df11_rans_encode",
    "df11_rans_build_table",
    "df11_rans_decompress",
    "df11_rans_decompress_timed",
    "df11_status_str",
]


class Df11Error(RuntimeError):
    """A DF11 C-ABI call returned a non-zero status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {STATUS_NAMES.get(status, status)}")


class Codebook(ctypes.Structure):
    _fields_ = [
        ("code_lengths", ctypes.c_uint8 * 256),
        ("codes", ctypes.c_uint32 * 256),
        ("luts", (ctypes.c_uint8 * 256) * MAX_LUTS),
        ("n_luts", ctypes.c_uint32),
        ("max_len", ctypes.c_uint32),
    ]


class Layout(ctypes.Structure):
    _fields_ = [("bytes_per_thread", ctypes.c_uint32), ("threads_per_group", ctypes.c_uint32)]


class Header(ctypes.Structure):
    _fields_ = [
        ("n_elements", ctypes.c_uint64),
        ("total_bits", ctypes.c_uint64),
        ("bytes_per_thread", ctypes.c_uint32),
        ("threads_per_group", ctypes.c_uint32),
        ("n_threads", ctypes.c_uint64),
        ("n_groups", ctypes.c_uint64),
        ("n_luts", ctypes.c_uint32),
        ("max_len", ctypes.c_uint32),
        ("enc_bytes", ctypes.c_uint64),
        ("sm_bytes", ctypes.c_uint64),
        ("gaps_bytes", ctypes.c_uint64),
        ("out_pos_bytes", ctypes.c_uint64),
        ("max_group_elems", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class DeviceStream(ctypes.Structure):
    _fields_ = [
        ("h", Header),
        ("enc", ctypes.c_void_p),
        ("sm", ctypes.c_void_p),
        ("gaps", ctypes.c_void_p),
        ("out_pos", ctypes.c_void_p),
        ("luts", ctypes.c_void_p),
        ("code_lengths", ctypes.c_void_p),
        ("decode_table", ctypes.c_void_p),
        ("decode_table_bits", ctypes.c_uint32),
        ("groups_per_workgroup", ctypes.c_uint32),
        ("schedule", ctypes.c_void_p),
        ("max_workgroups", ctypes.c_uint32),
        ("tile_cols", ctypes.c_uint32),
    ]


class RansHeader(ctypes.Structure):
    _fields_ = [
        ("n_elements", ctypes.c_uint64),
        ("n_segments", ctypes.c_uint64),
        ("n_words", ctypes.c_uint64),
        ("prob_bits", ctypes.c_uint32),
        ("lanes", ctypes.c_uint32),
        ("steps", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class RansDeviceStream(ctypes.Structure):
    _fields_ = [
        ("h", RansHeader),
        ("table", ctypes.c_void_p),
        ("states", ctypes.c_void_p),
        ("word_offsets", ctypes.c_void_p),
        ("words", ctypes.c_void_p),
        ("sm", ctypes.c_void_p),
    ]


_LIB = None


def load() -> ctypes.CDLL:
    """Load libdf11.so (after torch, so the HIP runtime torch loaded is shared)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          f"python -m entropy_decoding_df11_amd._build")
    try:
        import torch  # noqa: F401  (loads the HIP runtime first)
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    sig = {
        "df11_histogram": (ctypes.c_int, [u16p, ctypes.c_uint64, u64p]),
        "df11_build_codebook": (ctypes.c_int, [u64p, ctypes.POINTER(Codebook)]),
        "df11_plan": (ctypes.c_int, [ctypes.POINTER(Codebook), u64p, ctypes.c_uint64, ctypes.POINTER(Layout),
                                     ctypes.POINTER(Header)]),
        "df11_encode": (ctypes.c_int, [ctypes.POINTER(Codebook), u16p, ctypes.c_uint64, ctypes.POINTER(Layout),
                                       ctypes.POINTER(Header), u8p, u8p, u8p, u32p]),
        "df11_decode_table_bytes": (ctypes.c_uint64, [ctypes.c_uint32]),
        "df11_build_decode_table": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.c_uint32, ctypes.c_void_p,
                                                   ctypes.c_uint64]),
        "df11_decompress": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_void_p]),
        "df11_decompress_block": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_uint64,
                                                 ctypes.c_void_p]),
        "df11_decompress_batch": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
        "df11_decompress_timed": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p]),
        "df11_decompress_batch_timed": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_uint32,
                                                       ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                       ctypes.c_void_p, ctypes.c_void_p]),
        "df11_decompress_batch_noalloc": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_uint32,
                                                         ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
        "df11_tile_order": (ctypes.c_int, [u16p, ctypes.c_uint64, ctypes.c_uint64, u16p]),
        "df11_matmul": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]),
        "df11_matmul_acc": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_uint32,
                                           ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]),
        "df11_matmul_timed": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_uint32,
                                             ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]),
        "df11_matmul_batch": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_uint32,
                                             ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32, u32p, u32p,
                                             ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]),
        "df11_linear": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]),
        "df11_linear_acc": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_uint32,
                                           ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]),
        "df11_linear_timed": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_void_p, ctypes.c_uint32,
                                             ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]),
        "df11_linear_batch": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_uint32, ctypes.c_void_p,
                                             ctypes.c_uint32, ctypes.c_uint32, u32p,
                                             ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p]),
        "df11_linear_batch_acc": (ctypes.c_int, [ctypes.POINTER(DeviceStream), ctypes.c_uint32, ctypes.c_void_p,
                                                 ctypes.c_uint32, ctypes.c_uint32, u32p,
                                                 ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]),
        "df11_rans_quantize": (ctypes.c_int, [u64p, u32p]),
        "df11_rans_encode": (ctypes.c_int, [u32p, u16p, ctypes.c_uint64, u32p, u32p, u16p, ctypes.c_uint64, u8p,
                                            ctypes.POINTER(RansHeader)]),
        "df11_rans_build_table": (ctypes.c_int, [u32p, u32p]),
        "df11_rans_decompress": (ctypes.c_int, [ctypes.POINTER(RansDeviceStream), ctypes.c_void_p, ctypes.c_void_p]),
        "df11_rans_decompress_timed": (ctypes.c_int, [ctypes.POINTER(RansDeviceStream), ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
        "df11_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(status: int, what: str) -> None:
    if status != DF11_OK:
        raise Df11Error(status, what)
