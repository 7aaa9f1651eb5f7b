"""MI355X (gfx950) LSD radix sort: thin Python binding over the C ABI.

Every step of every sort runs in the HIP kernels of ``liblsd_radix_sort.so``;
this module only checks tensor shapes/dtypes, allocates outputs and the
workspace with torch, and passes raw device pointers and the current HIP
stream.  The entry points have the C ABI's names (include/lsd_radix_sort.h):

    radix_sort_keys(keys, begin_bit=0, end_bit=32, digit_bits=8)
    radix_sort_pairs(keys, values, begin_bit=0, end_bit=32, digit_bits=8)
    segmented_row_sort(x, descending=False, digit_bits=8)
    radix_sort_digit_histograms(keys, begin_bit, end_bit, digit_bits)

u32 data is accepted as torch.uint32 or torch.int32 (bit patterns); outputs
have the input's dtype.  There is no CPU fallback: without the built library or
a GPU these calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsd_radix_sort.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "lsd_radix_sort.h")

LRS_OK = 0
LRS_DTYPE_FP16 = 0
LRS_DTYPE_BF16 = 1
LRS_KEY_U32 = 0
LRS_KEY_I32 = 1
LRS_KEY_F32 = 2
LRS_KEY_U64 = 3
LRS_KEY_I64 = 4
LRS_KEY_F64 = 5
LRS_SCAN_LOOKBACK = 0
LRS_SCAN_REDUCE_THEN_SCAN = 1
_SCAN_STRATEGIES = {"lookback": LRS_SCAN_LOOKBACK, "reduce-then-scan": LRS_SCAN_REDUCE_THEN_SCAN}
STATUS_NAMES = {
    0: "LRS_OK", 1: "LRS_ERR_NULL_POINTER", 2: "LRS_ERR_BIT_RANGE", 3: "LRS_ERR_DIGIT_BITS",
    4: "LRS_ERR_SIZE", 5: "LRS_ERR_ALIASING", 6: "LRS_ERR_WORKSPACE_TOO_SMALL", 7: "LRS_ERR_DTYPE",
    8: "LRS_ERR_HIP", 9: "LRS_ERR_ALIGNMENT",
}
_VALUE_ERRORS = {1, 2, 3, 4, 5, 6, 7, 9}

_lib = None


class RadixSortError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class RadixSortArgumentError(RadixSortError, ValueError):
    pass


def load_library():
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m lsd_radix_sort_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, u64, i64, c_int, szt = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.radix_sort_workspace_size.argtypes = [u64, c_int, c_int, c_int, c_int]
    lib.radix_sort_workspace_size.restype = szt
    lib.radix_sort_keys.argtypes = [P, P, u64, c_int, c_int, c_int, P, szt, P]
    lib.radix_sort_keys.restype = c_int
    lib.radix_sort_pairs.argtypes = [P, P, P, P, u64, c_int, c_int, c_int, P, szt, P]
    lib.radix_sort_pairs.restype = c_int
    lib.segmented_row_sort_workspace_size.argtypes = [i64, i64, c_int]
    lib.segmented_row_sort_workspace_size.restype = szt
    lib.segmented_row_sort.argtypes = [P, P, P, i64, i64, c_int, c_int, c_int, P, szt, P]
    lib.segmented_row_sort.restype = c_int
    lib.segmented_row_sort_pairs.argtypes = [P, P, P, P, i64, i64, c_int, c_int, c_int, P, szt, P]
    lib.segmented_row_sort_pairs.restype = c_int
    lib.radix_sort_digit_histograms.argtypes = [P, u64, c_int, c_int, c_int, P, P]
    lib.radix_sort_digit_histograms.restype = c_int
    lib.radix_sort_copy_probe.argtypes = [P, P, szt, P]
    lib.radix_sort_copy_probe.restype = c_int
    lib.radix_sort_typed_workspace_size.argtypes = [u64, c_int, c_int, c_int, c_int, c_int]
    lib.radix_sort_typed_workspace_size.restype = szt
    lib.radix_sort_keys_typed.argtypes = [P, P, u64, c_int, c_int, c_int, c_int, c_int, P, szt, P]
    lib.radix_sort_keys_typed.restype = c_int
    lib.radix_sort_pairs_typed.argtypes = [P, P, P, P, u64, c_int, c_int, c_int, c_int, c_int, P, szt, P]
    lib.radix_sort_pairs_typed.restype = c_int
    lib.radix_sort_set_scan_strategy.argtypes = [c_int]
    lib.radix_sort_set_scan_strategy.restype = c_int
    lib.radix_sort_set_spin_limit.argtypes = [ctypes.c_uint32]
    lib.radix_sort_set_spin_limit.restype = ctypes.c_uint32
    lib.radix_sort_timing_begin.argtypes = []
    lib.radix_sort_timing_begin.restype = c_int
    lib.radix_sort_timing_end.argtypes = [P, P]
    lib.radix_sort_timing_end.restype = c_int
    lib.radix_sort_status_string.argtypes = [c_int]
    lib.radix_sort_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().radix_sort_status_string(status).decode()


def _check(status: int, what: str):
    if status != LRS_OK:
        if status in _VALUE_ERRORS:
            raise RadixSortArgumentError(status, what)
        raise RadixSortError(status, what)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _u32_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in (torch.uint32, torch.int32):
        raise ValueError(f"{name} must be uint32 or int32, got {t.dtype}")
    if t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D tensor")
    return t


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def radix_sort_workspace_size(n: int, begin_bit: int = 0, end_bit: int = 32, digit_bits: int = 8,
                              with_values: bool = False) -> int:
    return int(load_library().radix_sort_workspace_size(n, begin_bit, end_bit, digit_bits, int(with_values)))


def segmented_row_sort_workspace_size(rows: int, n: int, digit_bits: int = 8) -> int:
    return int(load_library().segmented_row_sort_workspace_size(rows, n, digit_bits))


def radix_sort_keys(keys: torch.Tensor, begin_bit: int = 0, end_bit: int = 32, digit_bits: int = 8,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Stable LSD sort of u32 keys by bits [begin_bit, end_bit); returns the sorted keys."""
    lib = load_library()
    keys = _u32_tensor(keys, "keys")
    n = keys.numel()
    if out is None:
        out = torch.empty_like(keys)
    if workspace is None:
        workspace = _workspace(lib.radix_sort_workspace_size(n, begin_bit, end_bit, digit_bits, 0), keys.device)
    _check(lib.radix_sort_keys(_ptr(keys), _ptr(out), n, begin_bit, end_bit, digit_bits,
                               _ptr(workspace), workspace.numel(), _stream(keys)), "radix_sort_keys")
    return out


def radix_sort_pairs(keys: torch.Tensor, values: torch.Tensor, begin_bit: int = 0, end_bit: int = 32,
                     digit_bits: int = 8, keys_out: torch.Tensor | None = None,
                     values_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Stable LSD sort of u32 keys carrying u32 values; returns (keys, values)."""
    lib = load_library()
    keys = _u32_tensor(keys, "keys")
    values = _u32_tensor(values, "values")
    n = keys.numel()
    if values.numel() != n:
        raise ValueError("keys and values differ in length")
    if keys_out is None:
        keys_out = torch.empty_like(keys)
    if values_out is None:
        values_out = torch.empty_like(values)
    if workspace is None:
        workspace = _workspace(lib.radix_sort_workspace_size(n, begin_bit, end_bit, digit_bits, 1), keys.device)
    _check(lib.radix_sort_pairs(_ptr(keys), _ptr(values), _ptr(keys_out), _ptr(values_out), n, begin_bit,
                                end_bit, digit_bits, _ptr(workspace), workspace.numel(), _stream(keys)),
           "radix_sort_pairs")
    return keys_out, values_out


_KEY_TYPES = {"u32": LRS_KEY_U32, "i32": LRS_KEY_I32, "f32": LRS_KEY_F32,
              "u64": LRS_KEY_U64, "i64": LRS_KEY_I64, "f64": LRS_KEY_F64}
_KEY_DTYPES = {torch.uint32: "u32", torch.int32: "i32", torch.float32: "f32",
               torch.uint64: "u64", torch.int64: "i64", torch.float64: "f64"}


def _typed_keys(keys: torch.Tensor, key_type: str | None):
    if not isinstance(keys, torch.Tensor) or not keys.is_cuda:
        raise ValueError("keys must be a GPU tensor")
    if keys.dtype not in _KEY_DTYPES:
        raise ValueError(f"keys must be a 32- or 64-bit integer or float tensor, got {keys.dtype}")
    if keys.dim() != 1 or not keys.is_contiguous():
        raise ValueError("keys must be a contiguous 1-D tensor")
    kt = _KEY_DTYPES[keys.dtype] if key_type is None else key_type
    if kt not in _KEY_TYPES:
        raise ValueError(f"key_type must be one of {sorted(_KEY_TYPES)}")
    if (kt.endswith("64")) != (keys.element_size() == 8):
        raise ValueError(f"key_type {kt} does not match a {keys.element_size() * 8}-bit tensor")
    return _KEY_TYPES[kt]


def radix_sort_typed_workspace_size(n: int, key_type: str, begin_bit: int = 0, end_bit: int | None = None,
                                    digit_bits: int = 8, with_values: bool = False) -> int:
    if end_bit is None:
        end_bit = 64 if key_type.endswith("64") else 32
    return int(load_library().radix_sort_typed_workspace_size(n, _KEY_TYPES[key_type], begin_bit, end_bit,
                                                              digit_bits, int(with_values)))


def radix_sort_keys_typed(keys: torch.Tensor, descending: bool = False, key_type: str | None = None,
                          begin_bit: int = 0, end_bit: int | None = None, digit_bits: int = 8,
                          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Stable sort of 32- or 64-bit keys as unsigned, signed or float (from the dtype
    unless key_type is given); end_bit defaults to the key width."""
    lib = load_library()
    kt = _typed_keys(keys, key_type)
    if end_bit is None:
        end_bit = 8 * keys.element_size()
    n = keys.numel()
    if out is None:
        out = torch.empty_like(keys)
    if workspace is None:
        workspace = _workspace(lib.radix_sort_typed_workspace_size(n, kt, begin_bit, end_bit, digit_bits, 0),
                               keys.device)
    _check(lib.radix_sort_keys_typed(_ptr(keys), _ptr(out), n, kt, int(descending), begin_bit, end_bit,
                                     digit_bits, _ptr(workspace), workspace.numel(), _stream(keys)),
           "radix_sort_keys_typed")
    return out


def radix_sort_pairs_typed(keys: torch.Tensor, values: torch.Tensor, descending: bool = False,
                           key_type: str | None = None, begin_bit: int = 0, end_bit: int | None = None,
                           digit_bits: int = 8, keys_out: torch.Tensor | None = None,
                           values_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """As radix_sort_keys_typed, carrying one 32-bit payload per key; returns (keys, values)."""
    lib = load_library()
    kt = _typed_keys(keys, key_type)
    if end_bit is None:
        end_bit = 8 * keys.element_size()
    values = _u32_tensor(values, "values")
    n = keys.numel()
    if values.numel() != n:
        raise ValueError("keys and values differ in length")
    if keys_out is None:
        keys_out = torch.empty_like(keys)
    if values_out is None:
        values_out = torch.empty_like(values)
    if workspace is None:
        workspace = _workspace(lib.radix_sort_typed_workspace_size(n, kt, begin_bit, end_bit, digit_bits, 1),
                               keys.device)
    _check(lib.radix_sort_pairs_typed(_ptr(keys), _ptr(values), _ptr(keys_out), _ptr(values_out), n, kt,
                                      int(descending), begin_bit, end_bit, digit_bits, _ptr(workspace),
                                      workspace.numel(), _stream(keys)), "radix_sort_pairs_typed")
    return keys_out, values_out


def segmented_row_sort(x: torch.Tensor, descending: bool = False, digit_bits: int = 8,
                       values_out: torch.Tensor | None = None, indices_out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None):
    """Sort every row of a 2-D fp16/bf16 GPU tensor; returns (values, int64 column indices)."""
    lib = load_library()
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if x.dtype == torch.float16:
        dtype = LRS_DTYPE_FP16
    elif x.dtype == torch.bfloat16:
        dtype = LRS_DTYPE_BF16
    else:
        raise ValueError(f"x must be float16 or bfloat16, got {x.dtype}")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D tensor")
    rows, n = x.shape
    if values_out is None:
        values_out = torch.empty_like(x)
    if indices_out is None:
        indices_out = torch.empty((rows, n), dtype=torch.int64, device=x.device)
    if workspace is None:
        workspace = _workspace(lib.segmented_row_sort_workspace_size(rows, n, digit_bits), x.device)
    _check(lib.segmented_row_sort(_ptr(x), _ptr(values_out), _ptr(indices_out), rows, n, dtype,
                                  int(descending), digit_bits, _ptr(workspace), workspace.numel(),
                                  _stream(x)), "segmented_row_sort")
    return values_out, indices_out


def segmented_row_sort_pairs(x: torch.Tensor, payload: torch.Tensor, descending: bool = False,
                             digit_bits: int = 8, values_out: torch.Tensor | None = None,
                             payload_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Sort every row of a 2-D fp16/bf16 GPU tensor carrying a same-shape 32-bit payload;
    returns (values, payload)."""
    lib = load_library()
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if x.dtype == torch.float16:
        dtype = LRS_DTYPE_FP16
    elif x.dtype == torch.bfloat16:
        dtype = LRS_DTYPE_BF16
    else:
        raise ValueError(f"x must be float16 or bfloat16, got {x.dtype}")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D tensor")
    if (not isinstance(payload, torch.Tensor) or not payload.is_cuda or payload.shape != x.shape
            or payload.element_size() != 4 or not payload.is_contiguous()):
        raise ValueError("payload must be a contiguous 32-bit GPU tensor of x's shape")
    rows, n = x.shape
    if values_out is None:
        values_out = torch.empty_like(x)
    if payload_out is None:
        payload_out = torch.empty_like(payload)
    if workspace is None:
        workspace = _workspace(lib.segmented_row_sort_workspace_size(rows, n, digit_bits), x.device)
    _check(lib.segmented_row_sort_pairs(_ptr(x), _ptr(payload), _ptr(values_out), _ptr(payload_out), rows, n,
                                        dtype, int(descending), digit_bits, _ptr(workspace), workspace.numel(),
                                        _stream(x)), "segmented_row_sort_pairs")
    return values_out, payload_out


def radix_sort_digit_histograms(keys: torch.Tensor, begin_bit: int = 0, end_bit: int = 32,
                                digit_bits: int = 8) -> torch.Tensor:
    """All passes' digit counts from one read of the keys: int32 [passes, 2^b] (u32 counts)."""
    lib = load_library()
    keys = _u32_tensor(keys, "keys")
    passes = -(-(end_bit - begin_bit) // digit_bits) if end_bit > begin_bit else 0
    hist = torch.empty((max(passes, 1), 1 << digit_bits), dtype=torch.int32, device=keys.device)
    _check(lib.radix_sort_digit_histograms(_ptr(keys), keys.numel(), begin_bit, end_bit, digit_bits,
                                           _ptr(hist), _stream(keys)), "radix_sort_digit_histograms")
    return hist


def copy_probe(src: torch.Tensor, dst: torch.Tensor) -> None:
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _check(lib.radix_sort_copy_probe(_ptr(src), _ptr(dst), nbytes, _stream(src)), "copy_probe")


def radix_sort_set_scan_strategy(strategy: str) -> str:
    """How single-row sorts find each tile's output offsets: "lookback" (default)
    or "reduce-then-scan".  Returns the previous strategy."""
    if strategy not in _SCAN_STRATEGIES:
        raise ValueError(f"strategy must be one of {sorted(_SCAN_STRATEGIES)}")
    old = load_library().radix_sort_set_scan_strategy(_SCAN_STRATEGIES[strategy])
    return {v: k for k, v in _SCAN_STRATEGIES.items()}[old]


def radix_sort_set_spin_limit(polls: int) -> int:
    """Bound, in polls, on a sweep tile's wait for an earlier tile's counts.

    Past it the tile counts its prefix from the keys (same result); 0 makes
    every tile do so.  Returns the previous bound.
    """
    if not 0 <= polls <= 0xFFFFFFFF:
        raise ValueError("polls must fit in 32 bits")
    return int(load_library().radix_sort_set_spin_limit(polls))


class KernelTimer:
    """Context manager: HIP-event times of every kernel the library enqueues inside it.

    After exit, ``ms`` and ``launches`` hold per-kind sums for the kinds
    "clear", "histogram", "sweep", "copy", "resident".
    """
    KINDS = ("clear", "histogram", "sweep", "copy", "resident")

    def __enter__(self):
        _check(load_library().radix_sort_timing_begin(), "timing_begin")
        return self

    def __exit__(self, *exc):
        ms = (ctypes.c_double * 5)()
        nl = (ctypes.c_int * 5)()
        _check(load_library().radix_sort_timing_end(ms, nl), "timing_end")
        self.ms = dict(zip(self.KINDS, list(ms)))
        self.launches = dict(zip(self.KINDS, list(nl)))
        return False
