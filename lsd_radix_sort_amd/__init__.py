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
have the input's dtype.  Outputs and the workspace may be passed in; each must
then be a contiguous GPU tensor on the input's device of the exact shape and
element size the call writes (the workspace: uint8, at least the
*_workspace_size() bytes), else RadixSortArgumentError is raised before
anything reaches the library.  Per-call options (scan strategy, look-back wait
bound, kernel timer) go in a SortOptions; nothing is global.  There is no CPU
fallback: without the built library or a GPU these calls raise.
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
    8: "LRS_ERR_HIP", 9: "LRS_ERR_ALIGNMENT", 10: "LRS_ERR_OPTION",
}
_VALUE_ERRORS = {1, 2, 3, 4, 5, 6, 7, 9, 10}


class RadixSortError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class RadixSortArgumentError(RadixSortError, ValueError):
    """An argument the library (or this binding, status None) rejects."""

    def __init__(self, status, what: str):
        if status is None:
            self.status = None
            ValueError.__init__(self, what)
        else:
            super().__init__(status, what)


class _Options(ctypes.Structure):
    # mirrors struct lrs_options
    _fields_ = [("scan_strategy", ctypes.c_int), ("spin_limit", ctypes.c_uint32),
                ("prefix_from_keys", ctypes.c_int), ("wide_from", ctypes.c_uint64),
                ("timer", ctypes.c_void_p)]


_lib = None


def load_library():
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m lsd_radix_sort_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, u64, i64, c_int, szt = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    O = ctypes.POINTER(_Options)
    sigs = {
        "radix_sort_workspace_size": ([u64, c_int, c_int, c_int, c_int, O], szt),
        "radix_sort_keys": ([P, P, u64, c_int, c_int, c_int, P, szt, P, O], c_int),
        "radix_sort_pairs": ([P, P, P, P, u64, c_int, c_int, c_int, P, szt, P, O], c_int),
        "segmented_row_sort_workspace_size": ([i64, i64, c_int, O], szt),
        "segmented_row_sort": ([P, P, P, i64, i64, c_int, c_int, c_int, P, szt, P, O], c_int),
        "segmented_row_sort_pairs": ([P, P, P, P, i64, i64, c_int, c_int, c_int, P, szt, P, O], c_int),
        "radix_sort_digit_histograms": ([P, u64, c_int, c_int, c_int, P, P, O], c_int),
        "radix_sort_copy_probe": ([P, P, szt, P, O], c_int),
        "radix_sort_typed_workspace_size": ([u64, c_int, c_int, c_int, c_int, c_int, O], szt),
        "radix_sort_keys_typed": ([P, P, u64, c_int, c_int, c_int, c_int, c_int, P, szt, P, O], c_int),
        "radix_sort_pairs_typed": ([P, P, P, P, u64, c_int, c_int, c_int, c_int, c_int, P, szt, P, O], c_int),
        "radix_sort_pairs_no_alloc": ([P, P, P, P, u64, c_int, c_int, c_int, P, O], c_int),
        "radix_sort_timer_create": ([], P),
        "radix_sort_timer_read": ([P, P, P], c_int),
        "radix_sort_timer_destroy": ([P], None),
        "radix_sort_timer_trace_tiles": ([P, P, u64], c_int),
        "radix_sort_timer_trace_used": ([P, P], c_int),
        "radix_sort_status_string": ([c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().radix_sort_status_string(status).decode()


def _check(status: int, what: str):
    if status != LRS_OK:
        if status in _VALUE_ERRORS:
            raise RadixSortArgumentError(status, what)
        raise RadixSortError(status, what)


def _bad(msg: str):
    raise RadixSortArgumentError(None, msg)


# ------------------------------------------------------------------ options

class KernelTimer:
    """A library kernel timer (lrs_timer): pass it in SortOptions(timer=...) and
    every kernel those calls enqueue is timed by a pair of HIP events on its
    stream (stamped by the dispatch; recorded around each launch for calls
    over at most 65,536 elements).

    As a context manager, ``ms`` and ``launches`` hold per-kind sums ("clear",
    "histogram", "sweep", "copy", "resident") after exit; ``read()`` returns
    them at any time and empties the timer.
    """
    KINDS = ("clear", "histogram", "sweep", "copy", "resident")

    def __init__(self):
        self._lib = load_library()
        self.handle = self._lib.radix_sort_timer_create()
        if not self.handle:
            raise MemoryError("radix_sort_timer_create failed")
        self.ms, self.launches = {}, {}

    def read(self):
        ms = (ctypes.c_double * 5)()
        nl = (ctypes.c_int * 5)()
        _check(self._lib.radix_sort_timer_read(self.handle, ms, nl), "radix_sort_timer_read")
        return dict(zip(self.KINDS, list(ms))), dict(zip(self.KINDS, list(nl)))

    TRACE_WORDS = 12  # LRS_TILE_TRACE_WORDS: one tile's phase record

    def trace_tiles(self, buf: "torch.Tensor | None") -> None:
        """Give the timer a device buffer (int64, contiguous) for tile phase
        records, or None to detach it (libraries built with LRS_TILE_TRACE=1;
        others raise RadixSortArgumentError)."""
        if buf is None:
            _check(self._lib.radix_sort_timer_trace_tiles(self.handle, None, 0), "radix_sort_timer_trace_tiles")
            return
        if not buf.is_cuda or buf.dtype != torch.int64 or not buf.is_contiguous():
            _bad("trace buffer must be a contiguous int64 GPU tensor")
        _check(self._lib.radix_sort_timer_trace_tiles(self.handle, _ptr(buf), buf.numel()),
               "radix_sort_timer_trace_tiles")

    def trace_used(self) -> int:
        """Words of the trace buffer taken since it was set."""
        w = ctypes.c_uint64(0)
        _check(self._lib.radix_sort_timer_trace_used(self.handle, ctypes.byref(w)), "radix_sort_timer_trace_used")
        return w.value

    def __enter__(self):
        self.read()  # start empty
        return self

    def __exit__(self, *exc):
        self.ms, self.launches = self.read()
        return False

    def close(self):
        if self.handle:
            self._lib.radix_sort_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class SortOptions:
    """Per-call options (struct lrs_options); a call given none uses the defaults.

    scan: "lookback" (default) or "reduce-then-scan" -- how single-row sorts get
        each tile's output offsets (the result is identical).
    spin_limit: bound, in polls, on a tile's wait for an earlier tile's counts
        (None: the library default); past it the tile counts its prefix from the keys.
    prefix_from_keys: every tile counts its prefix from the keys (tests that path).
    wide_from: rows of at least this many elements (sorted by sweeps) take the
        sweep with 64-bit look-back words and store addresses (a test hook).
    timer: a KernelTimer recording every kernel of the call.
    """

    def __init__(self, scan: str = "lookback", spin_limit: int | None = None, prefix_from_keys: bool = False,
                 wide_from: int = 0, timer: KernelTimer | None = None):
        if scan not in _SCAN_STRATEGIES:
            _bad(f"scan must be one of {sorted(_SCAN_STRATEGIES)}")
        if spin_limit is not None and not 1 <= spin_limit <= 0xFFFFFFFF:
            _bad("spin_limit must be in [1, 2^32)")
        if not 0 <= wide_from < 1 << 64:
            _bad("wide_from must be a non-negative 64-bit count")
        self.timer = timer  # keeps the timer alive while the options are
        self._c = _Options(_SCAN_STRATEGIES[scan], spin_limit or 0, int(bool(prefix_from_keys)), int(wide_from),
                           timer.handle if timer is not None else None)

    def _ptr(self):
        return ctypes.byref(self._c)


def _opt(options: SortOptions | None):
    if options is None:
        return None
    if not isinstance(options, SortOptions):
        _bad("options must be a SortOptions")
    return options._ptr()


# --------------------------------------------------------------- validation

# torch's own getter of the current stream's raw handle (the public
# torch.cuda.current_stream(...).cuda_stream builds a Stream object and costs
# about 2 us a call, as much as a small sort's whole launch)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    """The handle of torch's current stream on t's device."""
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _gpu_input(t, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        _bad(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        _bad(f"{name} must be contiguous")


def _u32_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    _gpu_input(t, name)
    if t.dtype not in (torch.uint32, torch.int32):
        _bad(f"{name} must be uint32 or int32, got {t.dtype}")
    if t.dim() != 1:
        _bad(f"{name} must be a 1-D tensor")
    return t


def _same_device(t, name: str, device):
    if not isinstance(t, torch.Tensor):
        _bad(f"{name} must be a tensor")
    if t.device != device:
        _bad(f"{name} is on {t.device}, the input on {device}")


def check_output(t, name: str, device, element_size: int, shape) -> torch.Tensor:
    """A caller-supplied output must be a contiguous tensor on the input's
    device with exactly the shape and element size the call writes."""
    _same_device(t, name, device)
    if not t.is_contiguous():
        _bad(f"{name} must be contiguous")
    if t.element_size() != element_size:
        _bad(f"{name} must have {element_size}-byte elements, got {t.element_size()}")
    if tuple(t.shape) != tuple(shape):
        _bad(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def check_workspace(t, device, nbytes: int) -> torch.Tensor:
    """A caller-supplied workspace must be a contiguous uint8 tensor on the
    input's device holding at least nbytes bytes."""
    _same_device(t, "workspace", device)
    if t.dtype != torch.uint8 or not t.is_contiguous():
        _bad("workspace must be a contiguous uint8 tensor")
    if t.numel() < nbytes:
        _bad(f"workspace holds {t.numel()} bytes, the call needs {nbytes}")
    return t


def _output(t, name, like: torch.Tensor, element_size=None, shape=None, dtype=None):
    if t is None:
        return torch.empty(tuple(like.shape) if shape is None else shape,
                           dtype=like.dtype if dtype is None else dtype, device=like.device)
    return check_output(t, name, like.device, like.element_size() if element_size is None else element_size,
                        like.shape if shape is None else shape)


def _workspace(t, nbytes: int, device) -> torch.Tensor:
    if t is None:
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    return check_workspace(t, device, int(nbytes))


# -------------------------------------------------------------------- sorts

def radix_sort_workspace_size(n: int, begin_bit: int = 0, end_bit: int = 32, digit_bits: int = 8,
                              with_values: bool = False, options: SortOptions | None = None) -> int:
    return int(load_library().radix_sort_workspace_size(n, begin_bit, end_bit, digit_bits, int(with_values),
                                                        _opt(options)))


def segmented_row_sort_workspace_size(rows: int, n: int, digit_bits: int = 8,
                                      options: SortOptions | None = None) -> int:
    return int(load_library().segmented_row_sort_workspace_size(rows, n, digit_bits, _opt(options)))


def radix_sort_keys(keys: torch.Tensor, begin_bit: int = 0, end_bit: int = 32, digit_bits: int = 8,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    options: SortOptions | None = None) -> torch.Tensor:
    """Stable LSD sort of u32 keys by bits [begin_bit, end_bit); returns the sorted keys."""
    lib = load_library()
    keys = _u32_tensor(keys, "keys")
    n = keys.numel()
    out = _output(out, "out", keys)
    workspace = _workspace(workspace, lib.radix_sort_workspace_size(n, begin_bit, end_bit, digit_bits, 0,
                                                                    _opt(options)), keys.device)
    _check(lib.radix_sort_keys(_ptr(keys), _ptr(out), n, begin_bit, end_bit, digit_bits, _ptr(workspace),
                               workspace.numel(), _stream(keys), _opt(options)), "radix_sort_keys")
    return out


def radix_sort_pairs(keys: torch.Tensor, values: torch.Tensor, begin_bit: int = 0, end_bit: int = 32,
                     digit_bits: int = 8, keys_out: torch.Tensor | None = None,
                     values_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     options: SortOptions | None = None):
    """Stable LSD sort of u32 keys carrying u32 values; returns (keys, values)."""
    lib = load_library()
    keys = _u32_tensor(keys, "keys")
    values = _u32_tensor(values, "values")
    _same_device(values, "values", keys.device)
    n = keys.numel()
    if values.numel() != n:
        _bad("keys and values differ in length")
    keys_out = _output(keys_out, "keys_out", keys)
    values_out = _output(values_out, "values_out", values)
    workspace = _workspace(workspace, lib.radix_sort_workspace_size(n, begin_bit, end_bit, digit_bits, 1,
                                                                    _opt(options)), keys.device)
    _check(lib.radix_sort_pairs(_ptr(keys), _ptr(values), _ptr(keys_out), _ptr(values_out), n, begin_bit,
                                end_bit, digit_bits, _ptr(workspace), workspace.numel(), _stream(keys),
                                _opt(options)), "radix_sort_pairs")
    return keys_out, values_out


NO_ALLOC_SCRATCH_BYTES = 64 << 20


def radix_sort_pairs_no_alloc(keys: torch.Tensor, values: torch.Tensor, begin_bit: int = 0, end_bit: int = 32,
                              digit_bits: int = 8, keys_out: torch.Tensor | None = None,
                              values_out: torch.Tensor | None = None, options: SortOptions | None = None):
    """radix_sort_pairs with the library's own per-GPU scratch as workspace (the
    C entry point allocates nothing; outputs are allocated here only if not
    given).  Calls that may overlap on one GPU race.  Returns (keys, values)."""
    lib = load_library()
    keys = _u32_tensor(keys, "keys")
    values = _u32_tensor(values, "values")
    _same_device(values, "values", keys.device)
    n = keys.numel()
    if values.numel() != n:
        _bad("keys and values differ in length")
    keys_out = _output(keys_out, "keys_out", keys)
    values_out = _output(values_out, "values_out", values)
    _check(lib.radix_sort_pairs_no_alloc(_ptr(keys), _ptr(values), _ptr(keys_out), _ptr(values_out), n, begin_bit,
                                         end_bit, digit_bits, _stream(keys), _opt(options)),
           "radix_sort_pairs_no_alloc")
    return keys_out, values_out


_KEY_TYPES = {"u32": LRS_KEY_U32, "i32": LRS_KEY_I32, "f32": LRS_KEY_F32,
              "u64": LRS_KEY_U64, "i64": LRS_KEY_I64, "f64": LRS_KEY_F64}
_KEY_DTYPES = {torch.uint32: "u32", torch.int32: "i32", torch.float32: "f32",
               torch.uint64: "u64", torch.int64: "i64", torch.float64: "f64"}


def _typed_keys(keys: torch.Tensor, key_type: str | None):
    _gpu_input(keys, "keys")
    if keys.dtype not in _KEY_DTYPES:
        _bad(f"keys must be a 32- or 64-bit integer or float tensor, got {keys.dtype}")
    if keys.dim() != 1:
        _bad("keys must be a 1-D tensor")
    kt = _KEY_DTYPES[keys.dtype] if key_type is None else key_type
    if kt not in _KEY_TYPES:
        _bad(f"key_type must be one of {sorted(_KEY_TYPES)}")
    if (kt.endswith("64")) != (keys.element_size() == 8):
        _bad(f"key_type {kt} does not match a {keys.element_size() * 8}-bit tensor")
    return _KEY_TYPES[kt]


def radix_sort_typed_workspace_size(n: int, key_type: str, begin_bit: int = 0, end_bit: int | None = None,
                                    digit_bits: int = 8, with_values: bool = False,
                                    options: SortOptions | None = None) -> int:
    if end_bit is None:
        end_bit = 64 if key_type.endswith("64") else 32
    return int(load_library().radix_sort_typed_workspace_size(n, _KEY_TYPES[key_type], begin_bit, end_bit,
                                                              digit_bits, int(with_values), _opt(options)))


def radix_sort_keys_typed(keys: torch.Tensor, descending: bool = False, key_type: str | None = None,
                          begin_bit: int = 0, end_bit: int | None = None, digit_bits: int = 8,
                          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                          options: SortOptions | None = None) -> torch.Tensor:
    """Stable sort of 32- or 64-bit keys as unsigned, signed or float (from the dtype
    unless key_type is given); end_bit defaults to the key width."""
    lib = load_library()
    kt = _typed_keys(keys, key_type)
    if end_bit is None:
        end_bit = 8 * keys.element_size()
    n = keys.numel()
    out = _output(out, "out", keys)
    workspace = _workspace(workspace, lib.radix_sort_typed_workspace_size(n, kt, begin_bit, end_bit, digit_bits, 0,
                                                                          _opt(options)), keys.device)
    _check(lib.radix_sort_keys_typed(_ptr(keys), _ptr(out), n, kt, int(descending), begin_bit, end_bit,
                                     digit_bits, _ptr(workspace), workspace.numel(), _stream(keys), _opt(options)),
           "radix_sort_keys_typed")
    return out


def radix_sort_pairs_typed(keys: torch.Tensor, values: torch.Tensor, descending: bool = False,
                           key_type: str | None = None, begin_bit: int = 0, end_bit: int | None = None,
                           digit_bits: int = 8, keys_out: torch.Tensor | None = None,
                           values_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           options: SortOptions | None = None):
    """As radix_sort_keys_typed, carrying one 32-bit payload per key; returns (keys, values)."""
    lib = load_library()
    kt = _typed_keys(keys, key_type)
    if end_bit is None:
        end_bit = 8 * keys.element_size()
    values = _u32_tensor(values, "values")
    _same_device(values, "values", keys.device)
    n = keys.numel()
    if values.numel() != n:
        _bad("keys and values differ in length")
    keys_out = _output(keys_out, "keys_out", keys)
    values_out = _output(values_out, "values_out", values)
    workspace = _workspace(workspace, lib.radix_sort_typed_workspace_size(n, kt, begin_bit, end_bit, digit_bits, 1,
                                                                          _opt(options)), keys.device)
    _check(lib.radix_sort_pairs_typed(_ptr(keys), _ptr(values), _ptr(keys_out), _ptr(values_out), n, kt,
                                      int(descending), begin_bit, end_bit, digit_bits, _ptr(workspace),
                                      workspace.numel(), _stream(keys), _opt(options)), "radix_sort_pairs_typed")
    return keys_out, values_out


def _rows_input(x):
    _gpu_input(x, "x")
    if x.dtype == torch.float16:
        dtype = LRS_DTYPE_FP16
    elif x.dtype == torch.bfloat16:
        dtype = LRS_DTYPE_BF16
    else:
        _bad(f"x must be float16 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        _bad("x must be a 2-D tensor")
    return dtype


def segmented_row_sort(x: torch.Tensor, descending: bool = False, digit_bits: int = 8,
                       values_out: torch.Tensor | None = None, indices_out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, options: SortOptions | None = None):
    """Sort every row of a 2-D fp16/bf16 GPU tensor; returns (values, int64 column indices)."""
    lib = load_library()
    dtype = _rows_input(x)
    rows, n = x.shape
    values_out = _output(values_out, "values_out", x)
    indices_out = _output(indices_out, "indices_out", x, element_size=8, dtype=torch.int64)
    workspace = _workspace(workspace, lib.segmented_row_sort_workspace_size(rows, n, digit_bits, _opt(options)),
                           x.device)
    _check(lib.segmented_row_sort(_ptr(x), _ptr(values_out), _ptr(indices_out), rows, n, dtype,
                                  int(descending), digit_bits, _ptr(workspace), workspace.numel(),
                                  _stream(x), _opt(options)), "segmented_row_sort")
    return values_out, indices_out


def segmented_row_sort_pairs(x: torch.Tensor, payload: torch.Tensor, descending: bool = False,
                             digit_bits: int = 8, values_out: torch.Tensor | None = None,
                             payload_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                             options: SortOptions | None = None):
    """Sort every row of a 2-D fp16/bf16 GPU tensor carrying a same-shape 32-bit payload;
    returns (values, payload)."""
    lib = load_library()
    dtype = _rows_input(x)
    _gpu_input(payload, "payload")
    _same_device(payload, "payload", x.device)
    if payload.shape != x.shape or payload.element_size() != 4:
        _bad("payload must be a 32-bit tensor of x's shape")
    rows, n = x.shape
    values_out = _output(values_out, "values_out", x)
    payload_out = _output(payload_out, "payload_out", payload)
    workspace = _workspace(workspace, lib.segmented_row_sort_workspace_size(rows, n, digit_bits, _opt(options)),
                           x.device)
    _check(lib.segmented_row_sort_pairs(_ptr(x), _ptr(payload), _ptr(values_out), _ptr(payload_out), rows, n,
                                        dtype, int(descending), digit_bits, _ptr(workspace), workspace.numel(),
                                        _stream(x), _opt(options)), "segmented_row_sort_pairs")
    return values_out, payload_out


def radix_sort_digit_histograms(keys: torch.Tensor, begin_bit: int = 0, end_bit: int = 32,
                                digit_bits: int = 8) -> torch.Tensor:
    """All passes' digit counts from one read of the keys: int32 [passes, 2^b] (u32 counts)."""
    lib = load_library()
    keys = _u32_tensor(keys, "keys")
    passes = -(-(end_bit - begin_bit) // digit_bits) if end_bit > begin_bit else 0
    hist = torch.empty((max(passes, 1), 1 << digit_bits), dtype=torch.int32, device=keys.device)
    _check(lib.radix_sort_digit_histograms(_ptr(keys), keys.numel(), begin_bit, end_bit, digit_bits,
                                           _ptr(hist), _stream(keys), None), "radix_sort_digit_histograms")
    return hist


def copy_probe(src: torch.Tensor, dst: torch.Tensor, options: SortOptions | None = None) -> None:
    """The bandwidth yardstick: copy src's bytes into dst with the library's streaming copy kernel."""
    lib = load_library()
    _gpu_input(src, "src")
    _same_device(dst, "dst", src.device)
    nbytes = src.numel() * src.element_size()
    if not dst.is_contiguous() or dst.numel() * dst.element_size() < nbytes:
        _bad("dst must be contiguous and at least as large as src")
    _check(lib.radix_sort_copy_probe(_ptr(src), _ptr(dst), nbytes, _stream(src), _opt(options)), "copy_probe")
