"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, sizes its workspace, and rejects bad arguments before it
enqueues anything.  No kernel runs here."""
import ctypes
import re

import pytest

import lsd_radix_sort_amd as lrs


def _declared_functions():
    text = open(lrs.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_functions_exported():
    names = _declared_functions()
    assert {"radix_sort_keys", "radix_sort_pairs", "segmented_row_sort"} <= set(names)
    lib = ctypes.CDLL(lrs.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    for s in range(0, 11):
        assert lrs.status_string(s)
    assert lrs.status_string(99) == "unknown status"


def test_workspace_sizes():
    lib = lrs.load_library()
    n = 1 << 20
    k = lib.radix_sort_workspace_size(n, 0, 32, 8, 0, None)
    p = lib.radix_sort_workspace_size(n, 0, 32, 8, 1, None)
    assert k >= 4 * n and p >= 8 * n and p > k
    # one pass needs no spare buffers
    assert lib.radix_sort_workspace_size(n, 0, 8, 8, 1, None) < 4 * n
    assert lib.radix_sort_workspace_size(0, 0, 32, 8, 0, None) == 0
    for args in ((n, 0, 32, 3, 0), (n, 0, 33, 8, 0), (n, 5, 5, 8, 0), (n, -1, 8, 8, 0)):
        assert lib.radix_sort_workspace_size(*args, None) == 0
    # segmented: spare values, two u32 index buffers when there are more than two passes
    s4 = lib.segmented_row_sort_workspace_size(1024, 65536, 4, None)
    s8 = lib.segmented_row_sort_workspace_size(1024, 65536, 8, None)
    assert s4 >= 1024 * 65536 * (2 + 4 + 4) and s8 >= 1024 * 65536 * (2 + 4) and s4 > s8
    assert lib.segmented_row_sort_workspace_size(4, 1 << 30, 8, None) == 0
    assert lib.segmented_row_sort_workspace_size(0, 16, 8, None) == 0
    # rows of at most 8192 elements are sorted whole in one workgroup: no workspace
    assert lib.radix_sort_workspace_size(8192, 0, 32, 8, 1, None) == 0
    assert lib.radix_sort_workspace_size(8193, 0, 32, 8, 1, None) > 0
    assert lib.segmented_row_sort_workspace_size(4096, 4096, 8, None) == 0
    assert lib.segmented_row_sort_workspace_size(4, 8193, 8, None) > 0


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Fake device addresses are only passed where validation must reject the call;
# on a machine with a GPU these cases are covered with real buffers instead.
FAKE = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(6)]


@pytest.mark.skipif(_gpu_present(), reason="fake-pointer validation runs only without a GPU")
def test_validation_before_launch():
    lib = lrs.load_library()
    k_in, k_out, v_in, v_out, ws, _ = FAKE
    big = 1 << 40

    def no_opts(fn):
        return lambda *a: fn(*a, None)
    st = no_opts(lib.radix_sort_keys)
    assert st(k_in, k_out, 100, 0, 32, 3, ws, big, None) == 3
    assert st(k_in, k_out, 100, 0, 33, 8, ws, big, None) == 2
    assert st(k_in, k_out, 100, 8, 8, 8, ws, big, None) == 2
    assert st(k_in, k_out, 1 << 32, 0, 32, 8, ws, big, None) == 4
    assert st(None, k_out, 100, 0, 32, 8, ws, big, None) == 1
    # inputs above 8192 elements need a workspace (smaller ones are sorted in one workgroup)
    assert st(k_in, k_out, 100_000, 0, 32, 8, None, big, None) == 1
    assert st(k_in, k_out, 100_000, 0, 32, 8, ws, 16, None) == 6
    assert st(k_in, k_in, 100, 0, 32, 8, ws, big, None) == 5
    assert st(k_in, ctypes.c_void_p(0x10000 + 200), 100, 0, 32, 8, ws, big, None) == 5
    assert st(None, None, 0, 0, 32, 8, None, 0, None) == 0  # n == 0: nothing to do
    assert st(ctypes.c_void_p(0x10002), k_out, 100, 0, 32, 8, ws, big, None) == 9
    assert st(k_in, k_out, 100, 0, 32, 8, ctypes.c_void_p(0x90010), big, None) == 9
    sp = no_opts(lib.radix_sort_pairs)
    assert sp(k_in, None, k_out, v_out, 100, 0, 32, 8, ws, big, None) == 1
    assert sp(k_in, v_in, k_out, k_out, 100, 0, 32, 8, ws, big, None) == 5
    assert sp(k_in, v_in, k_out, v_in, 100, 0, 32, 8, ws, big, None) == 5
    seg = no_opts(lib.segmented_row_sort)
    assert seg(k_in, k_out, v_out, 4, 100, 2, 0, 8, ws, big, None) == 7
    assert seg(k_in, k_out, v_out, 4, 100, 0, 0, 5, ws, big, None) == 3
    assert seg(k_in, k_out, v_out, 4, 1 << 30, 0, 0, 8, ws, big, None) == 4
    assert seg(k_in, k_out, v_out, -1, 100, 0, 0, 8, ws, big, None) == 4
    assert seg(k_in, k_out, None, 4, 100, 0, 0, 8, ws, big, None) == 1
    assert seg(k_in, k_out, v_out, 4, 100_000, 0, 0, 8, ws, 8, None) == 6
    assert seg(k_in, k_in, v_out, 4, 100, 0, 0, 8, ws, big, None) == 5
    assert seg(None, None, None, 0, 100, 0, 0, 8, None, 0, None) == 0
    h = no_opts(lib.radix_sort_digit_histograms)
    assert h(k_in, 100, 0, 32, 7, v_out, None) == 3
    assert h(k_in, 100, 0, 40, 8, v_out, None) == 2
    assert h(k_in, 100, 0, 32, 8, None, None) == 1
    kt = no_opts(lib.radix_sort_keys_typed)
    assert kt(k_in, k_out, 100, 9, 0, 0, 32, 8, ws, big, None) == 7      # unknown key type
    assert kt(k_in, k_out, 100, 1, 0, 0, 33, 8, ws, big, None) == 2      # i32: at most 32 bits
    assert kt(k_in, k_out, 100, 4, 0, 0, 65, 8, ws, big, None) == 2      # i64: at most 64 bits
    assert kt(k_in, k_out, 100, 5, 1, 0, 64, 3, ws, big, None) == 3      # f64: digit width
    assert kt(ctypes.c_void_p(0x10004), k_out, 100, 4, 0, 0, 64, 8, ws, big, None) == 9  # 8-byte keys
    assert kt(k_in, k_out, 100, 4, 0, 0, 64, 8, None, big, None) == 1    # 64-bit keys need a workspace
    assert kt(k_in, k_in, 100, 2, 0, 0, 32, 8, ws, big, None) == 5
    pt = no_opts(lib.radix_sort_pairs_typed)
    assert pt(k_in, None, k_out, v_out, 100, 2, 1, 0, 32, 8, ws, big, None) == 1
    assert pt(k_in, v_in, k_out, v_out, 100, 6, 0, 0, 32, 8, ws, big, None) == 7
    sg2 = no_opts(lib.segmented_row_sort_pairs)
    assert sg2(k_in, None, k_out, v_out, 4, 100, 0, 0, 8, ws, big, None) == 1
    assert sg2(k_in, v_in, k_out, v_in, 4, 100, 0, 0, 8, ws, big, None) == 5
    assert sg2(k_in, v_in, k_out, v_out, 4, 100, 3, 0, 8, ws, big, None) == 7
    assert sg2(None, None, None, None, 0, 100, 0, 0, 8, None, 0, None) == 0


def test_typed_workspace_sizes():
    lib = lrs.load_library()

    def tws(*a):
        return lib.radix_sort_typed_workspace_size(*a, None)
    # 32-bit types take the same workspace as the plain u32 sort
    for kt in (0, 1, 2):
        assert tws(1_000_000, kt, 0, 32, 8, 1) == lib.radix_sort_workspace_size(1_000_000, 0, 32, 8, 1, None)
    assert tws(1000, 0, 0, 32, 8, 0) == 0                       # resident: no workspace
    assert tws(1000, 3, 0, 64, 8, 0) > 0                        # 64-bit keys always need one
    assert tws(1_000_000, 4, 0, 64, 8, 1) > tws(1_000_000, 1, 0, 32, 8, 1)
    assert tws(100, 7, 0, 32, 8, 0) == 0 and tws(100, 4, 0, 65, 8, 0) == 0


@pytest.mark.skipif(_gpu_present(), reason="fake-pointer validation runs only without a GPU")
def test_invalid_options_rejected_before_launch():
    lib = lrs.load_library()
    k_in, k_out, v_in, v_out, ws, _ = FAKE
    bad = lrs._Options(7, 0, 0, 0, None)  # unknown scan strategy
    ok = lrs._Options(1, 5, 1, 1 << 20, None)
    r = ctypes.byref
    assert lib.radix_sort_keys(k_in, k_out, 100_000, 0, 32, 8, ws, 1 << 40, None, r(bad)) == 10
    assert lib.radix_sort_pairs(k_in, v_in, k_out, v_out, 100_000, 0, 32, 8, ws, 1 << 40, None, r(bad)) == 10
    assert lib.segmented_row_sort(k_in, k_out, v_out, 4, 100, 0, 0, 8, ws, 1 << 40, None, r(bad)) == 10
    assert lib.radix_sort_workspace_size(100_000, 0, 32, 8, 1, r(bad)) == 0
    assert lib.segmented_row_sort_workspace_size(4, 100_000, 8, r(bad)) == 0
    # a valid struct with an argument error still reports the argument error
    assert lib.radix_sort_keys(k_in, k_out, 100_000, 0, 32, 3, ws, 1 << 40, None, r(ok)) == 3
    with pytest.raises(ValueError):
        lrs.SortOptions(scan="bogus")
    with pytest.raises(ValueError):
        lrs.SortOptions(spin_limit=0)


def test_wide_option_sizes_workspace():
    """Forcing the wide sweep (64-bit look-back words) changes the workspace the
    query reports; rows short enough for the resident sort ignore it."""
    lib = lrs.load_library()
    n = 3_000_017
    narrow = lrs.radix_sort_workspace_size(n, 0, 32, 8, True)
    wide = lrs.radix_sort_workspace_size(n, 0, 32, 8, True, lrs.SortOptions(wide_from=1))
    assert narrow > 0 and wide > 0 and wide != narrow
    assert lrs.radix_sort_workspace_size(8192, 0, 32, 8, True, lrs.SortOptions(wide_from=1)) == 0
    assert lib.radix_sort_timer_read(None, None, None) == 1


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        lrs.radix_sort_keys(torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError):
        lrs.segmented_row_sort(torch.zeros(2, 4, dtype=torch.float16))


def test_python_binding_rejects_bad_outputs_and_workspace():
    """Every caller-supplied output and workspace is checked (device, element
    size, exact shape, contiguity, workspace bytes) before the library is called."""
    import torch
    cpu = torch.device("cpu")
    ok = torch.empty(10, dtype=torch.int32)
    assert lrs.check_output(ok, "out", cpu, 4, (10,)) is ok
    with pytest.raises(ValueError, match="shape"):
        lrs.check_output(torch.empty(9, dtype=torch.int32), "out", cpu, 4, (10,))
    with pytest.raises(ValueError, match="shape"):
        lrs.check_output(torch.empty(2, 5, dtype=torch.int32), "out", cpu, 4, (10,))
    with pytest.raises(ValueError, match="4-byte"):
        lrs.check_output(torch.empty(10, dtype=torch.int16), "out", cpu, 4, (10,))
    with pytest.raises(ValueError, match="contiguous"):
        lrs.check_output(torch.empty(20, dtype=torch.int32)[::2], "out", cpu, 4, (10,))
    with pytest.raises(ValueError, match="is on cpu"):
        lrs.check_output(ok, "out", torch.device("cuda:0"), 4, (10,))
    with pytest.raises(ValueError, match="must be a tensor"):
        lrs.check_output([0] * 10, "out", cpu, 4, (10,))
    ws = torch.empty(100, dtype=torch.uint8)
    assert lrs.check_workspace(ws, cpu, 100) is ws
    with pytest.raises(ValueError, match="needs 101"):
        lrs.check_workspace(ws, cpu, 101)
    with pytest.raises(ValueError, match="uint8"):
        lrs.check_workspace(torch.empty(100, dtype=torch.int32), cpu, 4)
    with pytest.raises(ValueError, match="is on cpu"):
        lrs.check_workspace(ws, torch.device("cuda:0"), 4)


def test_tile_trace_entry_points_in_the_default_build():
    # the phase records exist only in builds with LRS_TILE_TRACE=1; the default
    # library exports the entry points, refuses a trace buffer and records nothing
    lib = lrs.load_library()
    t = lib.radix_sort_timer_create()
    assert t
    try:
        used = ctypes.c_uint64(7)
        assert lib.radix_sort_timer_trace_tiles(None, None, 0) == 1      # LRS_ERR_NULL_POINTER
        assert lib.radix_sort_timer_trace_tiles(t, None, 0) == 10        # LRS_ERR_OPTION: not a trace build
        assert lib.radix_sort_timer_trace_used(None, ctypes.byref(used)) == 1
        assert lib.radix_sort_timer_trace_used(t, None) == 1
        assert lib.radix_sort_timer_trace_used(t, ctypes.byref(used)) == 0 and used.value == 0
    finally:
        lib.radix_sort_timer_destroy(t)
