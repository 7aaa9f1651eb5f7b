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
    for s in range(0, 10):
        assert lrs.status_string(s)
    assert lrs.status_string(99) == "unknown status"


def test_workspace_sizes():
    lib = lrs.load_library()
    n = 1 << 20
    k = lib.radix_sort_workspace_size(n, 0, 32, 8, 0)
    p = lib.radix_sort_workspace_size(n, 0, 32, 8, 1)
    assert k >= 4 * n and p >= 8 * n and p > k
    # one pass needs no spare buffers
    assert lib.radix_sort_workspace_size(n, 0, 8, 8, 1) < 4 * n
    assert lib.radix_sort_workspace_size(0, 0, 32, 8, 0) == 0
    for args in ((n, 0, 32, 3, 0), (n, 0, 33, 8, 0), (n, 5, 5, 8, 0), (n, -1, 8, 8, 0)):
        assert lib.radix_sort_workspace_size(*args) == 0
    # segmented: spare values, two u32 index buffers when there are more than two passes
    s4 = lib.segmented_row_sort_workspace_size(1024, 65536, 4)
    s8 = lib.segmented_row_sort_workspace_size(1024, 65536, 8)
    assert s4 >= 1024 * 65536 * (2 + 4 + 4) and s8 >= 1024 * 65536 * (2 + 4) and s4 > s8
    assert lib.segmented_row_sort_workspace_size(4, 1 << 30, 8) == 0
    assert lib.segmented_row_sort_workspace_size(0, 16, 8) == 0
    # rows of at most 8192 elements are sorted whole in one workgroup: no workspace
    assert lib.radix_sort_workspace_size(8192, 0, 32, 8, 1) == 0
    assert lib.radix_sort_workspace_size(8193, 0, 32, 8, 1) > 0
    assert lib.segmented_row_sort_workspace_size(4096, 4096, 8) == 0
    assert lib.segmented_row_sort_workspace_size(4, 8193, 8) > 0


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
    st = lib.radix_sort_keys
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
    sp = lib.radix_sort_pairs
    assert sp(k_in, None, k_out, v_out, 100, 0, 32, 8, ws, big, None) == 1
    assert sp(k_in, v_in, k_out, k_out, 100, 0, 32, 8, ws, big, None) == 5
    assert sp(k_in, v_in, k_out, v_in, 100, 0, 32, 8, ws, big, None) == 5
    seg = lib.segmented_row_sort
    assert seg(k_in, k_out, v_out, 4, 100, 2, 0, 8, ws, big, None) == 7
    assert seg(k_in, k_out, v_out, 4, 100, 0, 0, 5, ws, big, None) == 3
    assert seg(k_in, k_out, v_out, 4, 1 << 30, 0, 0, 8, ws, big, None) == 4
    assert seg(k_in, k_out, v_out, -1, 100, 0, 0, 8, ws, big, None) == 4
    assert seg(k_in, k_out, None, 4, 100, 0, 0, 8, ws, big, None) == 1
    assert seg(k_in, k_out, v_out, 4, 100_000, 0, 0, 8, ws, 8, None) == 6
    assert seg(k_in, k_in, v_out, 4, 100, 0, 0, 8, ws, big, None) == 5
    assert seg(None, None, None, 0, 100, 0, 0, 8, None, 0, None) == 0
    h = lib.radix_sort_digit_histograms
    assert h(k_in, 100, 0, 32, 7, v_out, None) == 3
    assert h(k_in, 100, 0, 40, 8, v_out, None) == 2
    assert h(k_in, 100, 0, 32, 8, None, None) == 1
    kt = lib.radix_sort_keys_typed
    assert kt(k_in, k_out, 100, 9, 0, 0, 32, 8, ws, big, None) == 7      # unknown key type
    assert kt(k_in, k_out, 100, 1, 0, 0, 33, 8, ws, big, None) == 2      # i32: at most 32 bits
    assert kt(k_in, k_out, 100, 4, 0, 0, 65, 8, ws, big, None) == 2      # i64: at most 64 bits
    assert kt(k_in, k_out, 100, 5, 1, 0, 64, 3, ws, big, None) == 3      # f64: digit width
    assert kt(ctypes.c_void_p(0x10004), k_out, 100, 4, 0, 0, 64, 8, ws, big, None) == 9  # 8-byte keys
    assert kt(k_in, k_out, 100, 4, 0, 0, 64, 8, None, big, None) == 1    # 64-bit keys need a workspace
    assert kt(k_in, k_in, 100, 2, 0, 0, 32, 8, ws, big, None) == 5
    pt = lib.radix_sort_pairs_typed
    assert pt(k_in, None, k_out, v_out, 100, 2, 1, 0, 32, 8, ws, big, None) == 1
    assert pt(k_in, v_in, k_out, v_out, 100, 6, 0, 0, 32, 8, ws, big, None) == 7
    sg2 = lib.segmented_row_sort_pairs
    assert sg2(k_in, None, k_out, v_out, 4, 100, 0, 0, 8, ws, big, None) == 1
    assert sg2(k_in, v_in, k_out, v_in, 4, 100, 0, 0, 8, ws, big, None) == 5
    assert sg2(k_in, v_in, k_out, v_out, 4, 100, 3, 0, 8, ws, big, None) == 7
    assert sg2(None, None, None, None, 0, 100, 0, 0, 8, None, 0, None) == 0


def test_typed_workspace_sizes_and_strategy_switch():
    lib = lrs.load_library()
    tws = lib.radix_sort_typed_workspace_size
    # 32-bit types take the same workspace as the plain u32 sort
    for kt in (0, 1, 2):
        assert tws(1_000_000, kt, 0, 32, 8, 1) == lib.radix_sort_workspace_size(1_000_000, 0, 32, 8, 1)
    assert tws(1000, 0, 0, 32, 8, 0) == 0                       # resident: no workspace
    assert tws(1000, 3, 0, 64, 8, 0) > 0                        # 64-bit keys always need one
    assert tws(1_000_000, 4, 0, 64, 8, 1) > tws(1_000_000, 1, 0, 32, 8, 1)
    assert tws(100, 7, 0, 32, 8, 0) == 0 and tws(100, 4, 0, 65, 8, 0) == 0
    assert lib.radix_sort_set_scan_strategy(2) == -1
    old = lrs.radix_sort_set_scan_strategy("reduce-then-scan")
    assert lrs.radix_sort_set_scan_strategy(old) == "reduce-then-scan"
    with pytest.raises(ValueError):
        lrs.radix_sort_set_scan_strategy("bogus")


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        lrs.radix_sort_keys(torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError):
        lrs.segmented_row_sort(torch.zeros(2, 4, dtype=torch.float16))
