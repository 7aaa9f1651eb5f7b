"""The entry point that allocates nothing (radix_sort_pairs_no_alloc), called
through the C ABI, against radix_sort_pairs on the same inputs: bit-exact keys
and values on two calls in a row, the second with a smaller input (the shared
scratch keeps the first call's contents), and the CPU oracle on both."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

lrs = pytest.importorskip("lsd_radix_sort_amd")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int32).copy()).cuda()


def _np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lrs.load_library()


def _no_alloc(lib, kt, vt, ko, vo, n, begin, end, b):
    return lib.radix_sort_pairs_no_alloc(kt.data_ptr(), vt.data_ptr(), ko.data_ptr(), vo.data_ptr(), n, begin, end,
                                         b, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), None)


def test_no_alloc_matches_the_workspace_entry_point():
    lib = lrs.load_library()
    # several 4096/8192-key tiles with a ragged end, then a smaller sort, then a
    # whole-row sort (no workspace) and a 4-bit sort over a bit window
    cases = [(5_000_011, 0, 32, 8, 1), (300_007, 0, 32, 8, 2), (6_000, 0, 32, 8, 3), (1_000_003, 3, 29, 4, 4)]
    for n, begin, end, b, seed in cases:
        log(f"no-alloc n={n} [{begin},{end}) b={b}")
        keys = workloads.random_u32(13_000 + seed, n)
        keys[::3] &= np.uint32(0x00FF00FF)  # ties
        vals = np.arange(n, dtype=np.uint32)
        kt, vt = _u32(keys), _u32(vals)
        ko, vo = torch.empty_like(kt), torch.empty_like(vt)
        st = _no_alloc(lib, kt, vt, ko, vo, n, begin, end, b)
        assert st == 0, lrs.status_string(st)
        ek, ev = lrs.radix_sort_pairs(kt, vt, begin, end, b)
        torch.cuda.synchronize()
        assert np.array_equal(_np(ko), _np(ek)), f"n={n}: keys differ from radix_sort_pairs"
        assert np.array_equal(_np(vo), _np(ev)), f"n={n}: values differ from radix_sort_pairs"
        ok, ov = oracle.radix_sort_pairs(keys, vals, begin, end, b)
        assert np.array_equal(_np(ko), ok) and np.array_equal(_np(vo), ov), f"n={n}: differs from the oracle"
        assert np.array_equal(_np(kt), keys), "input was written"


def test_no_alloc_rejects_sizes_beyond_its_scratch():
    lib = lrs.load_library()
    n = 9_000_000
    kt = torch.zeros(n, dtype=torch.int32, device="cuda")
    vt, ko, vo = torch.empty_like(kt), torch.empty_like(kt), torch.empty_like(kt)
    assert lib.radix_sort_workspace_size(n, 0, 32, 8, 1, None) > lrs.NO_ALLOC_SCRATCH_BYTES
    assert _no_alloc(lib, kt, vt, ko, vo, n, 0, 32, 8) == 4  # LRS_ERR_SIZE, nothing enqueued
    assert _no_alloc(lib, kt, vt, ko, vo, 100, 0, 32, 3) == 3  # LRS_ERR_DIGIT_BITS
    with pytest.raises(ValueError):
        lrs.radix_sort_pairs_no_alloc(kt, vt)
