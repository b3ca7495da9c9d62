"""C ABI checks of fa_bwd_noalloc that need no GPU: its argument errors and
its size limit are reported before any HIP call."""

import ctypes

import pytest

from exact_io_aware_55_amd import binding

FAKE = 0x10000  # a non-null, 256-byte aligned address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def call(lib, ptrs=None, B=1, H=2, N=64, d=64, scale=0.125):
    ptrs = [FAKE] * 9 if ptrs is None else ptrs
    return lib.fa_bwd_noalloc(*[ctypes.c_void_p(p) if p else None for p in ptrs], B, H, N, d, scale, 0,
                              None)


def test_noalloc_argument_errors(lib):
    for i in range(9):
        ptrs = [FAKE] * 9
        ptrs[i] = 0
        assert call(lib, ptrs) == binding.FA_ERR_INVALID_ARG
        ptrs[i] = FAKE + 8
        assert call(lib, ptrs) == binding.FA_ERR_MISALIGNED
    assert call(lib, B=0) == binding.FA_ERR_INVALID_ARG
    assert call(lib, scale=float("inf")) == binding.FA_ERR_INVALID_ARG
    assert call(lib, d=96) == binding.FA_ERR_UNSUPPORTED


def test_noalloc_size_limit(lib):
    """16 MiB of scratch: B * H * Npad up to 2^21 statistic rows; one more
    64-row block of one head is refused with FA_ERR_SCRATCH."""
    cap = lib.fa_bwd_noalloc_max_workspace()
    assert cap == 16 << 20
    assert lib.fa_bwd_workspace_size(1, 32, 65536, 64) == cap
    assert lib.fa_bwd_workspace_size(1, 32, 65536 + 1, 64) > cap
    assert call(lib, H=32, N=65536 + 1) == binding.FA_ERR_SCRATCH
    assert call(lib, B=4, H=64, N=16384) == binding.FA_ERR_SCRATCH
    assert "scratch" in binding.strerror(binding.FA_ERR_SCRATCH)
