"""The measurement-only ceilings library: it loads, exports its four entry
points, and refuses bad arguments before any launch (no GPU needed: every
call here returns from its argument checks)."""
import ctypes

import pytest

from dora_adapter_factored_amd import ceilings as CL

FAKE = ctypes.c_void_p(0x10000)


@pytest.fixture(scope="module")
def lib():
    return CL.load()


def test_exports(lib):
    for name in ("dora_ceiling_mfma", "dora_ceiling_stream", "dora_ceiling_cu_read", "dora_ceiling_w0_stream"):
        assert hasattr(lib, name)


def test_argument_checks(lib):
    assert lib.dora_ceiling_mfma(0, 0, 256, FAKE, None) == 1          # iters < 1
    assert lib.dora_ceiling_mfma(2, 10, 256, FAKE, None) == 1         # unknown kind
    assert lib.dora_ceiling_mfma(0, 10, 256, None, None) == 1
    assert lib.dora_ceiling_stream(0, FAKE, FAKE, None, FAKE, None, 24, 16, None) == 1   # not a multiple of 16
    assert lib.dora_ceiling_stream(1, FAKE, FAKE, None, FAKE, FAKE, 32, 16, None) == 1   # 3 reads need c
    assert lib.dora_ceiling_stream(2, FAKE, FAKE, None, FAKE, None, 32, 16, None) == 1   # 2 writes need z
    assert lib.dora_ceiling_stream(3, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 16, None) == 1
    assert lib.dora_ceiling_stream(0, FAKE, FAKE, None, FAKE, None, 32, -1, None) == 1   # negative grid
    assert lib.dora_ceiling_stream(1, FAKE, FAKE, None, FAKE, FAKE, 32, 0, None) == 1    # blocked form needs c too
    assert lib.dora_ceiling_cu_read(FAKE, 8, 0, 1, 256, 8, FAKE, None) == 1             # under 16 bytes
    assert lib.dora_ceiling_cu_read(FAKE, 1024, 0, 1, 256, 9, FAKE, None) == 1          # more than 8 waves
    assert lib.dora_ceiling_w0_stream(FAKE, FAKE, 8193 * 32, 8192, 384, 1, FAKE, None) == 1   # beyond 32 row tiles
    assert lib.dora_ceiling_w0_stream(FAKE, FAKE, 8192, 8190, 384, 1, FAKE, None) == 1   # d_in not a multiple of 8
    assert lib.dora_ceiling_w0_stream(FAKE, FAKE, 8192, 8192, 384, 4, FAKE, None) == 1   # unknown A layout
    assert lib.dora_ceiling_w0_stream(FAKE, FAKE, 8000, 8192, 384, 3, FAKE, None) == 1   # seven chunks: 32 row tiles
