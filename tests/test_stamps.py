"""The phase-stamp instrumentation is a separate build: the library's own build
exports no stamp entry, and the instrumented build (as the stamp tool builds it)
compiles and exports its buffer lookup. CPU only."""
import ctypes
import os
import shutil

import pytest

from mla_latent_kv_41_amd import build, mla, stamps


def test_product_build_has_no_stamps():
    assert not hasattr(ctypes.CDLL(mla.LIB_PATH), "mla_stamps_buffer")


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_instrumented_build_exports_the_stamp_buffer(tmp_path):
    lib = stamps.build_stamped(str(tmp_path))
    assert hasattr(ctypes.CDLL(lib), "mla_stamps_buffer")
