"""The C-ABI library loads on the CPU and exports every declared symbol.

No compute call is made here: the block-manager calls are host code, and the
device calls are only checked for presence and for argument validation that
returns before any HIP call.
"""

import ctypes
import os
import re

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("pa_write_kv", "pa_copy_blocks", "pa_decode", "pa_decode_workspace_bytes",
                 "pa_bm_create", "pa_bm_allocate", "pa_bm_append_slot", "pa_bm_free",
                 "pa_bm_fork", "pa_bm_slot", "pa_bm_num_free_blocks", "pa_bm_can_allocate",
                 "pa_bm_num_cached_tokens", "pa_bm_export_batch"):
        assert must in names


def test_library_exports_every_declared_symbol():
    from paged_kv_cache_136_amd import LIB_PATH
    from paged_kv_cache_136_amd._lib import SIGNATURES
    h = ctypes.CDLL(LIB_PATH)
    names = declared_functions()
    missing = [n for n in names if not hasattr(h, n)]
    assert not missing, missing
    # The binding declares exactly the header's functions.
    assert sorted(SIGNATURES) == names


def test_status_strings():
    from paged_kv_cache_136_amd import lib
    assert lib().pa_status_str(0) == b"PA_OK"
    assert lib().pa_status_str(1) == b"PA_ERR_OUT_OF_BLOCKS"


def test_device_calls_validate_before_touching_the_gpu():
    """Bad arguments are rejected on the host with PA_ERR_INVALID /
    PA_ERR_UNSUPPORTED before any HIP call (safe without a GPU)."""
    from paged_kv_cache_136_amd import lib
    L = lib()
    # negative T
    assert L.pa_write_kv(None, None, None, None, None, -1, 4, 16, 1, 64, 1, None) == 2
    # unsupported head_dim
    st = L.pa_decode(None, None, None, None, None, 1, None, 16, 1, 1, 1, 96, 16, 4, 1.0, 0, 1,
                     None, 0, None)
    assert st == 2  # null pointers are checked first
    assert b"null" in L.pa_last_error()
    # empty batch: nothing to do, OK
    assert L.pa_decode(None, None, None, None, None, 1, None, 16, 0, 1, 1, 64, 16, 4, 1.0, 0, 1,
                       None, 0, None) == 0
    assert L.pa_copy_blocks(None, None, 0, 16, 4, None, 0, None) == 0
    assert L.pa_decode_workspace_bytes(4, 8, 128, 4096, 512) == (
        ((4 * 8 * 8 * 128 * 4 + 255) // 256 * 256) + 2 * ((4 * 8 * 8 * 4 + 255) // 256 * 256))
    assert L.pa_decode_workspace_bytes(4, 8, 128, 512, 512) == 0
    assert L.pa_decode_workspace_bytes(4, 8, 128, 4096, 0) == 0
