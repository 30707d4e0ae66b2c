"""C ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and validates descriptors before touching any device."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decoupattn.h")


@pytest.fixture(scope="module")
def S():
    import sparse_attention_video_da_amd as S
    return S


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DA_API\s+[\w\s\*]+?\b(da_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared()
    for n in ("da_plan_create", "da_plan_destroy", "da_reassign", "da_forward", "da_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol(S):
    lib = ctypes.CDLL(S.LIB_PATH)
    for n in declared():
        assert hasattr(lib, n), n
    assert sorted(S.EXPORTED) == declared()


def test_status_strings(S):
    for code in range(5):
        assert S.da_status_str(code).startswith("DA_")
    assert S.da_status_str(99) == "unknown status"
    assert S.da_version() >= 100


def _ok_mask(n=8):
    return np.ones((1, n, n), np.uint8)


@pytest.mark.parametrize("field,value,code", [
    ("heads", 0, 1), ("seq_len", 0, 1), ("clusters", 0, 1), ("clusters", 1001, 1),
    ("mask_heads", 3, 1), ("scale", -1.0, 1), ("scale", float("nan"), 1),
    ("head_dim", 96, 2), ("block", 32, 2), ("dtype", 7, 2), ("clusters", 900, 0),
    ("key_block", -1, 1), ("key_block", 8, 2), ("key_block", 48, 2), ("key_block", 256, 2),
    ("key_block", 16, 0), ("key_block", 32, 0), ("key_block", 64, 0), ("key_block", 128, 0),
])
def test_descriptor_validation(S, field, value, code):
    d = S.make_desc(heads=2, seq_len=1000, head_dim=128, block=128, clusters=16)
    setattr(d, field, value)
    assert S.da_validate_desc(d, _ok_mask()) == code


def test_key_block_above_query_block_is_unsupported(S):
    d = S.make_desc(2, 1000, 128, 64, 16, key_block=128)
    assert S.da_validate_desc(d, _ok_mask()) == S.DA_ERR_UNSUPPORTED
    d.key_block = 64
    assert S.da_validate_desc(d, _ok_mask()) == S.DA_OK


def test_per_head_byte_size_limit(S):
    """One head's [N][d] tensor must be addressable with 32-bit byte offsets. (For bf16 the
    mask's nb x nkb limit binds first; fp32 at d = 128 reaches the byte limit.)"""
    d = S.make_desc(1, 4_194_304, 128, 128, 16, dtype="f32")   # exactly 2^31 bytes
    assert S.da_validate_desc(d, _ok_mask()) == S.DA_ERR_UNSUPPORTED
    d.seq_len = 4_194_303
    assert S.da_validate_desc(d, _ok_mask()) == S.DA_OK


def test_validation_rejects_null_mask_and_desc(S):
    d = S.make_desc(2, 1000, 128, 128, 16)
    assert S.da_validate_desc(d, None) == S.DA_ERR_INVALID_ARGUMENT
    assert S.da_validate_desc(None, _ok_mask()) == S.DA_ERR_INVALID_ARGUMENT


def test_cluster_limit_is_unsupported(S):
    d = S.make_desc(1, 100000, 64, 64, 8193)
    assert S.da_validate_desc(d, _ok_mask()) == S.DA_ERR_UNSUPPORTED


def test_plan_create_bad_desc_returns_before_device(S):
    d = S.make_desc(2, 1000, 96, 128, 16)
    st, h = S.da_plan_create(d, _ok_mask())
    assert st == S.DA_ERR_UNSUPPORTED and not h.value


def test_null_plan_is_rejected(S):
    assert S.da_forward(None, *([None] * 9)) == S.DA_ERR_INVALID_ARGUMENT
    assert S.da_reassign(None, *([None] * 9)) == S.DA_ERR_INVALID_ARGUMENT
    assert S.da_forward_var(None, *([None] * 10)) == S.DA_ERR_INVALID_ARGUMENT
    assert S.da_reassign_var(None, *([None] * 10)) == S.DA_ERR_INVALID_ARGUMENT
    assert S.da_plan_destroy(None) == S.DA_OK
