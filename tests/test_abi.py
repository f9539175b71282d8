"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
symbol include/mlaverify.h declares, and its pure-host functions (configuration
validation, workspace sizing, status strings) behave as documented."""

import ctypes
import math
import os
import re

import pytest

from mla_tree_verify_mlaverify_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mlaverify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from mla_tree_verify_mlaverify_amd import build

        build.build()
    return binding.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"MLAVERIFY_API\s+[\w\s\*]*?\b(mlaverify_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = declared_symbols()
    assert "mlaverify_create" in names and "mlaverify_run" in names and "mlaverify_destroy" in names
    assert sorted(names) == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(raw, name), name


def base_cfg(**kw):
    args = dict(num_heads=8, max_batch=8, max_tree_nodes=64, max_prefix_len=200000, pool_slots=262144)
    args.update(kw)
    return binding.make_config(**args)


@pytest.mark.parametrize("kw,expect", [
    ({}, binding.OK),
    (dict(max_tree_nodes=65), binding.OK),
    (dict(max_tree_nodes=256), binding.OK),
    (dict(max_tree_nodes=257), binding.ERR_UNSUPPORTED),
    (dict(max_tree_nodes=0), binding.ERR_INVALID_ARG),
    (dict(num_heads=0), binding.ERR_INVALID_ARG),
    (dict(num_heads=129), binding.ERR_INVALID_ARG),
    (dict(max_batch=0), binding.ERR_INVALID_ARG),
    (dict(max_batch=1025), binding.ERR_INVALID_ARG),
    (dict(max_prefix_len=-1), binding.ERR_INVALID_ARG),
    (dict(pool_slots=0), binding.ERR_INVALID_ARG),
    (dict(pool_slots=1 << 31), binding.ERR_INVALID_ARG),
    (dict(kv_row_stride=575), binding.ERR_INVALID_ARG),
    (dict(kv_row_stride=580), binding.ERR_INVALID_ARG),
    (dict(kv_row_stride=640), binding.OK),
    (dict(sm_scale=math.inf), binding.ERR_INVALID_ARG),
    (dict(sm_scale=0.0), binding.ERR_INVALID_ARG),
    (dict(sm_scale=-0.07), binding.ERR_INVALID_ARG),
    (dict(split_tokens=48), binding.ERR_INVALID_ARG),
    (dict(split_tokens=-32), binding.ERR_INVALID_ARG),
    (dict(split_tokens=1024), binding.OK),
    (dict(flags=0x80), binding.ERR_INVALID_ARG),
    (dict(flags=binding.FLAG_NO_FASTPATH), binding.OK),
    (dict(page_size=1), binding.OK),
    (dict(page_size=64), binding.OK),
    (dict(page_size=1024), binding.OK),
    (dict(page_size=3), binding.ERR_INVALID_ARG),     # not a power of two
    (dict(page_size=2048), binding.ERR_INVALID_ARG),  # larger than 1024
    (dict(page_size=-4), binding.ERR_INVALID_ARG),
    (dict(max_batch=1024, max_prefix_len=1 << 22), binding.ERR_UNSUPPORTED),  # 32-bit key offsets
    (dict(num_heads=128, max_batch=64, max_tree_nodes=256, max_prefix_len=1 << 24, split_tokens=1024),
     binding.ERR_UNSUPPORTED),  # key offsets fit, partial rows pass 2^31 (32-bit row indices)
])
def test_validate_config(lib, kw, expect):
    assert binding.validate_config(base_cfg(**kw)) == expect


def test_workspace_bytes(lib):
    assert binding.workspace_bytes(base_cfg(max_tree_nodes=0)) == 0
    small = binding.workspace_bytes(base_cfg(max_batch=1, max_tree_nodes=8, num_heads=8))
    big = binding.workspace_bytes(base_cfg(max_batch=8, max_tree_nodes=64, num_heads=16))
    assert 0 < small < big
    assert big % 256 == 0
    # partial outputs dominate: per unit and row 512 bf16 values and the lse
    row_bytes = 512 * 2 + 4
    assert binding.workspace_bytes(base_cfg(max_batch=1)) >= 64 * 512 * row_bytes
    fixed = binding.workspace_bytes(base_cfg(max_batch=2, max_prefix_len=4096, split_tokens=512))
    assert fixed >= 2 * 8 * 64 * 8 * row_bytes


def test_status_strings(lib):
    for code in (binding.OK, binding.ERR_INVALID_ARG, binding.ERR_UNSUPPORTED, binding.ERR_NO_MEMORY,
                 binding.ERR_WORKSPACE, binding.ERR_HIP):
        s = binding.status_string(code)
        assert s and s != "unknown status"
    assert binding.status_string(12345) == "unknown status"


def test_create_rejects_null_output_pointer(lib):
    assert lib.mlaverify_create(ctypes.byref(base_cfg()), None, 0, None) == binding.ERR_INVALID_ARG


def test_run_rejects_null_handle(lib):
    assert lib.mlaverify_run(None, 1, 1, *([None] * 8)) == binding.ERR_INVALID_ARG


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        binding.load_library(str(tmp_path / "nope.so"))


def test_run_static_refuses_oversize_calls_before_any_device_work(lib):
    # 128 heads x 256 nodes needs 2 x 32,768 rows of partials (about 67 MB), more than the
    # static workspace: refused on the host, so no GPU is needed for this check.  The device
    # pointers are never dereferenced.
    cfg = binding.make_config(128, 1, 256, 64, 1024)
    fake = [ctypes.c_void_p(1 << 20)] * 8
    assert lib.mlaverify_run_static(ctypes.byref(cfg), 1, 256, *fake) == binding.ERR_WORKSPACE
    assert lib.mlaverify_run_static(None, 1, 256, *fake) == binding.ERR_INVALID_ARG
    assert lib.mlaverify_run_static(ctypes.byref(cfg), 2, 256, *fake) == binding.ERR_INVALID_ARG  # batch > max_batch
