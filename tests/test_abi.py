"""The C-ABI library: it loads and exports every function include/mce.h declares
(no GPU needed: nothing here calls into the device)."""
import ctypes
import os
import re

import pytest

import maximal_clique_enumeration_amd as mce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mce.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mce_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not mce.lib_built():
        from maximal_clique_enumeration_amd import build
        build.build()
    return ctypes.CDLL(mce.LIB_PATH)


def test_header_declares_the_api():
    names = declared_functions()
    for want in ("mce_create", "mce_run", "mce_result", "mce_destroy", "mce_run_roots", "mce_ordering"):
        assert want in names
    assert sorted(mce.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_without_device(lib):
    lib.mce_status_string.restype = ctypes.c_char_p
    assert lib.mce_status_string(0) == b"MCE_OK"
    assert lib.mce_status_string(-2) == b"MCE_ERR_GRAPH"
    cfg = mce.mce_config()
    assert mce.mce_config_init(cfg) == 0
    assert (cfg.worker_list, cfg.donate_min_p, cfg.validate, cfg.timeout_ms) == (1, 1, 1, 120000)
    assert cfg.micro_donate_min_p == 10
    assert cfg.subgraph == mce.MCE_SUBGRAPH_AUTO
    assert cfg.struct_size == ctypes.sizeof(mce.mce_config)


def test_flag_values_match_the_header():
    text = open(os.path.join(ROOT, "include", "mce.h")).read()
    flags = dict(re.findall(r"#define (MCE_FLAG_[A-Z0-9_]+) (\d+)u", text))
    assert "MCE_FLAG_L2" in flags
    for name, value in flags.items():
        assert getattr(mce, name) == int(value), name


def test_unknown_flags_are_rejected_before_any_device_work(lib):
    cfg = mce.mce_config()
    assert mce.mce_config_init(cfg) == 0
    cfg.flags = 1 << 12
    h = ctypes.c_void_p()
    assert mce.mce_create(cfg, h) == mce.MCE_ERR_ARG
    assert not h.value


def test_null_arguments_are_rejected(lib):
    lib.mce_result.restype = ctypes.c_int
    assert lib.mce_result(None, None, None, None, 0, None) == mce.MCE_ERR_ARG
    lib.mce_destroy(None)   # ignored


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mce, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(mce, "_lib", None)
    with pytest.raises(mce.MceLibraryMissing):
        mce.load_library()
