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


@pytest.mark.parametrize("frames", [1, 63, 100, 3000, 1 << 21, -64])
def test_bad_micro_stack_sizes_are_rejected_before_any_device_work(lib, frames):
    cfg = mce.mce_config()
    assert mce.mce_config_init(cfg) == 0
    assert cfg.micro_stack_frames == 0          # 0: the default size
    cfg.micro_stack_frames = frames             # not a power of two in [64, 2^20]
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


LLVM_BIN = "/opt/rocm/llvm/bin"


def test_kernels_use_no_scratch_memory(lib, tmp_path):
    """Every kernel of the library keeps its state in registers and LDS. Scratch
    (private segment) memory in a kernel means spilled registers, or a structure
    handed by reference to a device function the compiler did not inline; in
    the peel that made the 45-vertex graph's ordering three times slower. The
    sizes come from the AMDGPU metadata of the library's own gfx950 code object."""
    import subprocess
    tools = [os.path.join(LLVM_BIN, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(os.path.exists(t) for t in tools):
        pytest.skip("ROCm LLVM tools not installed")
    objcopy, bundler, readelf = tools
    fatbin, code = str(tmp_path / "fatbin"), str(tmp_path / "gfx950.co")
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fatbin}", mce.LIB_PATH, str(tmp_path / "lib.so")],
                   check=True, capture_output=True)
    # one offload bundle per source file, each starting with the bundle magic
    blob = open(fatbin, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), blob)]
    assert starts
    names, sizes = [], []
    for i, a in enumerate(starts):
        piece = str(tmp_path / f"bundle{i}")
        with open(piece, "wb") as f:
            f.write(blob[a:starts[i + 1] if i + 1 < len(starts) else len(blob)])
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={piece}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={code}"], check=True,
                       capture_output=True)
        notes = subprocess.run([readelf, "--notes", code], check=True, capture_output=True, text=True).stdout
        names += re.findall(r"^\s+\.name:\s+(\S+)", notes, flags=re.M)
        sizes += [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)]
    assert len(names) == len(sizes) and len(names) >= 10
    assert any("k_peel" in n for n in names) and any("k_search_micro" in n for n in names)
    spilled = {n: s for n, s in zip(names, sizes) if s}
    assert not spilled, spilled
