"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
function the header declares, handles NULL arguments and reports missing devices; the
header is valid C; the product package never reaches into the oracle."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "anchor_attn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))
PKG = os.path.join(ROOT, "efficient_vision_transformer_amd")


@pytest.fixture(scope="module")
def lib():
    from efficient_vision_transformer_amd import anchor_attn
    if not os.path.exists(anchor_attn.library_path()):
        from efficient_vision_transformer_amd import build
        build.build()
    return anchor_attn.load_library()


def _declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"\b(anchor_attn_[a-z_]+)\s*\(", text)))


@pytest.mark.parametrize("header", HEADERS, ids=os.path.basename)
def test_header_is_valid_c(header):
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", header],
                   check=True)


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"anchor_attn_create", "anchor_attn_forward", "anchor_attn_destroy",
            "anchor_attn_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(PKG, "libanchor_attn.so")],
                         capture_output=True, text=True, check=True).stdout
    for name in names:
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings(lib):
    for code, name in enumerate(["SUCCESS", "ERROR_INVALID_VALUE", "ERROR_NOT_SUPPORTED",
                                 "ERROR_OUT_OF_MEMORY", "ERROR_HIP"]):
        assert lib.anchor_attn_status_string(code).decode() == "ANCHOR_ATTN_" + name
    assert lib.anchor_attn_status_string(99).decode() == "ANCHOR_ATTN_ERROR_UNKNOWN_STATUS"


def test_null_arguments(lib):
    assert lib.anchor_attn_create(None) == 1
    assert lib.anchor_attn_destroy(None) == 0
    assert lib.anchor_attn_set_plan(None, 0) == 1
    assert lib.anchor_attn_forward(None, None, None, None, None, 1, 1, 1, 1, 32, 0, None) == 1
    assert lib.anchor_attn_forward_noalloc(None, None, None, None, None, 1, 1, 1, 1, 32, 0,
                                           None) == 1
    assert lib.anchor_attn_forward_strided(None, None, None, None, None, None, None, None,
                                           1, 1, 1, 1, 32, 0, None) == 1
    assert lib.anchor_attn_relu_linear_forward(None, None, None, None, None, None, None, None,
                                               None, 1, 1, 1, 32, 100.0, 1.0, 1, None) == 1
    assert lib.anchor_attn_block_forward(None, None, None, None, None, None, None, None,
                                         1, 1, 1, 1, 32, 1, None) == 1
    assert lib.anchor_attn_backward_strided(None, None, None, None, None, None, None, None,
                                            None, None, None, None, None, 1, 1, 1, 1, 32, 1,
                                            None) == 1
    assert lib.anchor_attn_backward(None, None, None, None, None, None, None, None,
                                    1, 1, 1, 1, 32, 1, None) == 1
    buf = ctypes.create_string_buffer(64)
    assert lib.anchor_attn_describe_plan(None, 1, 1, 1, 1, 32, 0, buf, 64) == 1


def test_create_without_device_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    assert lib.anchor_attn_create(ctypes.byref(h)) == 4
    assert not h.value


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from efficient_vision_transformer_amd import anchor_attn
    monkeypatch.setattr(anchor_attn, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(anchor_attn, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        anchor_attn.load_library()


def test_product_code_never_touches_the_oracle():
    """No product source imports, loads or links the oracle."""
    pat = re.compile(r"(import\s+oracle|from\s+oracle|anchor_oracle|libanchor_oracle)")
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f"{f} reaches into the oracle"
