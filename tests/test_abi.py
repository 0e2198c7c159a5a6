"""The C-ABI library loads and exports every entry point include/psgd.h declares (CPU only),
and the ctypes structures match the C layout."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psgd.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psgd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_step_calls():
    names = _declared()
    for n in ("psgd_compress", "psgd_check_finite", "psgd_decompress_update", "psgd_create",
              "psgd_destroy", "psgd_plan_create", "psgd_plan_destroy", "psgd_last_error",
              "psgd_compress_p", "psgd_orthogonalize", "psgd_compress_q", "psgd_refresh_q",
              "psgd_factor_buffer", "psgd_reset_errors", "psgd_block_grad_enter", "psgd_block_grad_exit",
              "psgd_block_grad_exit_enter", "psgd_step_noalloc", "psgd_adam_attach", "psgd_adam_prepare",
              "psgd_decompress_adam", "psgd_adam_update"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from rank_gradient_compression_powersgd_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libpsgd.so is not built (run python -m rank_gradient_compression_powersgd_amd.build)")
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert binding.load_library().psgd_version() == 1


def test_binding_names_match_header():
    import rank_gradient_compression_powersgd_amd as pkg
    for n in _declared():
        assert hasattr(pkg, n) or n in ("psgd_debug_buffer",), n


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_struct_layout_matches_c(tmp_path):
    from rank_gradient_compression_powersgd_amd.binding import (
        psgd_adam_hparams, psgd_adam_matrix, psgd_adam_tensor, psgd_matrix, psgd_tensor)
    structs = (psgd_matrix, psgd_tensor, psgd_adam_hparams, psgd_adam_matrix, psgd_adam_tensor)
    src = tmp_path / "layout.c"
    body = ""
    for st in structs:
        body += f' printf("%zu\\n", sizeof({st.__name__}));\n'
        body += "".join(f' printf("%zu\\n", offsetof({st.__name__}, {f}));\n' for f, _ in st._fields_)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "psgd.h"\nint main(void){\n'
                   + body + " return 0; }\n")
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    k = 0
    for st in structs:
        assert vals[k] == ctypes.sizeof(st), st.__name__
        k += 1
        for f, _ in st._fields_:
            assert getattr(st, f).offset == vals[k], (st.__name__, f)
            k += 1
    assert k == len(vals)


def test_product_path_fails_loudly_without_library(tmp_path):
    from rank_gradient_compression_powersgd_amd import binding
    with pytest.raises(ImportError):
        binding.load_library(str(tmp_path / "missing.so"))


def test_oracle_is_not_imported_by_the_product():
    pkg = os.path.join(ROOT, "rank_gradient_compression_powersgd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), errors="ignore").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "oracle/" not in text, f


@pytest.mark.parametrize("call", ["enter", "exit", "exit_enter"])
def test_binding_argument_checks_raise_psgd_error(call):
    """The Python-side checks of the block-scaling wrappers (sizes, contiguity, dtype) run
    before any library call and raise PsgdError with the call's name and status."""
    import torch
    from rank_gradient_compression_powersgd_amd import binding as B
    dx = torch.zeros(16, dtype=torch.float32)
    g16 = torch.zeros(16, dtype=torch.float16)
    short = torch.zeros(8, dtype=torch.float16)
    f32 = torch.zeros(16, dtype=torch.float32)
    strided = torch.zeros(32, dtype=torch.float16)[::2]
    one = torch.ones(1)
    fn = {
        "enter": lambda out: B.psgd_block_grad_enter(0, dx, one, out),
        "exit": lambda g: B.psgd_block_grad_exit(0, dx, g, one),
        "exit_enter": lambda g: B.psgd_block_grad_exit_enter(0, dx, g, one, one, g16),
    }[call]
    name = "psgd_block_grad_" + call
    for bad, status in ((short, B.PSGD_EINVAL), (strided, B.PSGD_EINVAL), (f32, B.PSGD_EDTYPE)):
        with pytest.raises(B.PsgdError) as ei:
            fn(bad)
        assert ei.value.status == status and name in str(ei.value)
    if call == "exit_enter":
        with pytest.raises(B.PsgdError) as ei:
            B.psgd_block_grad_exit_enter(0, dx, g16, one, one, torch.zeros(16, dtype=torch.bfloat16))
        assert ei.value.status == B.PSGD_EDTYPE
