"""The C-ABI library loads without a GPU and exports every entry point that
include/dg.h declares; the binding covers the same set.  No compute calls."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_three_phase_calls():
    names = _declared()
    for n in ("dg_denoise_step", "dg_generate_canvas", "dg_commit_canvas", "dg_model_create"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from diffusion_decoding_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libdg.so not built")
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(_lib.ENTRY_POINTS) == _declared()


def test_status_strings_without_gpu():
    from diffusion_decoding_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libdg.so not built")
    lib = _lib.load()
    assert lib.dg_status_str(0) == b"ok"
    assert lib.dg_status_str(-2) == b"shape error"
    assert b"gfx950" in lib.dg_version()


def test_invalid_arguments_are_rejected_before_any_launch():
    """Host-side validation: bad configs fail with a status, nothing is launched."""
    from diffusion_decoding_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libdg.so not built")
    from diffusion_decoding_amd.runtime import make_config
    from workloads import get_config
    cfg = make_config(get_config("c0"))
    w = _lib.dg_weights(None, None, None)
    with pytest.raises(_lib.DGError) as e:
        _lib.dg_model_create(cfg, w, 1, 0, 0)
    assert e.value.status == -1
    bad = make_config(get_config("c0").replace(head_dim=12))
    with pytest.raises(_lib.DGError) as e:
        _lib.dg_model_create(bad, w, 1, 0, 0)
    assert e.value.status == -2
    bad = make_config(get_config("c0").replace(top_k=9))
    with pytest.raises(_lib.DGError) as e:
        _lib.dg_model_create(bad, w, 1, 0, 0)
    assert e.value.status == -2
    for mt in (512, -2):  # the [MASK] id must be a vocabulary id (c0: 512 ids) or -1
        bad = make_config(get_config("c0").replace(mask_token=mt))
        with pytest.raises(_lib.DGError) as e:
            _lib.dg_model_create(bad, w, 1, 0, 0)
        assert e.value.status == -1 and "mask_token" in str(e.value)
    lib = _lib.load()
    assert lib.dg_denoise_step(None, None, None, None, None) == -1
    assert lib.dg_commit_canvas(None, None, 0, None, None) == -1


STRUCTS = ["dg_config", "dg_layer_weights", "dg_weights", "dg_kv", "dg_canvas", "dg_step_out", "dg_segment"]


def _c_layout(tmp_path):
    """Size and field offsets of every ABI struct, as the C compiler lays out
    include/dg.h (a small program built with gcc here)."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    from diffusion_decoding_amd import _lib
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dg.h"', "int main(void) {"]
    for name in STRUCTS:
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in getattr(_lib, name)._fields_:
            lines.append(f'  printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ["  return 0;", "}"]
    src, exe = tmp_path / "layout.c", tmp_path / "layout"
    src.write_text("\n".join(lines) + "\n")
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    return {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}


def test_binding_structs_match_the_header_layout(tmp_path):
    """Every struct the binding passes across the ABI has the header's size and
    field offsets (a field added on one side only fails here)."""
    from diffusion_decoding_amd import _lib
    c = _c_layout(tmp_path)
    for name in STRUCTS:
        cls = getattr(_lib, name)
        assert c[(name, "size")] == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert c[(name, field)] == getattr(cls, field).offset, (name, field)
