"""The product path has no fallback: without the built HIP library every entry
point fails loudly, CPU tensors are refused, and nothing in the package or in
libh3fused.so refers to the oracle (which is test infrastructure only)."""
import os
import re
import subprocess
import sys

import pytest
import torch

import video_diffusion_transformer_h3f_amd as h3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.dirname(h3.__file__)


def test_missing_library_raises():
    code = (
        "import video_diffusion_transformer_h3f_amd as h3\n"
        "h3.LIB_PATH = '/nonexistent/libh3fused.so'\n"
        "try:\n"
        "    h3.abi_version()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('no error')\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=120)
    assert "raised:" in out.stdout and "not built" in out.stdout, out.stdout + out.stderr


def test_cpu_tensors_are_refused():
    a = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        h3.h3f_swiglu(torch.empty(4, 8, dtype=torch.bfloat16), a)
    with pytest.raises(ValueError):
        h3.h3f_adaln_modulate(torch.empty(4, 8), torch.zeros(4, 8), torch.zeros(1, 8),
                              torch.zeros(1, 8))


def _package_sources():
    for d, _, files in os.walk(PKG):
        if "_build" in d or "__pycache__" in d:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp", ".c")):
                yield os.path.join(d, f)


def test_package_sources_never_reach_the_oracle():
    pat = re.compile(r"\boracle\b|h3oracle|liboracle")
    hits = []
    for path in _package_sources():
        for i, line in enumerate(open(path, encoding="utf-8"), 1):
            if pat.search(line):
                hits.append(f"{os.path.relpath(path, ROOT)}:{i}: {line.strip()}")
    assert not hits, "\n".join(hits)


def test_library_links_no_oracle_code():
    if not os.path.exists(h3.LIB_PATH):
        pytest.skip("libh3fused.so not built")
    syms = subprocess.run(["nm", "-D", h3.LIB_PATH], capture_output=True, text=True,
                          check=True).stdout
    assert "oracle_" not in syms
    deps = subprocess.run(["readelf", "-d", h3.LIB_PATH], capture_output=True, text=True,
                          check=True).stdout
    assert "oracle" not in deps
