"""The oracle and the HIP path share no code.

The product (the package and its HIP sources) never imports, includes or
links anything under oracle/; the oracle never imports the package; the
seeded input generators in synth/ import neither.  Checked on the sources'
import statements and #include lines, so it runs without a GPU.  Without
libbsq.so the binding raises instead of computing anything.
"""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "block_scaled_precision_blockwise_amd"


def _files(top, exts):
    out = []
    for d, _, names in os.walk(os.path.join(ROOT, top)):
        if "__pycache__" in d:
            continue
        out += [os.path.join(d, n) for n in names if n.endswith(exts)]
    assert out, f"no {exts} files under {top}/"
    return out


def _py_imports(path):
    with open(path) as f:
        tree = ast.parse(f.read(), path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            mods.add(node.module.split(".")[0])
        elif isinstance(node, ast.Call) and getattr(node.func, "attr", None) == "import_module":
            if node.args and isinstance(node.args[0], ast.Constant):
                mods.add(str(node.args[0].value).split(".")[0])
    return mods


def _c_includes(path):
    with open(path, errors="replace") as f:
        return re.findall(r'^\s*#\s*include\s*[<"]([^>"]+)[>"]', f.read(), re.M)


@pytest.mark.parametrize("path", _files(PKG, (".py",)))
def test_package_python_never_imports_the_oracle(path):
    assert "oracle" not in _py_imports(path), path


@pytest.mark.parametrize("path", _files(PKG, (".hip", ".h", ".hpp", ".cpp", ".c")))
def test_hip_sources_never_include_the_oracle(path):
    bad = [i for i in _c_includes(path) if "oracle" in i]
    assert not bad, (path, bad)
    with open(path, errors="replace") as f:
        assert "oracle/" not in f.read(), path


@pytest.mark.parametrize("path", _files("oracle", (".py",)))
def test_oracle_never_imports_the_package(path):
    mods = _py_imports(path)
    assert PKG not in mods and "synth" not in mods, (path, mods)


@pytest.mark.parametrize("path", _files("synth", (".py",)))
def test_generators_import_neither_side(path):
    mods = _py_imports(path)
    assert PKG not in mods and "oracle" not in mods, (path, mods)


def test_build_links_no_oracle_code():
    """The library's build line names only the package's own sources."""
    with open(os.path.join(ROOT, "__graft_entry__.py")) as f:
        src = f.read()
    tree = ast.parse(src)
    for node in ast.walk(tree):
        if isinstance(node, ast.Constant) and isinstance(node.value, str) and node.value.endswith((".hip", ".c", ".o")):
            assert "oracle" not in node.value, node.value


def test_binding_fails_loudly_without_the_library():
    """With libbsq.so absent every call raises; nothing computes elsewhere."""
    import subprocess
    import sys
    code = (
        "import block_scaled_precision_blockwise_amd as b, torch\n"
        "b._LIB_PATH = '/nonexistent/libbsq.so'\n"
        "b._lib = None\n"
        "try:\n"
        "    b.bsq_version()\n"
        "    raise SystemExit('bsq_version returned without the library')\n"
        "except RuntimeError as e:\n"
        "    assert 'libbsq.so' in str(e), e\n"
        "x = torch.randn(4, 128)\n"
        "q = torch.empty(4, 128, dtype=torch.uint8)\n"
        "s = torch.empty(4, 1)\n"
        "try:\n"
        "    b.bsq_quant_fp8_rowblock(x, q, s, 128)\n"
        "    raise SystemExit('a quantizer returned without the library')\n"
        "except (RuntimeError, ValueError):\n"
        "    pass\n"
        "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
