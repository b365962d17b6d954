"""The oracle, the input generators and the HIP product path share no code."""

import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "kv_cache_quantization_codec_amd"


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    out = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            if node.level:
                out.add(".")
            elif node.module:
                out.add(node.module.split(".")[0])
    return out


def _py_files(d):
    for dp, _, fns in os.walk(os.path.join(ROOT, d)):
        for fn in fns:
            if fn.endswith(".py"):
                yield os.path.join(dp, fn)


def test_oracle_imports_only_stdlib_and_numpy():
    allowed = {".", "__future__", "fractions", "numpy", "math", "struct", "typing"}
    for f in _py_files("oracle"):
        assert _imports(f) <= allowed, (f, _imports(f) - allowed)


def test_oracle_has_no_native_or_hip_sources():
    for dp, _, fns in os.walk(os.path.join(ROOT, "oracle")):
        for fn in fns:
            assert not fn.endswith((".hip", ".cu", ".h", ".hpp", ".cpp", ".so")), fn


def test_generators_import_neither_codec_nor_oracle():
    for f in _py_files("kvsynth"):
        imps = _imports(f)
        assert "oracle" not in imps and PKG not in imps, f


def test_product_path_never_imports_the_oracle():
    files = list(_py_files(PKG))
    assert files, "package missing"
    for f in files:
        imps = _imports(f)
        assert "oracle" not in imps and "kvsynth" not in imps, f
        src = open(f).read()
        assert "oracle" not in src.replace("oracle-free", ""), f
