"""The oracle and the HIP path share no code, and the product path never reaches the oracle.

Static checks over the sources:
* nothing under the package (Python binding, build script, HIP sources) or the C header
  imports, includes or names the oracle module;
* the oracle imports nothing but numpy and the standard library, so it cannot reach the
  library, its build products or the shared input generators' device code;
* the seeded input module imports neither side.
"""
import ast
import pathlib
import re

ROOT = pathlib.Path(__file__).resolve().parent.parent


def _py_imports(path):
    tree = ast.parse(path.read_text())
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            mods.add(("." * node.level) + (node.module or ""))
    return mods


def test_package_never_reaches_the_oracle():
    pkg = ROOT / "nvfp4_bit_kv_amd"
    for path in pkg.rglob("*.py"):
        if "_build" in path.parts:
            continue
        mods = _py_imports(path)
        assert not any(m.split(".")[0] in ("oracle", "tests") for m in mods), (path, mods)
        assert "oracle" not in path.read_text(), path
    for path in list((pkg / "csrc").glob("*.hip")) + list((pkg / "csrc").glob("*.hpp")) + \
            list((ROOT / "include").glob("*.h")):
        text = path.read_text()
        includes = re.findall(r'#include\s+[<"]([^">]+)[">]', text)
        assert not any("oracle" in inc for inc in includes), (path, includes)
        assert "nvfp4_oracle" not in text, path


def test_oracle_imports_only_numpy_and_the_standard_library():
    allowed = {"__future__", "numpy", "math", "fractions", "itertools", "functools", "typing", "dataclasses",
               ".nvfp4_oracle", "."}
    for path in (ROOT / "oracle").glob("*.py"):
        mods = _py_imports(path)
        assert mods <= allowed, (path, mods - allowed)


def test_input_generators_import_neither_side():
    for path in (ROOT / "synth").glob("*.py"):
        mods = _py_imports(path)
        roots = {m.lstrip(".").split(".")[0] for m in mods}
        assert not roots & {"oracle", "nvfp4_bit_kv_amd", "tests", "bench"}, (path, mods)
