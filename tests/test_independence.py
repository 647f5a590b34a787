"""The HIP path and the oracle stay apart: no module of the package imports
the oracle (the tuner and the bench's after-run check use a plain float64
product instead), and the oracle imports nothing from the package.  The
seeded input generator (``inputs.py``) is the one module both sides call,
and it holds none of the GEMM's arithmetic."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "latency_decode_gemm_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _imported_modules(path):
    tree = ast.parse(open(path, encoding="utf-8").read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def _py_files(d):
    return [os.path.join(d, f) for f in sorted(os.listdir(d)) if f.endswith(".py")]


def test_package_sources_never_import_the_oracle():
    for f in _py_files(PKG):
        assert "oracle" not in _imported_modules(f), f


def test_oracle_sources_never_import_the_package():
    for f in _py_files(ORACLE):
        assert "latency_decode_gemm_amd" not in _imported_modules(f), f


def test_importing_every_package_module_loads_no_oracle():
    mods = [os.path.splitext(os.path.basename(f))[0] for f in _py_files(PKG)
            if not os.path.basename(f).startswith("__")]
    code = ("import sys, importlib\n"
            f"for m in {mods!r}:\n"
            "    importlib.import_module('latency_decode_gemm_amd.' + m)\n"
            "print(sorted(k for k in sys.modules if k == 'oracle' or k.startswith('oracle.')))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "[]", r.stdout


def test_input_generator_holds_no_gemm_arithmetic():
    src = open(os.path.join(PKG, "inputs.py"), encoding="utf-8").read()
    for op in ("@", "matmul", "einsum", ".dot(", "tensordot"):
        assert op not in src, op
