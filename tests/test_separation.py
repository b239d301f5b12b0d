"""The oracle and the HIP library stay apart (CPU only).

The product path (the package: its Python binding and every HIP/C++ source) never names
the oracle; the oracle never names the package or its sources; bench.py and the graft
entry import the oracle only inside the functions that time or check against it; and
the binding refuses to run without its compiled library instead of falling back."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_sparse_kv_csa_amd")


def _files(top, exts):
    for d, _, fs in os.walk(top):
        if "_build" in d or "__pycache__" in d:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(d, f)


def test_the_product_path_never_names_the_oracle():
    for path in list(_files(PKG, (".py", ".hip", ".cpp", ".h"))) + list(_files(os.path.join(ROOT, "include"), (".h",))):
        text = open(path, encoding="utf-8").read()
        assert "oracle" not in text.lower(), path


def test_the_oracle_never_names_the_library():
    for path in _files(os.path.join(ROOT, "oracle"), (".py",)):
        text = open(path, encoding="utf-8").read()
        for word in ("compressed_sparse_kv_csa_amd", "csrc", "libcsakv", "ctypes"):
            assert word not in text, (path, word)


def _module_level_imports(path):
    tree = ast.parse(open(path, encoding="utf-8").read())
    names = []
    for node in tree.body:  # top-level statements only
        if isinstance(node, ast.Import):
            names += [a.name for a in node.names]
        elif isinstance(node, ast.ImportFrom):
            names.append(node.module or "")
    return names


def _functions_importing(path, module):
    tree = ast.parse(open(path, encoding="utf-8").read())
    found = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, ast.ImportFrom) and (node.module or "").split(".")[0] == module:
                    found.add(fn.name)
                if isinstance(node, ast.Import) and any(a.name.split(".")[0] == module for a in node.names):
                    found.add(fn.name)
    return found


def test_bench_and_entry_import_the_oracle_only_where_they_use_it():
    bench = os.path.join(ROOT, "bench.py")
    entry = os.path.join(ROOT, "__graft_entry__.py")
    for path in (bench, entry):
        assert not any(n.split(".")[0] == "oracle" for n in _module_level_imports(path)), path
    users = _functions_importing(bench, "oracle")
    assert users and all("cpu" in f for f in users), users  # the cpu_baseline leg only
    assert _functions_importing(entry, "oracle") == {"smoke"}


def test_the_binding_fails_loudly_without_its_library(tmp_path):
    missing = str(tmp_path / "libcsakv.so")
    code = ("import compressed_sparse_kv_csa_amd as ck\n"
            "try:\n    ck.lib()\nexcept RuntimeError as e:\n    print('refused:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, CSAKV_LIBRARY=missing))
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.startswith("refused:") and "missing" in r.stdout
