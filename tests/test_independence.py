"""The HIP path and the CPU oracle are independent (CPU only).

* Importing the package, or loading and calling its binding, brings in no
  part of ``oracle/``, and nothing under ``dense_gemm_08_amd/`` or
  ``include/`` names it.
* The oracle names nothing of the package or its sources.
* The only module both sides import is ``dense_gemm_08_amd.inputs``, which
  holds the seeded generators and no GEMM arithmetic.
* Without the built library every entry point fails loudly: there is no
  fallback path.
"""
import os
import re
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "dense_gemm_08_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        if "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def test_product_sources_do_not_name_the_oracle():
    for path in list(_files(PKG, (".py", ".hip", ".h", ".cpp"))) + list(
            _files(os.path.join(ROOT, "include"), (".h",))):
        text = open(path).read()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), path
        assert not re.search(r"#include\s+[<\"][^>\"]*oracle", text), path


def test_oracle_does_not_name_the_product():
    for path in _files(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        text = open(path).read()
        assert "dense_gemm_08_amd" not in text, path
        assert not re.search(r"#include\s+[<\"][^>\"]*(dense_gemm|cdna_ops|tile_sched)", text), path


def test_inputs_module_has_no_gemm_arithmetic():
    # the shared generator module draws and encodes values: no matrix
    # product anywhere in its code (docstrings aside)
    import ast
    tree = ast.parse(open(os.path.join(PKG, "inputs.py")).read())
    for node in ast.walk(tree):
        assert not (isinstance(node, ast.BinOp) and isinstance(node.op, ast.MatMult)), node.lineno
        if isinstance(node, ast.Call):
            f = node.func
            name = f.attr if isinstance(f, ast.Attribute) else getattr(f, "id", "")
            assert name not in ("matmul", "dot", "einsum", "tensordot", "inner", "mm", "bmm"), \
                (name, node.lineno)


def test_importing_and_loading_the_package_leaves_the_oracle_out():
    code = ("import sys; import dense_gemm_08_amd as dg; from dense_gemm_08_amd import binding; "
            "binding.load_library(); "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "print('loaded:', bad); sys.exit(1 if bad else 0)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_missing_library_fails_loudly():
    code = ("import dense_gemm_08_amd as dg\n"
            "try:\n"
            "    dg.load_library()\n"
            "except FileNotFoundError as e:\n"
            "    print('raised', e)\n"
            "else:\n"
            "    raise SystemExit('no error without the library')\n")
    env = dict(os.environ, DENSE_GEMM_LIB=os.path.join(ROOT, "no-such-library.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "raised" in r.stdout, r.stdout + r.stderr


@pytest.mark.parametrize("fn", ["gemm_nt_f16", "gemm_nn_bf16", "gemm_nt_e4m3_mx"])
def test_entry_points_fail_without_the_library(fn):
    # the Python entry points reach the library before touching any tensor
    # data: with no library they raise instead of computing anything
    code = ("import dense_gemm_08_amd as dg\n"
            "try:\n"
            "    dg.%s(None, None, None, None) if '%s' == 'gemm_nt_e4m3_mx' else dg.%s(None, None)\n"
            "except FileNotFoundError:\n"
            "    print('raised')\n" % (fn, fn, fn))
    env = dict(os.environ, DENSE_GEMM_LIB=os.path.join(ROOT, "no-such-library.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, env=env)
    assert "raised" in r.stdout, r.stdout + r.stderr
