"""The product path has no fallback: without libkvq.so every call fails
loudly, and no module of the package reaches the oracle."""
import ast
import os

import pytest

import int2_rotated_kv_amd.kvq as K

PKG = os.path.dirname(os.path.abspath(K.__file__))


def test_missing_library_raises(tmp_path):
    saved_path, saved_lib = K._LIB_PATH, K._lib
    try:
        K._LIB_PATH = str(tmp_path / "libkvq.so")
        K._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            K.load_library()
        with pytest.raises(RuntimeError, match="not built"):
            K.kvq_decode_workspace_bytes(1, 1, 1, 128, 64)
    finally:
        K._LIB_PATH, K._lib = saved_path, saved_lib


def test_package_does_not_import_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)
