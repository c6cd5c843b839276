"""Separation rules, checked on the CPU.

* The product path (the package and the input generators) never imports the
  oracle, and the oracle never imports the product path: the two share no
  code beyond the seeded input module.
* The oracle is reached only from the tests, ``__graft_entry__.smoke`` and the
  benchmark's CPU-baseline leg.
* A missing library or a host tensor makes the binding raise: there is no CPU
  fallback that could compute a result.
"""
import ast
import glob
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    """(imported module, enclosing function name or None) for every import."""
    tree = ast.parse(open(path, encoding="utf-8").read(), filename=path)
    found = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else func
            if isinstance(child, ast.Import):
                found.extend((a.name, func) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                found.append((child.module or "", func))
            visit(child, f)

    visit(tree, None)
    return found


def _product_files():
    files = glob.glob(os.path.join(ROOT, "reduce_residual_add_amd", "**", "*.py"), recursive=True)
    files.append(os.path.join(ROOT, "workloads.py"))
    return files


def test_product_path_never_imports_the_oracle():
    for path in _product_files():
        for mod, _ in _imports(path):
            assert not mod.split(".")[0] == "oracle", f"{path} imports {mod}"
    for path in glob.glob(os.path.join(ROOT, "reduce_residual_add_amd", "csrc", "*")):
        text = open(path, encoding="utf-8", errors="replace").read().lower()
        assert "oracle" not in text, f"{path} mentions the oracle"


def test_oracle_never_imports_the_product_path():
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        for mod, _ in _imports(path):
            top = mod.split(".")[0]
            assert top not in ("reduce_residual_add_amd", "torch", "bench", "ctypes"), \
                f"{path} imports {mod}"


@pytest.mark.parametrize("path,allowed", [
    ("bench.py", {"cpu_baseline"}),
    ("__graft_entry__.py", {"smoke"}),
])
def test_oracle_reached_only_from_allowed_functions(path, allowed):
    uses = [(mod, func) for mod, func in _imports(os.path.join(ROOT, path))
            if mod.split(".")[0] == "oracle"]
    assert uses, f"{path} was expected to use the oracle somewhere"
    for mod, func in uses:
        assert func in allowed, f"{path} imports {mod} in {func!r}, outside {sorted(allowed)}"


def test_missing_library_raises(monkeypatch):
    import reduce_residual_add_amd as twn
    monkeypatch.setattr(twn, "_lib", None)
    with pytest.raises(ImportError, match="no CPU fallback"):
        twn.load(os.path.join(ROOT, "no_such_dir", "libtwnorm.so"))


def test_host_tensors_are_refused():
    """With CPU tensors the binding raises before any computation; if the
    library is not built it raises ImportError instead.  Either way no
    result is produced."""
    import torch
    import reduce_residual_add_amd as twn
    parts = [torch.zeros(4, 64, dtype=torch.bfloat16) for _ in range(2)]
    res = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises((ValueError, ImportError)):
        twn.fused_reduce_rmsnorm(parts, res, w, 1e-5)
    with pytest.raises((ValueError, ImportError)):
        twn.reduce(parts)
    with pytest.raises((ValueError, ImportError)):
        twn.rmsnorm(res, res, w, 1e-5)
    with pytest.raises((ValueError, ImportError)):
        twn.PreparedFused(parts, res, w, 1e-5, torch.empty_like(res), torch.empty_like(res))
    with pytest.raises((ValueError, ImportError)):
        twn.stream_copy(res, torch.empty_like(res))
    with pytest.raises((ValueError, ImportError)):
        twn.stream_mix([res], [torch.empty_like(res)])


def test_tensors_off_the_current_device_are_refused(monkeypatch):
    """The library launches on the current device and takes its CU count
    from it, so the binding refuses tensors or a stream on another device
    (checked here with a stand-in for torch's current-device query)."""
    import types
    import reduce_residual_add_amd as twn
    fake = types.SimpleNamespace(_C=types.SimpleNamespace(_cuda_getDevice=lambda: 0))
    monkeypatch.setattr(twn, "_torch", lambda: fake)
    twn._check_device(0)
    with pytest.raises(ValueError, match="current device is cuda:0"):
        twn._check_device(1)
    on1 = types.SimpleNamespace(device=types.SimpleNamespace(index=1))
    on0 = types.SimpleNamespace(device=types.SimpleNamespace(index=0))
    twn._check_device(0, on0)
    twn._check_device(0, object())      # a stream object that names no device
    with pytest.raises(ValueError, match="stream is on cuda:1"):
        twn._check_device(0, on1)
