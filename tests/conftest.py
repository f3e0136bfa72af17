import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _install_oracle_mutant():
    """When BSA_ORACLE_MUTANT holds a JSON [old, new] pair, load the oracle
    with that one textual change (a planted mistake) in place of the real
    one. Used only by the mutation test, which runs the oracle pins in a
    child process and expects them to fail."""
    spec = os.environ.get("BSA_ORACLE_MUTANT")
    if not spec:
        return
    import json
    import types
    old, new = json.loads(spec)
    path = os.path.join(ROOT, "oracle", "__init__.py")
    src = open(path).read()
    assert old in src, "mutation site not found"
    mod = types.ModuleType("oracle")
    mod.__file__ = path
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    sys.modules["oracle"] = mod


_install_oracle_mutant()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a visible device; on a CPU-only host they are skipped
    # (the product path itself raises loudly when the library or device is
    # missing, see block_sparse_matmul_amd._lib).
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
