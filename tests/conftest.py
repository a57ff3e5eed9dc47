import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    out = os.environ.get("QSA_MARGINS_OUT")
    if not out:
        return
    try:
        from tests import gpu_helpers
    except Exception:  # pragma: no cover
        return
    import json
    rows = {k: {"max_abs_d_out": v[0], "max_abs_d_lse": v[1], "comparisons": v[2]}
            for k, v in sorted(gpu_helpers.MARGINS.items())}
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    with open(out, "w") as f:
        json.dump({"tolerance": gpu_helpers.OUT_TOL, "margins": rows, "recall": gpu_helpers.RECALL}, f,
                  indent=1)
