import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip-free guard: a `gpu` test that runs without a GPU is an error, not a skip."""
    if not _gpu_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import torch
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    from tests import parity_log
    if not parity_log.RECORDS:
        return
    tr = terminalreporter
    tr.section("measured parity margins (value / bound)")
    worst = {}
    for r in parity_log.RECORDS:
        key = r["kind"]
        if key not in worst or r["value"] / r["bound"] > worst[key]["value"] / worst[key]["bound"]:
            worst[key] = r
    for r in parity_log.RECORDS:
        tr.write_line(f"{r['kind']:<18} {r['value']:.3e} / {r['bound']:.0e}  {r['test']} {r['what']}")
    for k, r in worst.items():
        tr.write_line(f"worst {k}: {r['value']:.3e} of {r['bound']:.0e} ({r['test']} {r['what']})")
    path = os.environ.get("SPECACHE_PARITY_LOG")
    if path:
        import json
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(parity_log.RECORDS, f, indent=1)
