import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of oracle time)")


@pytest.fixture(scope="session")
def oracle_c_built():
    """Make sure the oracle's plain-C generator exists (built on demand on the CPU)."""
    from oracle import build, rng
    if not rng.have_c():
        build.build()
    return True


@pytest.fixture(autouse=True)
def _report_worst_logits(request):
    """After each GPU test, print the worst logits cosine / max relative error it saw."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    try:
        from tests import gpu_util
    except Exception:
        return
    for kind, (cos, rel) in sorted(gpu_util.WORST.items()):
        print(f"[{request.node.name}] worst {kind}: cos {cos:.7f} rel {rel:.3e}", file=sys.stderr,
              flush=True)
    gpu_util.WORST.clear()
