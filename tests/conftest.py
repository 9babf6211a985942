import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, HERE):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded; GPU tests skip nothing silently: a missing build fails loudly."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    from block_diffusion_sparse_herald_amd import herald

    herald.load()
    return herald


def pytest_terminal_summary(terminalreporter):
    """Worst attention error per workload against its tolerance (GPU parity runs)."""
    from parity import MARGINS

    if not MARGINS:
        return
    terminalreporter.section("attention parity margins (max abs error vs the oracle / tolerance)")
    for name, (err, tol, count) in sorted(MARGINS.items()):
        terminalreporter.write_line(f"{name}: {err:.3g} / {tol:g} ({err / tol:.1%} of the tolerance, "
                                    f"{count} outputs)")
