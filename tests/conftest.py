import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(autouse=True)
def _poison_uninitialised_memory(request):
    """In GPU tests every tensor allocated without initialisation (torch.empty
    and its kind, in the tests and in the binding: workspaces, outputs, the
    sampler schedule, the modulation table) starts filled with NaN (floating
    point) or all-ones bytes (integers), so a kernel that reads memory it did
    not write first shows up as a non-finite or mismatching output."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch
    det = torch.are_deterministic_algorithms_enabled()
    warn = torch.is_deterministic_algorithms_warn_only_enabled()
    fill = torch.utils.deterministic.fill_uninitialized_memory
    torch.use_deterministic_algorithms(True, warn_only=True)
    torch.utils.deterministic.fill_uninitialized_memory = True
    try:
        yield
    finally:
        torch.use_deterministic_algorithms(det, warn_only=warn)
        torch.utils.deterministic.fill_uninitialized_memory = fill
