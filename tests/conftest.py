"""Shared pytest set-up: the repository root on sys.path and the `gpu` marker.

CPU tests (`-m "not gpu"`) check the oracle against what the pages and
mathematics fix, and check that the C-ABI library loads. GPU tests (`-m gpu`)
compare the HIP path with the oracle on an MI355X.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle():
    from oracle import build as obuild
    from oracle import oracle as O

    if not os.path.exists(O.LIB_PATH):
        obuild.build()
    return O
