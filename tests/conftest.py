"""Shared fixtures.  `gpu` marks tests that need an MI355X; everything else
runs on the CPU.  The C oracle and the input generator are compiled here on
first use if they are not built yet (gcc only, a second each)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def syn():
    import synth

    synth.lib()
    return synth
