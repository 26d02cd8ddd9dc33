"""Shared pytest set-up: the ``gpu`` marker, import paths and common fixtures."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; the parity tests proper")


@pytest.fixture(scope="session")
def oracle_lib():
    """The oracle library; ORACLE_LIB may point the pins at another build of it (the
    mutant tests use this to run the pins against oracles with planted mistakes)."""
    import oracle
    path = os.environ.get("ORACLE_LIB")
    return oracle.load(path, rebuild_if_missing=False) if path else oracle.load()
