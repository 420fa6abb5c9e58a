import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


# The mutation tests run the pin suites in a child process against an oracle
# build with a planted mistake; the child points the oracle at that build here.
_MUTANT = os.environ.get("PDA_ORACLE_MUTANT")
if _MUTANT:
    import oracle as _oracle
    _oracle.use_library(_MUTANT)
