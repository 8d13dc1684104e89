"""pytest configuration: the `gpu` marker and the import path.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything else runs on the
CPU (the oracle and its pins, the input generator, the host-side ABI checks)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU and the built HIP library")
