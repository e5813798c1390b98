import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# The mutation test (test_oracle_mutants.py) re-runs the oracle pins in a child
# process against a copy of the oracle compiled with one planted mistake.
_MUTANT = os.environ.get("MAMBA_ORACLE_MUTANT_LIB")
if _MUTANT:
    from oracle import oracle as _oracle

    _oracle.use_library(_MUTANT)
