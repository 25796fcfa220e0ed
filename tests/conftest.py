import json
import os
import sys
from collections import Counter

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

# How many test items each module must collect.  A parametrisation that
# silently collapses (an empty id list, a shape filter gone wrong) would
# otherwise still pass; this count is the suite's own sentinel (vllm.cpp PR
# #2556, section "Gates, read literally": the instrument asserts its own
# line count).  Changing a module's tests means rewriting that file with
# tests/golden/update_expected_counts.py, a deliberate step.
EXPECTED_COUNTS = os.path.join(HERE, "golden", "expected_counts.json")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.hookimpl(tryfirst=True)
def pytest_collection_modifyitems(session, config, items):
    """Before -m / -k deselection: every module collected whole must hold
    exactly its expected number of items.  Runs that name single tests
    (path::name) are not checked."""
    if any("::" in str(a) for a in config.args) or os.environ.get("DR_UPDATE_COUNTS"):
        return
    with open(EXPECTED_COUNTS) as f:
        want = json.load(f)
    got = Counter(os.path.basename(item.nodeid.split("::")[0]) for item in items)
    bad = {m: (n, want.get(m)) for m, n in got.items() if want.get(m) != n}
    if bad:
        lines = ", ".join(f"{m}: collected {n}, expected {w}" for m, (n, w) in sorted(bad.items()))
        raise pytest.UsageError(f"test counts differ from tests/golden/expected_counts.json: {lines}")
