"""Rewrites tests/golden/expected_counts.json: the number of test items each
module under tests/ collects (all of them, before any -m or -k selection).
Run it after adding or removing tests on purpose; the suite refuses to run
while a module's count differs from the file.

    python tests/golden/update_expected_counts.py
"""
import json
import os
import sys
from collections import Counter

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)


class _Collect:
    def __init__(self):
        self.items = []

    def pytest_collection_finish(self, session):
        self.items = list(session.items)


def main():
    os.environ["DR_UPDATE_COUNTS"] = "1"
    c = _Collect()
    rc = pytest.main([TESTS, "--collect-only", "-q", "-p", "no:cacheprovider"], plugins=[c])
    if rc != 0:
        sys.exit(rc)
    counts = dict(sorted(Counter(os.path.basename(i.nodeid.split("::")[0]) for i in c.items).items()))
    with open(os.path.join(HERE, "expected_counts.json"), "w") as f:
        json.dump(counts, f, indent=1)
        f.write("\n")
    print(f"{sum(counts.values())} items in {len(counts)} modules")


if __name__ == "__main__":
    main()
