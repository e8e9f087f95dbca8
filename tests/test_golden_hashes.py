"""Bitwise regression baseline, oracle side: the CPU oracle still produces the digests stored
in tests/golden/oracle_hashes.json (written by tests/golden/make_hashes.py, which calls only
the oracle).  A change to the oracle's arithmetic shows up here as drift."""
import json
import os
import sys

import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
if GOLDEN not in sys.path:
    sys.path.insert(0, GOLDEN)

import cases as golden  # noqa: E402
import make_hashes  # noqa: E402

STORED = json.load(open(golden.HASH_FILE))


@pytest.mark.parametrize("name", sorted(golden.cases()))
def test_oracle_matches_stored_digest(orc, name):
    desc, kind, build = golden.cases()[name]
    assert name in STORED and STORED[name]["kind"] == kind
    assert make_hashes.oracle_digest(kind, build()) == STORED[name]["sha256"], name
