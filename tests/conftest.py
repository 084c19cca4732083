"""Shared pytest configuration: markers, the oracle, golden-file readers."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def qref():
    import oracle
    return oracle.load()


@pytest.fixture(scope="session")
def mutant_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("qref_mutants"))


def golden_lines(name):
    """Non-comment, non-empty lines of a golden file, split on whitespace."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def golden_kv(name):
    """Golden file of 'key v1 v2 ...' lines -> dict key -> list of strings."""
    return {p[0]: p[1:] for p in golden_lines(name)}


def unpack_nibbles(wbytes, I):
    """[..., rb] packed bytes -> [..., I] nibbles, low nibble = even column.

    The byte layout stated for grouped int4 (colibri PR #457, section 3).
    """
    lo = wbytes & 0x0F
    hi = wbytes >> 4
    q = np.stack([lo, hi], axis=-1).reshape(*wbytes.shape[:-1], -1)
    return q[..., :I].astype(np.int64)
