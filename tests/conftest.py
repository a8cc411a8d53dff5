import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def load_golden(name):
    """Parse a tests/golden fixture: '# ...' lines are comments, 'key: values'
    lines hold whitespace-separated integers; a repeated key adds a row."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    out = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, vals = line.partition(":")
            row = [int(v) for v in vals.split()]
            out.setdefault(key.strip(), []).append(row)
    return {k: (v[0] if len(v) == 1 else v) for k, v in out.items()}
