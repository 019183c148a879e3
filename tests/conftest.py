import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Rows of a golden fixture: whitespace-split fields, comments dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture
def golden():
    return read_golden


@pytest.fixture(params=["auto", "chunks"])
def split(request):
    """Run the test under both decode work splits: the default (per-pair
    workgroups where the shape allows) and the persistent chunk split."""
    import paged_kv_cache_resolve_amd as pk
    mode = pk.SPLIT_AUTO if request.param == "auto" else pk.SPLIT_CHUNKS
    with pk.split_mode(mode):
        yield request.param
