"""The CPU oracle against its pins (brute force, closed forms, worked
examples from the pages, exhaustive decoder checks).  No GPU needed."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_oracle_rebuilds_on_source_change(tmp_path):
    """A library built from another source is rebuilt, not reused."""
    import os
    import shutil
    src = os.path.join(tmp_path, "o.c")
    lib = os.path.join(tmp_path, "libo.so")
    shutil.copy(oracle.SOURCE, src)
    oracle.build(src, lib)
    first = os.stat(lib).st_mtime_ns
    assert oracle.ensure_built(src, lib) == lib
    assert os.stat(lib).st_mtime_ns == first          # same source: reused
    with open(src, "a") as fh:
        fh.write("\n/* edited */\n")
    oracle.ensure_built(src, lib)
    with open(lib + ".sha256") as fh:
        assert fh.read().strip() == oracle.source_digest(src)
    os.remove(lib + ".sha256")                        # no record: rebuilt
    oracle.ensure_built(src, lib)
    assert os.path.exists(lib + ".sha256")
