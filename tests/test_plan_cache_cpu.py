"""The per-shape plan cache (trimul_tune's on-disk store), host side only:
entries round-trip through the file, a later entry for the same key replaces
the earlier one, other keys and devices are kept apart, malformed lines and
unknown plans are ignored, and the path follows TRIMUL_PLAN_CACHE."""
import os
import subprocess
import sys

import pytest

from triangle_multiplication_amd import binding as tb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_candidates_include_the_default_first():
    c = tb.plan_candidates()
    assert c[0] == (0, 1, 8, 256)
    assert len(c) == len(set(c)) >= 2
    assert {p[1] for p in c} == {0, 1} and {p[2] for p in c} == {4, 8, 16} and {p[3] for p in c} == {256, 128}


def test_round_trip_and_replace(tmp_path):
    path = str(tmp_path / "sub" / "plans.txt")   # directory created on first store
    dev = "gfx950-256cu"
    assert tb.cache_lookup(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False) is None
    tb.cache_store(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False, (0, 1, 16, 256), 24.5)
    tb.cache_store(path, dev, 256, 256, "bf16", 1, 4096, "incoming", False, (0, 0, 4, 128), 25.0)
    tb.cache_store(path, dev, 128, 128, "bf16", 1, 8192, "incoming", True, (0, 1, 8, 256), 90.0)
    assert tb.cache_lookup(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False) == (0, 1, 16, 256)
    assert tb.cache_lookup(path, dev, 256, 256, "bf16", 1, 4096, "incoming", False) == (0, 0, 4, 128)
    assert tb.cache_lookup(path, dev, 128, 128, "bf16", 1, 8192, "incoming", True) == (0, 1, 8, 256)
    # a different key of any field is a miss
    assert tb.cache_lookup(path, dev, 128, 128, "bf16", 1, 8192, "incoming", False) is None
    assert tb.cache_lookup(path, dev, 256, 256, "fp32", 1, 4096, "outgoing", False) is None
    assert tb.cache_lookup(path, "gfx950-32cu", 256, 256, "bf16", 1, 4096, "outgoing", False) is None
    assert tb.cache_lookup(path, dev, 256, 256, "bf16", 2, 4096, "outgoing", False) is None
    # replacing keeps one line per key
    tb.cache_store(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False, (0, 0, 8, 256), 23.0)
    assert tb.cache_lookup(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False) == (0, 0, 8, 256)
    lines = [l for l in open(path).read().splitlines() if l.strip()]
    assert len(lines) == 3
    assert not [f for f in os.listdir(os.path.dirname(path)) if ".tmp" in f]


def test_malformed_and_unknown_lines_are_ignored(tmp_path):
    path = str(tmp_path / "plans.txt")
    dev = "gfx950-256cu"
    with open(path, "w") as f:
        f.write("# comment\n")
        f.write("garbage line\n")
        f.write("trimul-plan v3 %s 256 256 0 1 4096 0 0 0 7 99 256 1.0\n" % dev)   # no such plan
        f.write("trimul-plan v3 %s 256 256 0 1 4096 0 0 0 0 8 64 1.0\n" % dev)     # no such tile
        f.write("trimul-plan v2 %s 256 256 0 1 4096 0 0 0 1 8 1.0\n" % dev)        # older version
        f.write("trimul-plan v3 %s 256 256 0 1 4096 0\n" % dev)                    # truncated
    assert tb.cache_lookup(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False) is None
    tb.cache_store(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False, (0, 1, 4, 128), 2.0)
    assert tb.cache_lookup(path, dev, 256, 256, "bf16", 1, 4096, "outgoing", False) == (0, 1, 4, 128)
    text = open(path).read()
    assert "# comment" in text and "garbage line" in text   # other lines survive a store


def test_store_rejects_unknown_plan(tmp_path):
    with pytest.raises(tb.TriMulError):
        tb.cache_store(str(tmp_path / "p.txt"), "d", 32, 32, "bf16", 1, 64, "outgoing", False, (0, 5, 8, 256), 1.0)
    with pytest.raises(tb.TriMulError):
        tb.cache_store(str(tmp_path / "p.txt"), "d", 32, 32, "bf16", 1, 64, "outgoing", False, (7, 0, 8, 256), 1.0)
    with pytest.raises(tb.TriMulError):
        tb.cache_store(str(tmp_path / "p.txt"), "d", 32, 32, "bf16", 1, 64, "outgoing", False, (0, 0, 8, 64), 1.0)


def test_unwritable_location_is_an_error_of_the_store_only(tmp_path):
    blocker = tmp_path / "file"
    blocker.write_text("x")
    with pytest.raises(tb.TriMulError):
        tb.cache_store(str(blocker / "plans.txt"), "d", 32, 32, "bf16", 1, 64, "outgoing", False, (0, 0, 8, 256), 1.0)


def _path_with_env(env):
    code = "from triangle_multiplication_amd import binding as tb; print(tb.cache_path())"
    e = {k: v for k, v in os.environ.items() if k not in ("TRIMUL_PLAN_CACHE", "XDG_CACHE_HOME", "HOME")}
    e.update(env)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=e, capture_output=True, text=True, check=True)
    return r.stdout.strip()


def test_cache_path_follows_environment():
    assert _path_with_env({"TRIMUL_PLAN_CACHE": "/x/y.txt", "HOME": "/h"}) == "/x/y.txt"
    assert _path_with_env({"TRIMUL_PLAN_CACHE": "0", "HOME": "/h"}) == ""
    assert _path_with_env({"XDG_CACHE_HOME": "/c", "HOME": "/h"}) == "/c/libtrimul/plans.txt"
    assert _path_with_env({"HOME": "/h"}) == "/h/.cache/libtrimul/plans.txt"
