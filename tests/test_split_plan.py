"""The grid-tail split plan of the bf16 attention launch (dit_amd/csrc/split_plan.h), built with
the host compiler: its structural guarantees on a sweep of shapes, and the plans of the
benchmark workloads that the measurements quote."""
import ctypes
import math
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dit_amd", "csrc")


@pytest.fixture(scope="module")
def plan(tmp_path_factory):
    out = tmp_path_factory.mktemp("split") / "libsplit.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC,
                    os.path.join(ROOT, "tests", "split_plan_host.cpp"), "-o", str(out)], check=True)
    lib = ctypes.CDLL(str(out))
    lib.split_plan_host.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]

    def f(tiles, cus, key_tiles):
        nw, p = ctypes.c_int32(), ctypes.c_int32()
        lib.split_plan_host(tiles, cus, key_tiles, ctypes.byref(nw), ctypes.byref(p))
        return nw.value, p.value

    f.max_parts = lib.split_plan_max_parts()
    f.max_tail = lib.split_plan_max_tail()
    return f


def test_plan_structure(plan):
    """Every plan: 1..kMaxParts parts; no split when the tiles fill whole rounds, when the tail
    exceeds the split limit or without a CU count; a split keeps every tile of the whole rounds
    whole (n_whole = tiles - tail), and the extra part slots fit the workspace's
    (kMaxParts - 1) x min(tiles, kMaxSplitTail)."""
    for cus in (0, 1, 8, 80, 256, 304):
        for tiles in list(range(1, 700, 7)) + [2960, 5000, 65536]:
            for key_tiles in (1, 3, 32, 128, 591, 2363, 40000):
                nw, p = plan(tiles, cus, key_tiles)
                assert 1 <= p <= plan.max_parts
                tail = tiles % cus if cus > 0 else 0
                if cus <= 0 or tail == 0 or tail > plan.max_tail:
                    assert (nw, p) == (tiles, 1)
                elif p > 1:
                    assert nw == tiles - tail
                    assert tail * (p - 1) <= (plan.max_parts - 1) * min(tiles, plan.max_tail)
                else:
                    assert nw == tiles


def test_plan_of_the_benchmark_workloads(plan):
    """On 256 compute units: the Wan 720p rank share (2,960 query tiles, 2,363 key tiles) in 7
    parts; the Wan block (640, 128) and the ragged 37,800-key workload (640, 1,182) in 2; 37 heads
    x 8 query tiles over 65 key tiles (the split-tail GPU tests) in 6."""
    assert plan(2960, 256, 2363) == (2816, 7)
    assert plan(640, 256, 128) == (512, 2)
    assert plan(640, 256, 1182) == (512, 2)
    assert plan(296, 256, 65) == (256, 6)


def test_short_items_split_less(plan):
    """The fixed cost of a work item weighs more when its key range is short: for the same grid
    the plan never takes more parts for fewer key tiles."""
    for tiles in (300, 640, 1000, 2960):
        parts = [plan(tiles, 256, kt)[1] for kt in (8, 32, 128, 512, 2048, 8192)]
        assert parts == sorted(parts), (tiles, parts)
