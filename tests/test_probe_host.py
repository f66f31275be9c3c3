"""Host-side checks of libzsprobe (the HBM stream probes bench.py --ceiling
times): it loads, exports what include/zsprobe.h declares, reports each
mix's read:write streams, and refuses bad arguments before any launch (no
GPU is touched here)."""

import ctypes as C
import os
import re

import pytest

from adam_zs_shard_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(_build.PROBE_PATH):
        pytest.fail(f"{_build.PROBE_PATH} is not built; run __graft_entry__.build()")
    L = C.CDLL(_build.PROBE_PATH)
    L.zsp_stream.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int32,
                             C.c_void_p, C.c_void_p]
    L.zsp_stream.restype = C.c_int32
    L.zsp_streams.argtypes = [C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
    L.zsp_streams.restype = C.c_int32
    return L


def test_exports_every_declared_function(probe):
    text = open(os.path.join(ROOT, "include", "zsprobe.h")).read()
    names = re.findall(r"^int32_t (\w+)\(", text, re.M)
    assert sorted(names) == ["zsp_step_reads", "zsp_step_reads_paced", "zsp_stream", "zsp_streams"]
    for n in names:
        assert hasattr(probe, n), n


def test_stream_counts_match_the_step_mixes(probe):
    # the read:write ratios of the step's bytes per element, 2P + 12 read and
    # 14 written: P = 64 -> 10:1, P = 16 -> 22:7, P = 8 -> 2:1
    for p, mix in ((64, 4), (16, 3), (8, 2)):
        nr, nw = C.c_int32(), C.c_int32()
        assert probe.zsp_streams(mix, C.byref(nr), C.byref(nw)) == 0
        assert nr.value * 14 == nw.value * (2 * p + 12)
        nr2, nw2 = C.c_int32(), C.c_int32()
        assert probe.zsp_streams(mix + 5, C.byref(nr2), C.byref(nw2)) == 0   # phased twin
        assert (nr2.value, nw2.value) == (nr.value, nw.value)
    expect = {0: (8, 0), 1: (1, 1), 10: (1, 0), 11: (2, 0), 12: (4, 0), 13: (8, 0), 14: (1, 0)}
    for mix, (r, w) in expect.items():
        nr, nw = C.c_int32(), C.c_int32()
        assert probe.zsp_streams(mix, C.byref(nr), C.byref(nw)) == 0
        assert (nr.value, nw.value) == (r, w)
    nr, nw = C.c_int32(), C.c_int32()
    assert probe.zsp_streams(15, C.byref(nr), C.byref(nw)) == 1
    assert probe.zsp_streams(-1, C.byref(nr), C.byref(nw)) == 1
    assert probe.zsp_streams(0, None, C.byref(nw)) == 1


def test_bad_arguments_launch_nothing(probe):
    fake = 1 << 40   # never dereferenced: every call below is refused first
    assert probe.zsp_stream(0, None, None, 1 << 20, 1024, 256, fake, None) == 1      # no src
    assert probe.zsp_stream(0, fake, None, 1 << 20, 1024, 256, None, None) == 1      # no sink
    assert probe.zsp_stream(0, fake, None, 1 << 20, 1024, 0, fake, None) == 1        # grid 0
    assert probe.zsp_stream(0, fake, None, 1 << 20, -1, 256, fake, None) == 1        # nvec < 0
    assert probe.zsp_stream(0, fake, None, 1000, 1024, 256, fake, None) == 1         # streams overlap
    assert probe.zsp_stream(1, fake, None, 1 << 20, 1024, 256, fake, None) == 1      # copy, no dst
    assert probe.zsp_stream(99, fake, fake, 1 << 20, 1024, 256, fake, None) == 1     # unknown mix
    probe.zsp_step_reads.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int32,
                                     C.c_void_p, C.c_void_p]
    probe.zsp_step_reads.restype = C.c_int32
    ranks = (C.c_void_p * 65)(*([fake] * 65))
    assert probe.zsp_step_reads(None, 8, 1 << 20, 256, fake, None) == 1             # no ranks
    assert probe.zsp_step_reads(ranks, 65, 1 << 20, 256, fake, None) == 1           # p > 64
    assert probe.zsp_step_reads(ranks, 0, 1 << 20, 256, fake, None) == 1            # p < 1
    assert probe.zsp_step_reads(ranks, 8, 1 << 20, 0, fake, None) == 1              # grid 0
    assert probe.zsp_step_reads(ranks, 8, -1, 256, fake, None) == 1                 # elems < 0
    assert probe.zsp_step_reads(ranks, 8, 1 << 20, 256, None, None) == 1            # no sink
    holes = (C.c_void_p * 8)(*([fake] * 7 + [None]))
    assert probe.zsp_step_reads(holes, 8, 1 << 20, 256, fake, None) == 1            # a null rank
    probe.zsp_step_reads_paced.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.c_int64,
                                           C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    probe.zsp_step_reads_paced.restype = C.c_int32
    assert probe.zsp_step_reads_paced(ranks, 8, 1 << 20, 256, 0, fake, None) == 1   # pace < 1
    assert probe.zsp_step_reads_paced(ranks, 65, 1 << 20, 256, 2, fake, None) == 1  # p > 64
    assert probe.zsp_step_reads_paced(holes, 8, 1 << 20, 256, 2, fake, None) == 1   # a null rank
