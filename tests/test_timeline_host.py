"""Host-side checks of the phase-stamp measurement build (no GPU needed).

libdsa.so must not carry the stamp entry points of include/dsa_timeline.h; the measurement build
libdsa_timeline.so (built on demand) must export them and validate their arguments without
touching the device.  The summary that profile_counters.py prints from a recorded file is checked
on a small hand-made record whose phase ends are known."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_timeline.h")
PKG = os.path.join(ROOT, "sparse_indexed_attention_amd")


def declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_plain_library_has_no_stamps():
    import sparse_indexed_attention_amd as m
    if not os.path.exists(m.LIB_PATH):
        from sparse_indexed_attention_amd.build import build
        build()
    lib = ctypes.CDLL(m.LIB_PATH)
    names = declared()
    assert names == ["dsa_timeline_bytes", "dsa_timeline_register"]
    for n in names:
        assert not hasattr(lib, n), n


@pytest.fixture(scope="module")
def tl_lib():
    path = os.path.join(PKG, "libdsa_timeline.so")
    if not os.path.exists(path):
        pytest.skip("libdsa_timeline.so not built (python -m sparse_indexed_attention_amd.build --timeline)")
    lib = ctypes.CDLL(path)
    lib.dsa_timeline_bytes.restype = ctypes.c_size_t
    lib.dsa_timeline_register.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.dsa_timeline_register.restype = ctypes.c_int32
    return lib


def test_timeline_build_exports_and_validates(tl_lib):
    nbytes = tl_lib.dsa_timeline_bytes()
    assert nbytes == 3 * 4096 * 32 * 8
    # the pointer is only recorded, never dereferenced on the host
    assert tl_lib.dsa_timeline_register(0x1000, nbytes - 8) == 5      # DSA_ERR_WORKSPACE
    assert tl_lib.dsa_timeline_register(0x1008, nbytes) == 6          # DSA_ERR_ALIGN
    assert tl_lib.dsa_timeline_register(0x1000, nbytes) == 0
    assert tl_lib.dsa_timeline_register(None, 0) == 0                 # stop recording


def test_summary_of_a_known_record(capsys):
    import profile_counters as pc
    # two indexer workgroups of one query (the second merges), one attention and one combine
    # workgroup; slots 8-12 (and 19) are cycle counts and clock readings, 13 the scoring loop's start
    def idx(scored, merged, last):
        v = [0.0, scored, scored + 1, scored + 2] + ([scored + 3, scored + 4, scored + 5, scored + 6]
                                                     if merged else [None] * 4)
        v += [100, 400, 5, 0, int(2000 * scored), 1.0, 0, 1 if last else 0]
        return v
    att = [30.0, 31.0, 35.0, 35.5, 39.0, 40.0, None, None, 50, 950, 2, 60000, 60000 + 2000 * 9, None, 0, 0,
           None, None, None, 300]
    comb = [42.0, None, None, None, None, 47.0] + [None] * 2 + [0, 0, 0, 0, 0, None, 0, 0]
    rec = {"indexer": {"0": idx(10.0, False, False), "1": idx(12.0, True, True)},
           "attention": {"0": att}, "combine": {"0": comb}}
    pc.timeline_summary({"workload": "toy", "queries": 1, "visible": [1], "clock": "", "steps": [rec, rec]})
    out = capsys.readouterr().out
    assert "| indexer | split scored | 2 | 11.00 |" in out
    assert "| indexer | merge: output written | 1 | 18.00 | 18.00 | 18.00 |" in out
    assert "| whole merge | 4.00 | 4.00 |" in out
    assert "| combine | written | 1 | 47.00 |" in out
    assert "| indexer | key groups (scoring) | 5 | 20 | 80 | - | 0.20 |" in out
    # attention: 25 cycles waiting, 475 computing and 150 issuing per step (slot 19)
    assert "| attention | tile pairs (64-head decode kernel) or tiles | 2 | 25 | 475 | 150 | 0.04 |" in out
    assert "attention: shader clock 2000 MHz" in out
