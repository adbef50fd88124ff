"""The build's staleness check: ensure_built() rebuilds the library when the
sources it was built from have changed."""

import os
import shutil

import __graft_entry__ as ge


def test_built_library_matches_its_sources():
    ge.ensure_built()
    assert not ge.is_stale()


def test_digest_follows_every_source_byte_and_flag(tmp_path):
    src = tmp_path / "csrc"
    inc = tmp_path / "include"
    shutil.copytree(ge.CSRC, src, ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(ge.INCLUDE, inc)
    d0 = ge.source_digest((str(src), str(inc)))
    assert d0 == ge.source_digest((str(src), str(inc)))
    with open(src / "la_api.cpp", "ab") as f:
        f.write(b"\n")                     # one byte more in a source
    d1 = ge.source_digest((str(src), str(inc)))
    with open(inc / "la_vr.h", "ab") as f:
        f.write(b" ")                      # and in the header
    d2 = ge.source_digest((str(src), str(inc)))
    assert len({d0, d1, d2}) == 3
    assert ge.source_digest((str(src), str(inc)), flags=ge.FLAGS + ["-DX"]) != d2


def test_ensure_built_rebuilds_a_stale_library(tmp_path, monkeypatch):
    lib, stamp = tmp_path / "lib.so", tmp_path / "lib.so.stamp"
    lib.write_bytes(b"x")
    stamp.write_text("not the digest\n")
    assert ge.is_stale(str(lib), str(stamp), digest="abc")
    stamp.write_text("abc\n")
    assert not ge.is_stale(str(lib), str(stamp), digest="abc")
    os.remove(stamp)
    assert ge.is_stale(str(lib), str(stamp), digest="abc")
    calls = []
    monkeypatch.setattr(ge, "build", lambda: calls.append(1))
    monkeypatch.setattr(ge, "is_stale", lambda: True)
    ge.ensure_built()
    monkeypatch.setattr(ge, "is_stale", lambda: False)
    ge.ensure_built()
    assert calls == [1]
