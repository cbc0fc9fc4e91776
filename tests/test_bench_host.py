"""bench.py's host logic: the hash of the kernel sources that ties a committed HBM traffic
summary to the code it was measured on, and the lookup that reports that traffic only
while the hash still matches."""
from __future__ import annotations

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "CSRC", str(tmp_path))
    k = tmp_path / "k.h"
    k.write_text("int f(int a) {\n  return a + 1;  // one\n}\n")
    h0 = b.kernel_sources_sha(["k.h"])
    k.write_text("/* a header\n   comment */\nint f(int a) {   return a + 1; // two\n\n}\n")
    assert b.kernel_sources_sha(["k.h"]) == h0
    k.write_text("int f(int a) {\n  return a + 2;\n}\n")
    assert b.kernel_sources_sha(["k.h"]) != h0


def test_traffic_reported_only_while_sources_match(tmp_path, monkeypatch):
    b = _bench()
    src, prof = tmp_path / "src", tmp_path / "prof"
    src.mkdir()
    prof.mkdir()
    monkeypatch.setattr(b, "CSRC", str(src))
    monkeypatch.setattr(b, "PROFILES", str(prof))
    monkeypatch.setitem(b.KERNEL_FILES, "decode", ("k.h",))
    (src / "k.h").write_text("int f() { return 1; }\n")
    sha = b.kernel_sources_sha(["k.h"])
    (prof / "traffic_fc1_decode_w.txt").write_text(
        f"kernel: k\ntraffic_bytes_per_launch: 1234\nkernel_sources_sha256: {sha}\n")
    assert b.committed_traffic("decode", "w") == 1234
    assert b.committed_traffic("decode", "other") is None
    (src / "k.h").write_text("int f() { return 2; }\n")
    assert b.committed_traffic("decode", "w") is None


def test_committed_traffic_summaries_parse():
    # each committed summary names a kernel kind bench.py hashes, a positive byte count and
    # the hash of the sources it was taken on
    b = _bench()
    names = [n for n in os.listdir(b.PROFILES) if n.startswith("traffic_fc1_")]
    assert names
    for name in names:
        kind = name[len("traffic_fc1_"):].split("_", 1)[0]
        assert kind in b.KERNEL_FILES, name
        vals = {}
        with open(os.path.join(b.PROFILES, name)) as fh:
            for line in fh:
                if ":" in line and not line.startswith(" "):
                    key, v = line.split(":", 1)
                    vals[key.strip()] = v.strip()
        assert int(vals["traffic_bytes_per_launch"]) > 0, name
        assert len(vals["kernel_sources_sha256"]) == 16, name
