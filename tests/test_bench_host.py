"""Host logic of bench.py that needs no GPU: the source digest that keys the
committed HBM-traffic records to the kernel source they were taken on."""
import json
import os

import bench


def _tree(tmp_path, header_text):
    (tmp_path / "a.hip").write_text('#include "b.h"\n#include "c.h"\nint k;\n')
    (tmp_path / "b.h").write_text('#pragma once\n#include "c.h"\n' + header_text)
    (tmp_path / "c.h").write_text("#pragma once\nint c;\n")
    return str(tmp_path / "a.hip")


def test_digest_follows_included_headers(tmp_path):
    src = _tree(tmp_path, "int b;\n")
    d0 = bench.source_digest(src)
    assert len(d0) == 16 and int(d0, 16) >= 0
    assert bench.source_digest(src) == d0
    (tmp_path / "c.h").write_text("#pragma once\nint c2;\n")
    d1 = bench.source_digest(src)
    assert d1 != d0, "a change two includes deep must change the digest"
    (tmp_path / "b.h").write_text('#pragma once\n#include "c.h"\nint b2;\n')
    assert bench.source_digest(src) not in (d0, d1)


def test_digest_ignores_system_headers(tmp_path):
    (tmp_path / "a.hip").write_text("#include <hip/hip_runtime.h>\nint k;\n")
    d0 = bench.source_digest(str(tmp_path / "a.hip"))
    (tmp_path / "a.hip").write_text("#include <stdint.h>\nint k;\n")
    assert bench.source_digest(str(tmp_path / "a.hip")) != d0


def test_every_traffic_record_names_a_source_and_profile():
    recs = json.load(open(os.path.join(bench.ROOT, "profiles", "traffic.txt")))
    assert recs
    for key, rec in recs.items():
        assert os.path.isfile(os.path.join(bench.ROOT, rec["src"])), key
        assert os.path.isfile(os.path.join(bench.ROOT, rec["profile"])), key
        assert rec["read_bytes"] > 0 and rec["write_bytes"] > 0, key


def test_record_valid_only_for_the_current_source(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    src = _tree(csrc, "int b;\n")
    rel = os.path.relpath(src, tmp_path)
    (tmp_path / "profiles").mkdir()
    rec = {"src": rel, "read_bytes": 1000, "write_bytes": 24, "profile": "profiles/x.md"}
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles" / "traffic.txt").write_text(
        json.dumps({"k|w": dict(rec, sha256_16=bench.source_digest(rel))}))
    assert bench.measured_traffic("k|w", rel) == 1024
    assert bench.measured_traffic("k|other", rel) is None
    assert bench.measured_traffic("k|w", "csrc/other.hip") is None
    (csrc / "c.h").write_text("#pragma once\nint changed;\n")
    assert bench.measured_traffic("k|w", rel) is None, "a header change must void the record"
