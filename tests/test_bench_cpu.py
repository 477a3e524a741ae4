"""Host-side logic of bench.py that needs no GPU."""
import hashlib
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _profile(tmp_path, sha, value=123456):
    files = "llama_decoder_only_amd/csrc/gemm.hip llama_decoder_only_amd/csrc/common.h"
    p = tmp_path / "traffic.md"
    p.write_text(f"text\n```\ndown-traffic-bytes-per-launch: {value}\nsource-sha256: {sha}\nsource-files: {files}\n```\n")
    return str(p)


def _sha(*rel):
    h = hashlib.sha256()
    for f in rel:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def test_traffic_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    b = _bench()
    good = _sha("llama_decoder_only_amd/csrc/gemm.hip", "llama_decoder_only_amd/csrc/common.h")
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", _profile(tmp_path, good))
    assert b.measured_traffic("down-traffic-bytes-per-launch") == 123456
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", _profile(tmp_path, "0" * 64))
    assert b.measured_traffic("down-traffic-bytes-per-launch") is None
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert b.measured_traffic("down-traffic-bytes-per-launch") is None


def test_committed_traffic_profile_is_well_formed():
    b = _bench()
    text = open(b.TRAFFIC_PROFILE).read()
    assert "down-traffic-bytes-per-launch: " in text and "source-sha256: " in text
    for f in text.split("source-files: ", 1)[1].split("\n", 1)[0].split():
        assert os.path.exists(os.path.join(ROOT, f)), f
