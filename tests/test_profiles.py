"""The committed rocprofv3 summaries are well formed (CPU only): every summary names the command
it comes from, and every `traffic-record:` / `counter-record:` line that bench.py reads parses,
names a kernel source that exists, and is unique for its (key, source)."""

import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
CSRC = os.path.join(ROOT, "io_aware_tiled_amd", "csrc")


def _records(kind):
    out = []
    for path in PROFILES:
        with open(path) as f:
            for line in f:
                if line.startswith(kind + ":"):
                    out.append((os.path.basename(path), json.loads(line.split(":", 1)[1])))
    return out


def test_there_are_summaries():
    assert PROFILES


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_summary_names_its_command(path):
    with open(path) as f:
        text = f.read()
    assert "rocprofv3" in text and "bench.py" in text
    # only text summaries: no raw trace output
    assert len(text) < 64 * 1024


@pytest.mark.parametrize("kind", ["traffic-record", "counter-record"])
def test_records_parse_and_are_unique(kind):
    recs = _records(kind)
    assert recs
    seen = set()
    for name, rec in recs:
        for field in ("key", "source", "source_sha256_16", "hbm_bytes_per_launch"):
            assert field in rec, (name, field)
        assert os.path.exists(os.path.join(CSRC, rec["source"])), (name, rec["source"])
        assert len(rec["source_sha256_16"]) == 16
        assert rec["hbm_bytes_per_launch"] > 0
        ident = (rec["key"], rec["source"])
        assert ident not in seen, (name, ident)
        seen.add(ident)


def test_counter_records_carry_utilisation():
    for name, rec in _records("counter-record"):
        per_kernel = rec.get("kernels", {"": rec})
        for k, u in per_kernel.items():
            assert 0.0 < u["mfma_busy"] <= 1.0, (name, k)
            assert u["lds_bank_conflict_per_lds_cycle"] >= 0.0, (name, k)


def test_headline_records_exist():
    keys = {rec["key"] for _, rec in _records("traffic-record")}
    assert {"prefill", "decode", "backward"} <= keys
    keys = {rec["key"] for _, rec in _records("counter-record")}
    assert {"prefill", "decode", "backward"} <= keys
