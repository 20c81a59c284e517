"""The launch table (csrc/tune_table.h) against the sweep record it is generated from (CPU only).

The table is a performance choice with no numerical effect; what these checks pin is that it is
reproducible: regenerating it from the committed sweep record gives the committed file byte for
byte, and the host planner then picks, for every swept shape, the configuration the record
measured fastest.
"""

import json

import pytest

import io_aware_tiled_amd as fa
from io_aware_tiled_amd import tune


@pytest.fixture(scope="module")
def record():
    with open(tune.SWEEP_PATH) as f:
        return json.load(f)


def test_header_is_the_one_the_record_generates(record):
    with open(tune.HEADER_PATH) as f:
        assert f.read() == tune.render(record, "tune_sweep.json")


def test_planner_picks_each_swept_shapes_fastest_configuration(record):
    by_shape = {}
    for r in record["records"]:
        if r["kind"] == "prefill":
            by_shape.setdefault(tuple(r["shape"]), []).append(r)
    assert set(by_shape) == {tuple(int(x) for x in s) for s in tune.PREFILL_SHAPES}
    for (B, Hq, Hkv, T, d, causal), recs in by_shape.items():
        best = tune._fastest(recs)
        p = fa.attn_fwd_plan(B, Hq, Hkv, T, T, d, bool(causal), fa.FATTN_BF16)
        assert [p["block_kv"], p["waves"], p["schedule"]] == best["cfg"], (B, Hq, Hkv, T, d)


def test_decode_split_count_is_the_sweeps_fastest(record):
    for shape in tune.DECODE_SHAPES:
        recs = [r for r in record["records"] if r["kind"] == "decode" and tuple(r["shape"]) == shape]
        assert {r["splits"] for r in recs} == set(tune.DECODE_SPLITS)
        B, Hq, Hkv, Tk, d = shape
        p = fa.attn_fwd_plan(B, Hq, Hkv, 1, Tk, d, False, fa.FATTN_BF16)
        assert p["splits"] == min(recs, key=lambda r: r["ms"])["splits"], shape


def test_every_configuration_was_timed(record):
    for shape in tune.PREFILL_SHAPES:
        cfgs = {tuple(r["cfg"]) for r in record["records"]
                if r["kind"] == "prefill" and tuple(r["shape"]) == tuple(int(x) for x in shape)}
        assert cfgs == set(tune.PREFILL_CFGS), shape
