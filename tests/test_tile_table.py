"""The compiled-in launch-shape table is what the sweep's measurements give:
regenerating the header from tune/sweep_gfx950.json reproduces the committed
csrc/pa_tile_table_gen.h byte for byte, and the choice rule behaves as its
docstring says on hand-made measurements (no GPU needed)."""
import json
import os

from paged_gqa_attention_pa_amd.tune import sweep


def test_header_regenerates_from_measurements(tmp_path):
    with open(sweep.DEFAULT_JSON) as f:
        results = json.load(f)
    out = tmp_path / "gen.h"
    sweep.emit_header(results, path=str(out))
    with open(sweep.GEN_HEADER) as f:
        committed = f.read()
    assert out.read_text() == committed


def test_every_decode_group_and_key_swept():
    with open(sweep.DEFAULT_JSON) as f:
        results = json.load(f)
    assert sorted(results["decode"]) == sorted(f"g{g}" for g in sweep.DECODE_GROUPS)
    for D, wide in sweep.SHORT_KEYS:
        for G, q in sweep.SHORT_SHAPES[wide][D]:
            assert f"d{D}_w{wide}_g{G}_q{q}" in results["short"]
    assert sorted(results["prefill"]) == sorted(f"d{d}" for d in sweep.PF_DIMS)


def test_choice_rule_ties_prefer_default_then_monotone():
    # ties within 2%: the default (4 waves, even grid) wins over a faster
    # 8-wave shape, and the split never drops below the previous bucket's
    # unless the measurements force it
    table = {
        "64x256": {"1,4,0": {"equal": 10.0, "varied": 10.0},
                   "2,4,6": {"equal": 9.0, "varied": 9.0}},
        "64x512": {"1,4,0": {"equal": 10.0, "varied": 10.0},
                   "2,4,6": {"equal": 10.1, "varied": 10.1},
                   "4,8,6": {"equal": 9.95, "varied": 9.95}},
        "64x1024": {"1,4,0": {"equal": 5.0, "varied": 5.0},
                    "4,4,6": {"equal": 9.0, "varied": 9.0}},
    }
    row = sweep.choose_decode_row(table, 64)
    assert row[256] == (2, 4, 6)
    assert row[512] == (2, 4, 6)       # tie: default shape, split kept at 2
    assert row[1024] == (1, 4, 0)      # a measured drop: the best, not monotone
