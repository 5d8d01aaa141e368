"""bench.py's host-side arithmetic, without a GPU: the tile-timeline summary on
synthetic records with known clocks, the step's FLOP accounting, and the
traffic entry's source-hash gate."""

import json
import os

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _records():
    """Two compute units, two 256x256 tiles each, four waves per tile.

    Per tile: 2 us of prologue, a 10-k-tile k-loop of 16 us that takes 25600
    shader cycles (1.6 GHz, 2560 cycles per k-tile against 2048 of MFMA
    work), a 5 us epilogue, and 1 us between a compute unit's tiles."""
    rows = []
    for tile_start in (1000, 3400):           # reference ticks (100 MHz)
        for cu in (0, 1):
            for _ in range(4):                # waves
                rt = [tile_start, tile_start + 200, tile_start + 1800, tile_start + 2300]
                ct = [50000, 50000 + 3200, 50000 + 3200 + 25600, 50000 + 3200 + 25600 + 8000]
                hw = cu << 8                  # HW_ID: compute unit in bits 11:8
                rows.append(rt + ct + [256, 10, hw, 3])
    return np.array(rows, dtype=np.int64)


def test_timeline_summary_known_clocks():
    s = bench.timeline_summary(_records())
    assert s["tiles"] == 4 and s["compute_units"] == 2 and s["k_tiles"] == 10
    assert s["prologue_us"] == pytest.approx(2.0)
    assert s["kloop_us"] == pytest.approx(16.0)
    assert s["epilogue_us"] == pytest.approx(5.0)
    assert s["gap_us"] == pytest.approx(1.0)
    assert s["cycles_per_ktile"] == pytest.approx(2560)
    assert s["sclk_ghz"] == pytest.approx(1.6)
    assert s["mfma_issue_in_kloop"] == pytest.approx(0.8)
    # span 1000 .. 5700 ticks = 47 us; four tiles of 23 us on two compute units
    assert s["span_us"] == pytest.approx(47.0)
    assert s["cu_busy"] == pytest.approx(4 * 23.0 / (2 * 47.0), abs=1e-3)
    assert s["kloop_us_first_round"] == pytest.approx(16.0)
    assert s["kloop_us_later_rounds"] == pytest.approx(16.0)


def test_timeline_summary_rounds():
    """The first round of tiles (one per compute unit) is reported apart from
    the later ones: here the later tiles' k-loops take 4 us longer."""
    r = _records()
    r[8:, 2] += 400                            # tiles 3 and 4 (records 8..15): k-loop end 4 us later
    r[8:, 3] += 400
    s = bench.timeline_summary(r)
    assert s["kloop_us_first_round"] == pytest.approx(16.0)
    assert s["kloop_us_later_rounds"] == pytest.approx(20.0)


def test_timeline_summary_half_tiles():
    r = _records()
    r[:, 8] = 128                              # 256 x 128 tiles: half the MFMA work per k-tile
    s = bench.timeline_summary(r)
    assert s["mfma_issue_in_kloop"] == pytest.approx(0.4)


def test_block_flops():
    M, d, F = bench.BLOCK_DIMS
    opf = bench.block_op_flops(M, d, F)
    assert set(opf) == set(bench.BLOCK_LAUNCHES) == set(bench.BLOCK_SHAPES)
    total = sum(opf[k] * bench.BLOCK_LAUNCHES[k] for k in opf)
    # per layer: gate/up 2*M*d*2F and down 2*M*F*d, forward, data and weight gradients (x3);
    # W0: 2*M*d*d forward, dgrad and wgrad (x3); two layers
    expect = 2 * 3 * (2 * M * d * 2 * F + 2 * M * F * d) + 3 * 2 * M * d * d
    assert total == expect
    assert round(total / 1e12, 2) == 18.14
    # each op's FLOPs match the M x N x K it reports
    for k, shape in bench.BLOCK_SHAPES.items():
        dims = [int(x) for x in shape.split()[0].split("x")]
        mult = 2 if "twice" in shape else 1
        assert opf[k] == mult * 2.0 * dims[0] * dims[1] * dims[2], k


def test_traffic_entry_needs_current_source(tmp_path, monkeypatch):
    h = bench.src_hash()
    assert len(h) == 16 and h == bench.src_hash()   # deterministic over csrc/
    prof = tmp_path / "profiles"
    prof.mkdir()
    ent = {"c5 swiglu": {"src_hash": h, "bytes_per_launch": 123}}
    (prof / "traffic.json").write_text(json.dumps(ent))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))   # profiles/ from tmp_path ...
    monkeypatch.setattr(bench, "src_hash", lambda: h)   # ... the kernels' hash as before
    assert bench.load_traffic("c5 swiglu") == 123
    ent["c5 swiglu"]["src_hash"] = "0" * 16
    (prof / "traffic.json").write_text(json.dumps(ent))
    assert bench.load_traffic("c5 swiglu") is None
    assert bench.load_traffic("missing") is None


def test_src_hash_ignores_comments():
    """The kernel-source hash changes with the code, not with its comments
    or layout (a measurement stays valid across a comment edit)."""
    a = {"k.hpp": 'int f(int x) { return x + 1; }  // add one\n/* note */ const char* s = "a//b";\n'}
    b = {"k.hpp": '/* other words */\nint f(int x) {\n  return x + 1;   // plus one\n}\nconst char* s = "a//b";\n'}
    c = {"k.hpp": 'int f(int x) { return x + 2; }\nconst char* s = "a//b";\n'}
    d = {"k.hpp": 'int f(int x) { return x + 1; }\nconst char* s = "a/ /b";\n'}
    assert bench.src_hash(a) == bench.src_hash(b)
    assert bench.src_hash(a) != bench.src_hash(c)
    assert bench.src_hash(a) != bench.src_hash(d)      # string literals are code
    assert bench.src_hash(a) != bench.src_hash({"j.hpp": a["k.hpp"]})


SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1393 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1769 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1717 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_parse_smi_metric():
    r = bench.parse_smi_metric(SMI_TEXT)
    assert r["socket_w"] == 1393.0
    assert r["gfx_mhz"] == [1769.0, 1717.0]          # graphics clocks only, not MIN/MAX or memory
    assert bench.parse_smi_metric("no GPU") == {"socket_w": None, "gfx_mhz": []}
