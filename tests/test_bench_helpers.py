"""Host-side helpers of bench.py on hand-built traces: the union of busy
intervals, the overlap figures E and hidden fraction, the per-step costs of
a trace spanning two forwards, the algorithmic work per launch, and the
lookup of counter-measured traffic (used only while the kernel source is the
one the counters were taken on)."""
import os

import pytest

import bench
import synth


def iv(kind, start, end, forward=0, block=0):
    return {"kind": kind, "start": float(start), "end": float(end), "forward": forward, "block": block}


def test_busy_is_the_union_of_intervals():
    assert bench.busy([]) == 0.0
    assert bench.busy([iv("h2d", 0, 2), iv("h2d", 1, 3), iv("h2d", 5, 6)]) == 4.0
    # nested and out of order
    assert bench.busy([iv("h2d", 4, 5), iv("h2d", 0, 10), iv("h2d", 2, 3)]) == 10.0


def test_overlap_figures():
    # copies 0-20 (two back to back), compute 5-15 and 20-30: forward 0-30
    rs = [iv("h2d", 0, 10), iv("h2d", 10, 20), iv("compute", 5, 15), iv("compute", 20, 30)]
    o = bench.overlap_of(rs)
    assert o["t_forward_ms"] == 30.0 and o["sum_h2d_ms"] == 20.0 and o["sum_compute_ms"] == 20.0
    assert o["E"] == pytest.approx(20.0 / 30.0)
    assert o["hidden_frac"] == pytest.approx((20 + 20 - 30) / 20.0)
    # fully serial: nothing hidden, E = max / sum
    rs = [iv("h2d", 0, 10), iv("compute", 10, 14)]
    o = bench.overlap_of(rs)
    assert o["hidden_frac"] == pytest.approx(0.0) and o["E"] == pytest.approx(10.0 / 14.0)
    assert o["hidden_side"] == "compute behind H2D"
    # compute-bound, copies entirely under compute
    rs = [iv("h2d", 1, 3), iv("compute", 0, 10)]
    o = bench.overlap_of(rs)
    assert o["hidden_frac"] == pytest.approx(1.0) and o["E"] == pytest.approx(1.0)
    assert o["hidden_side"] == "H2D behind compute"


def test_step_costs_across_a_forward_boundary():
    # two 2-block forwards; block 0 of forward 1 is reconstructed at 11, one
    # ms after the last block of forward 0 ended, and starts at 12
    tr = [iv("compute", 0, 5, 0, 0), iv("compute", 6, 10, 0, 1),
          iv("asm", 9, 11, 1, 0), iv("compute", 12, 15, 1, 0),
          iv("asm", 13, 14, 1, 1), iv("compute", 15, 20, 1, 1)]
    c = bench.step_costs(tr, 2, 1)
    assert c["step_ms"] == 10.0
    assert c["compute_idle_waiting_for_weights_ms"] == pytest.approx(1.0)
    assert c["stream_switch_ms"] == pytest.approx(1.0)
    assert c["step_boundary_gap_ms"] == pytest.approx(2.0)
    # block weights ready long before: no wait, only the switch
    tr[2] = iv("asm", 2, 3, 1, 0)
    c = bench.step_costs(tr, 2, 1)
    assert c["compute_idle_waiting_for_weights_ms"] == 0.0
    assert c["stream_switch_ms"] == pytest.approx(2.0)


def test_kernel_work_matches_the_per_block_closed_forms():
    for name in ("tiny", "image", "midvideo", "large"):
        shp = synth.workload(name).blocks[0]
        T, d, m = 1000, shp.d_model, shp.d_mlp
        w = bench.kernel_work(shp, T)
        gemm = sum(w[k][1] for k in ("k_qk", "k_v", "k_out", "k_fc1", "k_fc2"))
        # every projection is 2 flop per multiply-add: 2 T (3 d^2 + d^2 + 2 d m)
        assert gemm == 2.0 * T * (4 * d * d + 2 * d * m)
        if m == 4 * d:
            assert gemm == 24.0 * T * d * d
        assert w["k_attn"] == ("flop", 4.0 * T * T * d)
        assert all(w[k][0] == "byte" for k in ("k_adaln", "k_ln1", "k_ln2"))


def test_traffic_is_read_only_for_the_profiled_source(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic_demo_dit.txt").write_text(
        "k_fc2 aaaa000000000000 100 20\nk_ln bbbb000000000000 7 3\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda p: "bbbb000000000000" if p.endswith("norm.hip") else "aaaa000000000000")
    assert bench.traffic_from_profiles("k_fc2", "demo") == 120.0
    assert bench.traffic_from_profiles("k_ln2", "demo") == 10.0   # both LayerNorm launches share one kernel
    assert bench.traffic_from_profiles("k_qk", "demo") is None     # not profiled
    assert bench.traffic_from_profiles("k_fc2", "other") is None   # no file for this workload
    monkeypatch.setattr(bench, "source_hash", lambda p: "cccc000000000000")
    assert bench.traffic_from_profiles("k_fc2", "demo") is None    # the kernel changed since
