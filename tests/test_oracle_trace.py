"""Pins for oracle.trace: a simulated two-slot schedule passes; each planted
scheduling mistake is caught by the property it violates."""
import copy

import pytest

from oracle import trace as T


def _simulate(n_blocks=6, chunks=3, h2d=1.0, asm=0.2, comp=2.5, serialize=False, first_slot=0):
    """Event-driven model of the pipeline: one copy engine, one gather
    stream, one compute stream, two slots, two landing buffers."""
    tr = []
    copy_free = gather_free = comp_free = 0.0
    land_free = [0.0, 0.0]
    comp_end = {}
    j_global = 0
    for b in range(n_blocks):
        slot = (b + first_slot) % 2
        slot_ready = comp_end.get(b - 2, 0.0)
        if serialize:
            slot_ready = max(slot_ready, comp_end.get(b - 1, 0.0))
        asm_ends = []
        for j in range(chunks):
            lb = j_global % 2
            j_global += 1
            s = max(copy_free, land_free[lb], slot_ready if serialize else 0.0)
            e = s + h2d
            copy_free = e
            tr.append(dict(kind="h2d", block=b, chunk=j, slot=-1, landing=lb, start=s, end=e))
            s2 = max(gather_free, e, slot_ready)
            e2 = s2 + asm
            gather_free = e2
            land_free[lb] = e2
            asm_ends.append(e2)
            tr.append(dict(kind="asm", block=b, chunk=j, slot=slot, landing=lb, start=s2, end=e2))
        s3 = max(comp_free, max(asm_ends))
        e3 = s3 + comp
        comp_free = e3
        comp_end[b] = e3
        tr.append(dict(kind="compute", block=b, chunk=-1, slot=slot, landing=-1, start=s3, end=e3))
    return tr


NUMELS = [1000, 1003, 999, 1000, 1003, 999]


@pytest.mark.parametrize("serialize", [False, True])
@pytest.mark.parametrize("ratio", [0.2, 1.0, 5.0])
def test_valid_schedules_pass(serialize, ratio):
    tr = _simulate(comp=ratio * 3.2, serialize=serialize)
    assert T.check_trace(tr, 6, slot_capacity=4 * 251, numels=NUMELS, dp=4) == []
    assert T.residency_high_water(tr, 6) <= 2


def _find(tr, kind, block, chunk=None):
    for r in tr:
        if r["kind"] == kind and r["block"] == block and (chunk is None or r["chunk"] == chunk):
            return r
    raise KeyError


def test_wrong_slot_caught():
    tr = _simulate()
    _find(tr, "compute", 3)["slot"] = 1 - 3 % 2
    assert any(e.startswith("(i)") for e in T.check_trace(tr, 6))


def test_compute_before_reconstruction_caught():
    tr = _simulate()
    r = _find(tr, "compute", 2)
    last = max(x["end"] for x in tr if x["kind"] == "asm" and x["block"] == 2)
    r["start"] = last - 0.05
    assert any(e.startswith("(ii)") for e in T.check_trace(tr, 6))


def test_reconstruction_before_h2d_caught():
    tr = _simulate()
    a = _find(tr, "asm", 4, 1)
    a["start"] = _find(tr, "h2d", 4, 1)["end"] - 0.01
    assert any(e.startswith("(ii)") for e in T.check_trace(tr, 6))


def test_slot_reuse_too_early_caught():
    # Prefetch two blocks ahead: block b writes slot b%2 while b-2 still computes.
    tr = _simulate(comp=5.0)
    for r in tr:
        if r["kind"] == "asm" and r["block"] == 3:
            shift = _find(tr, "compute", 1)["end"] - 1.0 - min(
                x["start"] for x in tr if x["kind"] == "asm" and x["block"] == 3)
            r["start"] += shift
            r["end"] += shift
    errs = T.check_trace(tr, 6)
    assert any(e.startswith("(iii)") for e in errs)
    assert any(e.startswith("(iv)") and "resident" in e for e in errs)


def test_landing_double_occupancy_caught():
    tr = _simulate()
    h = _find(tr, "h2d", 1, 2)
    prev = _find(tr, "asm", 1, 0)  # same landing buffer, two chunks earlier
    assert h["landing"] == prev["landing"]
    h["start"] = prev["end"] - 0.1
    assert any("landing" in e for e in T.check_trace(tr, 6))


def test_missing_intervals_caught():
    tr = [r for r in _simulate() if not (r["kind"] == "compute" and r["block"] == 5)]
    assert T.check_trace(tr, 6)


def test_capacity_checked():
    tr = _simulate()
    assert T.slot_capacity_elems(NUMELS, 4) == 4 * 251
    assert any(e.startswith("(v)") for e in T.check_trace(tr, 6, slot_capacity=1003, numels=NUMELS, dp=4))


def test_forward_may_start_in_slot_one():
    # a forward that follows one with an odd block count starts in slot 1
    tr = _simulate(first_slot=1)
    assert T.check_trace(tr, 6, slot_capacity=4 * 251, numels=NUMELS, dp=4) == []


def test_broken_alternation_caught_from_either_start():
    for first in (0, 1):
        tr = _simulate(first_slot=first)
        _find(tr, "asm", 2)["slot"] = (2 + first + 1) % 2
        errs = T.check_trace(tr, 6)
        assert any(e.startswith("(i)") for e in errs), errs
