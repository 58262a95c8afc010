"""Pins for oracle.trace: a simulated two-slot schedule passes; each planted
scheduling mistake is caught by the property it violates."""
import copy

import pytest

from oracle import trace as T


def _simulate(n_blocks=6, chunks=3, h2d=1.0, asm=0.2, comp=2.5, serialize=False, first_slot=0,
              forwards=1, early_copy=False, chunk_bytes=100):
    """Event-driven model of the pipeline: one host link, one gather stream,
    one compute stream, two slots, two landing buffers.  The first copy of
    block instance g waits for compute(g-2), so no third block reaches the
    device; early_copy=True drops that wait (a copy then starts as soon as a
    landing buffer is free, and a third block's chunks can land while two
    blocks sit in the slots).  forwards > 1 continues the alternation across
    forwards, as back-to-back calls do."""
    tr = []
    copy_free = gather_free = comp_free = 0.0
    land_free = [0.0, 0.0]
    comp_end = {}
    j_global = 0
    for g in range(forwards * n_blocks):
        f, b = divmod(g, n_blocks)
        slot = (g + first_slot) % 2
        slot_ready = comp_end.get(g - 2, 0.0)
        copy_ready = 0.0 if early_copy else comp_end.get(g - 2, 0.0)
        if serialize:
            slot_ready = max(slot_ready, comp_end.get(g - 1, 0.0))
            copy_ready = max(copy_ready, comp_end.get(g - 1, 0.0))
        asm_ends = []
        for j in range(chunks):
            lb = j_global % 2
            j_global += 1
            s = max(copy_free, land_free[lb], copy_ready)
            e = s + h2d
            copy_free = e
            tr.append(dict(kind="h2d", block=b, forward=f, chunk=j, slot=-1, landing=lb, bytes=chunk_bytes,
                           start=s, end=e))
            s2 = max(gather_free, e, slot_ready)
            e2 = s2 + asm
            gather_free = e2
            land_free[lb] = e2
            asm_ends.append(e2)
            tr.append(dict(kind="asm", block=b, forward=f, chunk=j, slot=slot, landing=lb, bytes=chunk_bytes,
                           start=s2, end=e2))
        s3 = max(comp_free, max(asm_ends))
        e3 = s3 + comp
        comp_free = e3
        comp_end[g] = e3
        tr.append(dict(kind="compute", block=b, forward=f, chunk=-1, slot=slot, landing=-1, bytes=0,
                       start=s3, end=e3))
    return tr


NUMELS = [1000, 1003, 999, 1000, 1003, 999]


@pytest.mark.parametrize("forwards", [1, 3])
@pytest.mark.parametrize("serialize", [False, True])
@pytest.mark.parametrize("ratio", [0.2, 1.0, 5.0])
def test_valid_schedules_pass(serialize, ratio, forwards):
    tr = _simulate(comp=ratio * 3.2, serialize=serialize, forwards=forwards)
    assert T.check_trace(tr, 6, slot_capacity=4 * 251, numels=NUMELS, dp=4) == []
    assert T.residency_high_water(tr, 6) <= 2
    assert T.device_high_water(tr, 6) <= 2


# Exact residency values.  The page's TL;DR: exactly two layers' weights per
# device at any time.  Slot occupancy runs from a block's first
# reconstruction to its compute end; device occupancy from its first H2D.

def test_residency_compute_bound_is_two():
    # compute (5.0) outlasts the next block's staging (3 x 1.0 + 0.2): while
    # block g computes, block g+1 is already reconstructed into the other slot
    tr = _simulate(comp=5.0)
    assert T.residency_high_water(tr, 6) == 2
    assert T.device_high_water(tr, 6) == 2


def test_residency_link_bound():
    # compute (0.5) ends long before the next block's last chunk lands: the
    # next block enters its slot only after this one computed (slots: 1), but
    # its first chunks are already in a landing buffer (device: 2)
    tr = _simulate(comp=0.5)
    assert T.residency_high_water(tr, 6) == 1
    assert T.device_high_water(tr, 6) == 2


def test_residency_serialized_is_one():
    tr = _simulate(comp=2.0, serialize=True)
    assert T.residency_high_water(tr, 6) == 1
    assert T.device_high_water(tr, 6) == 1


def test_residency_early_copy_counts_three_on_device():
    # copies that start as soon as a landing buffer is free put block g+2's
    # first chunks on the device while g computes and g+1 waits in its slot
    tr = _simulate(comp=5.0, early_copy=True)
    assert T.residency_high_water(tr, 6) == 2
    assert T.device_high_water(tr, 6) == 3
    errs = T.check_trace(tr, 6)
    assert any(e.startswith("(iv)") and "on the device" in e for e in errs), errs


def test_residency_single_block_forwards():
    # one block per forward, three forwards: the instances still alternate
    # slots and overlap across forward boundaries exactly as within one
    tr = _simulate(n_blocks=1, comp=5.0, forwards=3)
    assert T.check_trace(tr, 1) == []
    assert T.residency_high_water(tr, 1) == 2


def test_weight_bytes_peak_hand_trace():
    # two blocks of 1000 padded bytes, two 500-byte chunks each
    iv = [
        dict(kind="h2d", block=0, chunk=0, slot=-1, landing=0, bytes=500, start=0.0, end=1.0),
        dict(kind="asm", block=0, chunk=0, slot=0, landing=0, bytes=500, start=1.0, end=2.0),
        dict(kind="h2d", block=0, chunk=1, slot=-1, landing=1, bytes=500, start=1.0, end=2.0),
        dict(kind="asm", block=0, chunk=1, slot=0, landing=1, bytes=500, start=2.0, end=3.0),
        dict(kind="compute", block=0, chunk=-1, slot=0, landing=-1, bytes=0, start=3.0, end=5.0),
        dict(kind="h2d", block=1, chunk=0, slot=-1, landing=0, bytes=500, start=2.0, end=4.0),
        dict(kind="asm", block=1, chunk=0, slot=1, landing=0, bytes=500, start=4.0, end=4.5),
        dict(kind="h2d", block=1, chunk=1, slot=-1, landing=1, bytes=500, start=4.0, end=5.0),
        dict(kind="asm", block=1, chunk=1, slot=1, landing=1, bytes=500, start=5.0, end=5.5),
        dict(kind="compute", block=1, chunk=-1, slot=1, landing=-1, bytes=0, start=5.5, end=6.0),
    ]
    # at t in [4, 4.5): block 0 (1000) and block 1 (1000) in slots, chunk
    # (1, 0) not yet reconstructed (500), chunk (1, 1) landing (500)
    assert T.weight_bytes_peak(iv, 2, [1000, 1000]) == 3000
    assert T.check_trace(iv, 2) == []
    assert T.residency_high_water(iv, 2) == 2
    assert T.device_high_water(iv, 2) == 2


def _bytes_by_sampling(tr, L, block_bytes):
    """Brute force: weight bytes in use at every interval endpoint and
    midpoint, summed directly from the definition."""
    pts = sorted({r[k] for r in tr for k in ("start", "end")})
    probes = pts + [(a + b) / 2 for a, b in zip(pts, pts[1:])]
    best = 0
    for t in probes:
        tot = 0
        for g in {(r.get("forward", 0), r["block"]) for r in tr}:
            a0 = min(r["start"] for r in tr if r["kind"] == "asm" and (r.get("forward", 0), r["block"]) == g)
            c1 = max(r["end"] for r in tr if r["kind"] == "compute" and (r.get("forward", 0), r["block"]) == g)
            if a0 <= t < c1:
                tot += block_bytes[g[1]]
        for r in tr:
            if r["kind"] != "h2d":
                continue
            a = [x for x in tr if x["kind"] == "asm" and x["block"] == r["block"]
                 and x.get("forward", 0) == r.get("forward", 0) and x["chunk"] == r["chunk"]][0]
            if r["start"] <= t < a["end"]:
                tot += r["bytes"]
        best = max(best, tot)
    return best


@pytest.mark.parametrize("comp,early,fw", [(0.5, False, 1), (5.0, False, 2), (2.0, True, 1), (3.3, False, 2)])
def test_weight_bytes_peak_matches_brute_force(comp, early, fw):
    tr = _simulate(n_blocks=4, chunks=3, comp=comp, early_copy=early, forwards=fw, chunk_bytes=70)
    bb = [210, 210, 210, 210]
    assert T.weight_bytes_peak(tr, 4, bb) == _bytes_by_sampling(tr, 4, bb)


def test_cross_forward_slot_reuse_caught():
    # block 1 of forward 1 reconstructs into its slot before block 5 of
    # forward 0 (two instances earlier, same slot) finished computing
    tr = _simulate(comp=5.0, forwards=2)
    last = _find(tr, "compute", 5, forward=0)
    for r in tr:
        if r["kind"] == "asm" and r["block"] == 1 and r["forward"] == 1:
            r["start"], r["end"] = last["end"] - 1.0, last["end"] - 0.8
    errs = T.check_trace(tr, 6)
    assert any(e.startswith("(iii)") and "forward 1" in e for e in errs), errs


def test_cross_forward_alternation_caught():
    # the second forward restarts in slot 0 after a 3-block forward
    tr = _simulate(n_blocks=3, forwards=2)
    for r in tr:
        if r["forward"] == 1 and r["kind"] in ("asm", "compute"):
            r["slot"] = r["block"] % 2
    assert any(e.startswith("(i)") for e in T.check_trace(tr, 3))


def _find(tr, kind, block, chunk=None, forward=0):
    for r in tr:
        if (r["kind"] == kind and r["block"] == block and (chunk is None or r["chunk"] == chunk)
                and r.get("forward", 0) == forward):
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
    # blocks 1, 2 and 3 in the two slots at once
    assert T.residency_high_water(tr, 6) == 3


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
