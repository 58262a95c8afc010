"""Checker for the two-slot streaming schedule (oracle).

Release page, section "Double-buffered prefetch with H2D + AllGather overlap":
exactly two device buffers (slots), each sized to the model's largest block,
allocated once and shared by every layer; while compute runs layer N from
one slot, layer N+1 is prepared into the other in two phases on side streams
(host-to-device copy of the shards, then the gather); compute waits on an
event for the gather before it switches slots; weight memory therefore stays
at two blocks whatever the depth.

Many interleavings are correct, so the checker verifies properties of a
measured trace instead of comparing against one timeline.  A trace is a list
of intervals (one per H2D chunk, per reconstruction chunk and per block
compute), each a mapping with keys:

    kind     'h2d' | 'asm' | 'compute'
    block    block index (position in the forward)
    forward  index of the forward the interval belongs to (optional, 0)
    chunk    chunk index within the block (h2d/asm), -1 for compute
    slot     slot written (asm) or read (compute); -1 for h2d
    landing  landing buffer written (h2d) or read (asm); -1 for compute
    bytes    bytes moved (h2d: the chunk's length; optional)
    start, end   times in ms on one clock

A trace may span several consecutive forwards of one model (a denoising loop
calls the forward once per step); block b of forward f is then the block
instance g = f * num_blocks + b of one long sequence, and every property below
is stated over that sequence, across forward boundaries too.

Properties (each violation is reported as a string):

 (i)   consecutive block instances alternate slots, starting from the slot
       of the first one traced (a forward with an odd block count hands its
       free slot to the next forward's first block);
 (ii)  compute(g) starts after every reconstruction chunk of g has ended,
       and reconstruction chunk j of g starts after H2D chunk j of g ended;
 (iii) the first reconstruction write into slot(g) starts after compute(g-2)
       has ended (the slot is free again only then);
 (iv)  residency -- the page's TL;DR puts exactly two layers' weights on each
       device at any time: at no instant do more than two block instances
       occupy the slots (g occupies its slot from its first reconstruction
       write to the end of its compute), nor have more than two any weight
       bytes on the device (g counts from its first H2D start, its chunks in
       the landing buffers included, to the end of its compute); and no
       landing buffer holds two chunks at once (a chunk holds its landing
       buffer from its H2D start to its reconstruction end);
 (v)   each slot's capacity equals dp * max_b shard_size(numel_b) elements.
"""

from __future__ import annotations

from collections import defaultdict
from typing import Dict, Iterable, List, Mapping, Optional, Sequence

from .shard import shard_size


def slot_capacity_elems(numels: Sequence[int], dp: int) -> int:
    return dp * max(shard_size(n, dp) for n in numels)


def _max_overlap(intervals: Iterable[tuple]) -> int:
    """Largest number of half-open [start, end) intervals alive at once."""
    ev = []
    for s, e in intervals:
        ev.append((s, 1))
        ev.append((e, -1))
    ev.sort(key=lambda t: (t[0], t[1]))  # ends before starts at equal times
    cur = best = 0
    for _, dlt in ev:
        cur += dlt
        best = max(best, cur)
    return best


def _seq(r: Mapping, num_blocks: int) -> int:
    """Block instance index of an interval: forward * num_blocks + block."""
    return int(r.get("forward", 0) or 0) * num_blocks + int(r["block"])


def _spans(trace: Sequence[Mapping], num_blocks: int):
    """Per block instance g: first reconstruction start, first H2D start and
    compute end (None where the trace holds no such interval)."""
    asm0: Dict[int, float] = {}
    h2d0: Dict[int, float] = {}
    comp1: Dict[int, float] = {}
    for r in trace:
        g = _seq(r, num_blocks)
        if r["kind"] == "asm":
            asm0[g] = min(asm0.get(g, r["start"]), r["start"])
        elif r["kind"] == "h2d":
            h2d0[g] = min(h2d0.get(g, r["start"]), r["start"])
        elif r["kind"] == "compute":
            comp1[g] = max(comp1.get(g, r["end"]), r["end"])
    return asm0, h2d0, comp1


def check_trace(trace: Sequence[Mapping], num_blocks: int,
                slot_capacity: Optional[int] = None, numels: Optional[Sequence[int]] = None,
                dp: Optional[int] = None, slack_ms: float = 0.0) -> List[str]:
    errs: List[str] = []
    by_kind: Dict[str, list] = defaultdict(list)
    for r in trace:
        if r["end"] < r["start"]:
            errs.append(f"interval ends before it starts: {dict(r)}")
        by_kind[r["kind"]].append(r)
    L = num_blocks

    comp = {_seq(r, L): r for r in by_kind["compute"]}
    h2d = {(_seq(r, L), r["chunk"]): r for r in by_kind["h2d"]}
    asm = defaultdict(list)
    for r in by_kind["asm"]:
        asm[_seq(r, L)].append(r)

    forwards = sorted({int(r.get("forward", 0) or 0) for r in trace}) or [0]
    seq = [f * L + b for f in forwards for b in range(L)]
    for g in seq:
        if g not in comp:
            errs.append(f"block {g % L} of forward {g // L}: no compute interval")
        if not asm.get(g):
            errs.append(f"block {g % L} of forward {g // L}: no reconstruction interval")
    if errs:
        return errs

    def name(g):
        return f"{g % L}" if len(forwards) == 1 else f"{g % L} of forward {g // L}"

    # (i) slot assignment: alternation from the first instance's slot
    g0 = seq[0]
    s0 = comp[g0]["slot"]
    if s0 not in (0, 1):
        errs.append(f"(i) block {name(g0)} uses slot {s0}")
    for r in list(by_kind["asm"]) + list(by_kind["compute"]):
        g = _seq(r, L)
        if r["slot"] != (s0 + g - g0) % 2:
            errs.append(f"(i) block {name(g)} {r['kind']} uses slot {r['slot']}")

    # (ii) ordering inside a block instance
    for g in seq:
        last_asm = max(r["end"] for r in asm[g])
        if comp[g]["start"] + slack_ms < last_asm:
            errs.append(f"(ii) compute({name(g)}) starts at {comp[g]['start']:.6f} before "
                        f"reconstruction ends at {last_asm:.6f}")
        for r in asm[g]:
            src = h2d.get((g, r["chunk"]))
            if src is None:
                errs.append(f"(ii) block {name(g)} chunk {r['chunk']}: no H2D interval")
            elif r["start"] + slack_ms < src["end"]:
                errs.append(f"(ii) block {name(g)} chunk {r['chunk']}: reconstruction starts "
                            f"before its H2D ends")
            elif r["landing"] != src["landing"]:
                errs.append(f"(ii) block {name(g)} chunk {r['chunk']}: landing buffer mismatch")

    # (iii) slot reuse only after compute(g-2), across forward boundaries too
    for g in seq:
        if g - 2 not in comp:
            continue
        first = min(r["start"] for r in asm[g])
        if first + slack_ms < comp[g - 2]["end"]:
            errs.append(f"(iii) block {name(g)} writes slot {comp[g]['slot']} at {first:.6f} before "
                        f"compute({name(g - 2)}) ends at {comp[g - 2]['end']:.6f}")

    # (iv) residency: two block instances in the slots and on the device at
    # most, one chunk per landing buffer
    hw = residency_high_water(trace, num_blocks)
    if hw > 2:
        errs.append(f"(iv) {hw} blocks resident in slots at once")
    dhw = device_high_water(trace, num_blocks)
    if dhw > 2:
        errs.append(f"(iv) {dhw} blocks with weights on the device at once")
    per_landing = defaultdict(list)
    for (g, j), r in h2d.items():
        a = [x for x in asm[g] if x["chunk"] == j]
        end = a[0]["end"] if a else r["end"]
        per_landing[r["landing"]].append((r["start"], end))
    for lb, iv in per_landing.items():
        if _max_overlap(iv) > 1:
            errs.append(f"(iv) landing buffer {lb} holds two chunks at once")

    # (v) slot capacity
    if slot_capacity is not None and numels is not None and dp is not None:
        want = slot_capacity_elems(numels, dp)
        if slot_capacity != want:
            errs.append(f"(v) slot capacity {slot_capacity} != dp * S_max = {want}")
    return errs


def residency_high_water(trace: Sequence[Mapping], num_blocks: int) -> int:
    """Most block instances in the two slots at one instant: an instance holds
    its slot from its first reconstruction start to its compute end.  Instances
    the trace does not show both ends of are left out."""
    asm0, _, comp1 = _spans(trace, num_blocks)
    return _max_overlap([(asm0[g], comp1[g]) for g in asm0 if g in comp1])


def device_high_water(trace: Sequence[Mapping], num_blocks: int) -> int:
    """Most block instances with any weight bytes on the device at one
    instant: an instance counts from its first H2D start (its chunks sit in
    the landing buffers before they reach its slot) to its compute end."""
    _, h2d0, comp1 = _spans(trace, num_blocks)
    return _max_overlap([(h2d0[g], comp1[g]) for g in h2d0 if g in comp1])


def weight_bytes_peak(trace: Sequence[Mapping], num_blocks: int, block_bytes: Sequence[int]) -> int:
    """Most weight bytes in use on the device at one instant: a block instance
    in its slot counts block_bytes[block] (its padded size) from its first
    reconstruction start to its compute end; an H2D chunk counts its `bytes`
    from its H2D start to the end of its reconstruction (it then sits in a
    landing buffer)."""
    asm0, _, comp1 = _spans(trace, num_blocks)
    ev = []
    for g in asm0:
        if g in comp1:
            ev.append((asm0[g], int(block_bytes[g % num_blocks])))
            ev.append((comp1[g], -int(block_bytes[g % num_blocks])))
    asm_end = {}
    for r in trace:
        if r["kind"] == "asm":
            asm_end[(_seq(r, num_blocks), r["chunk"])] = r["end"]
    for r in trace:
        if r["kind"] == "h2d":
            end = asm_end.get((_seq(r, num_blocks), r["chunk"]))
            if end is not None:
                ev.append((r["start"], int(r["bytes"])))
                ev.append((end, -int(r["bytes"])))
    ev.sort(key=lambda t: (t[0], t[1]))  # releases before acquisitions at equal times
    cur = best = 0
    for _, dlt in ev:
        cur += dlt
        best = max(best, cur)
    return best
