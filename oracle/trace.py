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
    chunk    chunk index within the block (h2d/asm), -1 for compute
    slot     slot written (asm) or read (compute); -1 for h2d
    landing  landing buffer written (h2d) or read (asm); -1 for compute
    start, end   times in ms on one clock

Properties (each violation is reported as a string):

 (i)   consecutive blocks alternate slots: block b uses slot (b + s0) mod 2,
       s0 the slot of block 0 (one forward may start in either slot, so that
       a forward with an odd block count hands its free slot to the next);
 (ii)  compute(b) starts after every reconstruction chunk of b has ended,
       and reconstruction chunk j of b starts after H2D chunk j of b ended;
 (iii) the first reconstruction write into slot(b) starts after compute(b-2)
       has ended (the slot is free again only then);
 (iv)  at no instant do more than two blocks occupy the slots (block b
       occupies its slot from its first reconstruction write to the end of its
       compute), and no landing buffer holds two chunks at once (a chunk holds
       its landing buffer from its H2D start to its reconstruction end);
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


def check_trace(trace: Sequence[Mapping], num_blocks: int,
                slot_capacity: Optional[int] = None, numels: Optional[Sequence[int]] = None,
                dp: Optional[int] = None, slack_ms: float = 0.0) -> List[str]:
    errs: List[str] = []
    by_kind: Dict[str, list] = defaultdict(list)
    for r in trace:
        if r["end"] < r["start"]:
            errs.append(f"interval ends before it starts: {dict(r)}")
        by_kind[r["kind"]].append(r)

    comp = {r["block"]: r for r in by_kind["compute"]}
    h2d = {(r["block"], r["chunk"]): r for r in by_kind["h2d"]}
    asm = defaultdict(list)
    for r in by_kind["asm"]:
        asm[r["block"]].append(r)

    for b in range(num_blocks):
        if b not in comp:
            errs.append(f"block {b}: no compute interval")
        if not asm.get(b):
            errs.append(f"block {b}: no reconstruction interval")
    if errs:
        return errs

    # (i) slot assignment: alternation from block 0's slot
    s0 = comp[0]["slot"]
    if s0 not in (0, 1):
        errs.append(f"(i) block 0 uses slot {s0}")
    for r in list(by_kind["asm"]) + list(by_kind["compute"]):
        if r["slot"] != (r["block"] + s0) % 2:
            errs.append(f"(i) block {r['block']} {r['kind']} uses slot {r['slot']}")

    # (ii) ordering inside a block
    for b in range(num_blocks):
        last_asm = max(r["end"] for r in asm[b])
        if comp[b]["start"] + slack_ms < last_asm:
            errs.append(f"(ii) compute({b}) starts at {comp[b]['start']:.6f} before "
                        f"reconstruction ends at {last_asm:.6f}")
        for r in asm[b]:
            src = h2d.get((b, r["chunk"]))
            if src is None:
                errs.append(f"(ii) block {b} chunk {r['chunk']}: no H2D interval")
            elif r["start"] + slack_ms < src["end"]:
                errs.append(f"(ii) block {b} chunk {r['chunk']}: reconstruction starts "
                            f"before its H2D ends")
            elif r["landing"] != src["landing"]:
                errs.append(f"(ii) block {b} chunk {r['chunk']}: landing buffer mismatch")

    # (iii) slot reuse only after compute(b-2)
    for b in range(2, num_blocks):
        first = min(r["start"] for r in asm[b])
        if first + slack_ms < comp[b - 2]["end"]:
            errs.append(f"(iii) block {b} writes slot {(b + s0) % 2} at {first:.6f} before "
                        f"compute({b - 2}) ends at {comp[b - 2]['end']:.6f}")

    # (iv) residency: at most two blocks in slots, one chunk per landing buffer
    occ = [(min(r["start"] for r in asm[b]), comp[b]["end"]) for b in range(num_blocks)]
    hw = _max_overlap(occ)
    if hw > 2:
        errs.append(f"(iv) {hw} blocks resident at once")
    per_landing = defaultdict(list)
    for (b, j), r in h2d.items():
        a = [x for x in asm[b] if x["chunk"] == j]
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
    asm = defaultdict(list)
    comp = {}
    for r in trace:
        if r["kind"] == "asm":
            asm[r["block"]].append(r["start"])
        elif r["kind"] == "compute":
            comp[r["block"]] = r["end"]
    return _max_overlap([(min(asm[b]), comp[b]) for b in range(num_blocks)])
