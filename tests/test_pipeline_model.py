"""Hazard check of the LDS pipelines of the attention kernels (CPU only).

Each kernel streams tiles through a ring of LDS stages with LDS-direct loads
that the compiler cannot see; their ordering rests on the schedule alone:
which tile a body loads, which tiles it reads, how many loads the wait at the
end of a body leaves in flight, and one barrier per body.  This module
restates those schedules as event lists and checks, for every body of a long
tile sequence:

* visibility: a tile is read only after the body whose wait covered its loads
  has ended with its barrier (all waves' loads have then landed);
* overwrite: a load into a stage is issued only after every read of the
  stage's previous tile, including reads still in flight across the barrier
  that precedes the load (the tail reads of the previous body).

The stage counts are read from the kernel headers, so a change there is
checked against the schedule.  Planted mistakes (a stage fewer, a wait that
leaves one more tile in flight) must fail the check.
"""
from __future__ import annotations

import os
import re
from dataclasses import dataclass, field

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "chiplet_numa_aware_amd", "csrc")


def _const(header: str, name: str) -> int:
    with open(os.path.join(CSRC, header)) as f:
        text = f.read()
    m = re.search(r"constexpr int " + name + r" = (\d+);", text)
    assert m, f"{name} not found in {header}"
    return int(m.group(1))


@dataclass
class Schedule:
    """One body per tile index t.  Offsets are relative to t.

    loads:   (stream, tile offset) issued in body t, in issue order;
    reads:   (stream, tile offset) read in body t after its opening barrier;
    tail:    (stream, tile offset) read at the end of body t, before its
             closing barrier, possibly still in flight after it;
    stages:  ring size per stream (a tile x of a stream lives in stage x % S);
    in_flight: loads of the most recent bodies the closing wait leaves
             outstanding, per stream, counted in bodies (loads retire in
             issue order, so a wait covers every earlier body)."""
    loads: list
    reads: list
    tail: list
    stages: dict
    in_flight: dict = field(default_factory=dict)


def check(s: Schedule, n_bodies: int = 40) -> list[str]:
    """All hazards of the schedule over bodies 0..n_bodies-1 (tiles >= 0)."""
    errors = []
    issued = {}   # (stream, tile) -> body that issued its load
    landed = {}   # (stream, tile) -> body whose closing barrier makes it visible
    # last body that reads (stream, tile), and whether a read is in its tail
    last_read = {}
    for t in range(-8, n_bodies):
        for stream, off in s.loads:
            issued[(stream, t + off)] = t
    for (stream, tile), b in issued.items():
        landed[(stream, tile)] = b + s.in_flight.get(stream, 0)
    for t in range(n_bodies):
        for stream, off in s.reads + s.tail:
            x = t + off
            if x < 0:
                continue
            tail = (stream, off) in s.tail
            # a main read needs the barrier that closed body t-1; a tail read
            # of body t happens before body t's barrier, after body t-1's
            need = t - 1
            if landed[(stream, x)] > need:
                errors.append(f"body {t}: {stream} tile {x} read before its loads are visible "
                              f"(landed at the end of body {landed[(stream, x)]})")
            prev = last_read.get((stream, x), (-1, False))
            last_read[(stream, x)] = max(prev, (t, tail))
    for (stream, tile), b in issued.items():
        if tile < 0 or b < 0 or b >= n_bodies:
            continue
        S = s.stages[stream]
        old = tile - S
        if old < 0 or (stream, old) not in last_read:
            continue
        rb, rtail = last_read[(stream, old)]
        # the load is issued after the barrier that closed body b-1: every
        # read of body <= b-1 has been issued by then, but a tail read of
        # body b-1 may still be in flight
        if rb > b - 1 or (rb == b - 1 and rtail):
            errors.append(f"body {b}: {stream} tile {tile} overwrites tile {old} "
                          f"(last read in body {rb}{' tail' if rtail else ''})")
    return errors


def forward_schedule(stages: int, ahead: int = 4) -> Schedule:
    # Steady tile j: K of tile j+4 and V of tile j+3 loaded (K first); score
    # MFMAs of tile j+1 read K of j+1, P V reads V of j; the ring head, the
    # first K fragments of tile j+2, is read before the closing barrier.  The
    # closing wait covers every load issued before body j-1 and the K loads
    # of body j-1: K in flight for one body, V for two.
    return Schedule(loads=[("K", ahead), ("V", ahead - 1)],
                    reads=[("K", 1), ("V", 0)], tail=[("K", 2)],
                    stages={"K": stages, "V": stages}, in_flight={"K": 1, "V": 2})


def dkv_schedule(stages: int) -> Schedule:
    # Body t: loads Q, dO and the statistics of tile t+3 into one stage; the
    # first part reads the transposed Q/dO fragments of tile t-1, the second
    # part the row fragments of tile t+1; the tail reads the first transposed
    # fragments of tile t and the statistics of tile t+1.  The closing wait
    # leaves the body's own loads in flight.
    return Schedule(loads=[("QdO", 3), ("st", 3)],
                    reads=[("QdO", -1), ("QdO", 1)], tail=[("QdO", 0), ("st", 1)],
                    stages={"QdO": stages, "st": stages}, in_flight={"QdO": 1, "st": 1})


def dq_schedule(stages: int) -> Schedule:
    # Tile j: K/V of tile j+3 loaded; every read is of tile j; the closing
    # wait leaves the loads of the last two bodies in flight.
    return Schedule(loads=[("KV", 3)], reads=[("KV", 0)], tail=[],
                    stages={"KV": stages}, in_flight={"KV": 2})


def test_forward_pipeline_is_hazard_free():
    stages = _const("attn_fwd_kernel.hpp", "kStages")
    assert check(forward_schedule(stages, ahead=stages)) == []


def test_dkv_pipeline_is_hazard_free():
    stages = _const("attn_bwd_kernel.hpp", "kDkvStages")
    assert check(dkv_schedule(stages)) == []


def test_dq_pipeline_is_hazard_free():
    with open(os.path.join(CSRC, "attn_bwd_kernel.hpp")) as f:
        m = re.search(r"constexpr int kDqStages = (\d+);", f.read())
    assert m
    assert check(dq_schedule(int(m.group(1)))) == []


@pytest.mark.parametrize("make, stages", [
    (forward_schedule, 3),   # a stage fewer: K of tile j+4 would overwrite K of j+1
    (dkv_schedule, 4),       # tile t+3 would overwrite tile t-1, read in body t
    (dq_schedule, 3),        # tile j+3 would overwrite tile j
])
def test_planted_stage_shortage_is_caught(make, stages):
    assert any("overwrites" in e for e in check(make(stages)))


def test_planted_short_wait_is_caught():
    s = dkv_schedule(5)
    s.in_flight = {"QdO": 2, "st": 2}   # wait leaves two bodies' loads in flight
    assert any("before its loads are visible" in e for e in check(s))
    f = forward_schedule(4)
    f.in_flight = {"K": 2, "V": 2}      # K of the ring head not yet covered
    assert any("K tile" in e and "visible" in e for e in check(f))


def test_planted_tail_read_of_the_next_load_target_is_caught():
    # With the kernel's five stages, body t+1 loads tile t+4 into the stage of
    # tile t-1: a tail read of tile t-1, still in flight across the barrier,
    # would race with that load (the kernel's tail reads tile t instead).
    s = dkv_schedule(5)
    assert check(s) == []
    s.tail = [("QdO", -1), ("st", 1)]
    errors = check(s)
    assert errors and all("tail" in e for e in errors)
