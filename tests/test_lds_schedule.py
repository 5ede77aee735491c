"""The LDS hand-off schedules of the matrix-core kernels, replayed on the CPU.

The causal prefill kernel (csrc/prefill.hip) and the backward's dq and dk/dv
kernels (csrc/prefill_bwd.hip) split each 32-row block between a score wave
and a value wave that hand tiles to each other through LDS, with one barrier
per tile.  This module restates, role by role and in each kernel's own order,
which LDS buffer every wave reads and writes between two barriers (an
"epoch"), which tile each buffer holds, and what the register stages of the
global loads hold when they are stored; then checks, over many grid shapes
(ragged tile counts, windows that start the loop late, pairs whose row
ranges differ):

  * every role passes the same number of barriers;
  * no buffer is written in an epoch in which another wave may read or
    write it (there is no ordering inside an epoch);
  * every read finds the tile it expects, written in an earlier epoch;
  * every register stage stored to LDS holds the tile the store expects.

A planted change (the dq kernel's K tiles double- instead of triple-
buffered, or the forward's register stages swapped) must be caught.  The
forward this kernel replaced (four waves, each doing both roles on its own
rows), which returned wrong results on some launches, is modelled too: the
model locates its race (K tile 2 stored over tile 0 in the epoch in which
the scores of tile 0 still read it).
"""
import itertools

import pytest


class Trace:
    """LDS events of one workgroup: (epoch, wave, 'r' | 'w', buffer, tile)."""

    def __init__(self):
        self.events = []
        self.barriers = {}
        self.stage_errors = []

    def wave(self, name):
        self.barriers.setdefault(name, 0)
        return Wave(self, name)


class Wave:
    def __init__(self, trace, name):
        self.t, self.name = trace, name
        self.stages = {}

    @property
    def epoch(self):
        return self.t.barriers[self.name]

    def read(self, buf, tile):
        self.t.events.append((self.epoch, self.name, "r", buf, tile))

    def write(self, buf, tile):
        self.t.events.append((self.epoch, self.name, "w", buf, tile))

    def barrier(self):
        self.t.barriers[self.name] += 1

    def load(self, stage, tile):  # global loads into a register stage
        self.stages[stage] = tile

    def store(self, stage, buf, tile):  # a register stage to LDS
        if self.stages.get(stage) != tile:
            self.t.stage_errors.append((self.name, stage, self.stages.get(stage), tile))
        self.write(buf, tile)


def check(trace):
    """The four properties above; returns a list of violations."""
    bad = []
    if len(set(trace.barriers.values())) != 1:
        bad.append(("barrier counts differ", trace.barriers))
    bad += [("register stage", e) for e in trace.stage_errors]
    by_epoch = {}
    for ev in trace.events:
        by_epoch.setdefault((ev[0], ev[3]), []).append(ev)
    for (ep, buf), evs in sorted(by_epoch.items(), key=repr):
        written = {e[4] for e in evs if e[2] == "w"}
        # all threads may store pieces of one tile together; a read, or a
        # second tile, beside a store in the same epoch is unordered
        if written and (len(written) > 1 or any(e[2] == "r" for e in evs)):
            bad.append(("unordered access", ep, buf, sorted(evs)))
    last = {}  # buffer -> (epoch, tile) of the latest store
    for ev in sorted(trace.events, key=lambda e: (e[0], e[2] == "r")):
        ep, who, op, buf, tile = ev
        if op == "w":
            last[buf] = (ep, tile)
        else:
            w = last.get(buf)
            if w is None or w[0] >= ep or w[1] != tile:
                bad.append(("stale read", ev, w))
    return bad


# ------------------------------------------------------------------ forward ---

def forward_trace(t_first, ntiles, pairs, swap_stages=False):
    """prefill_kernel: `pairs` = [(pair_lo, pair_tiles)] per score/value pair.
    Shared K and V tiles double-buffered (buffer t & 1); per-pair P operands
    and rescale factors double-buffered.  advance(t): K tile t+1 into K[(t+1)
    & 1] and V tile t into V[t & 1] from the register stages, then the loads
    of K tile t+3 and V tile t+2, then the barrier."""
    tr = Trace()
    roles = []
    for p, (lo, hi) in enumerate(pairs):
        roles.append(("score", p, lo, hi, tr.wave(f"score{p}")))
        roles.append(("value", p, lo, hi, tr.wave(f"value{p}")))

    def advance(w, t, P):
        Q = 1 - P
        ks, vs = (("k", Q), ("v", P)) if not swap_stages else (("k", P), ("v", Q))
        w.store(ks, ("K", (t + 1) & 1), t + 1)
        w.store(vs, ("V", t & 1), t)
        w.load(("k", Q), t + 3)
        w.load(("v", P), t + 2)
        w.barrier()

    for kind, p, lo, hi, w in roles:
        # prologue (every thread of both roles): K tile t_first to LDS, K
        # tiles t_first + 1, + 2 and V tiles t_first, + 1 in flight
        w.load(("k", 0), t_first)
        w.store(("k", 0), ("K", 0), t_first)
        w.load(("k", 1), t_first + 1)
        w.load(("v", 0), t_first)
        w.load(("k", 0), t_first + 2)
        w.load(("v", 1), t_first + 1)
        w.barrier()
        for t in range(t_first, ntiles + 1, 2):
            for tt, P in ((t, 0), (t + 1, 1)):
                if kind == "score":
                    if lo <= tt < hi:
                        w.read(("K", tt & 1), tt)
                        w.write(("P", p, tt & 1), tt)
                else:
                    u = tt - 1
                    if lo <= u < hi:
                        w.read(("P", p, u & 1), u)
                        w.read(("V", u & 1), u)
                advance(w, tt, P)
        # the statistics instantiation: the score wave hands its final
        # reference max to the value wave across one more barrier
        if kind == "score":
            w.write(("MFIN", p), "final")
        w.barrier()
        if kind == "value":
            w.read(("MFIN", p), "final")
    return tr


# ----------------------------------------------------------------------- dq ---

def dq_trace(t_first, ntiles, pairs, kslots=3):
    """bwd_dq_kernel: K tiles in kslots buffers (tile t in t % 3), V double-
    buffered, per-pair dS/dT operands double-buffered.  Score waves read K
    and V tile t and write dS, dT of tile t; value waves read dS, dT and K
    tile t - 1 (transposed), then store K and V tile t + 1 from the stage
    (two stages, tile j in stage j & 1) and load tile t + 3."""
    tr = Trace()
    for p, (lo, hi) in enumerate(pairs):
        s = tr.wave(f"score{p}")
        s.barrier()  # the value waves' prologue
        for t in range(t_first, ntiles + 1, 2):
            for tt in (t, t + 1):
                if lo <= tt < hi:
                    s.read(("K", tt % kslots), tt)
                    s.read(("V", tt & 1), tt)
                    s.write(("P", p, tt & 1), tt)
                s.barrier()
        v = tr.wave(f"value{p}")
        v.load(0, t_first)
        v.store(0, ("K", t_first % kslots), t_first)
        v.write(("V", 0), t_first)
        v.load(1, t_first + 1)
        v.load(0, t_first + 2)
        v.barrier()
        for t in range(t_first, ntiles + 1, 2):
            for tt, P in ((t, 0), (t + 1, 1)):
                u = tt - 1
                if lo <= u < hi:
                    v.read(("P", p, u & 1), u)
                    v.read(("K", u % kslots), u)
                v.store(1 - P, ("K", (tt + 1) % kslots), tt + 1)
                v.write(("V", (tt + 1) & 1), tt + 1)
                v.load(1 - P, tt + 3)
                v.barrier()
    return tr


# ---------------------------------------------------------------------- dkv ---

def dkv_trace(ntiles, active_sets):
    """bwd_dkv_kernel: q, rho, dout tiles and row statistics of tile t in
    buffer t % 3 (one register stage: tile t + 1 goes to LDS at the start of
    epoch t, the stage then loads tile t + 2); per-pair W, dS, dT operands
    double-buffered.  `active_sets` = the tiles each pair works on."""
    tr = Trace()
    for p, act in enumerate(active_sets):
        s = tr.wave(f"score{p}")
        s.barrier()
        for t in range(ntiles):
            if t in act:
                for a in ("Q", "R", "G", "STAT"):
                    s.read((a, t % 3), t)
                s.write(("P", p, t & 1), t)
            s.barrier()
        v = tr.wave(f"value{p}")
        v.load("st", 0)
        for a in ("Q", "R", "G", "STAT"):
            v.store("st", (a, 0), 0)
        v.load("st", 1)
        v.barrier()
        for t in range(ntiles):
            for a in ("Q", "R", "G", "STAT"):
                v.store("st", (a, (t + 1) % 3), t + 1)
            if t - 1 in act:
                v.read(("P", p, (t - 1) & 1), t - 1)
                for a in ("Q", "R", "G"):
                    v.read((a, (t - 1) % 3), t - 1)
            v.load("st", t + 2)
            v.barrier()
        if ntiles - 1 in act:  # after the last barrier
            v.read(("P", p, (ntiles - 1) & 1), ntiles - 1)
            for a in ("Q", "R", "G"):
                v.read((a, (ntiles - 1) % 3), ntiles - 1)
    return tr


# ------------------------------------------------- the replaced forward ---

def replaced_forward_trace(ntiles, wave_tiles):
    """The forward this kernel replaced: four waves, each doing both roles on
    its own rows.  Epoch t: the scores of tile t + 1 (K[(t+1) & 1]) and the
    value sums of tile t (V[t & 1]); then K tile t + 2 into K[t & 1] and V
    tile t + 1 into V[(t+1) & 1] from single register stages, and the loads
    of K tile t + 3 and V tile t + 2."""
    tr = Trace()
    for wv, wt in enumerate(wave_tiles):
        w = tr.wave(f"wave{wv}")
        w.load("k", 0)
        w.store("k", ("K", 0), 0)
        w.load("v", 0)
        w.store("v", ("V", 0), 0)
        if ntiles > 1:
            w.load("k", 1)
            w.store("k", ("K", 1), 1)
        if ntiles > 2:
            w.load("k", 2)
        if ntiles > 1:
            w.load("v", 1)
        w.barrier()
        w.read(("K", 0), 0)  # scores of tile 0 before the loop
        for t in range(ntiles):
            if t < wt:
                if t + 1 < ntiles:
                    w.read(("K", (t + 1) & 1), t + 1)
                w.read(("V", t & 1), t)
            if t + 2 < ntiles:
                w.store("k", ("K", t & 1), t + 2)
            if t + 1 < ntiles:
                w.store("v", ("V", (t + 1) & 1), t + 1)
            if t + 3 < ntiles:
                w.load("k", t + 3)
            if t + 2 < ntiles:
                w.load("v", t + 2)
            w.barrier()
    return tr


# ------------------------------------------------------------------- tests ---

def forward_cases():
    """(t_first, ntiles, pair ranges) as the kernels derive them: full causal
    (t_first = 0, pair_lo = 0, pair_tiles = the pair's last row tile + 1) and
    windows (t_first even, each pair_lo >= t_first)."""
    for ntiles in range(1, 11):
        for rows_per_pair in (1, 2):  # GQA groups give pairs of 32 or 64... rows per head
            pts = [min(ntiles, (i + 1) * rows_per_pair) for i in range(4)]
            yield 0, ntiles, [(0, max(1, x)) for x in pts]
        for t_first in range(0, ntiles, 2):
            for lo_off in range(0, 3):
                pairs = [(min(ntiles - 1, t_first + lo_off + i // 2), ntiles) for i in range(4)]
                yield t_first, ntiles, pairs


@pytest.mark.parametrize("t_first,ntiles,pairs", list(forward_cases()))
def test_forward_schedule(t_first, ntiles, pairs):
    assert check(forward_trace(t_first, ntiles, pairs)) == []


@pytest.mark.parametrize("t_first,ntiles,pairs", list(forward_cases()))
def test_dq_schedule(t_first, ntiles, pairs):
    assert check(dq_trace(t_first, ntiles, pairs)) == []


@pytest.mark.parametrize("ntiles", range(1, 13))
def test_dkv_schedule(ntiles):
    # pairs see contiguous runs of query tiles, per head of the group (G = 2:
    # two runs of nq tiles), some pairs none at all
    nq = max(1, ntiles // 2)
    sets = [set(range(ntiles)), {t for t in range(ntiles) if t % nq >= 1},
            {t for t in range(ntiles) if t % nq >= nq - 1}, set()]
    assert check(dkv_trace(ntiles, sets)) == []


@pytest.mark.parametrize("ntiles", range(1, 12))
def test_replaced_forward_race_is_located(ntiles):
    """The replaced forward computed the scores of tile 0 right after its
    prologue barrier, and in the same epoch every thread stored K tile 2
    into the buffer tile 0 occupies: a wave that ran ahead overwrote rows of
    K tile 0 that a slower wave was still reading.  With three or more tiles
    that is the one violation the model finds -- a whole wave's scores of
    tile 0 spoiled, which matches its wrong results (whole 32-row wave
    blocks, about one launch in eight at batch 4 x 8192)."""
    waves = [max(1, ntiles - i) for i in range(4)]
    bad = check(replaced_forward_trace(ntiles, waves))
    if ntiles < 3:
        assert bad == []
    else:
        unordered = [b for b in bad if b[0] == "unordered access"]
        assert [(b[1], b[2]) for b in unordered] == [(1, ("K", 0))]
        assert {e[4] for e in unordered[0][3]} == {0, 2}  # tile 0 read, tile 2 stored
        assert all(b[0] in ("unordered access", "stale read") and
                   (b[0] != "stale read" or b[1][:4] == (1, b[1][1], "r", ("K", 0)))
                   for b in bad)


def test_planted_double_buffered_dq_k_tiles_are_caught():
    """dq's K tile is read by the score waves in epoch t and by the value
    waves in epoch t + 1, so two buffers cannot hold it: the model must see
    the value waves' store of tile t + 1 overwrite tile t - 1 while it is
    still read."""
    bad = check(dq_trace(0, 6, [(0, 6)] * 4, kslots=2))
    assert any(b[0] == "unordered access" or b[0] == "stale read" for b in bad)


def test_planted_swapped_forward_stages_are_caught():
    bad = check(forward_trace(0, 6, [(0, 6)] * 4, swap_stages=True))
    assert any(b[0] == "register stage" for b in bad)


def test_checker_sees_a_write_beside_a_read():
    tr = Trace()
    a, b = tr.wave("a"), tr.wave("b")
    a.write("X", 0)
    a.barrier(), b.barrier()
    a.write("X", 1)
    b.read("X", 0)
    a.barrier(), b.barrier()
    assert any(x[0] == "unordered access" for x in check(tr))
