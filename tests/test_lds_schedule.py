"""The LDS hand-off schedules of the matrix-core kernels, replayed on the CPU.

The causal prefill kernel (csrc/prefill.hip) and the backward's dq and dk/dv
kernels (csrc/prefill_bwd.hip) split each 32-row block between a score wave
and a value wave that hand tiles to each other through LDS, with one barrier
per tile; the projection's large-tile GEMM (csrc/proj.hip) fills two LDS
stages with global->LDS loads that land at no fixed time, bounded only by
each wave's explicit wait counts.  This module restates, role by role and in each kernel's own order,
which LDS buffer every wave reads and writes between two barriers (an
"epoch"), which tile each buffer holds, and what the register stages of the
global loads hold when they are stored; then checks, over many grid shapes
(ragged tile counts, windows that start the loop late, pairs whose row
ranges differ, and for the prefill the work lists of its persistent
workgroups, whose items follow each other in one stream of positions):

  * every role passes the same number of barriers;
  * no buffer is written in an epoch in which another wave may read or
    write it (there is no ordering inside an epoch);
  * every read finds the tile it expects, written in an earlier epoch;
  * every register stage stored to LDS holds the tile the store expects.

A planted change (the dq kernel's K tiles double- instead of triple-
buffered, the forward's register stages swapped, its items shorter than
the three positions its loads run ahead, or the projection's waits one
chunk too loose, its loads issued before the barrier or the next tile's
before the output is read back) must be caught.  The
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
            bad.append(("unordered access", ep, buf, sorted(evs, key=repr)))
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

def forward_items(S, G, W, units, P, wg, min_len=4, persistent=True):
    """The work list of workgroup `wg` (prefill_kernel) when P persistent
    workgroups run: items k = (query block, unit), longest causal rows
    first.  With R = nitems // P - 1 >= 1 rounds, workgroup wg < P takes one
    item per round, in workgroup order in even rounds and in reverse order of
    8-workgroup groups in odd ones; workgroup wg >= P takes item R P + wg - P.
    (R < 1: every workgroup one item.)  Each item: (tiles t0, t1, stream
    positions it spans -- even, at least min_len, the last four being its
    tail --, [(pair_lo, pair_hi)] of the four pairs).  Not persistent (head
    dim 64): one item per workgroup."""
    pph = 4 // G
    qb_rows = 32 * pph
    nqb = -(-S // qb_rows)
    nitems = nqb * units
    R = nitems // P - 1 if persistent else 0
    if R < 1:
        P, R = 0, 0

    def item_id(i):
        if wg >= P:
            return R * P + wg - P
        off = wg
        if i & 1:
            off = P - 8 - (wg & ~7) + (wg & 7) if P % 8 == 0 else P - 1 - wg
        return i * P + off

    n_mine = R if wg < P else 1
    items = []
    for i in range(n_mine):
        qb = nqb - 1 - item_id(i) // units
        t1 = -(-min(S, (qb + 1) * qb_rows) // 32)
        t0 = max(0, qb * qb_rows - W + 1) // 32 if W > 0 else 0
        n = max(t1 - t0, min_len)
        n += n & 1
        pairs = []
        for p in range(4):
            r0 = qb * qb_rows + (p % pph) * 32
            hi = min(t1, -(-min(S, r0 + 32) // 32))
            lo = max(0, r0 - W + 1) // 32 if W > 0 else 0
            pairs.append((lo, hi))
        items.append((t0, t1, n, pairs))
    return items


def forward_grid(S, G, units, P):
    """Workgroups the launcher starts for P persistent ones (P <= items)."""
    nitems = -(-S // (32 * (4 // G))) * units
    R = nitems // P - 1
    return P + nitems - R * P if R >= 1 else nitems


def forward_trace(items, swap_stages=False, mfin_slots=2):
    """prefill_kernel over one workgroup's work list: an outer loop over the
    items, an inner loop over an item's positions t0 .. t0 + n - 1, all of
    them one stream of positions (so buffers go by the stream position's
    parity; items span an even number).  K and V tiles double-buffered;
    per-pair P operands and rescale factors double-buffered; the final
    reference max handed to the value wave per item (buffer = item parity).
    advance(t): K tile of position +1 into K[(j+1) & 1] and V tile of the
    position into V[j & 1] from the register stages, then the loads for
    positions +3 and +2, then the barrier.  Loads past an item's positions
    go to the next item's (its t0 + the overshoot), past the last item to
    the last position's tile again -- exactly as the kernel maps them, so a
    register stage stored to LDS is checked against the (item, tile) the
    position holds."""
    tr = Trace()
    pos = [(i, t) for i, (t0, t1, n, prs) in enumerate(items) for t in range(t0, t0 + n)]
    npos = len(pos)

    def fetched(j, d):  # (item, tile) the kernel loads at position j for position j + d
        i, t = pos[min(j, npos - 1)]
        t0, t1, n, prs = items[i]
        tt = t + d if j < npos else t0 + n + d  # past the end: the final advance
        if tt < t0 + n:
            return i, tt
        if i + 1 < len(items):
            return i + 1, items[i + 1][0] + tt - (t0 + n)
        return i, t0 + n - 1

    def want(j):
        return pos[j] if j < npos else None

    roles = []
    for p in range(4):
        roles.append(("score", p, tr.wave(f"score{p}")))
        roles.append(("value", p, tr.wave(f"value{p}")))

    def store_checked(w, stage, buf, j):
        if j < npos:
            w.store(stage, buf, want(j))
        else:
            w.write(buf, ("past", j))

    def advance(w, j, P):
        Q = 1 - P
        ks, vs = (("k", Q), ("v", P)) if not swap_stages else (("k", P), ("v", Q))
        store_checked(w, ks, ("K", Q), j + 1)
        store_checked(w, vs, ("V", P), j)
        w.load(("k", Q), fetched(j, 3))
        w.load(("v", P), fetched(j, 2))
        w.barrier()

    for kind, p, w in roles:
        # prologue: K tile of position 0 to LDS; K 1, 2 and V 0, 1 in flight
        w.load(("k", 0), fetched(0, 0))
        w.store(("k", 0), ("K", 0), want(0))
        w.load(("k", 1), fetched(0, 1))
        w.load(("v", 0), fetched(0, 0))
        w.load(("k", 0), fetched(0, 2))
        w.load(("v", 1), fetched(0, 1))
        w.barrier()
        j = 0
        for i, (t0, t1, n, prs) in enumerate(items):
            assert n % 2 == 0
            for t in range(t0, t0 + n):
                P = j & 1
                if kind == "score":
                    lo, hi = prs[p]
                    if lo <= t < hi:
                        w.read(("K", P), pos[j])
                        w.write(("P", p, P), pos[j])
                    if t == t0 + n - 1:
                        w.write(("MFIN", p, i % mfin_slots), i)
                else:
                    if j > 0:
                        pi, pt = pos[j - 1]
                        lo, hi = items[pi][3][p]
                        if lo <= pt < hi:
                            w.read(("P", p, (j - 1) & 1), pos[j - 1])
                            w.read(("V", (j - 1) & 1), pos[j - 1])
                        if pi != i:  # the previous item's outputs
                            w.read(("MFIN", p, pi % mfin_slots), pi)
                advance(w, j, P)
                j += 1
        # the position after the last: the value waves' last tile and outputs
        if kind == "value":
            pi, pt = pos[-1]
            lo, hi = items[pi][3][p]
            if lo <= pt < hi:
                w.read(("P", p, (npos - 1) & 1), pos[-1])
                w.read(("V", (npos - 1) & 1), pos[-1])
            w.read(("MFIN", p, pi % mfin_slots), pi)
        advance(w, npos, 0)
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

def dkv_trace(ntiles, active_sets, early_loads=False):
    """bwd_dkv_kernel: q, rho, dout tiles and row statistics of tile t in
    buffer t % 3 (one register stage: tile t + 1 goes to LDS at the start of
    epoch t, the stage then loads tile t + 2, after the value MFMAs' reads
    or, `early_loads` (head dim 64), before them); per-pair W, dS, dT
    operands double-buffered.  `active_sets` = the tiles each pair works on."""
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
            if early_loads:
                v.load("st", t + 2)
            if t - 1 in act:
                v.read(("P", p, (t - 1) & 1), t - 1)
                for a in ("Q", "R", "G"):
                    v.read((a, (t - 1) % 3), t - 1)
            if not early_loads:
                v.load("st", t + 2)
            v.barrier()
        if ntiles - 1 in act:  # after the last barrier
            v.read(("P", p, (ntiles - 1) & 1), ntiles - 1)
            for a in ("Q", "R", "G"):
                v.read((a, (ntiles - 1) % 3), ntiles - 1)
    return tr


# ----------------------------------------------------------- projection ---

def proj_trace(nsteps, waits=None, stages=2, early_loads=False, ntiles=1, early_next=False):
    """proj_big_kernel: four waves, each running `ntiles` tiles in turn; K
    chunk s of a tile's operands in stage s % stages, filled by global->LDS
    loads that each wave issues for its own rows.  Such a load lands at no
    fixed time: the model writes its stage in every epoch from its issue up
    to the one in which the issuing wave's explicit wait (pending loads at
    most `bound` chunks' worth, oldest first) covers it.

    Per tile: chunks 0 and 1 are loaded before the tile (the first tile's in
    the prologue, the next tile's during this tile's output), the tile
    starts with a wait for all loads and a barrier, then reads chunk 0's
    first k-step.  Chunk s reads its second k-step (same stage), waits for
    chunk s + 1's loads, passes the barrier, loads chunk s + 2 into its own
    stage and reads chunk s + 1's first k-step.  The output: a barrier,
    the accumulators written into both stages ([256 tokens][256 features],
    half h in stage h), a barrier, each half read back, a barrier, and that
    half's stage takes the next tile's chunk h.  (The kernel's wait at a
    tile's start leaves the previous tile's last 16 stores pending, which
    follow every load in issue order: for the loads it is the full wait
    modelled here.)  `waits[s]` = chunk s's
    bound; `early_loads` plants loads of chunk s + 2 issued before the
    barrier, `early_next` the next tile's loads issued before the output is
    read back."""
    if waits is None:
        waits = proj_waits(nsteps)
    tr = Trace()
    for w in range(4):
        wv = tr.wave(f"w{w}")
        issued, since, landed = [], {}, {}

        def issue(c):
            issued.append(c)
            since[c] = wv.epoch

        def wait(bound):
            for c in issued[:max(0, len(issued) - bound)]:
                landed.setdefault(c, wv.epoch)

        for c in range(min(stages, nsteps)):
            issue((0, c))
        for tl in range(ntiles):
            wait(0)
            wv.barrier()
            wv.read(("S", 0), (tl, 0))
            for st in range(nsteps):
                wv.read(("S", st % stages), (tl, st))  # the chunk's second k-step
                if waits[st] is not None:
                    if early_loads and st + stages < nsteps:
                        issue((tl, st + stages))
                    wait(waits[st])
                    wv.barrier()
                    if not early_loads and st + stages < nsteps:
                        issue((tl, st + stages))
                    wv.read(("S", (st + 1) % stages), (tl, st + 1))
            more = tl + 1 < ntiles
            wv.barrier()  # every wave's last operand reads are back
            for h in range(2):
                wv.write(("S", h), ("out", tl))
            if more and early_next:
                for h in range(2):
                    issue((tl + 1, h))
            wv.barrier()
            for h in range(2):
                wv.read(("S", h), ("out", tl))
                wv.barrier()
                if more and not early_next:
                    issue((tl + 1, h))
        end = wv.epoch
        for c in issued:
            for e in range(since[c], landed.get(c, end) + 1):
                tr.events.append((e, wv.name, "w", ("S", c[1] % stages), c))
    return tr


def proj_waits(nsteps):
    """The kernel's bounds: every chunk but the last waits for all of its
    loads (none are issued past the next chunk); the last reads nothing."""
    return [0] * (nsteps - 1) + [None]


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
    """Work lists as the kernel derives them: ragged sequence lengths around
    the tile and query-block edges, GQA groups 1, 2 and 4, full causal and
    local windows, and persistent workgroup counts from one to more than a
    round, multiples of 8 or not; the first, a middle and the last
    persistent workgroup and the first and last one-item workgroup."""
    seen = set()
    for S in (1, 31, 33, 64, 100, 257, 600):
        for G in (1, 2, 4):
            for W in (0, 40, 300):
                for units, P in ((1, 1), (3, 1), (3, 2), (2, 3), (5, 8), (4, 16)):
                    # the launcher never runs more persistent workgroups than items
                    P = min(P, -(-S // (32 * (4 // G))) * units)
                    n = forward_grid(S, G, units, P)
                    for wg in sorted({0, P // 2, P - 1, P, n - 1} & set(range(n))):
                        if (S, G, W, units, P, wg) not in seen:
                            seen.add((S, G, W, units, P, wg))
                            yield S, G, W, units, P, wg


def dq_cases():
    """(t_first, ntiles, pair ranges) as the dq kernel derives them: full
    causal (t_first = 0, pair_lo = 0, pair_tiles = the pair's last row tile
    + 1) and windows (t_first even, each pair_lo >= t_first)."""
    for ntiles in range(1, 11):
        for rows_per_pair in (1, 2):  # GQA groups give pairs of 32 or 64... rows per head
            pts = [min(ntiles, (i + 1) * rows_per_pair) for i in range(4)]
            yield 0, ntiles, [(0, max(1, x)) for x in pts]
        for t_first in range(0, ntiles, 2):
            for lo_off in range(0, 3):
                pairs = [(min(ntiles - 1, t_first + lo_off + i // 2), ntiles) for i in range(4)]
                yield t_first, ntiles, pairs


@pytest.mark.parametrize("S,G,W,units,P,wg", list(forward_cases()))
def test_forward_schedule(S, G, W, units, P, wg):
    items = forward_items(S, G, W, units, P, wg)
    assert check(forward_trace(items)) == []


def test_forward_work_lists_cover_every_item_once():
    """The workgroups' lists partition the items, and the odd-round order
    keeps item % 8 == workgroup % 8 when P is a multiple of 8."""
    for S, G, W, units in ((600, 2, 0, 8), (257, 4, 40, 3), (64, 1, 0, 16), (2048, 2, 0, 8)):
        qb_rows = 32 * (4 // G)
        nqb = -(-S // qb_rows)
        nitems = nqb * units
        for P in (1, 3, 8, 16, 24):
            P = min(P, nitems)
            seen = []
            for wg in range(forward_grid(S, G, units, P)):
                items = forward_items(S, G, W, units, P, wg)
                R = nitems // P - 1
                for i in range(len(items)):
                    if R >= 1 and wg < P:
                        off = (P - 8 - (wg & ~7) + (wg & 7) if P % 8 == 0 else P - 1 - wg) \
                            if i & 1 else wg
                        k = i * P + off
                    else:
                        k = R * P + wg - P if R >= 1 else wg
                    if P % 8 == 0 and R >= 1:
                        assert k % 8 == wg % 8
                    seen.append(k)
            assert sorted(seen) == list(range(nitems))


@pytest.mark.parametrize("t_first,ntiles,pairs", list(dq_cases()))
def test_dq_schedule(t_first, ntiles, pairs):
    assert check(dq_trace(t_first, ntiles, pairs)) == []


@pytest.mark.parametrize("early_loads", [False, True])
@pytest.mark.parametrize("ntiles", range(1, 13))
def test_dkv_schedule(ntiles, early_loads):
    # pairs see contiguous runs of query tiles, per head of the group (G = 2:
    # two runs of nq tiles), some pairs none at all
    nq = max(1, ntiles // 2)
    sets = [set(range(ntiles)), {t for t in range(ntiles) if t % nq >= 1},
            {t for t in range(ntiles) if t % nq >= nq - 1}, set()]
    assert check(dkv_trace(ntiles, sets, early_loads)) == []


@pytest.mark.parametrize("nsteps", [4, 8, 16, 32])
@pytest.mark.parametrize("ntiles", [1, 2, 3])
def test_projection_schedule(nsteps, ntiles):
    assert check(proj_trace(nsteps, ntiles=ntiles)) == []


def test_planted_projection_errors_are_caught():
    """A chunk that waits only for its older loads (one chunk still
    pending) reads the next chunk while it may still land; loads of chunk
    s + 2 issued before the barrier store over the stage others still read;
    the next tile's loads issued before the output is read back overwrite
    it."""
    w = proj_waits(16)
    w[5] = 1
    assert any(b[0] == "unordered access" for b in check(proj_trace(16, w)))
    assert any(b[0] == "unordered access" for b in check(proj_trace(16, early_loads=True)))
    assert any(b[0] == "unordered access" for b in check(proj_trace(8, ntiles=2, early_next=True)))


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
    items = forward_items(257, 2, 0, 3, 2, 0)
    bad = check(forward_trace(items, swap_stages=True))
    assert any(b[0] == "register stage" for b in bad)


def test_planted_short_items_are_caught():
    """The loads run three positions ahead and the kernel maps a position past
    an item's end into the next item only, so every item spans at least four
    positions (two would let a load for the item after next fetch a tile of
    the next item instead)."""
    bad = check(forward_trace(forward_items(100, 4, 0, 4, 1, 0, min_len=2)))
    assert any(b[0] == "register stage" for b in bad)
    assert check(forward_trace(forward_items(100, 4, 0, 4, 1, 0, min_len=4))) == []


def test_checker_sees_a_write_beside_a_read():
    tr = Trace()
    a, b = tr.wave("a"), tr.wave("b")
    a.write("X", 0)
    a.barrier(), b.barrier()
    a.write("X", 1)
    b.read("X", 0)
    a.barrier(), b.barrier()
    assert any(x[0] == "unordered access" for x in check(tr))
