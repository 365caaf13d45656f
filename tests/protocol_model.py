"""A CPU model of the two ring protocols, for exhaustive interleaving checks.

Test infrastructure: nothing in the library imports it.  It restates, as
per-wave instruction lists, the schedules that the kernels run:

* single schedule (Croqtile ch.6, "double buffering with swap", with the
  handles rotated over S slots): every wave issues asynchronous loads of its
  share of a tile into ring slot t mod S, waits for its own loads, meets the
  other waves at a workgroup barrier, and reads the slot; on the large
  tile's two-slot ring the barrier is split into a WAR barrier (the slot
  just read is free) and a RAW barrier (the next tile has landed);
* producer/consumer (Croqtile ch.6, "1P1C kernel with events" and the credit
  flow of one stage; Croqtile ch.5, the bootstrap protocol): producers wait
  for the slot's `empty` credit, load their share asynchronously, and add
  one to `full` once the loads have landed;
  consumers seed one `empty` credit per slot, wait for `full`, read the slot
  and add one to `empty`.  Credits are monotonic counters: round r of a slot
  waits for (r + 1) x (the number of waves that add to it).  Consumers that
  read one k32 step ahead (two fragment sets) issue the same credit events in
  the same order and, after their last tile, read the slot after it without
  a credit: data they never use, but a read that no write may overlap.

The explorer runs every interleaving of the waves (and, for asynchronous
loads, every moment at which an issued load may land) by depth-first search
over distinct states, and reports:

* deadlock: some wave cannot finish and nothing can move;
* RAW: a read of slot s for tile t while a share of the slot does not hold
  tile t (not written yet, or overwritten);
* WAR: a write or a landing load into slot s while another wave is reading
  the slot;
* order: a wave that reads tiles other than 0, 1, ..., n_k - 1 in order;
* leftover (producer/consumer): a tile written that no consumer read.

The hazards are the ones the pages name: the new copy must land in the
buffer that is not being read (Croqtile ch.6, swap); a missing bootstrap
credit deadlocks the producer, an early release lets the producer overwrite
a slot still being read, and both roles must run the same trip count
(Croqtile ch.6, credit flow; Croqtile ch.5, bootstrap protocol).
"""
from __future__ import annotations

import dataclasses
import random
from typing import List, Optional

# instruction kinds
WAIT, ADD, WBEGIN, WEND, RBEGIN, REND, ISSUE, WAITLOADS, BARRIER = range(9)


@dataclasses.dataclass
class Result:
    deadlock: bool = False
    raw: bool = False
    war: bool = False
    order: bool = False
    leftover: bool = False
    states: int = 0
    example: str = ""

    @property
    def ok(self) -> bool:
        return not (self.deadlock or self.raw or self.war or self.order or self.leftover)


# ----------------------------------------------------------- programs


def ws_programs(S: int, n_k: int, P: int, C: int, *, bootstrap: bool = True, early_release: bool = False,
                producer_trips: Optional[int] = None, consumer_trips: Optional[int] = None,
                lookahead: int = 0, no_sync: bool = False, lag: Optional[int] = None,
                read_after_last: bool = False, whole_tiles: bool = False, full_per_round: Optional[int] = None,
                publish_before_landing: bool = False):
    """Producer/consumer: P producers, C consumers.

    Shared tiles (whole_tiles=False; the kernel's K-split form): producer p
    issues its share of tile t as an asynchronous load once slot t mod S has
    its `empty` credit, and adds to `full` of tile t - lag after waiting for
    that tile's loads (lag = S - 2, at least 0); the last `lag` tiles are
    completed after the loop.  Consumers wait for P additions per round.

    Whole tiles (whole_tiles=True; the kernel's unsplit form): producer p
    loads tiles p, p + P, ... whole, each once its slot has its `empty`
    credit, and adds to `full` once that tile has landed.  Consumers wait
    for one addition per round (full_per_round overrides the count they
    wait for; publish_before_landing adds to `full` before the wait for the
    loads: both planted mistakes).

    Faults: bootstrap=False drops the consumers' initial `empty` credits;
    early_release adds to `empty` before the slot's reads finish; *_trips
    changes one role's trip count; lookahead=1 lets producers run one round
    ahead of their credits; lag sets another lag; no_sync drops every wait
    and credit.  read_after_last adds the consumers' uncredited read of slot
    n_k mod S after their last release (tile None: checked for WAR only)."""
    pt = n_k if producer_trips is None else producer_trips
    ct = n_k if consumer_trips is None else consumer_trips
    lg = max(S - 2, 0) if lag is None else lag
    progs = []
    if whole_tiles:
        for p in range(P):
            prog = []
            for t in range(p, pt, P):
                s, r = t % S, t // S
                if not no_sync:
                    prog.append((WAIT, "empty", s, C * (r + 1 - lookahead)))
                prog.append((ISSUE, s, t, 0))
                if not no_sync:
                    if publish_before_landing:
                        prog.append((ADD, "full", s))
                        prog.append((WAITLOADS, t))
                    else:
                        prog.append((WAITLOADS, t))
                        prog.append((ADD, "full", s))
            prog.append((WAITLOADS, 10 ** 9))
            progs.append(prog)
        fp = 1 if full_per_round is None else full_per_round
        progs += _consumers(S, ct, C, fp, bootstrap, no_sync, early_release, read_after_last)
        return progs, 1  # one share per slot: the whole tile
    for p in range(P):
        prog = []
        for t in range(pt):
            s, r = t % S, t // S
            if not no_sync:
                prog.append((WAIT, "empty", s, C * (r + 1 - lookahead)))
            prog.append((ISSUE, s, t, p))
            if not no_sync and t >= lg:
                prog.append((WAITLOADS, t - lg))
                prog.append((ADD, "full", (t - lg) % S))
        if not no_sync:
            for t in range(max(pt - lg, 0), pt):
                prog.append((WAITLOADS, t))
                prog.append((ADD, "full", t % S))
        prog.append((WAITLOADS, 10 ** 9))
        progs.append(prog)
    progs += _consumers(S, ct, C, P if full_per_round is None else full_per_round, bootstrap, no_sync,
                        early_release, read_after_last)
    return progs, P  # shares per slot: one per producer


def _consumers(S, ct, C, fp, bootstrap, no_sync, early_release, read_after_last):
    """C consumers: seed every slot's `empty`, then per tile wait for fp
    additions to `full` per round, read the slot, release it."""
    progs = []
    for c in range(C):
        prog = []
        if bootstrap and not no_sync:
            for s in range(S):
                prog.append((ADD, "empty", s))
        for t in range(ct):
            s, r = t % S, t // S
            if not no_sync:
                prog.append((WAIT, "full", s, fp * (r + 1)))
            if early_release and not no_sync:
                prog.append((ADD, "empty", s))
            prog.append((RBEGIN, s, t))
            prog.append((REND, s, t))
            if not early_release and not no_sync:
                prog.append((ADD, "empty", s))
        if read_after_last and ct > 0:
            prog.append((RBEGIN, ct % S, None))
            prog.append((REND, ct % S, None))
        progs.append(prog)
    return progs


def swap_programs(S: int, n_k: int, W: int, *, skip_barrier: bool = False, skip_wait: bool = False,
                  refill_before_barrier: bool = False, split_sync: bool = False, skip_raw_barrier: bool = False):
    """Single schedule with W waves, as the kernels run it.

    Each wave's share of a tile is two halves (shares 2w and 2w + 1), issued
    as asynchronous loads that land later.  S = 1: load, wait, barrier, read,
    barrier.  S >= 2: the prologue issues tiles 0 .. S-1; the wave reads
    tile t, waits for its own loads of tile t+1, meets the others at the
    barrier and then issues both halves of tile t+S into tile t's slot.
    Loads of tiles at or past n_k are issued too (they read zeros in the
    kernel); before the epilogue the wave waits for all of its loads.

    Faults: skip_barrier drops the per-tile barrier; skip_wait drops the
    wait for the wave's own loads; refill_before_barrier issues the refill
    of tile t's slot before the barrier instead of after it.

    split_sync (S = 2, the large tile's two-slot ring): a tile's reads are
    two parts, its first k32 step (read at the end of the previous tile)
    and its second (read at the start of its own).  After the second part
    a WAR barrier frees the tile's slot and the wave issues both halves of
    tile t+2 into it; then it waits for its own loads of tile t+1, meets
    the others at a RAW barrier and reads tile t+1's first part.  The last
    tile also reads the first part of tile n_k (loads of tiles past the end
    are issued too; the data is never used).  Only the second part of a
    read counts as reading the tile.  Faults: skip_barrier drops the WAR
    barrier, skip_raw_barrier the RAW barrier, skip_wait the wait before
    it, refill_before_barrier issues the refill before the WAR barrier."""
    if split_sync:
        return _split_sync_programs(n_k, W, skip_barrier, skip_wait, refill_before_barrier, skip_raw_barrier)
    progs = []
    for w in range(W):
        a, b = 2 * w, 2 * w + 1
        prog = []
        nb = 0
        if S == 1:
            for t in range(n_k):
                prog += [(ISSUE, 0, t, a), (ISSUE, 0, t, b)]
                if not skip_wait:
                    prog.append((WAITLOADS, t))
                if not skip_barrier:
                    prog.append((BARRIER, nb)); nb += 1
                prog += [(RBEGIN, 0, t), (REND, 0, t)]
                if not skip_barrier:
                    prog.append((BARRIER, nb)); nb += 1
            progs.append(prog)
            continue
        for j in range(S):
            prog += [(ISSUE, j % S, j, a), (ISSUE, j % S, j, b)]
        if not skip_wait:
            prog.append((WAITLOADS, 0))
        if not skip_barrier:
            prog.append((BARRIER, nb)); nb += 1
        for t in range(n_k):
            s = t % S
            prog += [(RBEGIN, s, t), (REND, s, t)]
            if t + 1 < n_k:
                refill = [(ISSUE, (t + S) % S, t + S, a), (ISSUE, (t + S) % S, t + S, b)]
                if refill_before_barrier:
                    prog += refill
                if not skip_wait:
                    prog.append((WAITLOADS, t + 1))
                if not skip_barrier:
                    prog.append((BARRIER, nb)); nb += 1
                if not refill_before_barrier:
                    prog += refill
        prog.append((WAITLOADS, 10 ** 9))  # the epilogue waits for every load
        progs.append(prog)
    return progs, 2 * W


def _split_sync_programs(n_k, W, skip_war, skip_wait, refill_before_war, skip_raw):
    progs = []
    for w in range(W):
        a, b = 2 * w, 2 * w + 1
        nb = 0
        prog = [(ISSUE, 0, 0, a), (ISSUE, 0, 0, b), (ISSUE, 1, 1, a), (ISSUE, 1, 1, b)]
        if not skip_wait:
            prog.append((WAITLOADS, 0))
        prog.append((BARRIER, nb)); nb += 1
        prog += [(RBEGIN, 0, 0), (REND, 0, 0, False)]  # first part of tile 0
        for t in range(n_k):
            s = t % 2
            prog += [(RBEGIN, s, t), (REND, s, t)]  # second part of tile t
            refill = [(ISSUE, s, t + 2, a), (ISSUE, s, t + 2, b)]
            if refill_before_war:
                prog += refill
            if not skip_war:
                prog.append((BARRIER, nb)); nb += 1
            if not refill_before_war:
                prog += refill
            if not skip_wait:
                prog.append((WAITLOADS, t + 1))
            if not skip_raw:
                prog.append((BARRIER, nb)); nb += 1
            prog += [(RBEGIN, (t + 1) % 2, t + 1), (REND, (t + 1) % 2, t + 1, False)]  # first part of tile t+1
        prog.append((WAITLOADS, 10 ** 9))
        progs.append(prog)
    return progs, 2 * W


# ----------------------------------------------------------- explorer


class _Explorer:
    def __init__(self, progs, shares: int, S: int, n_k: int, readers: List[int], max_states: int,
                 check_leftover: bool = False):
        self.progs = progs
        self.shares = shares
        self.S = S
        self.n_k = n_k
        self.readers = readers  # waves whose reads must cover 0..n_k-1 in order
        self.max_states = max_states
        self.res = Result()
        self.seen = set()
        self.n_waves = len(progs)
        self.check_leftover = check_leftover

    # state: (pcs, counters, slot tags, shares being written, waves reading,
    #         loads in flight, tiles read per wave, loads issued per wave)
    def initial(self):
        pcs = tuple(0 for _ in self.progs)
        ctr = (tuple(0 for _ in range(self.S)), tuple(0 for _ in range(self.S)))
        tags = tuple(tuple(None for _ in range(self.shares)) for _ in range(self.S))
        writing = tuple(tuple(None for _ in range(self.shares)) for _ in range(self.S))
        reading = tuple(frozenset() for _ in range(self.S))  # waves reading the slot
        inflight = frozenset()  # (wave, seq, slot, tile, share)
        log = tuple(() for _ in self.progs)
        issued = tuple(0 for _ in self.progs)
        return (pcs, ctr, tags, writing, reading, inflight, log, issued)

    def flag(self, kind: str, what: str):
        setattr(self.res, kind, True)
        if not self.res.example:
            self.res.example = f"{kind}: {what}"

    def moves(self, st):
        """Enabled moves: ('wave', w) or ('land', item)."""
        pcs, ctr, tags, writing, reading, inflight, log, issued = st
        out = []
        for w, prog in enumerate(self.progs):
            pc = pcs[w]
            if pc >= len(prog):
                continue
            ins = prog[pc]
            k = ins[0]
            if k == WAIT:
                which = 0 if ins[1] == "full" else 1
                if ctr[which][ins[2]] < ins[3]:
                    continue
            elif k == WAITLOADS:
                # all of this wave's loads of tiles <= ins[1] have landed
                if any(it[0] == w and it[3] <= ins[1] for it in inflight):
                    continue
            elif k == BARRIER:
                # enabled when every wave is at this barrier (or finished)
                ok = True
                for v, pv in enumerate(self.progs):
                    if pcs[v] >= len(pv) or pv[pcs[v]] != (BARRIER, ins[1]):
                        ok = False
                        break
                if not ok:
                    continue
            out.append(("wave", w))
        for it in inflight:
            out.append(("land", it))
        return out

    def step(self, st, mv):
        pcs, ctr, tags, writing, reading, inflight, log, issued = st
        pcs = list(pcs)
        if mv[0] == "land":
            w, seq, s, t, share = mv[1]
            if reading[s]:
                self.flag("war", f"load of tile {t} landed in slot {s} while it was read")
            tags = _set2(tags, s, share, t)
            inflight = inflight - {mv[1]}
            return (tuple(pcs), ctr, tags, writing, reading, inflight, log, issued)
        w = mv[1]
        ins = self.progs[w][pcs[w]]
        k = ins[0]
        if k == BARRIER:
            # all waves pass together
            for v in range(self.n_waves):
                pcs[v] += 1
            return (tuple(pcs), ctr, tags, writing, reading, inflight, log, issued)
        pcs[w] += 1
        if k == ADD:
            which = 0 if ins[1] == "full" else 1
            c = list(ctr)
            row = list(c[which])
            row[ins[2]] += 1
            c[which] = tuple(row)
            ctr = tuple(c)
        elif k == WBEGIN:
            _, s, t, share = ins
            if reading[s]:
                self.flag("war", f"write of tile {t} into slot {s} while it was read")
            writing = _set2(writing, s, share, t)
            tags = _set2(tags, s, share, None)
        elif k == WEND:
            _, s, t, share = ins
            writing = _set2(writing, s, share, None)
            tags = _set2(tags, s, share, t)
        elif k == RBEGIN:
            _, s, t = ins
            if t is not None and (any(x != t for x in tags[s]) or any(x is not None for x in writing[s])):
                self.flag("raw", f"read of tile {t} from slot {s} holding {tags[s]}")
            reading = _set1(reading, s, reading[s] | {w})
        elif k == REND:
            s, t = ins[1], ins[2]
            if t is not None and (any(x != t for x in tags[s]) or any(x is not None for x in writing[s])):
                self.flag("raw", f"slot {s} changed while tile {t} was read")
            reading = _set1(reading, s, reading[s] - {w})
            # a read of data that is never used, or the first part of a tile
            # read in two parts, is no tile read
            if t is not None and (len(ins) < 4 or ins[3]):
                log = _set1(log, w, log[w] + (t,))
        elif k == ISSUE:
            _, s, t, share = ins
            iss = list(issued)
            iss[w] += 1
            issued = tuple(iss)
            inflight = inflight | {(w, issued[w], s, t, share)}
        return (tuple(pcs), ctr, tags, writing, reading, inflight, log, issued)

    def finished(self, st):
        pcs = st[0]
        return all(pcs[w] >= len(p) for w, p in enumerate(self.progs)) and not st[5]

    def check_final(self, st):
        log = st[6]
        for w in self.readers:
            if log[w] != tuple(range(self.n_k)):
                self.flag("order", f"wave {w} read tiles {log[w]}")
        if self.check_leftover:
            read = set().union(*(set(log[w]) for w in self.readers))
            for row in st[2]:
                for t in row:
                    if t is not None and t not in read:
                        self.flag("leftover", f"tile {t} written but never read")

    def run(self, exhaustive: bool = True, walks: int = 0, rng: Optional[random.Random] = None,
            stop_at_first: bool = False):
        init = self.initial()
        if exhaustive:
            stack = [init]
            self.seen.add(init)
            while stack and not (stop_at_first and not self.res.ok):
                st = stack.pop()
                mv = self.moves(st)
                if not mv:
                    if self.finished(st):
                        self.check_final(st)
                    else:
                        self.flag("deadlock", f"stuck at pcs {st[0]}")
                    continue
                for m in mv:
                    nxt = self.step(st, m)
                    if nxt not in self.seen:
                        if len(self.seen) >= self.max_states:
                            raise RuntimeError("state space larger than the explorer's limit")
                        self.seen.add(nxt)
                        stack.append(nxt)
            self.res.states = len(self.seen)
        for _ in range(walks):
            st = init
            while True:
                mv = self.moves(st)
                if not mv:
                    if self.finished(st):
                        self.check_final(st)
                    else:
                        self.flag("deadlock", f"stuck at pcs {st[0]}")
                    break
                st = self.step(st, rng.choice(mv))
            self.res.states += 1
        return self.res


def _set1(tup, i, v):
    l = list(tup)
    l[i] = v
    return tuple(l)


def _set2(tup, i, j, v):
    row = list(tup[i])
    row[j] = v
    return _set1(tup, i, tuple(row))


def check_ws(S, n_k, P, C, *, exhaustive=True, walks=0, seed=0, max_states=2_000_000, stop_at_first=False,
             **faults) -> Result:
    """Explores the producer/consumer protocol (faults: see ws_programs)."""
    progs, shares = ws_programs(S, n_k, P, C, **faults)
    readers = list(range(P, P + C))
    ex = _Explorer(progs, shares, S, n_k, readers, max_states, check_leftover=True)
    return ex.run(exhaustive, walks, random.Random(seed), stop_at_first)


def check_swap(S, n_k, W, *, exhaustive=True, walks=0, seed=0, max_states=2_000_000, stop_at_first=False,
               **faults) -> Result:
    """Explores the single schedule (faults: see swap_programs)."""
    progs, shares = swap_programs(S, n_k, W, **faults)
    ex = _Explorer(progs, shares, S, n_k, list(range(W)), max_states)
    return ex.run(exhaustive, walks, random.Random(seed), stop_at_first)
