"""The ring protocols in a CPU model (no GPU): both schedules are free of
deadlock and slot hazards over every interleaving for small sizes, and each
protocol mistake the pages warn about is caught.

Pins: the pages' own statements (Croqtile ch.6, swap: the new copy lands in
the buffer not being read; credit flow of one stage: both roles must run
the same number of iterations, the producer waits for `empty` and the
consumer for `full`; Croqtile ch.5, bootstrap protocol: without the initial
`empty` credits the producer waits forever; releasing before the reads are
done lets the producer overwrite a slot in use), and the kernels' own wait
constants, checked against the model's wait points.
"""
import os

import pytest

from protocol_model import ISSUE, WAITLOADS, check_swap, check_ws, swap_programs

KERNELS = os.path.join(os.path.dirname(__file__), "..", "software_pipelined_tiled_pipeline_amd", "csrc", "kernels.hpp")


# ------------------------------------------------------ correct schedules

@pytest.mark.parametrize("S,n_k,W", [(1, 0, 2), (1, 1, 2), (1, 3, 2), (1, 4, 3),
                                     (2, 0, 2), (2, 1, 2), (2, 2, 2), (2, 3, 2), (2, 6, 2), (2, 3, 3),
                                     (3, 1, 2), (3, 2, 2), (3, 4, 2), (4, 1, 2), (4, 3, 2), (4, 4, 2)])
def test_swap_schedule_safe_in_every_interleaving(S, n_k, W):
    r = check_swap(S, n_k, W)
    assert r.ok, r.example
    assert r.states > 0


@pytest.mark.parametrize("S,n_k,W", [(2, 12, 2), (3, 10, 3), (4, 9, 2), (4, 7, 4)])
def test_swap_schedule_safe_on_random_interleavings(S, n_k, W):
    r = check_swap(S, n_k, W, exhaustive=False, walks=300, seed=S * 100 + n_k)
    assert r.ok, r.example


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("n_k", [0, 1, 2, 3, 5, 6])
@pytest.mark.parametrize("P,C", [(1, 1), (1, 2), (2, 2), (1, 4)])
def test_ws_protocol_safe_in_every_interleaving(S, n_k, P, C):
    if P * C >= 4 and n_k >= 5 and S >= 3:
        pytest.skip("covered by the random walks below")
    r = check_ws(S, n_k, P, C)
    assert r.ok, r.example


@pytest.mark.parametrize("S,n_k,P,C", [(4, 16, 2, 8), (2, 20, 2, 8), (3, 12, 2, 4), (1, 8, 2, 8), (4, 16, 4, 8)])
def test_ws_protocol_safe_on_random_interleavings(S, n_k, P, C):
    # the kernels' own role counts: 2 producers and 8 consumers (256 x 256
    # tiles), 2 and 4 (128 x 128 tiles)
    r = check_ws(S, n_k, P, C, exhaustive=False, walks=200, seed=S + n_k)
    assert r.ok, r.example


def test_kernel_wait_constants_match_the_model():
    # nt_swap_kernel waits with s_waitcnt vmcnt(N) for static N: (S-2)*PER
    # before each barrier and (S-1)*PER in the prologue, PER loads per wave
    # and tile.  In the model one ISSUE is half of them, so at each wait for
    # "tiles <= u landed" exactly 2(S-2) issues (2(S-1) in the prologue) of
    # later tiles may still be in flight, and every issue of a tile <= u
    # comes before them (loads complete in order).
    for S in (2, 3, 4):
        for n_k in (1, 2, 5, 9):
            prog = swap_programs(S, n_k, 1)[0][0]
            waits = [i for i, ins in enumerate(prog) if ins[0] == WAITLOADS and ins[1] < 10 ** 9]
            assert waits
            for j, i in enumerate(waits):
                u = prog[i][1]
                issues = [ins for ins in prog[:i] if ins[0] == ISSUE]
                later = [ins for ins in issues if ins[2] > u]
                expect = 2 * (S - 1) if j == 0 else 2 * (S - 2)
                assert len(later) == expect, (S, n_k, u)
                first_later = next((k for k, ins in enumerate(issues) if ins[2] > u), len(issues))
                assert all(ins[2] > u for ins in issues[first_later:])
    src = open(KERNELS).read()
    assert "wait_vmcnt<(S - 1) * PER>();  // tile 0 landed" in src
    assert "wait_vmcnt<(S - 2) * PER>();  // tile t+1 landed" in src


def test_reading_ahead_consumer_matches_the_model():
    # the two-fragment-set consumer of nt_ws_kernel issues, per tile, the
    # release of slot s after its reads have landed, then the wait for `full`
    # of the next tile, then the reads of the next tile's first step: the
    # order that ws_programs(read_after_last=True) explores.  The counter it
    # waits on may be read earlier in the tile: counters only grow, so that
    # value is a lower bound, and the wait is skipped only when even the
    # lower bound has reached the target (the model's wait succeeds then too)
    src = open(KERNELS).read()
    body = src[src.index("if constexpr (kTwoSets) {"):src.index("w.settle();", src.index("if constexpr (kTwoSets) {"))]
    early = body.index("const uint32_t next = credit_load(&full[s1]);")
    release = body.index("wait_lgkmcnt0();  // the last fragment reads of slot s are done")
    trigger = body.index("credit_trigger(&empty[s]);", release)
    check = body.index("if (t + 1 < n_k && __builtin_amdgcn_readfirstlane(next) < target)", trigger)
    wait_next = body.index("credit_wait(&full[s1], target", check)
    read_next = body.index("lane_a(s1), lane_b(s1), 0, chunk", wait_next)
    assert early < release < trigger < check < wait_next < read_next
    assert "next" not in body[early + 60:check]  # the early value is not used before the check
    # the first tile waits for its credit before any read
    assert body.index("credit_wait(&full[0]") < body.index("W::read_frags(f[0]")


# ------------------------------------------------------ planted mistakes

@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("n_k", [1, 2, 3, 5])
@pytest.mark.parametrize("P,C", [(1, 1), (1, 2), (2, 2)])
def test_ws_consumers_reading_ahead_safe_in_every_interleaving(S, n_k, P, C):
    # consumers with two fragment sets (the 128 x 128 tile: 2 producers, 4
    # consumers) keep the credit events in order and, after their last tile,
    # read the slot after it with no credit
    if P * C >= 4 and n_k >= 5 and S >= 3:
        pytest.skip("covered by the random walks below")
    r = check_ws(S, n_k, P, C, read_after_last=True)
    assert r.ok, r.example


@pytest.mark.parametrize("S,n_k", [(4, 16), (3, 12), (2, 9), (1, 8)])
def test_ws_consumers_reading_ahead_safe_on_random_interleavings(S, n_k):
    r = check_ws(S, n_k, 2, 4, exhaustive=False, walks=200, seed=S + n_k, read_after_last=True)
    assert r.ok, r.example


def test_read_after_the_last_tile_is_checked_for_overwrites():
    # a producer running one tile more than the consumers refills the slot
    # that the consumers read after their last tile
    r = check_ws(2, 3, 1, 1, read_after_last=True, producer_trips=4)
    assert r.war, r.example


def test_missing_bootstrap_deadlocks():
    for S, P, C in [(1, 1, 1), (2, 1, 2), (4, 2, 2)]:
        r = check_ws(S, 4, P, C, bootstrap=False)
        assert r.deadlock and not r.raw and not r.war


def test_release_before_reads_finish_lets_the_producer_overwrite():
    for S in (1, 2, 3):
        r = check_ws(S, S + 2, 1, 2, early_release=True)
        assert r.war


def test_producer_running_one_round_ahead_overwrites():
    for S in (1, 2, 3):
        r = check_ws(S, S + 2, 1, 2, lookahead=1)
        assert r.raw or r.war


@pytest.mark.parametrize("who,trips,expect", [
    ("consumer_trips", 3, "order"),     # a tile is left unread
    ("consumer_trips", 5, "deadlock"),  # a consumer waits for a tile never produced
    ("producer_trips", 3, "deadlock"),
    ("producer_trips", 5, "leftover"),  # a tile produced that nobody reads
    ("producer_trips", 8, "deadlock"),  # ... and past the ring's slack the producer blocks
])
def test_mismatched_trip_counts(who, trips, expect):
    r = check_ws(2, 4, 1, 2, **{who: trips})
    assert getattr(r, expect), r.example
    assert not r.ok


@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_producer_lag(S):
    # full of tile t may trail its loads by up to S - 1 tiles; at S tiles the
    # producer waits for a slot the consumers can only free after that full
    for lag in range(S):
        assert check_ws(S, S + 2, 1, 2, lag=lag, exhaustive=S < 4, walks=0 if S < 4 else 300).ok
    r = check_ws(S, S + 2, 1, 2, lag=S)
    assert r.deadlock


def test_no_synchronisation_races():
    assert not check_ws(2, 4, 1, 2, no_sync=True).ok
    assert not check_swap(2, 3, 2, skip_barrier=True, skip_wait=True, stop_at_first=True).ok


@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_swap_without_barrier_or_wait_is_caught(S):
    n_k = S + 1
    assert check_swap(S, n_k, 2, skip_barrier=True, stop_at_first=True).raw
    assert check_swap(S, n_k, 2, skip_wait=True, stop_at_first=True).raw


@pytest.mark.parametrize("S", [2, 3, 4])
def test_refill_before_the_barrier_is_caught(S):
    # the refill of tile t's slot issued before every wave has finished
    # reading tile t: the copy may land in the buffer still being read
    r = check_swap(S, S + 1, 2, refill_before_barrier=True, stop_at_first=True)
    assert r.raw or r.war


# ------------------------------------------- whole tiles, one producer each

@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("n_k", [0, 1, 2, 3, 5, 6])
@pytest.mark.parametrize("P,C", [(1, 1), (2, 1), (2, 2), (3, 1)])
def test_ws_whole_tiles_safe_in_every_interleaving(S, n_k, P, C):
    # producer p loads tiles p, p + P, ... whole and publishes each once it
    # has landed; consumers wait for one addition to `full` per round
    if P * C >= 4 and n_k >= 5 and S >= 3:
        pytest.skip("covered by the random walks below")
    r = check_ws(S, n_k, P, C, whole_tiles=True)
    assert r.ok, r.example
    r = check_ws(S, n_k, P, C, whole_tiles=True, read_after_last=True)
    assert r.ok, r.example


@pytest.mark.parametrize("S,n_k,P,C", [(4, 16, 2, 8), (3, 12, 2, 8), (4, 9, 2, 4), (3, 10, 2, 4), (1, 8, 2, 8), (4, 16, 4, 8),
                                       (3, 12, 4, 8)])
def test_ws_whole_tiles_safe_on_random_interleavings(S, n_k, P, C):
    # the kernels' role counts (2 producers / 8 consumers, 2 / 4), with more
    # producers than slots as well (S = 1 with two, S = 3 with four)
    r = check_ws(S, n_k, P, C, whole_tiles=True, exhaustive=False, walks=200, seed=S * 7 + n_k)
    assert r.ok, r.example
    r = check_ws(S, n_k, P, C, whole_tiles=True, read_after_last=True, exhaustive=False, walks=100, seed=n_k)
    assert r.ok, r.example


def test_whole_tiles_waiting_for_every_producer_deadlocks():
    # consumers that still wait for P additions per round never see them
    r = check_ws(2, 3, 2, 1, whole_tiles=True, full_per_round=2, stop_at_first=True)
    assert r.deadlock, r.example


def test_whole_tiles_published_before_landing_is_caught():
    r = check_ws(2, 3, 2, 1, whole_tiles=True, publish_before_landing=True, stop_at_first=True)
    assert r.raw, r.example


def test_kernel_whole_tile_producer_matches_the_model():
    # the unsplit nt_ws_kernel's producer: tiles p, p + P, ... whole, wait
    # for the slot's `empty`, load, wait for every load of the tile, then
    # one addition to `full`; consumers wait for one addition per round
    src = open(KERNELS).read()
    body = src[src.index("if constexpr (kWholeTiles) {"):src.index("} else {", src.index("if constexpr (kWholeTiles) {"))]
    loop = body.index("for (int t = wave - C; t < n_k; t += P) {")
    wait = body.index("credit_wait(&empty[s], (uint32_t)C * ((uint32_t)(t / S) + 1u)", loop)
    load = body.index("ld.template load<Loader::INSTR>(slot_ptr(s), t, 0, lane);", wait)
    landed = body.index("wait_vmcnt<0>();  // tile t landed", load)
    publish = body.index("credit_trigger(&full[s]);", landed)
    assert loop < wait < load < landed < publish
    assert "constexpr int FP = kWholeTiles ? 1 : P;" in src
    assert "constexpr bool kWholeTiles = !SPLIT && Loader::INSTR < 64;" in src


# ------------------------------------------- single schedule, split barriers

@pytest.mark.parametrize("n_k", [0, 1, 2, 3, 5])
@pytest.mark.parametrize("W", [2, 3])
def test_split_sync_schedule_safe_in_every_interleaving(n_k, W):
    # the two-slot ring of the large tile with a WAR and a RAW barrier per tile
    r = check_swap(2, n_k, W, split_sync=True)
    assert r.ok, r.example
    assert r.states > 0


@pytest.mark.parametrize("n_k,W", [(12, 2), (9, 4)])
def test_split_sync_schedule_safe_on_random_interleavings(n_k, W):
    # W = 4: the kernel's own wave count
    r = check_swap(2, n_k, W, split_sync=True, exhaustive=False, walks=250, seed=n_k)
    assert r.ok, r.example


@pytest.mark.parametrize("fault", ["skip_barrier", "skip_raw_barrier", "skip_wait", "refill_before_barrier"])
def test_split_sync_mistakes_are_caught(fault):
    # skip_barrier drops the WAR barrier: a refill lands while another wave
    # still reads the tile's second part; the RAW barrier or the wait before
    # it dropped: a wave reads a tile another wave's loads have not filled
    r = check_swap(2, 3, 2, split_sync=True, stop_at_first=True, **{fault: True})
    assert r.raw or r.war, r.example


def test_kernel_split_sync_wait_constants_match_the_model():
    # The two-barrier kernel waits with vmcnt(PER) in the prologue and before
    # each RAW barrier: one tile's loads (2 issues in the model) may still be
    # in flight, and every issue of an earlier tile comes before them.
    for n_k in (1, 2, 5, 9):
        prog = swap_programs(2, n_k, 1, split_sync=True)[0][0]
        waits = [i for i, ins in enumerate(prog) if ins[0] == WAITLOADS and ins[1] < 10 ** 9]
        assert len(waits) == n_k + 1
        for i in waits:
            u = prog[i][1]
            issues = [ins for ins in prog[:i] if ins[0] == ISSUE]
            later = [ins for ins in issues if ins[2] > u]
            assert len(later) == 2, (n_k, u)
            first_later = next(k for k, ins in enumerate(issues) if ins[2] > u)
            assert all(ins[2] > u for ins in issues[first_later:])
    src = open(KERNELS).read()
    assert "wait_vmcnt<PER>();  // tile 0 landed" in src
    assert "wait_vmcnt<PER>();  // still in flight: the PER loads of tile t+2" in src
