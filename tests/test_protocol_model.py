"""Pins for the protocol oracle (CPU only).

The brute-force checkers must accept the protocol as the pages state it and
reject each mutant that drops one of its safety rules (page "arx.cu":
protocol comment on parity buffers and in-order posting, the comment on
separate per-phase counters, and the go wait; page "triton_barrier.py":
send_signal / wait_signal CAS semantics and the zero-filled pad). The
sequential single-GPU model is pinned by closed-form final states.
"""
import numpy as np
import pytest

from oracle import protocol as P
from oracle import reduce as R
from signal_pad_sync_amd import workloads as WL

SIZES = [(2, 1, 4), (2, 2, 3), (3, 1, 3), (3, 2, 2), (4, 1, 2)]


@pytest.mark.parametrize("W,G,S", SIZES)
def test_protocol_safe_and_live(W, G, S):
    r = P.check_protocol(W, G, S)
    assert r.ok, r.violation
    assert r.finals == 1      # every run ends in the same final state


@pytest.mark.parametrize("mutant", ["M1", "M2", "M3", "M4", "M5"])
def test_each_protocol_mutant_is_caught(mutant):
    # at least one small configuration must expose every mutant
    found = [P.check_protocol(W, G, S, mutant=mutant) for W, G, S in [(2, 2, 3), (3, 2, 2)]]
    assert any(not r.ok for r in found), mutant
    assert all(r.violation for r in found if not r.ok)


def test_mutant_kinds():
    """Each mutant fails the way the page says it would."""
    assert "stale" in P.check_protocol(2, 1, 3, mutant="M1").violation   # skipped seq -> stale data
    assert "stale" in P.check_protocol(2, 1, 3, mutant="M2").violation   # one buffer -> overwritten data
    assert "stale" in P.check_protocol(2, 1, 3, mutant="M3").violation   # flag before data
    assert P.check_protocol(2, 2, 3, mutant="M4").violation               # shared counter
    assert "stale" in P.check_protocol(2, 2, 3, mutant="M5").violation   # no go wait


@pytest.mark.parametrize("W,G,S,C", [(2, 2, 3, 1), (2, 3, 2, 1), (2, 3, 2, 2), (3, 2, 2, 1), (2, 4, 2, 2)])
def test_protocol_with_fewer_copying_workgroups(W, G, S, C):
    """The kernel's variant: only the first C of G workgroups copy (each a
    stride of C workgroups' slices) and count arrival; the publish comes
    with the C-th arrival and every workgroup still waits for go."""
    r = P.check_protocol(W, G, S, copiers=C)
    assert r.ok, r.violation
    assert r.finals == 1


def test_publish_before_the_last_copier_is_caught():
    """M6: publishing at the (C-1)-th arrival lets the proxy send a slice
    the last copier has not written; caught with C = G and with C < G."""
    for W, G, S, C in [(2, 2, 3, 2), (2, 3, 2, 2), (2, 4, 2, 2)]:
        r = P.check_protocol(W, G, S, mutant="M6", copiers=C)
        assert not r.ok and "stale" in r.violation, (W, G, S, C)
    with pytest.raises(ValueError):
        P.check_protocol(2, 2, 2, copiers=3)


@pytest.mark.parametrize("W,G,S,C", [(2, 1, 4, None), (2, 2, 3, None), (3, 1, 3, None), (3, 2, 2, None),
                                     (4, 1, 2, None), (2, 2, 3, 1), (2, 3, 2, 2), (3, 2, 2, 1)])
def test_protocol_with_early_finish(W, G, S, C):
    """The kernel's order: workgroups other than 0 count themselves finished
    once they have read the seq and passed the arrival step, workgroup 0 once
    it has seen the flags. Still safe and live, counters zero at every kernel
    end, and the finished seq is recorded only after workgroup 0's flag wait."""
    r = P.check_protocol(W, G, S, copiers=C, early_finish=True)
    assert r.ok, r.violation
    assert r.finals == 1


def test_early_finish_mutants_are_caught():
    """M7: workgroup 0 counting itself finished before its flag wait records
    the seq as finished before the flags came. M8: a workgroup counting
    itself finished before reading the seq can read the next call's seq and
    reduce stale data (or wedge the protocol)."""
    for W, G, S, C in [(2, 2, 3, None), (2, 2, 2, 1), (2, 3, 2, 2)]:
        m7 = P.check_protocol(W, G, S, copiers=C, early_finish=True, mutant="M7")
        assert not m7.ok and "before workgroup 0 saw its flags" in m7.violation, (W, G, S, C)
        m8 = P.check_protocol(W, G, S, copiers=C, early_finish=True, mutant="M8")
        assert not m8.ok, (W, G, S, C)
    with pytest.raises(ValueError):
        P.check_protocol(2, 2, 2, mutant="M7")


@pytest.mark.parametrize("W,G,S,C,early", [(2, 2, 3, None, False), (2, 3, 2, 1, False), (3, 2, 2, None, False),
                                           (2, 2, 3, None, True), (2, 3, 2, None, True), (2, 3, 2, 1, True),
                                           (3, 2, 1, None, True)])
def test_protocol_with_poll_workgroup(W, G, S, C, early):
    """The kernel's grid, at every size (G = 2 is its smallest: the poll
    workgroup and one reducing workgroup): workgroup 0 only waits for the
    flags (possibly before any arrival, when a peer is ahead), gives
    go and counts itself finished; workgroups 1 .. G-1 hold the slices, the
    first C of them copy. Checked as the kernel runs it, with the poll
    workgroup's own arrival from a second wave (poll_arrives), with go held
    back until this rank's publish as well (the rule past 4 vectors per
    copying thread), and without that arrival. Safe, live, counters zero at
    every kernel end, and the finished seq recorded only after the flag
    wait."""
    for kw in (dict(poll_arrives=True), dict(poll_arrives=True, go_after_publish=True), {}):
        r = P.check_protocol(W, G, S, copiers=C, early_finish=early, poller=True, **kw)
        assert r.ok, (kw, r.violation)
        assert r.finals == 1, kw


def test_poll_workgroup_mutants_are_caught():
    """Every mutant still fails with a poll workgroup and its arrival wave;
    M9 (go on this rank's own publish, the published word, instead of the
    peers' flags) reduces stale data, with or without a poll workgroup: the
    published word can only say when to poll. M10 (the poll workgroup counts
    itself finished before its arrival wave has arrived) lets that wave read
    the next seq, arrive for the next call and publish it before its copies:
    stale data."""
    for kw in (dict(poll_arrives=True), {}):
        for mutant in ["M1", "M2", "M3", "M4", "M5", "M9"]:
            found = [P.check_protocol(W, G, S, mutant=mutant, poller=True, **kw) for W, G, S in [(2, 2, 3), (2, 3, 2)]]
            assert all(not r.ok and r.violation for r in found), (mutant, kw)
        for W, G, S, C in [(2, 3, 2, 2), (2, 3, 3, 2)]:
            r = P.check_protocol(W, G, S, mutant="M6", copiers=C, poller=True, **kw)
            assert not r.ok and "stale" in r.violation, (W, G, S, C, kw)
        for W, G, S, C in [(2, 2, 3, None), (2, 3, 2, 1), (2, 3, 2, 2)]:
            m7 = P.check_protocol(W, G, S, copiers=C, early_finish=True, mutant="M7", poller=True, **kw)
            assert not m7.ok and "before workgroup 0 saw its flags" in m7.violation, (W, G, S, C, kw)
            m8 = P.check_protocol(W, G, S, copiers=C, early_finish=True, mutant="M8", poller=True, **kw)
            assert not m8.ok, (W, G, S, C, kw)
    for poller in (False, True):
        assert "stale" in P.check_protocol(2, 2, 3, mutant="M9", poller=poller).violation
    # M6 with a single copier: the poll workgroup's arrival makes two
    r = P.check_protocol(2, 2, 3, mutant="M6", poller=True, poll_arrives=True)
    assert not r.ok and "stale" in r.violation
    for W, G, S, C in [(2, 2, 3, None), (2, 3, 2, 1)]:
        for early in (False, True):
            m10 = P.check_protocol(W, G, S, copiers=C, early_finish=early, mutant="M10", poller=True,
                                   poll_arrives=True)
            assert not m10.ok and "stale" in m10.violation, (W, G, S, C, early)
    with pytest.raises(ValueError):
        P.check_protocol(2, 1, 2, poller=True)          # no reducing workgroup
    with pytest.raises(ValueError):
        P.check_protocol(2, 3, 2, copiers=3, poller=True)
    with pytest.raises(ValueError):
        P.check_protocol(2, 2, 2, poll_arrives=True)    # an arrival wave needs a poll workgroup


@pytest.mark.parametrize("W,K", [(2, 1), (2, 3), (2, 4), (3, 2), (3, 3)])
def test_barrier_safe_live_and_zero(W, K):
    r = P.check_barrier(W, K)
    assert r.ok, r.violation
    assert r.finals == 1


def test_barrier_mutants_are_caught():
    b1 = P.check_barrier(2, 2, mutant="B1")
    assert not b1.ok and "deadlock" in b1.violation       # lost signal
    b2 = P.check_barrier(2, 2, mutant="B2")
    assert not b2.ok and "not zero" in b2.violation       # pad left dirty
    assert not P.check_barrier(3, 2, mutant="B1").ok
    assert not P.check_barrier(3, 2, mutant="B2").ok
    b3 = P.check_barrier(2, 2, mutant="B3")                # tags read before consuming
    assert not b3.ok and "before rank" in b3.violation and "wrote it" in b3.violation
    assert not P.check_barrier(3, 2, mutant="B3").ok


def test_barrier_tag_format():
    """Tags as the library documents them: 0x80000000 | round << 16 |
    block << 4 | rank, worked by hand."""
    assert P.barrier_tag(0, 0, 0) == 0x80000000
    assert P.barrier_tag(3, 5, 2) == 0x80020053
    assert P.barrier_tag(7, 1023, 63) == 0x803F3FF7
    assert P.barrier_tag(1, 16, 1) == 0x80010101


def test_barrier_tags_seen_prediction():
    """After round r every rank's block b sees rank p's round-r tag for block
    b, whoever reads it; the tag rows hold each rank's own tags."""
    W, nb, R = 3, 4, 2
    written = P.barrier_tags_written(W, nb, R)
    seen = P.barrier_tags_seen(W, nb, R)
    assert written.shape == (W, R, nb) and seen.shape == (W, R, nb, W)
    assert written[2, 1, 3] == 0x80010032
    for v in range(W):
        for r in range(R):
            for b in range(nb):
                assert [int(x) for x in seen[v, r, b]] == [P.barrier_tag(p, b, r) for p in range(W)]


def _recv(cfg, W, n):
    return [WL.recv_partials(cfg, par, n, W) for par in (0, 1)]


@pytest.mark.parametrize("mode", [P.LOCKSTEP, P.RUNAHEAD])
def test_sequential_model_final_state(mode):
    """K calls leave seq_dev = go = ctl.seq = ctl.done = K, both counters 0,
    every peer flag at K (lockstep) or K + 1 (run-ahead), this rank's flag
    untouched, and the send slots holding the inputs of calls K and K - 1."""
    W, n, K = 8, 4096, 25
    recv = _recv(2, W, n)
    calls = [(WL.own_partial(2, k, n), n) for k in range(1, K + 1)]
    st, outs = P.sequential_model(calls, recv, W, rank=0, mode=mode)
    assert st.seq_dev == st.go == st.ctl_seq == st.ctl_done == K
    assert st.cnt == [0, 0]
    lead = 1 if mode == P.RUNAHEAD else 0
    assert st.flags == [0] + [K + lead] * (W - 1)
    assert st.ctl_bytes == [2 * n, 2 * n]
    assert np.array_equal(st.send[K & 1], calls[K - 1][0])
    assert np.array_equal(st.send[(K - 1) & 1], calls[K - 2][0])
    # call k reduces with the recv slots of parity k & 1
    for k in (1, 2, K):
        parts = [calls[k - 1][0]] + [recv[k & 1][s] for s in range(1, W)]
        assert np.array_equal(outs[k - 1], R.reduce(parts, n=n))


def test_sequential_model_rank_placement():
    """With rank r, this GPU's partial takes position r in the sum."""
    W, n = 4, 1000
    recv = _recv(3, W, n)
    x = WL.recv_partials(3, 1, n)[2]
    st, outs = P.sequential_model([(x, n)], recv, W, rank=2)
    parts = [recv[1][0], recv[1][1], x, recv[1][3]]
    assert np.array_equal(outs[0], R.reduce(parts))
    assert st.flags == [1, 1, 0, 1]


def test_sequential_model_manual_needs_flags():
    W, n = 2, 64
    recv = _recv(1, W, n)
    with pytest.raises(RuntimeError):
        P.sequential_model([(recv[1][0], n)], recv, W, mode=P.MANUAL)


@pytest.mark.parametrize("W,K", [(2, 1), (2, 3), (3, 1), (3, 2), (3, 3)])
def test_counter_barrier_safe_live_and_final(W, K):
    """Page "common.cuh", PullController::sync: every rank has entered a
    stage before any rank leaves it; no deadlock; flags end at 2WK and each
    owner's base follows them."""
    r = P.check_counter_barrier(W, K)
    assert r.ok, r.violation
    assert r.finals == 1


@pytest.mark.parametrize("mutant", ["C1", "C2", "C3"])
def test_counter_barrier_mutants_are_caught(mutant):
    assert not P.check_counter_barrier(2, 2, mutant=mutant).ok
    assert not P.check_counter_barrier(3, 2, mutant=mutant).ok


def test_counter_barrier_per_flag_pairing():
    """The stronger property a fenced end stage needs (every rank's add to
    my own flag for this stage happened before I leave) holds at W = 2 for
    any number of rounds, and for one round at any W, but not at W = 3 over
    two rounds: a rank already in the next round's start stage adds to my
    flag in place of a slow rank's pending end-stage add."""
    assert P.check_counter_barrier(2, 3, strong="all").ok
    assert P.check_counter_barrier(3, 1, strong="end").ok
    r = P.check_counter_barrier(3, 2, strong="end")
    assert not r.ok and "left stage 1" in r.violation


def test_counter_barrier_split_stages_restore_the_pairing():
    """A repair, not the page's design: with one semaphore for start stages
    and one for end stages, a rank a stage ahead cannot add to the flag a
    slow rank's pending add is due on, and the per-flag pairing holds where
    the single-semaphore design loses it (W = 3 over two rounds) and at
    W = 4."""
    for W, K in [(3, 2), (3, 3), (4, 2)]:
        r = P.check_counter_barrier(W, K, strong="all", split_stages=True)
        assert r.ok, (W, K, r.violation)
        assert r.finals == 1
    assert not P.check_counter_barrier(3, 2, strong="end").ok   # the page's design, for contrast


def test_epochs_alternate():
    assert [P.epochs_after(k) for k in range(5)] == [0, 1, 0, 1, 0]


@pytest.mark.parametrize("W,iters", [(2, 1), (2, 3), (3, 1), (3, 2)])
def test_symm_patterns_safe(W, iters):
    """Page "triton_barrier.py", usage patterns: write, acq_rel barrier, read
    every rank's buffer, relaxed barrier; every read sees its iteration's
    data, nothing deadlocks, pads end zero."""
    r = P.check_symm_patterns(W, iters)
    assert r.ok, r.violation
    assert r.finals == 1


def test_symm_pattern_mutants():
    """Without pattern 1 a rank reads a buffer before its owner wrote it;
    without pattern 2 a fast rank overwrites its buffer with the next
    iteration while a peer still reads the current one."""
    p1 = P.check_symm_patterns(2, 2, mutant="P1")
    assert not p1.ok and "holding nothing" in p1.violation
    p2 = P.check_symm_patterns(2, 2, mutant="P2")
    assert not p2.ok and "holding iteration 1" in p2.violation
