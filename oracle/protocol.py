"""Protocol oracle: models of the seq/parity/flag protocol and of the signal-pad
barrier (test infrastructure only; only tests/, the smoke check and the
benchmark's CPU-baseline leg may import it).

Three models, each written from the pages' description, none sharing code
with the HIP library:

``sequential_model``
    One rank (this GPU) whose W-1 peers are virtual: their partials already
    sit in recv slots and a host proxy posts their flags. Runs K calls one
    after the other and predicts every output and the final state of every
    protocol word (page "arx.cu": protocol comment steps 1-3, arx_kernel).

``check_protocol``
    Brute-force exploration of every interleaving of a symmetric W-rank
    system (page "arx.cu"): per rank, G workgroups run the copy, arrival
    count, publish, flag wait (workgroup 0), go broadcast, reduction and
    last-block-out steps of arx_kernel, and a proxy posts, for every
    published seq in order, the partial into each peer's recv slot and then
    the flag. Checks that every reduction reads exactly the data of its own
    seq from every rank, that no reachable state is stuck before all calls
    finish, that both counters are zero whenever a kernel ends, and that a
    peer's flag never runs more than one seq ahead of this rank's publish.
    Mutants switch off one safety rule each; each must fail.

``check_counter_barrier``
    Brute-force exploration of the counter barrier (page "common.cuh",
    Semaphore and PullController::sync): every rank adds 1 to each rank's
    semaphore flag for its block, then the rank's own lane waits until its
    flag, minus a base only it keeps, reaches W (start stage) or 2W (end
    stage); the end stage then advances the base by 2W. Flags only grow.
    Checks barrier safety per stage (every rank has entered the stage; the
    stronger per-flag form holds only for W = 2), freedom from deadlock, and
    the final flag and base values. Mutants C1-C3 must fail.

``check_symm_patterns``
    Brute-force exploration of a symmetric-buffer exchange fenced by the
    pad barrier's usage patterns (page "triton_barrier.py", blockwise_barrier
    docstring): each iteration a rank writes its own buffer, passes a
    barrier (pattern 1, publishing the write), reads every rank's buffer,
    and passes a barrier (pattern 2, so the next iteration's write cannot
    clobber a buffer a peer still reads). Mutants P1 / P2 drop one barrier.

``check_barrier``
    Brute-force exploration of the blockwise signal-pad barrier (page
    "triton_barrier.py", send_signal / wait_signal / blockwise_barrier): W
    ranks, lane s of rank r CASes 0->1 on slot r of rank s's pad and then
    CASes 1->0 on slot s of its own pad, for K consecutive rounds on one block
    id. Checks that no rank leaves a round before every rank entered it, that
    nothing deadlocks, and that every pad is all zero whenever no barrier is
    in flight. Mutants B1 and B2 must fail.

The brute-force models are sequentially consistent: they check the protocol's
logic, not the memory ordering of any particular GPU.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import reduce as _reduce

U32 = 0xFFFFFFFF

# --------------------------------------------------------------------------
# Sequential single-GPU model with virtual peers
# --------------------------------------------------------------------------

LOCKSTEP = "lockstep"   # peers post seq s once this rank has published s
RUNAHEAD = "runahead"   # peers post seq s once this rank has published s - 1
MANUAL = "manual"       # flags are posted by the caller


@dataclass
class ProtocolState:
    """Every protocol word of one rank (page "arx.cu": struct Ctl, struct Dev)."""
    W: int
    rank: int
    seq_dev: int = 0            # device u64: last completed seq
    cnt: List[int] = field(default_factory=lambda: [0, 0])  # arrival / finish counters
    go: int = 0                 # device u32: low 32 bits of the seq whose peers' partials are all in place
    ctl_seq: int = 0            # pinned u64: last published seq
    ctl_bytes: List[int] = field(default_factory=lambda: [0, 0])  # bytes per parity
    ctl_done: int = 0           # pinned u64: last seq summed
    flags: List[int] = None     # pinned u64 per source rank (own entry unused)
    posted: int = 0             # last seq the proxy posted
    send: List[np.ndarray] = None  # send slot per parity

    def __post_init__(self):
        if self.flags is None:
            self.flags = [0] * self.W


def _post(st: ProtocolState, s: int) -> None:
    """The virtual peers publish seq s: every flag but this rank's becomes s.
    Seqs are posted in order, none skipped (page "arx.cu", the protocol
    comment on the proxy)."""
    if s != st.posted + 1:
        raise ValueError(f"seq {s} posted out of order after {st.posted}")
    for src in range(st.W):
        if src != st.rank:
            st.flags[src] = s
    st.posted = s


def sequential_model(calls: Sequence[Tuple[np.ndarray, int]], recv, W: int, rank: int = 0,
                     max_n: Optional[int] = None, mode: str = LOCKSTEP,
                     state: Optional[ProtocolState] = None, threads: int = 1):
    """Runs the calls (each ``(in_bits, n)``) through the one-shot path in order.

    recv[par][src] holds peer src's partial for parity par. Returns
    ``(state, outs)`` where outs[k] holds the first n elements of call k's
    output. In MANUAL mode no flags are posted, so a call whose flags are
    missing raises (the GPU would wait for them). threads: host threads of
    each call's reduction (contiguous index ranges; the same bits for any
    count).
    """
    if max_n is None:
        max_n = max((n for _, n in calls), default=0)
    st = state or ProtocolState(W=W, rank=rank)
    if st.send is None:
        st.send = [np.zeros(max_n, np.uint16), np.zeros(max_n, np.uint16)]
    if mode == RUNAHEAD and st.posted == st.ctl_seq:
        _post(st, st.ctl_seq + 1)          # the next seq needs only the last published one
    outs = []
    for x, n in calls:
        seq = st.seq_dev + 1
        par = seq & 1
        st.send[par][:n] = np.asarray(x, dtype=np.uint16)[:n]       # copy into the send slot
        st.ctl_bytes[par] = 2 * n
        st.ctl_seq = seq                   # last arriver publishes
        if mode == LOCKSTEP:
            _post(st, seq)
        elif mode == RUNAHEAD:
            _post(st, seq + 1)
        if any(st.flags[src] < seq for src in range(W) if src != rank):
            raise RuntimeError(f"seq {seq}: a peer flag never reached seq (flags {st.flags})")
        st.go = seq & U32                  # workgroup 0 releases the others
        parts = [st.send[par] if src == rank else recv[par][src] for src in range(W)]
        outs.append(_reduce.reduce(parts, n=n, threads=threads))
        st.seq_dev = seq                   # last block out
        st.ctl_done = seq
    return st, outs


# --------------------------------------------------------------------------
# Brute-force interleavings of the symmetric W-rank protocol
# --------------------------------------------------------------------------

# Workgroup program counters, in program order.
READSEQ, COPY, ARRIVE, WAIT, REDUCE, LASTOUT, DONE, FIN = range(8)

MUTANTS = {
    None: "the protocol as the page states it",
    "M1": "proxy posts only the latest published seq, skipping the ones between",
    "M2": "one send/recv buffer (parity always 0)",
    "M3": "proxy writes the flag before the data",
    "M4": "one counter shared by the arrival and the finish phase",
    "M5": "workgroups other than 0 do not wait for go",
    "M6": "the arrival count publishes one copying workgroup early",
    "M7": "with early_finish, workgroup 0 also counts itself finished before its flag wait",
    "M8": "with early_finish, a workgroup other than 0 counts itself finished before it reads the seq",
    "M9": "workgroup 0 gives go once this rank has published the seq, without the peers' flags",
    "M10": "with poll_arrives, the poll workgroup counts itself finished before its arrival wave has arrived",
}


def _tag(src: int, s: int) -> int:
    return src * 64 + s   # 0 = never written


@dataclass
class CheckResult:
    ok: bool
    states: int
    violation: Optional[str] = None
    finals: int = 0


def check_protocol(W: int, G: int, S: int, mutant: Optional[str] = None,
                   max_states: int = 5_000_000, copiers: Optional[int] = None,
                   early_finish: bool = False, poller: bool = False,
                   go_after_publish: bool = False, poll_arrives: bool = False) -> CheckResult:
    """Explores every interleaving of W ranks x G workgroups x S calls.

    copiers: the number C of workgroups that copy and count arrival (default
    G, as on the page). Workgroup c < C copies every slice g with g % C == c
    (a thread loop over a stride of C workgroups' vectors); the others skip
    the copy and the arrival, and wait for go. The publish comes with the
    C-th arrival. A workgroup reduces its own rank's partial from the
    caller's input, which holds this call's data throughout the call; the
    send slot is what the peers receive, through the proxy after the
    publish. (With C < G a workgroup's own slice of the send slot may be
    copied after its reduction: go follows the peers' flags, which do not
    wait for this rank's copies.)

    early_finish: where the last-block-out count comes (page "arx.cu",
    arx_kernel: the finish counter, the last block out records the finished
    seq). By default every workgroup counts itself finished after its
    reduction, as on the page. With early_finish a workgroup other than 0
    counts itself finished as soon as it has read the seq and passed the
    arrival step, and workgroup 0 right after its flag wait: the count only
    has to follow every workgroup's read of seq_dev (the last one to count
    advances it) and, so that the recorded finished seq means the peers'
    flags were seen, workgroup 0's flag wait. Checked in every mode: when the
    last workgroup to count records seq s as finished, workgroup 0 has passed
    its flag wait for s.

    poller: workgroup 0 only waits for the flags and gives go (page "arx.cu",
    protocol comment: one block reads the flags); it neither copies nor
    reduces and has no slice. Workgroups 1 .. G-1 hold the slices; the first
    C of them copy (workgroup 1 + k copies every slice 1 + i with i % C ==
    k; C defaults to G - 1) and count arrival, and all of them wait for go
    and reduce. Workgroup 0 reads the seq, waits for the flags (possibly
    before any arrival: a peer may be ahead) and counts itself finished
    (M7: before its wait).

    go_after_publish: workgroup 0's wait also needs this rank's own publish
    of the seq (the kernel's rule past a few vectors per copying thread).

    poll_arrives: the poll workgroup also counts one arrival (it stores the
    call's size for the proxy before it), from a wave of its own that runs
    beside its flag wait: one more process, which reads the seq and arrives
    and does nothing else; the publish then comes with the (C + 1)-th
    arrival, whichever process makes it. The poll workgroup counts itself
    finished only once that wave has arrived: otherwise, with a peer ahead,
    the call can be recorded finished before the wave reads the seq, and it
    then arrives for the next call and publishes it (M10).

    Rank state tuple: (c, pcs, ss, cnt0, cnt1, go, seq_dev, ctl_seq, done,
    send, recv, flag, posted, pcur, ppos) where c is the running call (S + 1
    after the last), pcs/ss the per-workgroup program counter and seq,
    send[par*G+g] / recv[(par*W+src)*G+g] data tags, flag[src] the flags this
    rank received, and (posted, pcur, ppos) the proxy's last posted seq, the
    seq it is posting (0 when idle) and its position in that post's actions.
    """
    if mutant not in MUTANTS:
        raise ValueError(mutant)
    if mutant in ("M7", "M8") and not early_finish:
        raise ValueError(f"{mutant} is a mutant of early_finish")
    if poller and G < 2:
        raise ValueError("a poll workgroup needs at least one reducing workgroup")
    first = 1 if poller else 0          # the first workgroup that holds a slice
    C = G - first if copiers is None else copiers
    if not 1 <= C <= G - first:
        raise ValueError(f"copiers {C} not in [1, {G - first}]")
    if poll_arrives and not poller:
        raise ValueError("poll_arrives needs a poll workgroup")
    NP = G + 1 if poll_arrives else G    # processes: the workgroups, and the poll workgroup's arrival wave
    arrivals = C + 1 if poll_arrives else C
    if mutant == "M6" and arrivals < 2:
        raise ValueError("M6 needs at least two arrivals")
    last_arrival = arrivals - 2 if mutant == "M6" else arrivals - 1
    nbuf = 1 if mutant == "M2" else 2

    def par_of(s):
        return 0 if mutant == "M2" else s & 1

    def start_pc(g):
        # M8: a workgroup other than 0 counts itself finished before it reads the seq
        return LASTOUT if (mutant == "M8" and 0 < g < G) else READSEQ

    def after_seq(g):
        if g == G:                      # the poll workgroup's arrival wave
            return ARRIVE
        if poller and g == 0:
            return LASTOUT if mutant == "M7" else WAIT
        if first <= g < first + C:
            return COPY
        return LASTOUT if (early_finish and g != 0 and mutant != "M8") else WAIT

    def after_arrive(g):
        if g == G:
            return DONE
        if early_finish and (g != 0 or mutant == "M7") and not (mutant == "M8" and g != 0):
            return LASTOUT
        return WAIT

    def after_lastout(g):
        if poller and g == 0:
            return WAIT if mutant == "M7" else DONE
        if not early_finish:
            return DONE
        if g == 0:
            return WAIT if mutant == "M7" else REDUCE
        return READSEQ if mutant == "M8" else WAIT

    def wg0_past_wait(pc0):
        if pc0 in (REDUCE, DONE):
            return True
        return pc0 == LASTOUT and mutant != "M7"   # otherwise workgroup 0 counts after its flag wait

    # Proxy actions for one seq, staggered peer order r+1, r+2, ... (page
    # "arx.cu": each rank sends to the next ranks in turn). Data first, then
    # the flag on the same ordered channel; M3 swaps them.
    def actions(r):
        acts = []
        for step in range(1, W):
            j = (r + step) % W
            data = [("data", j, g) for g in range(first, G)]
            flag = [("flag", j, 0)]
            acts += (flag + data) if mutant == "M3" else (data + flag)
        return acts

    acts = [actions(r) for r in range(W)]

    init_rank = (1, tuple(start_pc(g) for g in range(NP)), (0,) * NP, 0, 0, 0, 0, 0, 0,
                 (0,) * (2 * G), (0,) * (2 * W * G), (0,) * W, 0, 0, 0)
    init = tuple(init_rank for _ in range(W))

    seen = {init}
    stack = [init]
    finals = 0

    def replace(state, r, rs):
        return state[:r] + (rs,) + state[r + 1:]

    while stack:
        st = stack.pop()
        succ = []
        for r in range(W):
            (c, pcs, ss, cnt0, cnt1, go, seq_dev, ctl_seq, done,
             send, recv, flag, posted, pcur, ppos) = st[r]
            # ---- GPU workgroups of rank r
            if c <= S:
                for g in range(NP):
                    pc = pcs[g]
                    s = ss[g]
                    ns = None
                    if pc == READSEQ:
                        s2 = seq_dev + 1
                        nxt = after_seq(g)
                        ns = (c, pcs[:g] + (nxt,) + pcs[g + 1:], ss[:g] + (s2,) + ss[g + 1:],
                              cnt0, cnt1, go, seq_dev, ctl_seq, done, send, recv, flag, posted, pcur, ppos)
                    elif pc == COPY:
                        send2 = list(send)
                        for g2 in range(g, G, C):   # copier g: slices g, g + C, ...
                            send2[par_of(s) * G + g2] = _tag(r, s)
                        send2 = tuple(send2)
                        ns = (c, pcs[:g] + (ARRIVE,) + pcs[g + 1:], ss, cnt0, cnt1, go, seq_dev,
                              ctl_seq, done, send2, recv, flag, posted, pcur, ppos)
                    elif pc == ARRIVE:
                        old = cnt0
                        n0 = cnt0 + 1
                        cs = ctl_seq
                        if old == last_arrival:   # last copier publishes and resets
                            n0 = 0
                            cs = s
                        nxt = after_arrive(g)
                        if mutant == "M4":    # one counter for both phases
                            ns = (c, pcs[:g] + (nxt,) + pcs[g + 1:], ss, n0, n0, go, seq_dev, cs,
                                  done, send, recv, flag, posted, pcur, ppos)
                        else:
                            ns = (c, pcs[:g] + (nxt,) + pcs[g + 1:], ss, n0, cnt1, go, seq_dev, cs,
                                  done, send, recv, flag, posted, pcur, ppos)
                    elif pc == WAIT:
                        if g == 0:
                            flags_in = all(flag[j] >= s for j in range(W) if j != r)
                            if go_after_publish:
                                flags_in = flags_in and ctl_seq >= s
                            if (ctl_seq >= s) if mutant == "M9" else flags_in:
                                if poller:
                                    nxt = DONE if mutant == "M7" else LASTOUT
                                else:
                                    nxt = LASTOUT if (early_finish and mutant != "M7") else REDUCE
                                ns = (c, pcs[:g] + (nxt,) + pcs[g + 1:], ss, cnt0, cnt1, s, seq_dev,
                                      ctl_seq, done, send, recv, flag, posted, pcur, ppos)
                        elif mutant == "M5" or go >= s:
                            ns = (c, pcs[:g] + (REDUCE,) + pcs[g + 1:], ss, cnt0, cnt1, go, seq_dev,
                                  ctl_seq, done, send, recv, flag, posted, pcur, ppos)
                    elif pc == REDUCE:
                        p = par_of(s)
                        for j in range(W):
                            if j == r:
                                continue          # own partial: the caller's input
                            t = recv[(p * W + j) * G + g]
                            if t != _tag(j, s):
                                return CheckResult(False, len(seen), (
                                    f"rank {r} wg {g} reduced seq {s} with stale data from rank {j} "
                                    f"(tag {t // 64},{t % 64})"))
                        nxt = DONE if early_finish else LASTOUT
                        ns = (c, pcs[:g] + (nxt,) + pcs[g + 1:], ss, cnt0, cnt1, go, seq_dev,
                              ctl_seq, done, send, recv, flag, posted, pcur, ppos)
                    elif pc == LASTOUT:
                        if poll_arrives and g == 0 and pcs[G] != DONE and mutant != "M10":
                            continue          # wait for the arrival wave
                        base = cnt0 if mutant == "M4" else cnt1
                        n1 = base + 1
                        sd, dn = seq_dev, done
                        if base == G - 1:     # last block out
                            n1 = 0
                            sd = ss[0] if (mutant == "M8" and g != 0) else s
                            dn = sd
                            if not wg0_past_wait(pcs[0]) or (g == 0 and mutant == "M7"):
                                return CheckResult(False, len(seen), (
                                    f"rank {r} recorded seq {sd} finished before workgroup 0 saw its flags"))
                        if mutant == "M4":
                            ns = (c, pcs[:g] + (after_lastout(g),) + pcs[g + 1:], ss, n1, n1, go, sd,
                                  ctl_seq, dn, send, recv, flag, posted, pcur, ppos)
                        else:
                            ns = (c, pcs[:g] + (after_lastout(g),) + pcs[g + 1:], ss, cnt0, n1, go, sd,
                                  ctl_seq, dn, send, recv, flag, posted, pcur, ppos)
                    if ns is not None and all(x == DONE for x in ns[1]):   # the kernel ends
                        c2 = c + 1
                        pcs2 = tuple(start_pc(g2) if c2 <= S else FIN for g2 in range(NP))
                        final_cnt = (ns[3], ns[4])
                        if final_cnt != (0, 0):
                            return CheckResult(False, len(seen), (
                                f"rank {r} kernel {c} ended with counters {final_cnt}"))
                        ns = (c2, pcs2) + ns[2:]
                    if ns is not None:
                        succ.append(replace(st, r, ns))
            # ---- proxy of rank r
            if pcur == 0:
                nxt = None
                if mutant == "M1":
                    if ctl_seq > posted:
                        nxt = ctl_seq
                elif ctl_seq >= posted + 1:
                    nxt = posted + 1
                if nxt is not None:
                    ns = st[r][:13] + (nxt, 0)
                    succ.append(replace(st, r, ns))
            else:
                kind, j, g = acts[r][ppos]
                p = par_of(pcur)
                rj = st[j]
                if kind == "data":
                    tag = send[p * G + g]
                    i = (p * W + r) * G + g
                    rrecv = rj[10][:i] + (tag,) + rj[10][i + 1:]
                    rj2 = rj[:10] + (rrecv,) + rj[11:]
                else:
                    rflag = rj[11][:r] + (pcur,) + rj[11][r + 1:]
                    rj2 = rj[:11] + (rflag,) + rj[12:]
                st2 = replace(st, j, rj2)
                me = st2[r]
                if ppos + 1 == len(acts[r]):
                    me2 = me[:12] + (pcur, 0, 0)
                else:
                    me2 = me[:14] + (ppos + 1,)
                succ.append(replace(st2, r, me2))

        # invariant: a peer's flag at rank r never exceeds r's published seq + 1
        for r in range(W):
            ctl_seq = st[r][7]
            for j in range(W):
                if j != r and st[r][11][j] > ctl_seq + 1 and mutant is None:
                    return CheckResult(False, len(seen), (
                        f"flag from rank {j} at rank {r} is {st[r][11][j]}, more than one "
                        f"ahead of published {ctl_seq}"))

        if not succ:
            all_done = all(st[r][0] == S + 1 and st[r][13] == 0 and st[r][12] >= S for r in range(W))
            if not all_done:
                desc = "; ".join(f"r{r}: call {st[r][0]} pcs {st[r][1]} seqs {st[r][2]} posted {st[r][12]} "
                                 f"published {st[r][7]} flags {st[r][11]}" for r in range(W))
                return CheckResult(False, len(seen), f"deadlock: {desc}")
            finals += 1
        for s2 in succ:
            if s2 not in seen:
                seen.add(s2)
                stack.append(s2)
                if len(seen) > max_states:
                    raise RuntimeError(f"state space exceeds {max_states}")
    return CheckResult(True, len(seen), None, finals)


# --------------------------------------------------------------------------
# Brute-force interleavings of the blockwise signal-pad barrier
# --------------------------------------------------------------------------

SEND, WAITSIG, LANEDONE = range(3)

BARRIER_MUTANTS = {
    None: "CAS 0->1 to signal, CAS 1->0 to consume (page triton_barrier.py)",
    "B1": "signal with a plain store of 1 instead of a CAS from 0",
    "B2": "wait reads the 1 without clearing it",
    "B3": "the peers' tags are read once this rank's signals are sent, before it consumes theirs",
}


def check_barrier(W: int, K: int, mutant: Optional[str] = None,
                  max_states: int = 5_000_000) -> CheckResult:
    """Explores every interleaving of W ranks' lanes over K barrier rounds.

    Tags: on entering round k a rank writes its tag for round k (before any
    of its lanes signals, as the workgroup barrier of the page's usage
    pattern 1 orders it), and on leaving round k it reads every rank's tag
    for round k; the read must find it written. A rank has written its
    round-k tag exactly when it has entered round k, so this is the check
    that no rank leaves a round before every rank entered it. Mutant B3 moves
    the read to the moment this rank's last signal is sent.

    State: (rounds, lanes, pad). rounds[r] = rounds rank r has entered
    (1..K, K + 1 once finished); lanes[r*W+s] = lane s's step in rank r's
    current round; pad[q*W+s] = rank q's pad slot for signals from rank s.
    A rank starts its next round only when all its lanes finished the current
    one (the workgroup barrier after blockwise_barrier).
    """
    if mutant not in BARRIER_MUTANTS:
        raise ValueError(mutant)
    init = ((1,) * W, (SEND,) * (W * W), (0,) * (W * W))
    seen = {init}
    stack = [init]
    finals = 0
    while stack:
        st = stack.pop()
        rounds, lanes, pad = st
        succ = []
        for r in range(W):
            if rounds[r] > K:
                continue
            for s in range(W):
                li = r * W + s
                step = lanes[li]
                if step == SEND:
                    pi = s * W + r          # slot r of rank s's pad
                    if mutant == "B1" or pad[pi] == 0:
                        pad2 = pad[:pi] + (1,) + pad[pi + 1:]
                        lanes2 = lanes[:li] + (WAITSIG,) + lanes[li + 1:]
                        if mutant == "B3" and all(lanes2[r * W + x] != SEND for x in range(W)):
                            k = rounds[r]
                            for q in range(W):
                                if rounds[q] < k:
                                    return CheckResult(False, len(seen), (
                                        f"rank {r} read rank {q}'s round-{k} tag before rank {q} wrote it"))
                        succ.append((rounds, lanes2, pad2))
                elif step == WAITSIG:
                    pi = r * W + s          # slot s of this rank's pad
                    if pad[pi] == 1:
                        pad2 = pad if mutant == "B2" else pad[:pi] + (0,) + pad[pi + 1:]
                        lanes2 = lanes[:li] + (LANEDONE,) + lanes[li + 1:]
                        succ.append((rounds, lanes2, pad2))
            if all(lanes[r * W + s] == LANEDONE for s in range(W)):
                k = rounds[r]
                # rank r leaves round k and reads every rank's round-k tag:
                # every rank must have entered round k (written that tag)
                for q in range(W):
                    if rounds[q] < k and mutant != "B3":
                        return CheckResult(False, len(seen), (
                            f"rank {r} left round {k} before rank {q} entered it (read an unwritten tag)"))
                nxt = (SEND,) if k + 1 <= K else (LANEDONE,)
                rounds2 = rounds[:r] + (k + 1,) + rounds[r + 1:]
                lanes2 = lanes[:r * W] + nxt * W + lanes[r * W + W:]
                succ.append((rounds2, lanes2, pad))
        # quiescence: every rank between rounds (all lanes of its current round
        # still at SEND, or finished) and all at the same round -> pads zero
        quiet = all(rounds[r] > K or all(lanes[r * W + s] == SEND for s in range(W)) for r in range(W))
        if quiet and len(set(rounds)) == 1 and any(pad):
            return CheckResult(False, len(seen), f"pad not zero between barriers: {pad}")
        if not succ:
            if not all(x == K + 1 for x in rounds):
                return CheckResult(False, len(seen), f"deadlock: rounds {rounds} lanes {lanes} pad {pad}")
            if any(pad):
                return CheckResult(False, len(seen), f"pad not zero after the last barrier: {pad}")
            finals += 1
        for s2 in succ:
            if s2 not in seen:
                seen.add(s2)
                stack.append(s2)
                if len(seen) > max_states:
                    raise RuntimeError(f"state space exceeds {max_states}")
    return CheckResult(True, len(seen), None, finals)


def barrier_tag(rank: int, block: int, rnd: int) -> int:
    """The tag rank `rank`'s workgroup for block `block` writes before round
    `rnd` of a tagged barrier launch: 0x80000000 | rnd << 16 | block << 4 |
    rank (the library's documented tag format)."""
    return 0x80000000 | (rnd << 16) | (block << 4) | rank


def barrier_tags_written(W: int, nblocks: int, rounds: int) -> np.ndarray:
    """The tag rows after a tagged launch, u32 [W, rounds, nblocks]: rank v's
    slot for round r and block b holds barrier_tag(v, b, r)."""
    out = np.zeros((W, rounds, nblocks), np.uint32)
    for v in range(W):
        for r in range(rounds):
            for b in range(nblocks):
                out[v, r, b] = barrier_tag(v, b, r)
    return out


def barrier_tags_seen(W: int, nblocks: int, rounds: int) -> np.ndarray:
    """What a tagged barrier launch reads back, u32 [W, rounds, nblocks, W]:
    after round r, rank v's block b reads rank p's round-r tag for block b.
    check_barrier shows that every rank has written it by then (no rank
    leaves a round before every rank entered it), and the acquire / release
    pairing of each signal makes the write visible, so the read returns
    barrier_tag(p, b, r) for every p (page "triton_barrier.py",
    blockwise_barrier docstring, usage pattern 1)."""
    written = barrier_tags_written(W, nblocks, rounds)       # [p, r, b]
    return np.broadcast_to(np.transpose(written, (1, 2, 0))[None], (W, rounds, nblocks, W)).copy()


def barrier_pads_after(W: int, nblocks: int, rounds: int = 1) -> List[np.ndarray]:
    """Expected pads after `rounds` complete barriers on every block id from
    zero-filled pads: all zero (page "triton_barrier.py", blockwise_barrier
    docstring on graph friendliness)."""
    return [np.zeros((nblocks, W), np.uint32) for _ in range(W)]


# --------------------------------------------------------------------------
# Brute-force interleavings of the counter barrier (two stages per round)
# --------------------------------------------------------------------------

COUNTER_MUTANTS = {
    None: "flag - base >= W * stage, end stage advances base by 2W (page common.cuh)",
    "C1": "the end stage does not advance the base",
    "C2": "the wait tests flag - base == W * stage instead of >=",
    "C3": "the start stage also advances the base, by W",
}

# per-rank program counter within a stage: lanes still to add, then wait
ADDING, WAITING, STAGE_DONE = range(3)


def check_counter_barrier(W: int, K: int, mutant: Optional[str] = None, strong: str = "",
                          max_states: int = 5_000_000, split_stages: bool = False) -> CheckResult:
    """Explores every interleaving of W ranks running K rounds of (start
    stage, end stage) on one block id.

    Safety, by default: no rank leaves a stage before every rank has entered
    it (made at least one of its adds for it). With strong="all" (every
    stage) or "end" (end stages only, the fenced ones): no rank r leaves such
    a stage before every rank's add to r's own flag for that stage has
    happened, which is what a release / acquire pairing through r's flag
    needs. The weak form holds for any W; the strong form holds for W = 2
    but not for W >= 3, where a rank that is a stage ahead can add to r's
    flag in place of a slow rank's pending add.

    split_stages: a repair, not the page's design. Every rank has two
    semaphores per block, one that start stages add to and one for end
    stages, each waited for up to W per stage; a rank a stage ahead then
    cannot add to the flag a slow rank's pending add is due on.

    State: (stage_idx, added, waiting, flag, base). stage_idx[r] counts the
    stages rank r has entered (0-based; stage 2k is round k's start, 2k+1
    its end; 2K once finished); added[r] is the set (bitmask) of lanes of
    rank r that have added in the current stage; waiting[r] tells whether
    rank r's own lane is now waiting; flag[r] and base[r] are rank r's
    semaphore flag and its owner-only base counter.
    """
    if mutant not in COUNTER_MUTANTS:
        raise ValueError(mutant)
    full = (1 << W) - 1
    nf = 2 if split_stages else 1           # semaphores per rank
    init = ((0,) * W, (0,) * W, (0,) * W, (0,) * (nf * W), (0,) * (nf * W))
    seen = {init}
    stack = [init]
    finals = 0
    while stack:
        st = stack.pop()
        stage_idx, added, waiting, flag, base = st
        succ = []
        for r in range(W):
            si = stage_idx[r]
            if si >= 2 * K:
                continue
            start = si % 2 == 0
            sem = (0 if start else 1) if split_stages else 0   # which of a rank's semaphores
            # a lane that has not added yet adds 1 to its rank's flag
            if not waiting[r]:
                for w in range(W):
                    if not added[r] >> w & 1:
                        fw = w * nf + sem
                        flag2 = flag[:fw] + (flag[fw] + 1,) + flag[fw + 1:]
                        added2 = added[:r] + (added[r] | (1 << w),) + added[r + 1:]
                        waiting2 = waiting
                        if added2[r] == full:
                            waiting2 = waiting[:r] + (1,) + waiting[r + 1:]
                        succ.append((stage_idx, added2, waiting2, flag2, base))
            else:
                fr = r * nf + sem
                target = W if split_stages else W * (1 if start else 2)
                have = flag[fr] - base[fr]
                ok = have == target if mutant == "C2" else have >= target
                if ok:
                    # rank r leaves this stage: every rank must have added for it
                    for q in range(W):
                        if strong == "all" or (strong == "end" and not start):
                            q_added = stage_idx[q] > si or (stage_idx[q] == si and added[q] >> r & 1)
                        else:
                            q_added = stage_idx[q] > si or (stage_idx[q] == si and added[q] != 0)
                        if not q_added:
                            return CheckResult(False, len(seen), (
                                f"rank {r} left stage {si} before rank {q} arrived at it"))
                    b = base[fr]
                    if split_stages:
                        b = base[fr] + W
                    else:
                        if not start and mutant != "C1":
                            b = base[fr] + 2 * W
                        if start and mutant == "C3":
                            b = base[fr] + W
                    base2 = base[:fr] + (b,) + base[fr + 1:]
                    stage2 = stage_idx[:r] + (si + 1,) + stage_idx[r + 1:]
                    added2 = added[:r] + (0,) + added[r + 1:]
                    waiting2 = waiting[:r] + (0,) + waiting[r + 1:]
                    succ.append((stage2, added2, waiting2, flag, base2))
        if not succ:
            if not all(x == 2 * K for x in stage_idx):
                return CheckResult(False, len(seen), (
                    f"deadlock: stages {stage_idx} flags {flag} bases {base}"))
            want = W * K if split_stages else 2 * W * K
            if any(f != want for f in flag) or any(b != want for b in base):
                return CheckResult(False, len(seen), f"final flags {flag} bases {base}, want {want}")
            finals += 1
        for s2 in succ:
            if s2 not in seen:
                seen.add(s2)
                stack.append(s2)
                if len(seen) > max_states:
                    raise RuntimeError(f"state space exceeds {max_states}")
    return CheckResult(True, len(seen), None, finals)


def epochs_after(launches: int) -> int:
    """Page "common.cuh", PushController: each launch's exit flips a block's
    epoch between 0 and 1 (kNumStages = 2), so after k launches from 0 the
    epoch is k mod 2 and launch i (0-based) saw epoch i mod 2."""
    return launches % 2


# --------------------------------------------------------------------------
# Brute-force interleavings of a pattern-fenced symmetric-buffer exchange
# --------------------------------------------------------------------------

SYMM_MUTANTS = {
    None: "write, barrier (pattern 1), read all, barrier (pattern 2)",
    "P1": "no barrier between the write and the reads",
    "P2": "no barrier between the reads and the next iteration's write",
}

# rank program counter within an iteration
S_WRITE, S_B1_SEND, S_B1_WAIT, S_READ, S_B2_SEND, S_B2_WAIT, S_NEXT = range(7)


def check_symm_patterns(W: int, iters: int, mutant: Optional[str] = None,
                        max_states: int = 5_000_000) -> CheckResult:
    """Explores every interleaving of W ranks (one block each, its W barrier
    lanes modelled as one send step per peer and one consume step per peer)
    running `iters` iterations of the exchange. A read of rank j's buffer in
    iteration k must see exactly the tag (j, k).

    State: (pc, it, sent, consumed, pad, buf) per rank: pc and iteration,
    bitmasks of the peers signalled / consumed in the current barrier, the
    pad slots (pad[r*W+s] = rank r's slot for rank s), and buf[r] = the tag
    rank r last wrote.
    """
    if mutant not in SYMM_MUTANTS:
        raise ValueError(mutant)
    full = (1 << W) - 1
    init = ((S_WRITE,) * W, (0,) * W, (0,) * W, (0,) * W, (0,) * (W * W), (-1,) * W)
    seen = {init}
    stack = [init]
    finals = 0

    def setr(t, r, v):
        return t[:r] + (v,) + t[r + 1:]

    while stack:
        st = stack.pop()
        pc, it, sent, cons, pad, buf = st
        succ = []
        for r in range(W):
            p, k = pc[r], it[r]
            if k >= iters:
                continue
            if p == S_WRITE:
                nxt = S_READ if mutant == "P1" else S_B1_SEND
                succ.append((setr(pc, r, nxt), it, sent, cons, pad, setr(buf, r, r * 64 + k)))
            elif p in (S_B1_SEND, S_B2_SEND):
                for s_ in range(W):                 # lane s_ signals rank s_
                    if not sent[r] >> s_ & 1:
                        i = s_ * W + r
                        if pad[i] == 0:             # CAS 0 -> 1
                            sent2 = setr(sent, r, sent[r] | (1 << s_))
                            pc2 = setr(pc, r, p + 1) if sent2[r] == full else pc
                            succ.append((pc2, it, sent2 if sent2[r] != full else setr(sent, r, 0),
                                         cons, setr(pad, i, 1), buf))
            elif p in (S_B1_WAIT, S_B2_WAIT):
                for s_ in range(W):                 # lane s_ consumes rank s_'s signal
                    if not cons[r] >> s_ & 1:
                        i = r * W + s_
                        if pad[i] == 1:             # CAS 1 -> 0
                            cons2 = setr(cons, r, cons[r] | (1 << s_))
                            if cons2[r] == full:
                                nxt = S_READ if p == S_B1_WAIT else S_NEXT
                                succ.append((setr(pc, r, nxt), it, sent, setr(cons, r, 0), setr(pad, i, 0), buf))
                            else:
                                succ.append((pc, it, sent, cons2, setr(pad, i, 0), buf))
            elif p == S_READ:
                for j in range(W):
                    if buf[j] != j * 64 + k:
                        return CheckResult(False, len(seen), (
                            f"rank {r} iteration {k} read rank {j}'s buffer holding "
                            f"{'nothing' if buf[j] < 0 else f'iteration {buf[j] % 64}'}"))
                nxt = S_NEXT if mutant == "P2" else S_B2_SEND
                succ.append((setr(pc, r, nxt), it, sent, cons, pad, buf))
            elif p == S_NEXT:
                succ.append((setr(pc, r, S_WRITE), setr(it, r, k + 1), sent, cons, pad, buf))
        if not succ:
            if not all(x >= iters for x in it):
                return CheckResult(False, len(seen), f"deadlock: pcs {pc} iterations {it} pad {pad}")
            if any(pad):
                return CheckResult(False, len(seen), f"pad not zero at the end: {pad}")
            finals += 1
        for s2 in succ:
            if s2 not in seen:
                seen.add(s2)
                stack.append(s2)
                if len(seen) > max_states:
                    raise RuntimeError(f"state space exceeds {max_states}")
    return CheckResult(True, len(seen), None, finals)

