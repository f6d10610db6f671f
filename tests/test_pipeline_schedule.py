"""CPU model of the MFMA kernels' K-loop schedules: the order in which one
wave issues direct loads into LDS stages, waits, passes barriers and reads
fragments.  Every wave runs the same program, so a barrier between two
events in program order separates them in every wave.  Checked:

* read after write: a stage is read for step k only after the direct loads
  of step k into it were waited for and a barrier followed;
* write after read: a stage is overwritten only after a barrier that follows
  every read of its previous contents (the barrier waits for the wave's LDS
  reads).

The generators mirror the loop control of `tile_accumulate` (the two-stage
fragment-prefetch loop and the S-stage loop) and of the aligned loop of
`lp_tile_accumulate` (16- and 8-bit operands) step for step."""

import pytest


def prefetch_schedule(s0, e):
    ev = []
    if s0 < e:
        ev.append(("dma", s0, 0))
    if s0 + 1 < e:
        ev.append(("dma", s0 + 1, 1))
    ev.append(("wait", 0))
    ev.append(("bar",))
    if s0 < e:
        ev.append(("read", s0, 0))
    ev.append(("bar",))

    def step(kt, st):
        if kt + 1 < e:
            ev.append(("read", kt + 1, st ^ 1))
        if kt + 2 < e:
            ev.append(("dma", kt + 2, st))
        ev.append(("wait", 0))
        ev.append(("bar",))

    kt = s0
    while kt + 1 < e:
        step(kt, 0)
        step(kt + 1, 1)
        kt += 2
    if kt < e:
        step(kt, 0)
    return ev


def staged_schedule(s0, e, nst):
    ev = []
    for s in range(nst - 1):
        if s0 + s < e:
            ev.append(("dma", s0 + s, s))
    ev.append(("wait", nst - 2 if e - s0 >= nst - 1 else 0))
    ev.append(("bar",))
    stage, nxt = 0, nst - 1
    for kt in range(s0, e):
        issue = kt + nst - 1 < e
        if issue:
            ev.append(("dma", kt + nst - 1, nxt))
        ev.append(("read", kt, stage))
        ev.append(("wait", nst - 2 if issue else 0))
        ev.append(("bar",))
        stage = (stage + 1) % nst
        nxt = (nxt + 1) % nst
    return ev


def check(ev):
    """Replay the events; `wait n` leaves the n most recent direct-load steps
    in flight (a step's loads are issued together)."""
    issued = []          # steps in issue order
    landed = set()       # steps waited for
    visible = set()      # steps waited for, then a barrier
    holder = {}          # stage -> step written into it last
    reads_since_bar = {}  # stage -> steps read from it since the last barrier
    read_before = {}     # stage -> steps read from it before the last barrier
    for x in ev:
        if x[0] == "dma":
            _, k, st = x
            assert not reads_since_bar.get(st), f"step {k} overwrites stage {st} " \
                f"read without a barrier in between: {ev}"
            holder[st] = k
            issued.append(k)
        elif x[0] == "wait":
            n = x[1]
            done = issued[:len(issued) - n] if n else issued
            landed.update(done)
        elif x[0] == "bar":
            visible.update(landed)
            for st, ks in reads_since_bar.items():
                read_before.setdefault(st, set()).update(ks)
            reads_since_bar = {}
        elif x[0] == "read":
            _, k, st = x
            if k is not None:  # (None: a read whose values are never used)
                assert holder.get(st) == k, f"stage {st} holds {holder.get(st)}, read for {k}"
                assert k in visible, f"step {k} read before it was waited for and a barrier passed"
            reads_since_bar.setdefault(st, set()).add(k)
    return ev


@pytest.mark.parametrize("s0", [0, 1, 5])
@pytest.mark.parametrize("n", range(0, 9))
def test_prefetch_loop_hazards(s0, n):
    ev = check(prefetch_schedule(s0, s0 + n))
    assert sorted(x[1] for x in ev if x[0] == "read") == list(range(s0, s0 + n))


@pytest.mark.parametrize("nst", [2, 3, 4])
@pytest.mark.parametrize("n", range(0, 9))
def test_staged_loop_hazards(nst, n):
    ev = check(staged_schedule(3, 3 + n, nst))
    assert sorted(x[1] for x in ev if x[0] == "read") == list(range(3, 3 + n))


def test_the_model_sees_a_missing_barrier():
    """Without the barrier after the prologue's read, the first step's
    direct load overwrites stage 0 while other waves may still read it."""
    ev = prefetch_schedule(0, 4)
    i = max(j for j, x in enumerate(ev[:6]) if x == ("bar",))
    with pytest.raises(AssertionError, match="overwrites stage 0"):
        check(ev[:i] + ev[i + 1:])


def lowp_schedule(kd, nst, qg, tail=False):
    """The aligned loop of the 16- and 8-bit kernels over kd direct-load
    steps: S = nst stages, QG groups of MFMAs per step, the barrier before
    group H = QG/2.  Look-ahead loads past the last step repeat the last step
    (clamped) into stages never read again; at the last step the groups after
    the barrier still read the next stage (values never used).  `tail`: the
    edge kernels' register-staged last step into stage 0."""
    h = qg // 2
    ev = []
    if kd > 0:
        for st in range(nst):
            ev.append(("dma", min(st, kd - 1), st))
        ev.append(("wait", nst - 1))
        ev.append(("bar",))
        for _ in range(h):  # groups 0 .. H-1 of step 0
            ev.append(("read", 0, 0))
        for kt in range(kd):
            st, st1 = kt % nst, (kt + 1) % nst
            kl = min(kt + nst, kd - 1)
            for _ in range(h):  # groups 0 .. H-1: reads of groups H .. QG-1 of step kt
                ev.append(("read", kt, st))
            ev.append(("wait", nst - 2))
            ev.append(("bar",))
            for _ in range(qg - h):  # groups H .. QG-1
                ev.append(("read", kt + 1 if kt + 1 < kd else None, st1))
                ev.append(("dma", kl, st))
    if tail:
        ev.append(("wait", 0))
        ev.append(("bar",))
        ev.append(("dma", kd, 0))  # register stores, waited for (lgkmcnt(0))
        ev.append(("wait", 0))
        ev.append(("bar",))
        ev.append(("read", kd, 0))
    return ev


@pytest.mark.parametrize("qg", [2, 4])
@pytest.mark.parametrize("nst", [2, 4])
@pytest.mark.parametrize("kd", range(0, 10))
@pytest.mark.parametrize("tail", [False, True])
def test_lowp_loop_hazards(qg, nst, kd, tail):
    if kd == 0 and not tail:
        return
    ev = check(lowp_schedule(kd, nst, qg, tail))
    want = list(range(kd + (1 if tail else 0)))
    assert sorted({x[1] for x in ev if x[0] == "read" and x[1] is not None}) == want


def test_the_lowp_model_sees_a_load_before_the_barrier():
    """A step's first direct load issued before the step's barrier instead of
    after it overwrites the stage other waves may still be reading."""
    ev = lowp_schedule(6, 2, 4)
    i = ev.index(("bar",), 4)          # the first step's barrier
    j = next(k for k in range(i, len(ev)) if ev[k][0] == "dma")
    moved = ev[:i] + [ev[j]] + ev[i:j] + ev[j + 1:]
    with pytest.raises(AssertionError, match="overwrites stage 0"):
        check(moved)
