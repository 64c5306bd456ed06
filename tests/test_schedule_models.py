"""Host models of the LDS ring schedules of three kernels (no GPU).

Each model lists, in program order, what one wave issues: direct-to-LDS loads
(operand, slab, ring unit), `vmcnt` waits, workgroup barriers and fragment
reads, exactly in the order the kernel's source issues them.  Loads retire in
issue order (no load of these kernels is out of range in all its lanes), so a
`vmcnt(N)` wait leaves the wave's last N loads in flight.  Every wave issues the
same pattern for its own rows, so a barrier publishes what each wave had
completed when it arrived.  The checks, for every slab count up to 40:
- every fragment read of slab i from unit u finds u holding slab i, loaded
  and completed by every wave before the barrier that precedes the read;
- no load into a unit is issued before the barrier that follows the last read
  of the slab the unit held (no wave can still be reading it);
- slabs past the split's end are loaded only into units no real slab reads
  afterwards (the kernels re-read the last slab there to keep wait counts
  uniform).
The ping-pong kernel's two wave groups run different programs; its model
(at the end) checks the same two properties across the groups, a load being
published by the barrier after the issuing group's wait that covers it.
"""
import pytest


class Wave:
    """One wave's program: a list of events."""

    def __init__(self):
        self.ev = []

    def load(self, op, slab, unit):
        self.ev.append(("load", op, slab, unit))

    def wait(self, n):
        self.ev.append(("wait", n))

    def barrier(self):
        self.ev.append(("barrier",))

    def read(self, op, slab, unit):
        self.ev.append(("read", op, slab, unit))


def check(prog, nk):
    """Run the checks on one wave's program (all waves run the same one)."""
    from collections import Counter
    issued = []                  # (op, slab, unit) in issue order
    done = 0                     # loads completed at the last wait
    published = Counter()        # loads per (op, slab, unit) completed by every wave at the last barrier
    barriers = 0
    last_read = {}               # (op, unit) -> barrier count at that unit's latest read
    holds = {}                   # (op, unit) -> slab most recently loaded there
    for e in prog.ev:
        if e[0] == "load":
            _, op, slab, unit = e
            key = (op, unit)
            # WAR: the unit's previous contents were last read before a barrier
            # that has since passed
            if key in last_read:
                assert barriers > last_read[key], ("load over a unit still being read", e)
            holds[key] = slab
            issued.append((op, slab, unit))
        elif e[0] == "wait":
            done = max(done, len(issued) - e[1])
        elif e[0] == "barrier":
            barriers += 1
            published = Counter(issued[:done])
        else:
            _, op, slab, unit = e
            assert slab < nk
            assert holds.get((op, unit)) == slab, ("unit holds another slab", e, holds.get((op, unit)))
            # every load of this slab into this unit, by every wave, published
            n = sum(1 for x in issued if x == (op, slab, unit))
            assert n > 0 and published[(op, slab, unit)] == n, ("read before its loads were published", e)
            last_read[(op, unit)] = barriers
    # no dummy load lands where a real slab is read afterwards: holds at the end
    # may be dummies, but every read above matched its slab


# ---------------------------------------------------------------------------
# The four-wave 256x128 kernel (gemm_nt_w4.hpp): 3 A units, 4 B units, a slab
# is LA A loads and LB B loads per wave, a k-step issues its share of loads
# between MFMAs, and one barrier per slab before the last MFMAs of k-step 2.

LA, LB, NUA, NUB = 8, 4, 3, 4


def w4_program(nk):
    w = Wave()
    # (a load past the split's end re-reads the last slab in the kernel; the
    # model records it under the index it stands for, so a read that met such a
    # load would fail the slab check)

    def A(i, u, half):
        for _ in range(LA // 2):
            w.load("A", i, u)

    def B(i, u, half):
        for _ in range(LB // 2):
            w.load("B", i, u)

    # prologue: A(0)a, B(0), A(0)b, B(1), A(1), B(2), A(2)a
    A(0, 0, 0); B(0, 0, 0); B(0, 0, 1); A(0, 0, 1)
    B(1, 1, 0); B(1, 1, 1); A(1, 1, 0); A(1, 1, 1)
    B(2, 2, 0); B(2, 2, 1); A(2, 2, 0)
    w.wait(2 * LB + 3 * LA // 2)
    w.barrier()
    w.read("A", 0, 0); w.read("B", 0, 0)              # slab 0, k-step 0 fragments
    ua = ub = 0
    for i in range(nk):
        ua1 = (ua + 1) % NUA
        ua2 = (ua1 + 1) % NUA
        ub1 = (ub + 1) % NUB
        ubp = (ub - 1) % NUB
        # k-step 0: reads of k-step 1, second half of A(i + 2)
        w.read("A", i, ua); w.read("B", i, ub)
        A(i + 2, ua2, 1)
        # k-step 1: reads of k-step 2, first half of B(i + 3)
        w.read("A", i, ua); w.read("B", i, ub)
        B(i + NUB - 1, ubp, 0)
        # k-step 2 (before the barrier): reads of k-step 3, second half of B(i + 3)
        w.read("A", i, ua); w.read("B", i, ub)
        B(i + NUB - 1, ubp, 1)
        w.wait(LA + 2 * LB)
        w.barrier()
        # k-step 3: reads of slab i + 1's k-step 0, first half of A(i + 3)
        if i + 1 < nk:
            w.read("A", i + 1, ua1); w.read("B", i + 1, ub1)
        A(i + 3, ua, 0)
        ua, ub = ua1, ub1
    return w


@pytest.mark.parametrize("nk", range(1, 41))
def test_four_wave_ring(nk):
    check(w4_program(nk), nk)


def test_four_wave_ring_model_catches_a_short_wait():
    # the same schedule with one load fewer allowed in flight at the barrier
    # passes; with one more it must fail (the model is not vacuous)
    w = w4_program(12)
    bad = Wave()
    bad.ev = [("wait", LA + 2 * LB + 1) if e == ("wait", LA + 2 * LB) else e for e in w.ev]
    with pytest.raises(AssertionError):
        check(bad, 12)
    ok = Wave()
    ok.ev = [("wait", LA + 2 * LB - 1) if e == ("wait", LA + 2 * LB) else e for e in w.ev]
    check(ok, 12)


# ---------------------------------------------------------------------------
# The tile kernels (gemm_nt_kernel.hpp): a STAGES-deep ring, NL loads per wave
# and slab; loads issued at once after the barrier (B streamed, or two stages)
# or spread between the MFMAs of the slab (with uniform re-reads past the end).

def tile_program(nk, stages, nl, early):
    w = Wave()

    def slab_loads(i, s):
        for _ in range(nl):
            w.load("T", i, s)

    for s in range(stages - 1):
        if not early or s < nk:
            slab_loads(s, s)
    for i in range(nk):
        s = i % stages
        if early and i + stages - 2 >= nk:
            w.wait(0)
        else:
            w.wait((stages - 2) * nl)
        w.barrier()
        nxt, snx = i + stages - 1, (i + stages - 1) % stages
        if early:
            if nxt < nk:
                slab_loads(nxt, snx)
            w.read("T", i, s)
        else:
            # loads between the MFMAs of the k-steps, reads of the slab beside them
            w.read("T", i, s)
            slab_loads(nxt, snx)
            w.read("T", i, s)
    return w


@pytest.mark.parametrize("stages,nl", [(2, 8), (4, 8), (6, 5)])
@pytest.mark.parametrize("early", [True, False])
def test_tile_ring(stages, nl, early):
    if stages == 2 and not early:
        pytest.skip("two-stage rings always issue at once")
    for nk in range(1, 41):
        check(tile_program(nk, stages, nl, early), nk)


def test_tile_ring_model_catches_a_short_wait():
    w = tile_program(10, 4, 8, False)
    bad = Wave()
    bad.ev = [("wait", 2 * 8 + 1) if e == ("wait", 2 * 8) else e for e in w.ev]
    with pytest.raises(AssertionError):
        check(bad, 10)


# ---------------------------------------------------------------------------
# The ping-pong kernel (gemm_nt_pp2.hpp): two groups of waves, each with its own
# program; a workgroup barrier ends every phase, so the programs are cut into
# the same number of segments.  Group 0 loads B and reads A_0 and B; group 1
# loads A (both halves) and reads A_1 and B.  A wave's waits count its own
# loads only; a load is published at the barrier ending the segment of the
# wait that completed it.  Units: B slot s = units ("B", 2 s), ("B", 2 s + 1);
# A_0 slot s = ("A0", s), s < 2; A_1 slot s = ("A1", s), s < 3.

PP_LOADS = 8          # wave-wide loads per wave and slab (4 per half)


def pp2_programs(nk, am=False, a_exact=True, g1_wait=PP_LOADS, b_slots=2, a1_slots=3):
    """Per group, a list of segments; a segment is a list of events
    ("load", key, slab), ("wait", n), ("read", key, slab)."""
    g0, g1 = [[]], [[]]

    def b_load(seg, i):
        for half in (0, 1):
            for _ in range(PP_LOADS // 2):
                seg.append(("load", ("B", 2 * (i % b_slots) + half), i))

    def a_load(seg, i):
        for _ in range(PP_LOADS // 2):
            seg.append(("load", ("A0", i % 2), i))
        for _ in range(PP_LOADS // 2):
            seg.append(("load", ("A1", i % a1_slots), i))

    # prologue: B(0) by group 0; A(0), A(1) by group 1
    b_load(g0[-1], 0)
    g0[-1].append(("wait", 0))
    a_load(g1[-1], 0)
    if nk > 1:
        a_load(g1[-1], 1)
    g1[-1].append(("wait", g1_wait if a_exact and (nk > 2 or (nk == 2 and not am)) else 0))
    for i in range(nk):
        # phase 2i: group 0 loads B(i+1), reads A_0(i) and B(i); group 1 computes
        g0.append([])
        if i + 1 < nk:
            b_load(g0[-1], i + 1)
        g0[-1] += [("read", ("A0", i % 2), i), ("read", ("B", 2 * (i % b_slots)), i),
                   ("read", ("B", 2 * (i % b_slots) + 1), i)]
        g1.append([])
        # phase 2i+1: group 0 computes, then waits for B(i+1); group 1 loads
        # A(i+2), reads A_1(i) and B(i), waits for A(i+1)
        g0.append([("wait", 0)])
        g1.append([])
        if i + 2 < nk:
            a_load(g1[-1], i + 2)
        g1[-1] += [("read", ("A1", i % a1_slots), i), ("read", ("B", 2 * (i % b_slots)), i),
                   ("read", ("B", 2 * (i % b_slots) + 1), i)]
        exact = a_exact and (i + 3 < nk or (i + 2 < nk and not am))
        g1[-1].append(("wait", g1_wait if exact else 0))
    return g0, g1


def pp2_check(groups, nk):
    nseg = len(groups[0])
    assert all(len(g) == nseg for g in groups)
    # completion segment of every load, per group (a wait completes all but the
    # last n loads that group issued)
    published = {}          # (key, slab) -> list of segments at whose end each load is published
    for g in groups:
        issued = []         # (key, slab, segment issued)
        done = 0
        for k, seg in enumerate(g):
            for e in seg:
                if e[0] == "load":
                    issued.append((e[1], e[2]))
                elif e[0] == "wait":
                    upto = max(done, len(issued) - e[1])
                    for key, slab in issued[done:upto]:
                        published.setdefault((key, slab), []).append(k)
                    done = upto
        assert done == len(issued), "loads left in flight at the end"
    # what each unit holds, in segment order (loads of a segment land before
    # its reads by another group only if published earlier: checked below)
    last_read = {}          # (key, slab) -> latest segment it is read in
    loads_at = {}           # key -> list of (segment, slab)
    for gi, g in enumerate(groups):
        for k, seg in enumerate(g):
            for e in seg:
                if e[0] == "load":
                    loads_at.setdefault(e[1], []).append((k, e[2]))
                elif e[0] == "read":
                    last_read[(e[1], e[2])] = max(last_read.get((e[1], e[2]), -1), k)
    for gi, g in enumerate(groups):
        for k, seg in enumerate(g):
            for e in seg:
                if e[0] != "read":
                    continue
                key, slab = e[1], e[2]
                assert slab < nk
                # every load of this slab into this unit published before segment k
                segs = published.get((key, slab))
                assert segs, ("read of a slab never loaded", e)
                assert len(segs) == PP_LOADS // 2 and max(segs) <= k - 1, ("read before publication", gi, k, e, segs)
                # the unit still holds this slab: no later slab loaded into it
                # in a segment up to k
                later = [s for s, sl in loads_at[key] if sl != slab and sl > slab and s <= k]
                assert not later, ("unit overwritten before the read", gi, k, e)
    # WAR: a load into a unit only after every read of its previous slab
    for key, lst in loads_at.items():
        for k, slab in lst:
            prev = [sl for s, sl in lst if sl < slab]
            if prev:
                p = max(prev)
                assert last_read.get((key, p), -1) <= k - 1, ("load over a unit still read", key, slab, k)


@pytest.mark.parametrize("am", [False, True])
def test_ping_pong_ring(am):
    for nk in range(1, 41):
        pp2_check(pp2_programs(nk, am=am), nk)


def test_ping_pong_ring_model_catches_mistakes():
    # one load fewer allowed in flight passes; one more reads A before it lands
    pp2_check(pp2_programs(12, g1_wait=PP_LOADS - 1), 12)
    with pytest.raises(AssertionError):
        pp2_check(pp2_programs(12, g1_wait=PP_LOADS + 1), 12)
    # B with one slot, or A_1 with two, overwrites a unit that is still read
    with pytest.raises(AssertionError):
        pp2_check(pp2_programs(12, b_slots=1), 12)
    with pytest.raises(AssertionError):
        pp2_check(pp2_programs(12, a1_slots=2), 12)
