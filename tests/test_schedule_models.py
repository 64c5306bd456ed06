"""Host models of the LDS ring schedules of two kernels (no GPU).

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
