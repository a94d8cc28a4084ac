"""CPU models of the two inter-wave schedules of the NVFP4 readers.

* The MLA decode's wave-pair handshake (csrc/mla_decode.hip): each wave of a
  pair owns a page image and a P slot in LDS. Step k: wait until the partner
  has published 2k (its PV of step k-1 has read this wave's image and P),
  write image and P of step k, publish 2k+1, wait for the partner's 2k+1,
  read the partner's image and P (PV), publish 2k+2. The model runs the two
  waves under many interleavings (every schedule for short runs, random and
  adversarial ones for long runs) and checks that no wait can block forever,
  that every read sees the step it expects and that no write destroys data
  the partner has still to read.

* The MLA prefill's barrier schedule (csrc/mla_prefill.hip): one barrier per
  step, three page-image buffers and outer-scale tables indexed by step mod 3,
  P and shift exchange slots indexed by step mod 2. Within one barrier
  interval the waves are unordered, so the model checks the schedule
  statically: a slot read in interval i holds the step the reader expects
  (written in an earlier interval, not overwritten since) and no slot is
  written in the interval in which another wave reads or writes it.

These are models of the kernels' orderings, written from the kernels'
comments; the GPU tests check the kernels' results.
"""
import random

import pytest


# ---------------------------------------------------------------- decode pair

class PairModel:
    """Two waves with their program counters over the handshake protocol."""

    def __init__(self, nsteps):
        self.n = nsteps
        self.flag = [0, 0]
        self.image = [None, None]     # step whose rows/P a wave's slot holds
        self.pc = [0, 0]              # index into the op list
        self.ops = self._program()
        self.errors = []

    def _program(self):
        ops = []
        for k in range(self.n):
            ops += [("wait", 2 * k), ("write", k), ("publish", 2 * k + 1),
                    ("wait", 2 * k + 1), ("read", k), ("publish", 2 * k + 2)]
        return ops

    def runnable(self, w):
        if self.pc[w] >= len(self.ops):
            return False
        op, v = self.ops[self.pc[w]]
        return op != "wait" or self.flag[1 - w] >= v

    def step(self, w):
        op, v = self.ops[self.pc[w]]
        p = 1 - w
        if op == "write":
            # the partner must have read the previous step's contents
            if self.image[w] is not None and self.flag[p] < 2 * self.image[w] + 2:
                self.errors.append("wave %d overwrote step %d before the partner read it" % (w, self.image[w]))
            self.image[w] = v
        elif op == "read":
            if self.image[p] != v:
                self.errors.append("wave %d read step %s, expected %d" % (w, self.image[p], v))
        elif op == "publish":
            assert v > self.flag[w]
            self.flag[w] = v
        self.pc[w] += 1

    def done(self):
        return all(pc >= len(self.ops) for pc in self.pc)


def run_schedule(n, choose):
    m = PairModel(n)
    while not m.done():
        ready = [w for w in (0, 1) if m.runnable(w)]
        assert ready, "deadlock at pcs %s flags %s" % (m.pc, m.flag)
        m.step(choose(m, ready))
    assert not m.errors, m.errors[:3]
    return m


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
def test_pair_handshake_every_interleaving(n):
    """Every interleaving of the two waves for runs of up to 8 steps: the
    reachable states (program counters, counters, slot contents) are explored
    exhaustively, so every schedule's transitions are checked once."""
    def key(m):
        return (tuple(m.pc), tuple(m.flag), tuple(m.image))
    start = PairModel(n)
    seen = {key(start)}
    todo = [start]
    finals = 0
    while todo:
        m = todo.pop()
        if m.done():
            finals += 1
            continue
        ready = [w for w in (0, 1) if m.runnable(w)]
        assert ready, "deadlock at pcs %s flags %s" % (m.pc, m.flag)
        for w in ready:
            c = PairModel(n)
            c.flag, c.image, c.pc = list(m.flag), list(m.image), list(m.pc)
            c.step(w)
            assert not c.errors, c.errors[:3]
            if key(c) not in seen:
                seen.add(key(c))
                todo.append(c)
    assert finals == 1 and len(seen) > 2 * len(start.ops)


@pytest.mark.parametrize("n", list(range(1, 65)))
def test_pair_handshake_random_and_adversarial(n):
    """1-64 steps: random interleavings, one wave always first, and the
    laggard-first order."""
    rng = random.Random(n)
    for _ in range(20):
        run_schedule(n, lambda m, ready: rng.choice(ready))
    for first in (0, 1):
        run_schedule(n, lambda m, ready, f=first: f if f in ready else ready[0])
    run_schedule(n, lambda m, ready: min(ready, key=lambda w: m.pc[w]))
    run_schedule(n, lambda m, ready: max(ready, key=lambda w: m.pc[w]))


def test_pair_model_catches_a_missing_wait():
    """The model is not vacuous: dropping the 2k wait lets a wave overwrite
    rows its partner has not read."""
    m = PairModel(3)
    m.ops = [op for op in m.ops if not (op[0] == "wait" and op[1] % 2 == 0 and op[1] > 0)]
    # wave 0 runs ahead as far as it can
    while not m.done():
        ready = [w for w in (0, 1) if m.runnable(w)]
        m.step(0 if 0 in ready else ready[0])
    assert m.errors


# ----------------------------------------------------------- prefill barriers

WAVES = 8


def prefill_schedule(nsteps):
    """Barrier intervals of the prefill kernel as lists of
    (wave, 'r'|'w', slot, step). Slots: ('img', buf), ('s2', buf),
    ('xp', parity, owner), ('xs', parity, owner), ('fin', owner).
    The prologue dequantizes steps 0 and 1 and runs the softmax of step 0;
    interval k then holds PV of step k (reads its image and both P slots of
    the pair), the dequant of step k+2 and the softmax of step k+1."""
    intervals = []
    if nsteps == 0:
        return intervals
    iv = []
    for s in range(min(2, nsteps)):
        for w in range(WAVES):
            iv += [(w, "w", ("img", s % 3), s), (w, "w", ("s2", s % 3), s)]
    intervals.append(iv)
    iv = []
    for w in range(WAVES):
        iv += [(w, "r", ("img", 0), 0), (w, "r", ("s2", 0), 0),
               (w, "w", ("xp", 0, w), 0), (w, "w", ("xs", 0, w), 0)]
    intervals.append(iv)
    for k in range(nsteps):
        iv = []
        for w in range(WAVES):
            partner = w ^ 1
            iv += [(w, "r", ("img", k % 3), k),
                   (w, "r", ("xp", k & 1, w), k), (w, "r", ("xp", k & 1, partner), k),
                   (w, "r", ("xs", k & 1, partner), k)]
            if k + 2 < nsteps:
                iv += [(w, "w", ("img", (k + 2) % 3), k + 2), (w, "w", ("s2", (k + 2) % 3), k + 2)]
            if k + 1 < nsteps:
                s = k + 1
                iv += [(w, "r", ("img", s % 3), s), (w, "r", ("s2", s % 3), s),
                       (w, "w", ("xp", s & 1, w), s), (w, "w", ("xs", s & 1, w), s)]
        intervals.append(iv)
    # the row sums go where the P exchange was, behind a barrier, and are
    # read behind another
    intervals.append([(w, "w", ("fin", w), -1) for w in range(WAVES)])
    intervals.append([(w, "r", ("fin", w ^ 1), -1) for w in range(WAVES)]
                     + [(w, "r", ("fin", w), -1) for w in range(WAVES)])
    return intervals


def check_barrier_schedule(intervals, alias=None):
    """Static check; alias maps a slot to every slot sharing its storage."""
    alias = alias or (lambda slot: [slot])
    content = {}
    for i, iv in enumerate(intervals):
        written = set()
        for w, kind, slot, step in iv:
            if kind == "w":
                written.update(alias(slot))
        for w, kind, slot, step in iv:
            if kind == "r":
                assert not (set(alias(slot)) & written), \
                    "interval %d: wave %d reads %s while it is written" % (i, w, slot)
                if step >= 0:
                    assert content.get(slot) == step, \
                        "interval %d: wave %d reads %s expecting step %d, holds %s" % (i, w, slot, step, content.get(slot))
        for w, kind, slot, step in iv:
            if kind == "w":
                for st in alias(slot):
                    content[st] = step if st == slot else None


def fin_alias(slot):
    # the row sums reuse the bytes of the P exchange slots of parity 0
    if slot[0] == "fin":
        return [slot, ("xp", 0, slot[1])]
    if slot[:2] == ("xp", 0):
        return [slot, ("fin", slot[2])]
    return [slot]


@pytest.mark.parametrize("nsteps", list(range(0, 65)))
def test_prefill_barrier_schedule(nsteps):
    check_barrier_schedule(prefill_schedule(nsteps), alias=fin_alias)


def test_prefill_model_catches_two_image_buffers():
    """With two image buffers the dequant of step k+2 would land on the image
    PV of step k reads in the same interval."""
    sched = prefill_schedule(6)
    # re-index the buffers by step mod 2
    bad = []
    for iv in sched:
        nv = []
        for (w, kind, slot, step) in iv:
            if slot[0] in ("img", "s2") and step >= 0:
                slot = (slot[0], step % 2)
            nv.append((w, kind, slot, step))
        bad.append(nv)
    with pytest.raises(AssertionError):
        check_barrier_schedule(bad, alias=fin_alias)
