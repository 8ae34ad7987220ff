"""The offloaded step's stream schedule, checked on the host.

A small model of the three streams: ops run in issue order on their stream
(STREAM[kind]), and a wait makes an op follow another.  Every pair of ops that
touch the same buffer, one of them writing, must be ordered by those two
relations, in the order the step means (copy-in, compute, copy-out of one
micro-bucket; all of a slot's users one after the other; the previous step
before the next).  Waits are implemented with one event per (kind, slot), so
each wait must name the op that last recorded that event when the wait is
issued."""
import itertools

import pytest

from newton_schulz_amd.offload import KINDS, STREAM, Op, offload_schedule


def accesses(op: Op):
    """(resource, writes) pairs of one op.  Device slot buffers: gradient G,
    momentum M, update U (with its sum-of-squares partials).  Host buffers
    per micro-bucket: gradient hg, momentum hm, update hu; device master W."""
    s, i = op.slot, op.bucket
    return {
        "h2d": [(("G", s), True), (("M", s), True), (("hg", i), False), (("hm", i), False)],
        "mom": [(("G", s), False), (("M", s), True), (("U", s), True)],
        "d2h_mom": [(("M", s), False), (("hm", i), True)],
        "nsa": [(("U", s), True), (("W", i), True)],
        "d2h_upd": [(("U", s), False), (("hu", i), True)],
    }[op.kind]


def build(steps_ops, slots):
    """Issue-ordered node list over several steps, with the start/end syncs
    the executor adds, and the happens-before closure."""
    nodes, preds = [], []
    last_on = {}
    ev = {}          # (kind, slot) -> node index of the op that last recorded it
    for t, ops in enumerate(steps_ops):
        start = len(nodes)
        nodes.append(("start", t, None))
        preds.append({last_on["main"]} if "main" in last_on else set())
        last_on["main"] = start
        for st in ("h2d", "d2h"):
            last_on.setdefault(st, None)
        first_on = {"h2d": True, "d2h": True}
        for op in ops:
            idx = len(nodes)
            st = STREAM[op.kind]
            p = set()
            if last_on.get(st) is not None:
                p.add(last_on[st])
            if st != "main" and first_on[st]:
                p.add(start)
                first_on[st] = False
            for kind, j in op.waits:
                key = (kind, j % slots)
                assert key in ev, f"{op} waits for {kind} {j}, which was never recorded"
                k = ev[key]
                assert nodes[k][0] == "op" and nodes[k][2].bucket == j and nodes[k][1] == t, (
                    f"{op} waits on the event of {kind} {j}, but it holds {nodes[k]}")
                p.add(k)
            nodes.append(("op", t, op))
            preds.append(p)
            last_on[st] = idx
            ev[(op.kind, op.slot)] = idx
        if ops:
            end = len(nodes)
            last_d2h = ev[("d2h_upd", ops[-1].slot)]
            assert nodes[last_d2h][2] == [o for o in ops if STREAM[o.kind] == "d2h"][-1]
            nodes.append(("end", t, None))
            preds.append({last_on["main"], last_d2h})
            last_on["main"] = end
    # transitive closure (nodes are in issue order and every predecessor was
    # issued earlier, so one forward pass suffices)
    before = []
    for i, p in enumerate(preds):
        assert all(q < i for q in p), "a wait names an op issued later: possible deadlock"
        b = set(p)
        for q in p:
            b |= before[q]
        before.append(b)
    return nodes, before


def check(steps_ops, slots):
    nodes, before = build(steps_ops, slots)
    ops = [(i, n) for i, n in enumerate(nodes) if n[0] == "op"]
    rank = {"h2d": 0, "mom": 1, "d2h_mom": 2, "nsa": 2, "d2h_upd": 3}
    for (i, (_, ti, a)), (j, (_, tj, b)) in itertools.combinations(ops, 2):
        ra, rb = dict(accesses(a)), dict(accesses(b))
        shared = [r for r in ra if r in rb and (ra[r] or rb[r])]
        if not shared:
            continue
        # the order the step means: by step, then (for a slot's buffers) by
        # micro-bucket, then copy-in < compute < copy-out
        ka = (ti, a.bucket, rank[a.kind])
        kb = (tj, b.bucket, rank[b.kind])
        if ka < kb:
            assert i in before[j], f"{a} (step {ti}) and {b} (step {tj}) race on {shared}"
        else:
            assert j in before[i], f"{b} (step {tj}) and {a} (step {ti}) race on {shared}"


@pytest.mark.parametrize("n,slots", [(1, 1), (1, 2), (2, 2), (5, 1), (5, 2), (15, 2), (7, 3), (3, 5)])
def test_schedule_is_race_free(n, slots):
    ops = offload_schedule(n, slots)
    # every micro-bucket once per stage, in its slot
    for kind in KINDS:
        assert [o.bucket for o in ops if o.kind == kind] == list(range(n))
    assert all(o.slot == o.bucket % slots for o in ops)
    check([ops, ops], slots)


@pytest.mark.parametrize("n,slots", [(6, 2), (9, 3)])
def test_inflight_bound(n, slots):
    """At most `slots` micro-buckets are between their copy-in and the end of
    their update's copy-out at any point of the issue order, and the copy-in
    runs slots - 1 micro-buckets ahead of the compute."""
    ops = offload_schedule(n, slots)
    live = set()
    for k, o in enumerate(ops):
        if o.kind == "h2d":
            live.add(o.bucket)
            assert len(live) <= slots
        elif o.kind == "d2h_upd":
            live.discard(o.bucket)
        elif o.kind == "mom":
            h2d_issued = [p.bucket for p in ops[:k] if p.kind == "h2d"]
            assert max(h2d_issued) == min(o.bucket + slots - 1, n - 1)


def test_one_slot_is_serial():
    ops = offload_schedule(4, 1)
    assert [(o.kind, o.bucket) for o in ops] == [
        (k, i) for i in range(4) for k in ("h2d", "mom", "d2h_mom", "nsa", "d2h_upd")]


def test_momentum_leaves_before_newton_schulz_ends():
    """The slot's momentum is released by its copy-out, which waits only for
    the momentum kernel: the next copy-in into the slot never waits for the
    update's copy-out."""
    for o in offload_schedule(8, 2):
        if o.kind == "h2d":
            assert all(k in ("mom", "d2h_mom") for k, _ in o.waits)
        if o.kind == "d2h_mom":
            assert o.waits == (("mom", o.bucket),)


def test_checker_catches_planted_mistakes():
    """The model must reject a schedule that drops the slot-reuse wait, the
    compute's wait for its copy-in or for the slot's last update copy-out,
    the momentum copy-out's wait for the momentum kernel, or one that waits
    for an op issued later."""
    ops = offload_schedule(6, 2)
    no_reuse_wait = [o._replace(waits=()) if o.kind == "h2d" else o for o in ops]
    with pytest.raises(AssertionError, match="race"):
        check([no_reuse_wait], 2)
    no_copy_wait = [o._replace(waits=o.waits[1:]) if o.kind == "mom" else o for o in ops]
    with pytest.raises(AssertionError, match="race"):
        check([no_copy_wait], 2)
    no_update_wait = [o._replace(waits=o.waits[:1]) if o.kind == "mom" else o for o in ops]
    with pytest.raises(AssertionError, match="race"):
        check([no_update_wait], 2)
    early_mom_copy = [o._replace(waits=()) if o.kind == "d2h_mom" else o for o in ops]
    with pytest.raises(AssertionError, match="race"):
        check([early_mom_copy], 2)
    # copy-in of micro-bucket 3 issued before the copy-out of 1 it waits for
    i3 = next(k for k, o in enumerate(ops) if o.kind == "h2d" and o.bucket == 3)
    early = ops[:]
    op = early.pop(i3)
    early.insert(1, op)
    with pytest.raises(AssertionError):
        check([early], 2)
    with pytest.raises(ValueError):
        offload_schedule(3, 0)


def test_inflight_must_be_positive():
    """Both steps reject zero micro-buckets in flight before touching a GPU."""
    from newton_schulz_amd import MuonStep
    from newton_schulz_amd.offload import MuonOffloadStep
    for cls in (MuonStep, MuonOffloadStep):
        with pytest.raises(ValueError, match="inflight"):
            cls([(8, 8, 0)], "cuda:0", inflight=0)
