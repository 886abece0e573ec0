"""Event normalisation (the MPK scheme the megakernel page's Q&A describes:
at most one wait and one trigger event per task, events fused by
predecessor and successor sets, breadth-first numbering with the tasks one
event releases contiguous).

Random DAGs are checked against properties computed here independently
(reachability by boolean matrix closure, a brute-force transitive
reduction); small graphs against their exact expected events; the plans
mk_plan_create builds against the event structure of a decoder layer."""
import numpy as np
import pytest

import synth_inputs as si
from persistent_megakernel_decode_02_amd import mk
from test_abi_plan import SHAPES, plan_opts, shape_struct


def _closure(preds):
    n = len(preds)
    reach = np.zeros((n, n), dtype=bool)  # reach[a, b]: a precedes b
    for t, ps in enumerate(preds):
        for q in ps:
            reach[q, t] = True
    for k in range(n):  # Warshall
        reach |= np.outer(reach[:, k], reach[k, :])
    return reach


def _check_normalised(preds, out):
    n = len(preds)
    wait, trig, slot, count, order, ne = (out[k] for k in ("wait", "trigger", "slot", "count", "order", "n_events"))
    assert all(-1 <= w < ne for w in wait) and all(-1 <= g < ne for g in trig)
    # trigger counts and slots
    for e in range(ne):
        ts = [t for t in range(n) if trig[t] == e]
        assert count[e] == len(ts) > 0
        assert sorted(slot[t] for t in ts) == list(range(len(ts)))
        assert any(w == e for w in wait)  # no event without a waiter
    # every raw edge q -> t is ordered by the events: q's trigger releases t
    # or a task that precedes t
    hb = [[] for _ in range(n)]
    for t in range(n):
        if wait[t] >= 0:
            hb[t] = [q for q in range(n) if trig[q] == wait[t]]
    reach_hb = _closure(hb)
    for t, ps in enumerate(preds):
        for q in ps:
            assert reach_hb[q, t], (q, t)
    # no deadlock: the events fire in some order that runs every task
    done, remaining = [False] * n, list(count)
    ready = [t for t in range(n) if wait[t] < 0]
    while ready:
        t = ready.pop()
        done[t] = True
        if trig[t] >= 0:
            remaining[trig[t]] -= 1
            if remaining[trig[t]] == 0:
                ready += [u for u in range(n) if wait[u] == trig[t]]
    assert all(done)
    # breadth-first order: a permutation; every task after its event's
    # triggers; the waiters of one event contiguous; events fire in id order
    assert sorted(order) == list(range(n))
    pos = {t: k for k, t in enumerate(order)}
    for t in range(n):
        if wait[t] >= 0:
            assert all(pos[q] < pos[t] for q in range(n) if trig[q] == wait[t])
    firsts = []
    for e in range(ne):
        ks = sorted(pos[t] for t in range(n) if wait[t] == e)
        assert ks == list(range(ks[0], ks[0] + len(ks)))
        firsts.append(ks[0])
    assert firsts == sorted(firsts)


def _reduced(preds, reach):
    return [sorted(q for q in set(ps) if not any(reach[q, r] for r in set(ps) if r != q)) for ps in preds]


def _layered_dag(rng):
    """Tasks in layers, each with predecessors in the layer just above, plus
    skip edges that other paths already imply (the reduction removes them)."""
    n_layers = int(rng.integers(2, 7))
    layers, preds = [], []
    for k in range(n_layers):
        width = int(rng.integers(1, 9))
        ids = list(range(len(preds), len(preds) + width))
        for _ in ids:
            ps = []
            if k > 0:
                above = layers[-1]
                ps = sorted({int(x) for x in rng.choice(above, size=int(rng.integers(1, len(above) + 1)))})
            preds.append(ps)
        layers.append(ids)
    reach = _closure(preds)
    for t in range(len(preds)):
        anc = [q for q in range(len(preds)) if reach[q, t] and q not in preds[t]]
        if anc and rng.random() < 0.5:
            preds[t] = preds[t] + [int(rng.choice(anc))]
    return preds


def _permuted(preds, rng):
    n = len(preds)
    perm = rng.permutation(n)  # task ids need not be topological
    inv = np.argsort(perm)
    return [[int(perm[q]) for q in preds[int(inv[t])]] for t in range(n)]


@pytest.mark.parametrize("seed", range(16))
def test_random_layered_dags(seed):
    rng = np.random.default_rng(seed)
    preds = _permuted(_layered_dag(rng), rng)
    n = len(preds)
    rc, out = mk.mk_events_normalize(preds)
    assert rc == mk.MK_OK
    _check_normalised(preds, out)
    # tasks with the same reduced predecessors share their wait event, and an
    # event's triggers are exactly the union of its waiters' reduced
    # predecessors
    red = _reduced(preds, _closure(preds))
    for a in range(n):
        for b in range(n):
            if red[a] and red[a] == red[b]:
                assert out["wait"][a] == out["wait"][b]
    for e in range(out["n_events"]):
        union = sorted({q for t in range(n) if out["wait"][t] == e for q in red[t]})
        assert union == sorted(t for t in range(n) if out["trigger"][t] == e)


@pytest.mark.parametrize("seed", range(16))
def test_random_dags_valid_or_refused(seed):
    # arbitrary DAGs: a task whose successors sit at different depths may
    # need events that cannot be fused without a cycle; the pass must then
    # refuse, never return events that deadlock or miss a dependency
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(5, 70))
    density = rng.uniform(0.02, 0.3)
    preds = []
    for t in range(n):
        ps = [int(q) for q in range(t) if rng.random() < density]
        if ps and rng.random() < 0.3:
            ps.append(ps[0])  # duplicates are allowed
        preds.append(ps)
    preds = _permuted(preds, rng)
    rc, out = mk.mk_events_normalize(preds)
    assert rc in (mk.MK_OK, mk.MK_ERR_PLAN)
    if rc == mk.MK_OK:
        _check_normalised(preds, out)


def test_diamond_exact():
    #  0,1 -> 2,3 -> 4
    rc, out = mk.mk_events_normalize([[], [], [0, 1], [1, 0], [2, 3]])
    assert rc == mk.MK_OK
    assert out["n_events"] == 2
    assert out["wait"] == [-1, -1, 0, 0, 1] and out["trigger"] == [0, 0, 1, 1, -1]
    assert out["count"] == [2, 2] and out["order"] == [0, 1, 2, 3, 4]


def test_implied_edge_is_dropped():
    # 0 -> 1 -> 2 and 0 -> 2: task 2 waits for 1 only
    rc, out = mk.mk_events_normalize([[], [0], [0, 1]])
    assert rc == mk.MK_OK
    assert out["n_events"] == 2 and out["count"] == [1, 1]
    assert out["trigger"][0] == out["wait"][1] and out["trigger"][1] == out["wait"][2]


def test_shared_predecessor_fuses_events():
    # 0 -> 1 and {0, 2} -> 3: task 0 would trigger two events, so they fuse
    # and task 1 also waits for task 2
    rc, out = mk.mk_events_normalize([[], [0], [], [0, 2]])
    assert rc == mk.MK_OK
    assert out["n_events"] == 1 and out["count"] == [2]
    assert out["wait"] == [-1, 0, -1, 0] and out["trigger"] == [0, -1, 0, -1]
    _check_normalised([[], [0], [], [0, 2]], out)


def test_fusion_cycle_is_reported():
    # 0 -> 1 -> 2, {0, 2} -> 3.  Reduced, task 3 waits for 2 only.  Without
    # the reduction, 0 triggers for both 1 and 3: the fused event would have
    # task 1 wait for task 2, its own successor
    preds = [[], [0], [1], [0, 2]]
    rc, out = mk.mk_events_normalize(preds)
    assert rc == mk.MK_OK
    _check_normalised(preds, out)
    rc, _ = mk.mk_events_normalize(preds, flags=mk.MK_NORM_NO_REDUCTION)
    assert rc == mk.MK_ERR_PLAN


def test_bad_graphs():
    assert mk.mk_events_normalize([[1], [0]])[0] == mk.MK_ERR_PLAN   # cycle
    assert mk.mk_events_normalize([[0]])[0] == mk.MK_ERR_PLAN        # self edge
    assert mk.mk_events_normalize([[3]])[0] == mk.MK_ERR_INVALID_ARG  # no such task
    rc, out = mk.mk_events_normalize([])
    assert rc == mk.MK_OK and out["n_events"] == 0


def test_rank_breaks_ties():
    rc, out = mk.mk_events_normalize([[], [], [0, 1], [0, 1]], rank=[5, 1, 9, 3])
    assert rc == mk.MK_OK and out["order"] == [1, 0, 3, 2]


@pytest.mark.parametrize("name", ["tiny", "llama1b_pos1024", "llama1b_b16", "llama8b_pos2048"])
@pytest.mark.parametrize("exec_mode", [mk.MK_EXEC_FLAT, mk.MK_EXEC_MEGA])
def test_plan_events_are_the_decoder_dataflow(name, exec_mode):
    shape, batch, max_ctx = SHAPES[name]
    if exec_mode == mk.MK_EXEC_MEGA and batch > 4:
        pytest.skip("the role engine runs up to 4 sequences")
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256, exec_mode=exec_mode))
    try:
        d = mk.mk_plan_export(plan)
        q = mk.mk_plan_get_queue(plan)
        L, nkv, nq, hd = shape.n_layers, shape.n_kv_heads, shape.n_q_heads, shape.head_dim
        G = nq // nkv
        ne = 1 + max(x.signal_event for x in d)
        assert ne == L * (nkv + 4)  # per layer: one per kv group, attention, O, gate/up, down
        trig, waiters = {}, {}
        for i, x in enumerate(d):
            if x.signal_event >= 0:
                trig.setdefault(x.signal_event, set()).add(i)
            if x.wait_event >= 0:
                waiters.setdefault(x.wait_event, set()).add(i)

        def ids(op, layer, pred=lambda x: True):
            return {i for i, x in enumerate(d) if x.op == op and x.layer == layer and pred(x)}

        def group_of_row(r):
            if r < nq * hd:
                return r // hd // G
            return (r - nq * hd) // hd % nkv

        def one_event(waiting, triggering):
            evs = {d[i].wait_event for i in waiting}
            assert len(evs) == 1
            e = evs.pop()
            assert trig[e] == triggering and waiters[e] == waiting
            return e

        for l in range(L):
            if l > 0:
                one_event(ids(mk.MK_OP_QKV, l), ids(mk.MK_OP_DOWN, l - 1))
            else:
                assert all(d[i].wait_event < 0 for i in ids(mk.MK_OP_QKV, 0))
            for g in range(nkv):
                units = ids(mk.MK_OP_ATTN, l, lambda x: x.r1 == g)
                qkv_g = ids(mk.MK_OP_QKV, l, lambda x: group_of_row(x.r0) == g)
                evs = {d[i].wait_event for i in units}
                assert len(evs) == 1
                e = evs.pop()
                assert trig[e] == qkv_g and waiters[e] == units
            one_event(ids(mk.MK_OP_OPROJ, l), ids(mk.MK_OP_ATTN, l))
            one_event(ids(mk.MK_OP_GATEUP, l), ids(mk.MK_OP_OPROJ, l))
            one_event(ids(mk.MK_OP_DOWN, l), ids(mk.MK_OP_GATEUP, l))
        one_event({i for i, x in enumerate(d) if x.op == mk.MK_OP_LMHEAD}, ids(mk.MK_OP_DOWN, L - 1))
        # the queue: breadth-first, each event's waiters contiguous, in firing order
        assert sorted(q) == list(range(len(d)))
        pos = {i: k for k, i in enumerate(q)}
        firsts = []
        for e in range(ne):
            ks = sorted(pos[i] for i in waiters[e])
            assert ks == list(range(ks[0], ks[0] + len(ks)))
            assert max(pos[i] for i in trig[e]) < ks[0]
            firsts.append(ks[0])
        assert firsts == sorted(firsts)
        assert mk.mk_plan_validate(plan) == mk.MK_OK
    finally:
        mk.mk_plan_destroy(plan)
