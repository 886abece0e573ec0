"""The homogeneous engine's multi-launch baseline: one launch per dependency
level (MK_EXEC_FLAT_MULTI), enqueued per step or captured once as a hipGraph
and replayed.

Graph replays are checked against the oracle on every step (logits, greedy
tokens, appended cache values) and must be bit-identical to the same
launches enqueued one by one.  Between replays the host runs its own eager
work (feeding the token back, advancing the position) and synchronises; one
run also interleaves eagerly enqueued steps with replays, which the graph's
device-side step record has to follow."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from decode_harness import check_kv, run_decode
from oracle import oracle as orc
from persistent_megakernel_decode_02_amd import engine, mk

pytestmark = pytest.mark.gpu

TINY = si.WORKLOADS["tiny"]
LEVELS = dict(exec_mode=mk.MK_EXEC_FLAT_MULTI, sync_mode=mk.MK_SYNC_COUNTER)


@pytest.fixture(scope="module")
def tiny_setup():
    w = si.make_weights(TINY.shape, master=0)
    return w, engine.to_gpu(w), orc.Model(TINY.shape, w)


@pytest.fixture(scope="module")
def tiny_levels(tiny_setup):
    w, gw, model = tiny_setup
    return run_decode(TINY, TINY.steps, weights=w, gpu_weights=gw, model=model, advance=False, **LEVELS)


def _same(a, b):
    assert a.tokens == b.tokens
    assert all(np.array_equal(x, y) for x, y in zip(a.logits_all, b.logits_all))
    assert np.array_equal(a.kv_gpu, b.kv_gpu)


@pytest.mark.parametrize("advance", [False, True], ids=["host-feeds", "device-advance"])
def test_tiny_graph_replays_match_oracle_and_launches(tiny_setup, tiny_levels, advance):
    w, gw, model = tiny_setup
    res = run_decode(TINY, TINY.steps, weights=w, gpu_weights=gw, model=model, advance=advance, use_graph=True,
                     **LEVELS)
    assert res.max_rel_err <= 1e-4
    assert res.near_ties == 0
    check_kv(res)
    _same(res, tiny_levels)


def test_tiny_graph_with_eager_steps_between(tiny_setup, tiny_levels):
    w, gw, model = tiny_setup
    res = run_decode(TINY, TINY.steps, weights=w, gpu_weights=gw, model=model, advance=False, use_graph=True,
                     eager_steps=(0, 5, 6, 30), **LEVELS)
    _same(res, tiny_levels)


def test_tiny_graph_split_attention(tiny_setup):
    # forced key-range splits: the ticketed merge inside one level launch
    w, gw, model = tiny_setup
    res = run_decode(TINY, TINY.steps, weights=w, gpu_weights=gw, model=model, advance=False, use_graph=True,
                     kv_splits=5, **LEVELS)
    assert res.max_rel_err <= 1e-4
    check_kv(res)


def test_graph_host_checks(tiny_setup):
    s = TINY.shape
    eng = engine.Engine(s, tiny_setup[1], max_batch=1, max_ctx=128, exec_mode=mk.MK_EXEC_FLAT,
                        sync_mode=mk.MK_SYNC_FLAG)
    try:
        kv = eng.kv_cache()
        t = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        lg = torch.empty((1, s.vocab), dtype=torch.float32, device="cuda:0")
        with pytest.raises(mk.MkError) as e:  # only the per-level build is captured
            eng.graph(t, t.clone(), kv, lg)
        assert e.value.code == mk.MK_ERR_UNSUPPORTED
    finally:
        eng.close()
