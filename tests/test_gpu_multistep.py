"""Multi-token persistent decode (mk_decode_steps): several greedy steps in
one launch of the homogeneous engine, the device feeding each step's token
to the next.

Every multi-step run is compared bit for bit with the same mode's
one-launch-per-step run (same kernels, same reduction orders): logits of
every step, every greedy token and the whole KV cache afterwards.  That
per-step run is itself checked against the oracle over every step (logits,
greedy tokens, appended cache values), so the multi-step tokens are the
oracle's too.  Launch splits of 1, 7 and all steps cover a launch boundary
inside the sequence and a single launch for the whole sequence."""
import dataclasses

import numpy as np
import pytest
import torch

import synth_inputs as si
from decode_harness import check_kv, run_decode, run_multistep
from oracle import oracle as orc
from persistent_megakernel_decode_02_amd import engine, mk

pytestmark = pytest.mark.gpu

MODES = {"flat-counter": (mk.MK_EXEC_FLAT, mk.MK_SYNC_COUNTER), "flat-flag": (mk.MK_EXEC_FLAT, mk.MK_SYNC_FLAG),
         "flat-sentinel": (mk.MK_EXEC_FLAT, mk.MK_SYNC_SENTINEL)}
# the tiny model without its teacher-forced prompt: greedy from position 0
TINY_FREE = dataclasses.replace(si.WORKLOADS["tiny"], name="tiny_free", prompt_len=0, steps=40)
TINY_FREE_B3 = dataclasses.replace(TINY_FREE, name="tiny_free_b3", batch=3)

_PER_STEP = {}


@pytest.fixture(scope="module")
def tiny_setup():
    w = si.make_weights(TINY_FREE.shape, master=0)
    return w, engine.to_gpu(w), orc.Model(TINY_FREE.shape, w)


def _per_step(setup, wl, mode):
    """The one-launch-per-step run of `mode`, checked against the oracle."""
    key = (wl.name, mode)
    if key not in _PER_STEP:
        w, gw, model = setup
        res = run_decode(wl, wl.steps, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                         sync_mode=MODES[mode][1])
        assert res.max_rel_err <= 1e-3
        assert res.near_ties == 0
        # batched projections run on the matrix cores (bf16 hi/lo split): the
        # bound the batched decode tests use
        check_kv(res, max_rel_err=1e-3 if wl.batch >= 2 else 1e-4)
        _PER_STEP[key] = res
    return _PER_STEP[key]


def _same(ms, res):
    assert ms.tokens == res.tokens
    assert np.array_equal(ms.logits, np.stack(res.logits_all))
    assert np.array_equal(ms.kv_gpu, res.kv_gpu)


@pytest.mark.parametrize("chunk", [1, 7, 40])
@pytest.mark.parametrize("mode", list(MODES))
def test_tiny_multistep_bit_identical_to_per_step(tiny_setup, mode, chunk):
    res = _per_step(tiny_setup, TINY_FREE, mode)
    ms = run_multistep(TINY_FREE, TINY_FREE.steps, chunk, exec_mode=MODES[mode][0], sync_mode=MODES[mode][1],
                       gpu_weights=tiny_setup[1])
    print(f"tiny {mode}: {TINY_FREE.steps} steps in {ms.launches} launches, tokens {[t[0] for t in ms.tokens[:8]]}")
    _same(ms, res)


@pytest.mark.parametrize("mode", ["flat-counter", "flat-flag"])
def test_tiny_batched_multistep(tiny_setup, mode):
    # three sequences per step: the projections run on the matrix cores
    res = _per_step(tiny_setup, TINY_FREE_B3, mode)
    ms = run_multistep(TINY_FREE_B3, TINY_FREE_B3.steps, 40, exec_mode=MODES[mode][0], sync_mode=MODES[mode][1],
                       gpu_weights=tiny_setup[1])
    _same(ms, res)


def test_multistep_host_checks(tiny_setup):
    s = TINY_FREE.shape
    eng = engine.Engine(s, tiny_setup[1], max_batch=1, max_ctx=128, exec_mode=mk.MK_EXEC_FLAT,
                        sync_mode=mk.MK_SYNC_FLAG)
    role = engine.Engine(s, tiny_setup[1], max_batch=1, max_ctx=128, exec_mode=mk.MK_EXEC_MEGA)
    try:
        kv = eng.kv_cache()
        toks = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        pos = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        lg = torch.empty((4, 1, s.vocab), dtype=torch.float32, device="cuda:0")
        nx = torch.empty((4, 1), dtype=torch.int32, device="cuda:0")
        st = eng.stream.cuda_stream
        for n in (0, -1, mk.MK_MAX_STEPS + 1):
            assert mk.mk_decode_steps(eng.ctx, toks.data_ptr(), pos.data_ptr(), 1, kv.data_ptr(), lg.data_ptr(),
                                      nx.data_ptr(), n, st) == mk.MK_ERR_INVALID_ARG
        # a cache that is 16- but not 128-byte aligned
        big = torch.zeros(kv.numel() + 64, dtype=torch.bfloat16, device="cuda:0")
        assert mk.mk_decode_steps(eng.ctx, toks.data_ptr(), pos.data_ptr(), 1, big.data_ptr() + 16, lg.data_ptr(),
                                  nx.data_ptr(), 2, st) == mk.MK_ERR_ALIGN
        assert mk.mk_decode_steps(role.ctx, toks.data_ptr(), pos.data_ptr(), 1, kv.data_ptr(), lg.data_ptr(),
                                  nx.data_ptr(), 2, role.stream.cuda_stream) == mk.MK_ERR_UNSUPPORTED
        assert mk.mk_ctx_epoch(eng.ctx) == 0  # nothing was enqueued
    finally:
        role.close()
        eng.close()


@pytest.mark.parametrize("mode", list(MODES))
def test_multistep_stops_at_context_end(tiny_setup, mode):
    # steps from position 120 with max_ctx 128: the step at position 128 finds
    # no cache slot; the device reports an input error and the launch ends
    s = TINY_FREE.shape
    eng = engine.Engine(s, tiny_setup[1], max_batch=1, max_ctx=128, exec_mode=MODES[mode][0],
                        sync_mode=MODES[mode][1])
    try:
        kv = eng.kv_cache()
        toks = torch.tensor([5], dtype=torch.int32, device="cuda:0")
        pos = torch.tensor([120], dtype=torch.int32, device="cuda:0")
        lg = torch.empty((12, 1, s.vocab), dtype=torch.float32, device="cuda:0")
        nx = torch.empty((12, 1), dtype=torch.int32, device="cuda:0")
        eng.steps(toks, pos, kv, lg, nx, 12)
        rc, detail = eng.device_error()
        assert rc == mk.MK_ERR_INPUT, (rc, detail)
        assert int(pos.item()) == 128  # eight steps completed
        eng.reset()
        pos.fill_(0)
        eng.steps(toks, pos, kv, lg, nx, 3)  # usable again after a reset
        assert eng.device_error()[0] == 0
    finally:
        eng.close()


@pytest.fixture(scope="module")
def llama1b():
    wl = si.WORKLOADS["llama1b_pos1024"]
    w = si.make_weights(wl.shape, master=0)
    return w, engine.to_gpu(w), orc.Model(wl.shape, w)


# the benchmarked sequence: 128 passes from position 1024 in ONE launch
@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["flat-sentinel", "flat-flag"])
def test_llama1b_pos1024_one_launch(llama1b, mode):
    wl = si.WORKLOADS["llama1b_pos1024"]
    res = _per_step(llama1b, wl, mode)
    ms = run_multistep(wl, wl.steps, wl.steps, exec_mode=MODES[mode][0], sync_mode=MODES[mode][1],
                       gpu_weights=llama1b[1])
    print(f"llama1b@1024 {mode}: {wl.steps} steps in {ms.launches} launch(es)")
    _same(ms, res)
