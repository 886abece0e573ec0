"""GPU parity of the decode path against the CPU oracle, through the C ABI.

Tiny model: all 47 passes (16 teacher-forced prompt tokens, then greedy),
in every execution and synchronisation mode, plus forced key-range splits.
Llama-1B shape at position 1024 and 8192: full-logit parity on the first
passes of the benchmarked configuration (same plan and launch shape as
bench.py).  Modes must agree bit for bit with each other (same ops, same
reduction orders)."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from decode_harness import LOGIT_TOL, check_kv, run_decode
from oracle import oracle as orc
from persistent_megakernel_decode_02_amd import engine, mk

pytestmark = pytest.mark.gpu

TINY = si.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def tiny_setup():
    w = si.make_weights(TINY.shape, master=0)
    return w, engine.to_gpu(w), orc.Model(TINY.shape, w)


def _run_tiny(tiny_setup, **kw):
    w, gw, model = tiny_setup
    return run_decode(TINY, TINY.steps, weights=w, gpu_weights=gw, model=model, **kw)


def test_device_is_mi355x():
    info = mk.mk_device_query(0)
    import sys
    print(f"device {info.arch.decode()} cus={info.num_cus} lds/block={info.lds_per_block} "
          f"lds/cu={info.lds_per_cu} clock={info.clock_khz}kHz mega_blocks_per_cu={info.mega_blocks_per_cu}",
          file=sys.stderr)
    assert info.arch.decode().startswith("gfx950")
    assert info.num_cus >= 1


MODES = {"mega-counter": (mk.MK_EXEC_MEGA, mk.MK_SYNC_COUNTER), "mega-flag": (mk.MK_EXEC_MEGA, mk.MK_SYNC_FLAG),
         "mega-sentinel": (mk.MK_EXEC_MEGA, mk.MK_SYNC_SENTINEL), "multi": (mk.MK_EXEC_MULTI, mk.MK_SYNC_COUNTER),
         "flat-counter": (mk.MK_EXEC_FLAT, mk.MK_SYNC_COUNTER), "flat-flag": (mk.MK_EXEC_FLAT, mk.MK_SYNC_FLAG)}


@pytest.mark.parametrize("mode", list(MODES.values()), ids=list(MODES))
def test_tiny_decode_matches_oracle(tiny_setup, mode):
    res = _run_tiny(tiny_setup, exec_mode=mode[0], sync_mode=mode[1])
    print(f"tiny {mode}: max rel logit err {res.max_rel_err:.3e}, near ties {res.near_ties}, "
          f"tokens {[t[0] for t in res.tokens]}")
    assert res.max_rel_err <= LOGIT_TOL
    assert res.max_rel_err <= 1e-4  # fp32 accumulation is far tighter than the bound
    assert res.near_ties == 0
    exact = check_kv(res)
    print(f"kv exact fraction {exact:.6f}")


@pytest.mark.parametrize("group", [("mega-counter", "mega-flag", "mega-sentinel", "multi"),
                                   ("flat-counter", "flat-flag")], ids=["roles", "flat"])
def test_tiny_modes_bit_identical(tiny_setup, group):
    # the same ops under different synchronisation / launch schemes give the same bits
    runs = [_run_tiny(tiny_setup, exec_mode=MODES[m][0], sync_mode=MODES[m][1]) for m in group]
    for r in runs[1:]:
        assert r.tokens == runs[0].tokens
        assert np.array_equal(r.logits_last, runs[0].logits_last)
        assert np.array_equal(r.kv_gpu, runs[0].kv_gpu)


@pytest.mark.parametrize("splits", [2, 5, 16])
def test_tiny_split_attention_matches_oracle(tiny_setup, splits):
    res = _run_tiny(tiny_setup, kv_splits=splits)
    assert res.max_rel_err <= 1e-4, res.max_rel_err
    assert res.near_ties == 0
    check_kv(res)


def test_tiny_host_driven_positions(tiny_setup):
    # without MK_ADVANCE the host feeds tokens and positions itself
    res = _run_tiny(tiny_setup, advance=False)
    assert res.max_rel_err <= 1e-4
    check_kv(res)


@pytest.fixture(scope="module")
def llama1b():
    wl = si.WORKLOADS["llama1b_pos1024"]
    w = si.make_weights(wl.shape, master=0)
    return w, engine.to_gpu(w), orc.Model(wl.shape, w)


@pytest.mark.parametrize("mode", ["flat-flag", "flat-counter", "mega-counter", "mega-sentinel"])
def test_llama1b_pos1024_first_passes(llama1b, mode):
    wl = si.WORKLOADS["llama1b_pos1024"]
    w, gw, model = llama1b
    res = run_decode(wl, 4, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"llama1b@1024 {mode}: errs {['%.2e' % e for e in res.per_step_err]} tokens {res.tokens}")
    assert res.max_rel_err <= LOGIT_TOL
    assert res.max_rel_err <= 1e-3
    check_kv(res)


@pytest.mark.parametrize("mode", ["flat-flag", "mega-sentinel"])
def test_llama1b_pos8192_split_attention(llama1b, mode):
    wl = si.WORKLOADS["llama1b_pos8192"]
    w, gw, model = llama1b
    res = run_decode(wl, 2, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"llama1b@8192: errs {['%.2e' % e for e in res.per_step_err]} tokens {res.tokens}")
    assert res.max_rel_err <= 1e-3
    check_kv(res)


# Batched decode (projections on the matrix cores): per-sequence context
# lengths drawn uniformly, every sequence checked against the oracle.
TINY_BATCHED = {b: si.Workload(f"tiny_b{b}", TINY.shape, batch=b, steps=6, start_pos=-1, len_lo=1, len_hi=100,
                               max_ctx=TINY.max_ctx) for b in (2, 5, 16)}


@pytest.mark.parametrize("batch", sorted(TINY_BATCHED))
@pytest.mark.parametrize("mode", ["flat-counter", "flat-flag"])
def test_tiny_batched_decode_matches_oracle(tiny_setup, batch, mode):
    wl = TINY_BATCHED[batch]
    w, gw, model = tiny_setup
    res = run_decode(wl, wl.steps, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"tiny b={batch} {mode}: max rel logit err {res.max_rel_err:.3e}, near ties {res.near_ties}")
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    check_kv(res)


def test_tiny_batched_split_attention(tiny_setup):
    wl = TINY_BATCHED[16]
    w, gw, model = tiny_setup
    res = run_decode(wl, 3, weights=w, gpu_weights=gw, model=model, exec_mode=mk.MK_EXEC_FLAT, kv_splits=4)
    assert res.max_rel_err <= 1e-3
    check_kv(res)


def test_llama1b_batch16_first_passes(llama1b):
    # the batched configuration as the benchmark runs it: 16 sequences with
    # context lengths 512..4096, FLAT engine, projections on MFMA
    wl = si.WORKLOADS["llama1b_b16"]
    w, gw, model = llama1b
    res = run_decode(wl, 2, weights=w, gpu_weights=gw, model=model, exec_mode=mk.MK_EXEC_FLAT)
    print(f"llama1b b16: errs max {res.max_rel_err:.2e} near ties {res.near_ties} tokens {res.tokens}")
    assert res.max_rel_err <= 1e-3
    print(f"kv exact fraction {check_kv(res, min_exact=0.97):.5f}")


@pytest.mark.parametrize("mode", ["mega-counter", "mega-sentinel", "multi", "flat-counter"])
def test_invalid_token_reports_input_error_and_poisons(tiny_setup, mode):
    w, gw, model = tiny_setup
    s = TINY.shape
    eng = engine.Engine(s, gw, max_batch=1, max_ctx=TINY.max_ctx, exec_mode=MODES[mode][0],
                        sync_mode=MODES[mode][1])
    try:
        kv = eng.kv_cache()
        logits = torch.empty((1, s.vocab), dtype=torch.float32, device="cuda:0")
        pos = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        bad = torch.tensor([s.vocab + 5], dtype=torch.int32, device="cuda:0")
        eng.step(bad, pos, kv, logits)
        rc, _ = eng.device_error()
        assert rc == mk.MK_ERR_INPUT
        with pytest.raises(mk.MkError) as e:
            eng.step(bad, pos, kv, logits)
        assert e.value.code == mk.MK_ERR_STATE
        eng.reset()
        good = torch.tensor([3], dtype=torch.int32, device="cuda:0")
        eng.step(good, pos, kv, logits)
        assert eng.device_error()[0] == 0
        bad_pos = torch.tensor([TINY.max_ctx], dtype=torch.int32, device="cuda:0")
        eng.step(good, bad_pos, kv, logits)
        assert eng.device_error()[0] == mk.MK_ERR_INPUT
    finally:
        eng.close()


@pytest.mark.parametrize("mode", ["mega-counter", "flat-counter"])
def test_watchdog_turns_unmet_wait_into_timeout(tiny_setup, mode):
    # the host claims more steps ran than the device counted, so the first
    # counter wait can never be met; a 2 ms watchdog ends the step cleanly.
    # (Flag and sentinel waits compare against what this step's producers
    # write, so a skipped host epoch cannot starve them.)
    w, gw, model = tiny_setup
    s = TINY.shape
    eng = engine.Engine(s, gw, max_batch=1, max_ctx=TINY.max_ctx, exec_mode=MODES[mode][0],
                        sync_mode=MODES[mode][1])
    try:
        kv = eng.kv_cache()
        logits = torch.empty((1, s.vocab), dtype=torch.float32, device="cuda:0")
        pos = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        tok = torch.tensor([3], dtype=torch.int32, device="cuda:0")
        mk.mk_ctx_set_watchdog_us(eng.ctx, 2000, eng.stream.cuda_stream)
        mk.mk_ctx_set_epoch(eng.ctx, 5)
        eng.step(tok, pos, kv, logits)
        rc, detail = eng.device_error()
        assert rc == mk.MK_ERR_TIMEOUT, rc
        eng.reset()
        mk.mk_ctx_set_watchdog_us(eng.ctx, 2_000_000, eng.stream.cuda_stream)
        eng.step(tok, pos, kv, logits)
        assert eng.device_error()[0] == 0
    finally:
        eng.close()


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5])
def test_gridsync_variants_are_correct(variant):
    info = mk.mk_device_query(0)
    n = info.num_cus
    scratch = torch.empty(mk.mk_gridsync_scratch_bytes(n) + 256, dtype=torch.uint8, device="cuda:0")
    base = (scratch.data_ptr() + 255) // 256 * 256
    res = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nb = 2000
    mk.mk_gridsync_bench(variant, 10, n, base, res.data_ptr(), st.cuda_stream)
    e0.record(st)
    mk.mk_gridsync_bench(variant, nb, n, base, res.data_ptr(), st.cuda_stream)
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / nb
    r = res.cpu().tolist()
    print(f"gridsync {mk.GRIDSYNC_VARIANTS[variant]}: {us:.2f} us/barrier at {n} blocks, errors {r[0]}, "
          f"timeouts {r[1]}, blocks off the XCD b % 8: {r[2]}")
    assert r[1] == 0
    assert r[0] == 0
