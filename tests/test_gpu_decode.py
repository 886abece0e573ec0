"""GPU parity of the decode path against the CPU oracle, through the C ABI.

Tiny model: all 47 passes (16 teacher-forced prompt tokens, then greedy),
in every execution and synchronisation mode, plus forced key-range splits,
host-driven positions, a NaN-filled cache and a batch below the plan's bound.
Llama-1B shape: every pass of the benchmarked sequences (128 from position
1024 in every engine, 64 from 8192 with split attention), and 8 passes of
16 sequences with context lengths 512..4096, in the plan and launch shape
bench.py times.  Modes of one engine must agree bit for bit with each other
(same ops, same reduction orders).  Error paths: bad inputs, the watchdog, a
grid wider than the device, misaligned pointers."""
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
         "flat-counter": (mk.MK_EXEC_FLAT, mk.MK_SYNC_COUNTER), "flat-flag": (mk.MK_EXEC_FLAT, mk.MK_SYNC_FLAG),
         "flat-sentinel": (mk.MK_EXEC_FLAT, mk.MK_SYNC_SENTINEL),
         "flat-levels": (mk.MK_EXEC_FLAT_MULTI, mk.MK_SYNC_COUNTER),
         "queue-counter": (mk.MK_EXEC_QUEUE, mk.MK_SYNC_COUNTER), "queue-flag": (mk.MK_EXEC_QUEUE, mk.MK_SYNC_FLAG),
         "stream-counter": (mk.MK_EXEC_STREAM, mk.MK_SYNC_COUNTER),
         "stream-flag": (mk.MK_EXEC_STREAM, mk.MK_SYNC_FLAG)}


@pytest.mark.parametrize("mode", list(MODES.values()), ids=list(MODES))
def test_tiny_decode_matches_oracle(tiny_setup, mode):
    res = _run_tiny(tiny_setup, exec_mode=mode[0], sync_mode=mode[1])
    print(f"tiny {mode}: max rel logit err {res.max_rel_err:.3e}, near ties {res.near_ties}, "
          f"tokens {[t[0] for t in res.tokens]}")
    assert res.max_rel_err <= LOGIT_TOL
    assert res.max_rel_err <= 1e-4  # fp32 accumulation is far tighter than the bound
    assert res.near_ties == 0
    print(f"kv exact fraction {check_kv(res):.6f}")


@pytest.mark.parametrize("group", [("mega-counter", "mega-flag", "mega-sentinel", "multi"),
                                   ("flat-counter", "flat-flag", "flat-sentinel"),
                                   ("stream-counter", "stream-flag"), ("flat-levels", "queue-counter", "queue-flag")],
                         ids=["roles", "flat", "stream", "queue"])
def test_tiny_modes_bit_identical(tiny_setup, group):
    # the same ops under different synchronisation / launch schemes give the same bits
    runs = [_run_tiny(tiny_setup, exec_mode=MODES[m][0], sync_mode=MODES[m][1]) for m in group]
    for r in runs[1:]:
        assert r.tokens == runs[0].tokens
        assert np.array_equal(r.logits_last, runs[0].logits_last)
        assert np.array_equal(r.kv_gpu, runs[0].kv_gpu)


@pytest.mark.parametrize("splits", [2, 5, 16])
@pytest.mark.parametrize("mode", ["mega-counter", "stream-flag"])
def test_tiny_split_attention_matches_oracle(tiny_setup, splits, mode):
    res = _run_tiny(tiny_setup, kv_splits=splits, exec_mode=MODES[mode][0], sync_mode=MODES[mode][1])
    assert res.max_rel_err <= 1e-4, res.max_rel_err
    assert res.near_ties == 0
    check_kv(res)


def test_tiny_host_driven_positions(tiny_setup):
    # without MK_ADVANCE the host feeds tokens and positions itself
    res = _run_tiny(tiny_setup, advance=False)
    assert res.max_rel_err <= 1e-4
    check_kv(res)


# Tiny model with every not-yet-written cache slot holding a NaN bit
# pattern: attention reads only slots [0, p]; padding rows of a key block
# must not carry the stale NaN of slot p into the value product.
@pytest.mark.parametrize("mode", ["flat-flag", "mega-counter", "stream-flag"])
def test_tiny_nan_filled_cache(tiny_setup, mode):
    res = _run_tiny(tiny_setup, exec_mode=MODES[mode][0], sync_mode=MODES[mode][1], kv_fill=0x7FC1)
    assert np.isfinite(res.logits_last).all()
    assert res.max_rel_err <= 1e-4
    check_kv(res)


@pytest.fixture(scope="module")
def llama1b():
    wl = si.WORKLOADS["llama1b_pos1024"]
    w = si.make_weights(wl.shape, master=0)
    return w, engine.to_gpu(w), orc.Model(wl.shape, w)


# Llama-1B shape at position 1024: every generated token of the benchmarked
# sequence (128 passes), in every engine; the oracle trajectory is computed
# once and shared by the modes whose tokens agree.
@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["stream-flag", "stream-counter", "flat-flag", "flat-counter", "flat-sentinel",
                                  "flat-levels", "queue-flag", "mega-counter",
                                  "mega-flag", "mega-sentinel", "multi"])
def test_llama1b_pos1024_full_sequence(llama1b, mode):
    wl = si.WORKLOADS["llama1b_pos1024"]
    w, gw, model = llama1b
    res = run_decode(wl, wl.steps, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"llama1b@1024 {mode}: {wl.steps} passes, max err {res.max_rel_err:.2e}, near ties {res.near_ties}, "
          f"tokens {[t[0] for t in res.tokens[:8]]}...")
    assert res.max_rel_err <= LOGIT_TOL
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    print(f"kv exact fraction {check_kv(res):.6f}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["stream-flag", "flat-flag", "flat-sentinel", "mega-sentinel"])
def test_llama1b_pos8192_full_sequence(llama1b, mode):
    # long context: split attention over the key range, 64 passes
    wl = si.WORKLOADS["llama1b_pos8192"]
    w, gw, model = llama1b
    res = run_decode(wl, wl.steps, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"llama1b@8192 {mode}: max err {res.max_rel_err:.2e}, near ties {res.near_ties}")
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    print(f"kv exact fraction {check_kv(res):.6f}")


# Batched decode (projections on the matrix cores): per-sequence context
# lengths drawn uniformly, every sequence checked against the oracle.
TINY_BATCHED = {b: si.Workload(f"tiny_b{b}", TINY.shape, batch=b, steps=6, start_pos=-1, len_lo=1, len_hi=100,
                               max_ctx=TINY.max_ctx) for b in (2, 4, 5, 16)}


@pytest.mark.parametrize("batch", [2, 5, 16])
@pytest.mark.parametrize("mode", ["flat-counter", "flat-flag", "queue-flag"])
def test_tiny_batched_decode_matches_oracle(tiny_setup, batch, mode):
    wl = TINY_BATCHED[batch]
    w, gw, model = tiny_setup
    res = run_decode(wl, wl.steps, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"tiny b={batch} {mode}: max rel logit err {res.max_rel_err:.3e}, near ties {res.near_ties}")
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    print(f"kv exact fraction {check_kv(res, max_rel_err=1e-3):.5f}")


# Wider FFNs at batch size >= 2.  Width 4608: the batched down projection
# stages its input in three 2048-column chunks (the last one ragged, 512
# columns).  Width 6144: each down slice is split by input columns into three
# parts of one chunk, merged by the last part to finish (ticket).
WIDE = {ffn: si.ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=ffn, vocab=4096)
        for ffn in (4608, 6144)}


@pytest.fixture(scope="module", params=[4608, 6144])
def wide_setup(request):
    s = WIDE[request.param]
    w = si.make_weights(s, master=3)
    return s, w, engine.to_gpu(w), orc.Model(s, w)


@pytest.mark.parametrize("batch", [3, 16])
@pytest.mark.parametrize("mode", ["flat-counter", "flat-flag", "queue-flag", "flat-levels"])
def test_tiny_wide_ffn_batched_decode_matches_oracle(wide_setup, batch, mode):
    s, w, gw, model = wide_setup
    wl = si.Workload(f"wide{s.ffn}_b{batch}", s, batch=batch, steps=4, start_pos=-1, len_lo=1, len_hi=100,
                     max_ctx=TINY.max_ctx)
    res = run_decode(wl, wl.steps, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"wide ffn={s.ffn} b={batch} {mode}: max rel logit err {res.max_rel_err:.3e}, near ties {res.near_ties}")
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    check_kv(res, max_rel_err=1e-3)


@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("mode", ["flat-counter", "flat-flag", "queue-flag"])
def test_tiny_wide_ffn_batch_below_plan_bound(wide_setup, batch, mode):
    # a plan for 4 sequences stepped with 1 or 2: with one sequence the
    # projections take the vector path, except a down slice split by input
    # columns, which still runs as parts merged by the last one
    s, w, gw, model = wide_setup
    wl = si.Workload(f"wide{s.ffn}_b4", s, batch=4, steps=3, start_pos=-1, len_lo=1, len_hi=100,
                     max_ctx=TINY.max_ctx)
    res = run_decode(wl, 3, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1], batch=batch, max_batch=4)
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    check_kv(res, max_rel_err=1e-3)
    assert np.array_equal(res.kv_gpu[:, :, batch:], res.kv_before[:, :, batch:])


def test_tiny_batched_split_attention(tiny_setup):
    wl = TINY_BATCHED[16]
    w, gw, model = tiny_setup
    res = run_decode(wl, 3, weights=w, gpu_weights=gw, model=model, exec_mode=mk.MK_EXEC_FLAT, kv_splits=4)
    assert res.max_rel_err <= 1e-3
    check_kv(res, max_rel_err=1e-3)


def test_tiny_batched_nan_filled_cache(tiny_setup):
    wl = TINY_BATCHED[5]
    w, gw, model = tiny_setup
    res = run_decode(wl, 4, weights=w, gpu_weights=gw, model=model, exec_mode=mk.MK_EXEC_FLAT,
                     sync_mode=mk.MK_SYNC_FLAG, kv_fill=0xFFC3)
    assert np.isfinite(res.logits_last).all()
    assert res.max_rel_err <= 1e-3
    check_kv(res, max_rel_err=1e-3)


# A plan for 4 sequences stepped with 2: the sequence slots past the batch
# are neither read nor written (their caches stay byte-identical).
@pytest.mark.parametrize("mode", ["flat-flag", "flat-counter", "mega-counter", "mega-sentinel"])
def test_batch_below_plan_bound_leaves_other_slots_alone(tiny_setup, mode):
    wl = TINY_BATCHED[4]
    w, gw, model = tiny_setup
    for splits in (0, 3):
        res = run_decode(wl, 4, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                         sync_mode=MODES[mode][1], batch=2, max_batch=4, kv_splits=splits)
        assert res.max_rel_err <= 1e-3
        assert res.near_ties == 0
        check_kv(res, max_rel_err=1e-3)
        assert np.array_equal(res.kv_gpu[:, :, 2:], res.kv_before[:, :, 2:])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["flat-flag", "flat-counter"])
def test_llama1b_batch16(llama1b, mode):
    # the batched configuration as the benchmark runs it: 16 sequences with
    # context lengths 512..4096, projections on MFMA; 8 passes
    wl = si.WORKLOADS["llama1b_b16"]
    w, gw, model = llama1b
    res = run_decode(wl, 8, weights=w, gpu_weights=gw, model=model, exec_mode=MODES[mode][0],
                     sync_mode=MODES[mode][1])
    print(f"llama1b b16 {mode}: errs max {res.max_rel_err:.2e} near ties {res.near_ties}")
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    print(f"kv exact fraction {check_kv(res, max_rel_err=1e-3):.5f}")


@pytest.mark.parametrize("mode", ["mega-counter", "mega-sentinel", "multi", "flat-counter", "flat-sentinel",
                                  "stream-flag"])
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


@pytest.mark.parametrize("mode", ["mega-counter", "flat-counter", "stream-counter"])
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


@pytest.mark.parametrize("exec_mode", [mk.MK_EXEC_FLAT, mk.MK_EXEC_MEGA, mk.MK_EXEC_STREAM])
def test_plan_wider_than_the_device_is_refused(exec_mode):
    # persistence needs every workgroup resident at once: a plan for twice
    # the device's CUs must be refused before anything is launched
    info = mk.mk_device_query(0)
    s = TINY.shape
    plan = mk.mk_plan(engine.shape_struct(s), engine.plan_opts(1, TINY.max_ctx, exec_mode=exec_mode,
                                                               num_cus=2 * info.num_cus))
    try:
        ws, _, _, _ = mk.mk_plan_sizes(plan)
        buf = torch.empty(ws + 256, dtype=torch.uint8, device="cuda:0")
        base = (buf.data_ptr() + 255) // 256 * 256
        with pytest.raises(mk.MkError) as e:
            mk.mk_ctx_create(plan, base, ws, torch.cuda.current_stream().cuda_stream)
        assert e.value.code == mk.MK_ERR_NOT_RESIDENT
    finally:
        mk.mk_plan_destroy(plan)


def test_misaligned_pointers_are_refused(tiny_setup):
    w, gw, model = tiny_setup
    s = TINY.shape
    eng = engine.Engine(s, gw, max_batch=1, max_ctx=TINY.max_ctx, exec_mode=mk.MK_EXEC_FLAT,
                        sync_mode=mk.MK_SYNC_FLAG)
    try:
        st = eng.stream.cuda_stream
        # a weight tensor 2 bytes off its 16-byte alignment
        raw = torch.empty(gw["layers"][0]["wq"].numel() + 8, dtype=torch.bfloat16, device="cuda:0")
        shifted = raw[1:1 + gw["layers"][0]["wq"].numel()].view(gw["layers"][0]["wq"].shape)
        bad = dict(gw)
        bad["layers"] = [dict(ld) for ld in gw["layers"]]
        bad["layers"][1]["wq"] = shifted
        with pytest.raises(mk.MkError) as e:
            eng._bind(bad)
        assert e.value.code == mk.MK_ERR_ALIGN
        eng._bind(gw)  # the previous binding still works
        kv = eng.kv_cache()
        kv_raw = torch.zeros(kv.numel() + 8, dtype=torch.bfloat16, device="cuda:0")
        logits = torch.empty((1, s.vocab), dtype=torch.float32, device="cuda:0")
        pos = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        tok = torch.tensor([3], dtype=torch.int32, device="cuda:0")
        rc = mk.mk_decode_step(eng.ctx, tok.data_ptr(), pos.data_ptr(), 1, kv_raw.data_ptr() + 2, logits.data_ptr(),
                               None, 0, st)
        assert rc == mk.MK_ERR_ALIGN
        rc = mk.mk_decode_step(eng.ctx, tok.data_ptr(), pos.data_ptr(), 1, kv.data_ptr(), logits.data_ptr() + 2,
                               None, 0, st)
        assert rc == mk.MK_ERR_ALIGN
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
