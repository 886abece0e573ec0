"""The allocation-free context (mk_ctx_create_scratch): its workspace is the
library's static device array.  Checked against the ordinary context
(mk_ctx_create with a caller workspace) on the same inputs: logits, greedy
tokens and the KV cache must be bit-identical (same plan, same kernels), on
two contexts in a row, the second with a smaller input (fewer sequences and
a shorter cache), which re-initialises the shared array."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from persistent_megakernel_decode_02_amd import engine, mk

pytestmark = pytest.mark.gpu

TINY = si.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def tiny_gpu():
    return engine.to_gpu(si.make_weights(TINY.shape, master=0))


def _decode(gw, batch, max_ctx, exec_mode, sync_mode, scratch, steps=5):
    s = TINY.shape
    eng = engine.Engine(s, gw, max_batch=batch, max_ctx=max_ctx, exec_mode=exec_mode, sync_mode=sync_mode,
                        scratch=scratch)
    try:
        lens = [3 + 7 * b for b in range(batch)]
        kv = si.make_kv_cache(s, batch, max_ctx, lens, master=1).to("cuda:0")
        toks = torch.tensor(si.uniform_ints(batch, 0, s.vocab, 2, "noalloc/tokens"), dtype=torch.int32,
                            device="cuda:0")
        pos = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
        logits = torch.empty((batch, s.vocab), dtype=torch.float32, device="cuda:0")
        nxt = torch.empty(batch, dtype=torch.int32, device="cuda:0")
        out_logits, out_tokens = [], []
        for _ in range(steps):
            eng.step(toks, pos, kv, logits, nxt, advance=True)
            rc, det = eng.device_error()
            assert rc == 0, (rc, det)
            out_logits.append(logits.cpu().numpy().copy())
            out_tokens.append(nxt.cpu().numpy().copy())
        return out_logits, out_tokens, kv.view(torch.int16).cpu().numpy()
    finally:
        eng.close()


@pytest.mark.parametrize("mode", [(mk.MK_EXEC_FLAT, mk.MK_SYNC_FLAG), (mk.MK_EXEC_STREAM, mk.MK_SYNC_FLAG)],
                         ids=["flat-flag", "stream-flag"])
def test_scratch_context_matches_workspace_context(tiny_gpu, mode):
    # two calls in a row on the shared array, the second with a smaller input
    cases = [(1, 128), (1, 64)] if mode[0] == mk.MK_EXEC_STREAM else [(4, 128), (2, 64)]
    for batch, max_ctx in cases:
        ref = _decode(tiny_gpu, batch, max_ctx, *mode, scratch=False)
        got = _decode(tiny_gpu, batch, max_ctx, *mode, scratch=True)
        for a, b in zip(ref[0], got[0]):
            assert np.array_equal(a, b)
        for a, b in zip(ref[1], got[1]):
            assert np.array_equal(a, b)
        assert np.array_equal(ref[2], got[2])


def test_scratch_limits_and_replacement(tiny_gpu):
    s = TINY.shape
    # a plan whose workspace exceeds the static array is refused before any device work
    big = si.WORKLOADS["llama1b_b16"]
    plan = mk.mk_plan(engine.shape_struct(big.shape), engine.plan_opts(16, 65536, exec_mode=mk.MK_EXEC_FLAT))
    try:
        assert mk.mk_plan_sizes(plan)[0] > 32 << 20
        with pytest.raises(mk.MkError) as e:
            mk.mk_ctx_create_scratch(plan, torch.cuda.current_stream().cuda_stream)
        assert e.value.code == mk.MK_ERR_SCRATCH
    finally:
        mk.mk_plan_destroy(plan)
    # a newer scratch context ends the older one on the same device
    a = engine.Engine(s, tiny_gpu, max_batch=1, max_ctx=64, exec_mode=mk.MK_EXEC_FLAT, sync_mode=mk.MK_SYNC_FLAG,
                      scratch=True)
    b = engine.Engine(s, tiny_gpu, max_batch=1, max_ctx=64, exec_mode=mk.MK_EXEC_FLAT, sync_mode=mk.MK_SYNC_FLAG,
                      scratch=True)
    try:
        kv = b.kv_cache()
        logits = torch.empty((1, s.vocab), dtype=torch.float32, device="cuda:0")
        pos = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        tok = torch.tensor([5], dtype=torch.int32, device="cuda:0")
        with pytest.raises(mk.MkError) as e:
            a.step(tok, pos, kv, logits)
        assert e.value.code == mk.MK_ERR_STATE
        b.step(tok, pos, kv, logits)
        assert b.device_error()[0] == 0
    finally:
        a.close()
        b.close()
