"""GPU parity of the Llama-8B-shaped decode (32 layers, hidden 4096, 32/8
heads, head_dim 128, SwiGLU 14336, vocab 128256, untied LM head) against the
CPU oracle, through the C ABI, at position 2048 with a random-filled cache:
the only workload with head_dim 128 (the attention instruction's 128-wide
tiles), 4096-wide vectors and a separate LM-head matrix.  ~16 GB of weights
are drawn once for the module."""
import pytest

import synth_inputs as si
from decode_harness import LOGIT_TOL, check_kv, run_decode
from oracle import oracle as orc
from persistent_megakernel_decode_02_amd import engine, mk

pytestmark = pytest.mark.gpu

WL = si.WORKLOADS["llama8b_pos2048"]


@pytest.fixture(scope="module")
def llama8b():
    w = si.make_weights(WL.shape, master=0)
    return w, engine.to_gpu(w), orc.Model(WL.shape, w)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("mode", [(mk.MK_EXEC_STREAM, mk.MK_SYNC_FLAG), (mk.MK_EXEC_FLAT, mk.MK_SYNC_FLAG),
                                  (mk.MK_EXEC_FLAT, mk.MK_SYNC_SENTINEL)],
                         ids=["stream-flag", "flat-flag", "flat-sentinel"])
def test_llama8b_pos2048_decode(llama8b, mode):
    w, gw, model = llama8b
    res = run_decode(WL, 4, weights=w, gpu_weights=gw, model=model, exec_mode=mode[0], sync_mode=mode[1])
    print(f"llama8b@2048: errs {['%.2e' % e for e in res.per_step_err]} near ties {res.near_ties} "
          f"tokens {res.tokens}")
    assert res.max_rel_err <= LOGIT_TOL
    assert res.max_rel_err <= 1e-3
    assert res.near_ties == 0
    print(f"kv exact fraction {check_kv(res):.6f}")
