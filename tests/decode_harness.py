"""Shared driver for the GPU parity tests: runs the HIP decode path through
the C ABI, then the CPU oracle teacher-forced on the tokens the GPU fed, on
the same seeded inputs, and compares them step by step.

Comparison rules (written here once, used by every GPU test):
  * logits: per step and sequence, max_i |gpu_i - ref_i| / max_i |ref_i| must
    not exceed LOGIT_TOL = 2e-2 (bf16 weights, fp32 accumulation vs an fp64
    oracle); the observed value is returned so tests can assert tighter bounds;
  * greedy tokens, every step of the run: the GPU runs free (its own argmax
    feeds the next step); the oracle is teacher-forced on the GPU's tokens, so
    a flip cannot cascade.  The GPU token must equal the oracle's argmax
    unless the oracle logit of the GPU token is within the step's measured
    logit error of the oracle's maximum (a near tie), which is counted and
    reported;
  * KV cache (check_kv): the bytes that changed are exactly the slots of the
    decoded positions, on both sides, and every other byte is unchanged
    (indexing is bit-exact).  Every appended bf16 value must be the
    round-to-nearest-even of a number within the GPU's measured fp32 error of
    the oracle's unrounded value: rne(u - e) <= gpu <= rne(u + e).  For a
    value whose error is below half its bf16 spacing this allows the oracle's
    own rounding or, when u lies within e of a rounding boundary, the
    neighbour across that boundary (one ulp); only values much smaller than
    the error of their dot product (near zero) may differ by more.  The fp32
    error e is measured on the run: the GPU's pre-rotation keys and values
    are read back from the workspace after every step and compared with the
    oracle's unrounded ones (per step, sequence and layer), and the largest
    error relative to the layer's largest value is reported and bounded.

The oracle side of a run is cached by its inputs (workload, seed, cache
geometry, the tokens fed), so several GPU modes that produce the same tokens
share one oracle trajectory.
"""
from __future__ import annotations

import dataclasses
import math
from collections import OrderedDict
from typing import List, Optional

import numpy as np
import torch

import synth_inputs as si
from oracle import oracle as orc
from persistent_megakernel_decode_02_amd import engine, mk

LOGIT_TOL = 2e-2


@dataclasses.dataclass
class RunResult:
    tokens: List[List[int]]        # generated tokens per step [step][b]
    max_rel_err: float
    per_step_err: List[float]
    near_ties: int
    kv_gpu: np.ndarray
    kv_ref: np.ndarray
    kv_written: np.ndarray          # bool mask of slots written by the steps
    logits_last: np.ndarray
    logits_all: List[np.ndarray]    # fp32 logits of every step [step] -> [B][V]
    kv_before: np.ndarray
    kv_idx: tuple                   # flat indices (into the cache) of every appended value
    kv_unrounded: np.ndarray        # the oracle's unrounded value at each of them
    kv_bound: np.ndarray            # the GPU's measured fp32 error bound at each of them
    kv_rel_err: float               # largest measured k/v error relative to its layer's largest value


@dataclasses.dataclass
class _OracleRun:
    logits: List[np.ndarray]
    nxt: List[np.ndarray]
    probe: List[np.ndarray]
    kv_ref: np.ndarray


_ORACLE_CACHE: "OrderedDict[tuple, _OracleRun]" = OrderedDict()
_ORACLE_CACHE_MAX = 2


def ulp_diff_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in bf16 units in the last place (sign-magnitude ordering)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(key(a) - key(b))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (as float64;
    normal range)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    spacing = np.exp2(np.maximum(e, -126.0) - 7.0)
    return np.where(mag > 0, np.rint(x / spacing) * spacing, 0.0)


def _fill_unwritten(kv: torch.Tensor, prefill: List[int], bits: int):
    """Give every slot at or above a sequence's first position the bf16 bit
    pattern `bits` (e.g. a NaN): memory the path must never let into a result."""
    v = kv.view(torch.int16)
    val = bits - 0x10000 if bits >= 0x8000 else bits
    for b, n in enumerate(prefill):
        v[:, :, b, :, n:, :] = val


def run_decode(wl: si.Workload, n_steps: int, exec_mode=mk.MK_EXEC_MEGA, sync_mode=mk.MK_SYNC_COUNTER,
               kv_splits: int = 0, weights=None, gpu_weights=None, model: Optional[orc.Model] = None,
               advance: bool = True, master: int = 0, batch: Optional[int] = None,
               max_batch: Optional[int] = None, kv_fill: Optional[int] = None, use_graph: bool = False,
               eager_steps=()) -> RunResult:
    """Decode n_steps passes of `wl` on the GPU, then check every step against
    the oracle.  batch / max_batch: sequences per step and the plan's bound
    (defaults: the workload's batch for both); sequence slots past `batch`
    keep their prefill and must stay untouched.  kv_fill: bf16 bits stored in
    every not-yet-written cache slot of both sides.  use_graph: the step is
    captured once as a hipGraph (MK_EXEC_FLAT_MULTI) and replayed, except the
    steps listed in eager_steps, which are enqueued by mk_decode_step."""
    s = wl.shape
    B = batch or wl.batch
    Bmax = max_batch or B
    assert B <= Bmax
    w = weights if weights is not None else si.make_weights(s, master=master)
    gw = gpu_weights if gpu_weights is not None else engine.to_gpu(w)
    model = model if model is not None else orc.Model(s, w)
    pos_all = wl.positions0(master)
    pos_all = (pos_all * ((Bmax + len(pos_all) - 1) // len(pos_all)))[:Bmax]
    pos0 = pos_all[:B]
    prefill = pos_all if wl.start_pos != 0 else [0] * Bmax
    kv_cpu = si.make_kv_cache(s, Bmax, wl.max_ctx, prefill, master=master)
    if kv_fill is not None:
        _fill_unwritten(kv_cpu, prefill, kv_fill)
    kv0 = si.bf16_bits(kv_cpu).reshape(kv_cpu.shape).copy()  # cache before the run
    first = si.workload_tokens(wl, master)
    prompt = first if wl.prompt_len else None
    if prompt is None and len(first) < B:
        first = (first * B)[:B]

    # ---------------------------------------------------------------- GPU
    eng = engine.Engine(s, gw, max_batch=Bmax, max_ctx=wl.max_ctx, kv_splits=kv_splits, sync_mode=sync_mode,
                        exec_mode=exec_mode)
    R = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    lay = mk.mk_plan_get_layout(eng.plan)
    try:
        kv = kv_cpu.to("cuda:0")
        toks = torch.tensor(first[:B] if prompt is None else [prompt[0]], dtype=torch.int32, device="cuda:0")
        pos = torch.tensor(pos0, dtype=torch.int32, device="cuda:0")
        logits = torch.empty((B, s.vocab), dtype=torch.float32, device="cuda:0")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda:0")
        graph = eng.graph(toks, pos, kv, logits, nxt, advance=advance) if use_graph else None
        feeds, poss, g_tokens, g_logits, g_kv = [], [], [], [], []
        cur_tok = list(toks.cpu().numpy())
        cur_pos = list(pos0)
        for t in range(n_steps):
            feed = cur_tok
            if prompt is not None and t < len(prompt):
                feed = [prompt[t]]
                toks.copy_(torch.tensor(feed, dtype=torch.int32))
            epoch = mk.mk_ctx_epoch(eng.ctx)
            if graph is not None and t not in eager_steps:
                graph.launch()
            else:
                eng.step(toks, pos, kv, logits, nxt, advance=advance)
            rc, detail = eng.device_error()
            assert rc == 0, f"device error {rc} ({mk.mk_strerror(rc)}), detail {detail}, step {t}"
            g_next = [int(v) for v in nxt.cpu().numpy()]
            feeds.append([int(x) for x in feed])
            poss.append(list(cur_pos))
            g_tokens.append(g_next)
            g_logits.append(logits.cpu().numpy().copy())
            # this step's pre-rotation keys and values, fp32 [L][Bmax][R] in the workspace
            off = lay[0] + (epoch & 1) * lay[7]
            qkv = eng.workspace_view(off, s.n_layers * Bmax * R).view(s.n_layers, Bmax, R)
            g_kv.append(qkv[:, :B, qd:].cpu().numpy().copy())
            if advance:
                assert [int(v) for v in pos.cpu().numpy()] == [p + 1 for p in cur_pos]
                assert [int(v) for v in toks.cpu().numpy()] == g_next
            else:
                toks.copy_(nxt)
                pos.add_(1)
            cur_tok = g_next
            cur_pos = [p + 1 for p in cur_pos]
        torch.cuda.synchronize()
        kv_gpu = kv.view(torch.int16).cpu().numpy().view(np.uint16)
        if graph is not None:
            graph.close()
    finally:
        eng.close()

    # ------------------------------------------------------------- oracle
    key = (wl.name, master, Bmax, wl.max_ctx, kv_fill, tuple(map(tuple, feeds)), tuple(map(tuple, poss)))
    orun = _ORACLE_CACHE.get(key)
    if orun is None:
        kv_ref = kv0.copy()
        orun = _OracleRun([], [], [], kv_ref)
        for t in range(n_steps):
            probe = np.empty((B, s.n_layers, 3, s.n_kv_heads, s.head_dim), dtype=np.float64)
            lg, nx = model.step(feeds[t], poss[t], kv_ref, Bmax, wl.max_ctx, probe=probe)
            orun.logits.append(lg)
            orun.nxt.append(nx)
            orun.probe.append(probe)
        _ORACLE_CACHE[key] = orun
        while len(_ORACLE_CACHE) > _ORACLE_CACHE_MAX:
            _ORACLE_CACHE.popitem(last=False)
    else:
        _ORACLE_CACHE.move_to_end(key)

    # ------------------------------------------------------------ compare
    errs, near = [], 0
    for t in range(n_steps):
        got, ref = g_logits[t].astype(np.float64), orun.logits[t]
        for b in range(B):
            err = float(np.max(np.abs(got[b] - ref[b])) / np.max(np.abs(ref[b])))
            errs.append(err)
            gt, rt = g_tokens[t][b], int(orun.nxt[t][b])
            if gt != rt:
                gap = ref[b].max() - ref[b][gt]
                tol = float(np.max(np.abs(got[b] - ref[b])))
                assert gap <= tol, (f"step {t} seq {b}: gpu token {gt} vs oracle {rt}, "
                                    f"gap {gap:.3e} > logit error {tol:.3e}")
                near += 1

    # appended values: their flat cache indices, the oracle's unrounded value
    # and the GPU's measured fp32 error at each
    L, nkv, d = s.n_layers, s.n_kv_heads, s.head_dim
    shp = kv0.shape
    written = np.zeros(shp, dtype=bool)
    idx, unr, bnd = [], [], []
    rel = 0.0
    li, gi, ii = np.meshgrid(np.arange(L), np.arange(nkv), np.arange(d), indexing="ij")
    for t in range(n_steps):
        pr = orun.probe[t]
        for b in range(B):
            p = poss[t][b]
            written[:, :, b, :, p, :] = True
            kg = g_kv[t][:, b, :kd].astype(np.float64).reshape(L, nkv, d)       # GPU keys before rotation
            vg = g_kv[t][:, b, kd:].astype(np.float64).reshape(L, nkv, d)
            k_pre, k_post, v_ref = pr[b, :, 0], pr[b, :, 1], pr[b, :, 2]         # [L][nkv][d]
            e_k = np.max(np.abs(kg - k_pre), axis=(1, 2))                         # per layer
            e_v = np.max(np.abs(vg - v_ref), axis=(1, 2))
            # the rotation is linear with |cos| + |sin| <= sqrt(2); its own fp32
            # products and difference add at most a few ulps of the operands
            bk = math.sqrt(2.0) * e_k + 2.0 ** -20 * np.max(np.abs(k_pre), axis=(1, 2))
            bv = e_v * (1 + 1e-12)
            rel = max(rel, float(np.max(e_k / np.max(np.abs(k_pre), axis=(1, 2)))),
                      float(np.max(e_v / np.max(np.abs(v_ref), axis=(1, 2)))))
            for plane, vals, bb in ((0, k_post, bk), (1, v_ref, bv)):
                flat = np.ravel_multi_index((li, np.full_like(li, plane), np.full_like(li, b), gi,
                                             np.full_like(li, p), ii), shp)
                idx.append(flat.ravel())
                unr.append(vals.ravel())
                bnd.append(np.broadcast_to(bb[:, None, None], (L, nkv, d)).ravel())
    return RunResult(g_tokens, max(errs), errs, near, kv_gpu, orun.kv_ref, written, g_logits[-1], g_logits, kv0,
                     np.concatenate(idx), np.concatenate(unr), np.concatenate(bnd), rel)


def check_kv(res: RunResult, max_rel_err: float = 1e-4):
    """Cache parity (the rules in the module docstring).  Returns the fraction
    of appended values that are bit-identical to the oracle's; prints the
    counts of one-ulp and wider (explained) differences.

    max_rel_err: bound on the measured fp32 error of the appended keys and
    values relative to their layer's largest value (the fp32 vector path
    stays near 1e-6; the matrix-core path, whose inputs are split into bf16
    high and low parts, near 1e-5)."""
    kg, kr = res.kv_gpu.reshape(-1), res.kv_ref.reshape(-1)
    m = res.kv_written
    # nothing outside the appended slots moved, on either side
    assert np.array_equal(res.kv_gpu[~m], res.kv_before[~m])
    assert np.array_equal(res.kv_ref[~m], res.kv_before[~m])
    g, r = kg[res.kv_idx], kr[res.kv_idx]
    assert int(m.sum()) == g.size  # every written slot is accounted for once
    assert res.kv_rel_err <= max_rel_err, res.kv_rel_err
    # the oracle's own rounding is what it stored
    assert np.array_equal(rne_bf16(res.kv_unrounded), bf16_to_f64(r))
    same = g == r
    exact = float(np.mean(same))
    dg = ~same
    wide = 0
    if dg.any():
        u, e = res.kv_unrounded[dg], res.kv_bound[dg]
        gv = bf16_to_f64(g[dg])
        lo, hi = rne_bf16(u - e), rne_bf16(u + e)
        bad = (gv < lo) | (gv > hi)
        assert not bad.any(), (f"{int(bad.sum())} of {int(dg.sum())} differing appended values are not the rounding "
                               f"of a value within the measured error of the oracle's (first: gpu {gv[bad][0]!r}, "
                               f"oracle {u[bad][0]!r}, error bound {e[bad][0]!r})")
        wide = int(np.sum(ulp_diff_bf16(g[dg], r[dg]) > 1))
    print(f"kv: {g.size} appended values, {exact:.5f} bit-identical, {int(dg.sum()) - wide} one ulp apart, "
          f"{wide} wider (near zero), measured relative error {res.kv_rel_err:.2e}")
    # a written value may coincide with the prefill by chance; nearly all differ
    before = res.kv_before.reshape(-1)[res.kv_idx]
    assert np.mean(g != before) > 0.99 and np.mean(r != before) > 0.99
    return exact


@dataclasses.dataclass
class MultiStepResult:
    tokens: List[List[int]]       # [step][b]
    logits: np.ndarray            # fp32 [step][B][V]
    kv_gpu: np.ndarray            # cache bits after the run
    launches: int


def run_multistep(wl: si.Workload, n_steps: int, chunk: int, exec_mode=mk.MK_EXEC_FLAT,
                  sync_mode=mk.MK_SYNC_FLAG, kv_splits: int = 0, weights=None, gpu_weights=None,
                  master: int = 0) -> MultiStepResult:
    """The same free-running greedy decode as run_decode (same seeded inputs,
    prompt-free workloads), but `chunk` steps per launch through
    mk_decode_steps: the device feeds each step's token to the next."""
    assert not wl.prompt_len
    s = wl.shape
    B = wl.batch
    gw = gpu_weights if gpu_weights is not None else engine.to_gpu(
        weights if weights is not None else si.make_weights(s, master=master))
    pos0 = wl.positions0(master)
    prefill = pos0 if wl.start_pos != 0 else [0] * B
    kv_cpu = si.make_kv_cache(s, B, wl.max_ctx, prefill, master=master)
    first = si.workload_tokens(wl, master)
    if len(first) < B:
        first = (first * B)[:B]
    eng = engine.Engine(s, gw, max_batch=B, max_ctx=wl.max_ctx, kv_splits=kv_splits, sync_mode=sync_mode,
                        exec_mode=exec_mode)
    try:
        kv = kv_cpu.to("cuda:0")
        toks = torch.tensor(first[:B], dtype=torch.int32, device="cuda:0")
        pos = torch.tensor(pos0, dtype=torch.int32, device="cuda:0")
        logits = torch.empty((n_steps, B, s.vocab), dtype=torch.float32, device="cuda:0")
        nxt = torch.empty((n_steps, B), dtype=torch.int32, device="cuda:0")
        done, launches = 0, 0
        while done < n_steps:
            n = min(chunk, n_steps - done)
            eng.steps(toks, pos, kv, logits[done:], nxt[done:], n)
            launches += 1
            done += n
        rc, detail = eng.device_error()
        assert rc == 0, f"device error {rc} ({mk.mk_strerror(rc)}), detail {detail}"
        assert [int(v) for v in pos.cpu().numpy()] == [p + n_steps for p in pos0]
        torch.cuda.synchronize()
        res = MultiStepResult([[int(v) for v in row] for row in nxt.cpu().numpy()], logits.cpu().numpy(),
                              kv.view(torch.int16).cpu().numpy().view(np.uint16), launches)
        assert [int(v) for v in toks.cpu().numpy()] == res.tokens[-1]
        return res
    finally:
        eng.close()
