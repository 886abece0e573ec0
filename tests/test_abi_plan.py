"""Host-side checks of libmk.so (no GPU): every symbol include/mk.h declares
is exported, the planner builds valid plans for all workload shapes and CU
counts, the validator and the schedule simulator accept them, and they
reject plans corrupted on purpose (missing wait, wrong event, broken level
order, dropped instruction)."""
import ctypes as C
import os
import re

import pytest

import synth_inputs as si
from persistent_megakernel_decode_02_amd import mk
from persistent_megakernel_decode_02_amd.engine import plan_opts, shape_struct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "mk.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_\w+)\s*\(", txt)))


def test_every_declared_symbol_is_exported_and_bound():
    lib = mk.load_library()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
        assert n in mk.SIGNATURES, n
    assert set(mk.SIGNATURES) == set(names)


def test_strerror_texts():
    for code in range(0, -12, -1):
        assert mk.mk_strerror(code) != "unknown error"
    assert mk.mk_strerror(-99) == "unknown error"


SHAPES = {k: (wl.shape, wl.batch, wl.max_ctx) for k, wl in si.WORKLOADS.items()}


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("n_cu", [8, 80, 256, 304])
def test_plan_builds_and_validates(name, n_cu):
    shape, batch, max_ctx = SHAPES[name]
    # the role engine stages up to 4 sequences; larger batches run the flat kernel
    exec_mode = mk.MK_EXEC_MEGA if batch <= 4 else mk.MK_EXEC_FLAT
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=n_cu, exec_mode=exec_mode))
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_OK
        info = mk.mk_plan_get_info(plan)
        assert info.num_cus == n_cu and info.n_levels == 5 * shape.n_layers + 1
        assert info.lds_bytes <= 160 * 1024
        descs = mk.mk_plan_export(plan)
        assert len(descs) == info.n_instructions
        # lists are level-sorted per CU and every CU index is in range
        last = {}
        for d in descs:
            assert 0 <= d.cu < n_cu
            assert d.level >= last.get(d.cu, -1)
            last[d.cu] = d.level
        # weights streamed once per pass: matches the parameter count
        d, L, H = shape.head_dim, shape.n_layers, shape.hidden
        P = L * (H * (shape.n_q_heads + 2 * shape.n_kv_heads) * d + shape.n_q_heads * d * H + 3 * H * shape.ffn
                 + 2 * H) + shape.vocab * H + H
        assert info.weight_bytes == 2 * P
        if n_cu <= 80 or name == "tiny":
            assert mk.mk_plan_simulate(plan, 20, 1) == mk.MK_OK
    finally:
        mk.mk_plan_destroy(plan)


def test_plan_llama1b_one_gemv_slice_per_cu():
    shape, batch, max_ctx = SHAPES["llama1b_pos1024"]
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256))
    try:
        descs = mk.mk_plan_export(plan)
        for op in (mk.MK_OP_OPROJ, mk.MK_OP_GATEUP, mk.MK_OP_DOWN, mk.MK_OP_LMHEAD):
            cus = [d.cu for d in descs if d.op == op and d.layer in (0, shape.n_layers)]
            assert len(cus) == 256 and len(set(cus)) == 256
        assert mk.mk_plan_simulate(plan, 3, 7) == mk.MK_OK
    finally:
        mk.mk_plan_destroy(plan)


def test_flat_plan_keeps_attention_cus_out_of_o_and_gateup():
    """Homogeneous engine, one sequence: every layer's O and gate/up slices go
    to CUs that run none of that layer's attention, while every row is still
    covered exactly once and the plan validates and simulates.  At position
    8192 the default splits stop at 3/8 of the CUs (12 splits, 96 units:
    the exclusion holds); with 22 splits asked for (176 units, over half the
    CUs) the exclusion is off."""
    shape, batch, max_ctx = SHAPES["llama1b_pos1024"]
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256,
                                                           exec_mode=mk.MK_EXEC_FLAT,
                                                           sync_mode=mk.MK_SYNC_FLAG))
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_OK
        descs = mk.mk_plan_export(plan)
        for layer in range(shape.n_layers):
            attn = {d.cu for d in descs if d.op == mk.MK_OP_ATTN and d.layer == layer}
            assert len(attn) == shape.n_kv_heads * 3  # 3 splits at this context bound
            for op, rows in ((mk.MK_OP_OPROJ, shape.hidden), (mk.MK_OP_GATEUP, shape.ffn)):
                sl = [d for d in descs if d.op == op and d.layer == layer]
                assert not attn & {d.cu for d in sl}
                assert len({d.cu for d in sl}) == len(sl)  # one slice per CU
                cover = sorted((d.r0, d.r1) for d in sl)
                assert cover[0][0] == 0 and cover[-1][1] == rows
                assert all(a[1] == b[0] for a, b in zip(cover, cover[1:]))
        assert mk.mk_plan_simulate(plan, 3, 11) == mk.MK_OK
    finally:
        mk.mk_plan_destroy(plan)
    shape, batch, max_ctx = SHAPES["llama1b_pos8192"]
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256,
                                                           exec_mode=mk.MK_EXEC_FLAT))
    try:
        descs = mk.mk_plan_export(plan)
        attn = {d.cu for d in descs if d.op == mk.MK_OP_ATTN and d.layer == 0}
        assert max(d.n_splits for d in descs if d.op == mk.MK_OP_ATTN) == 12 and len(attn) == 96
        o_cus = {d.cu for d in descs if d.op == mk.MK_OP_OPROJ and d.layer == 0}
        assert len(o_cus) <= 256 - 96 and not attn & o_cus
    finally:
        mk.mk_plan_destroy(plan)
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, kv_splits=22, num_cus=256,
                                                           exec_mode=mk.MK_EXEC_FLAT))
    try:
        descs = mk.mk_plan_export(plan)
        assert len({d.cu for d in descs if d.op == mk.MK_OP_OPROJ and d.layer == 0}) == 256
    finally:
        mk.mk_plan_destroy(plan)


def _tiny_plan(n_cu=8, **kw):
    shape, batch, max_ctx = SHAPES["tiny"]
    return mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=n_cu, **kw))


def _mutated(mutate):
    plan = _tiny_plan()
    descs = mk.mk_plan_export(plan)
    mutate(descs)
    assert mk.mk_plan_set_instructions(plan, descs) == mk.MK_OK
    return plan


def test_unmodified_roundtrip_stays_valid():
    plan = _mutated(lambda d: None)
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_OK
        assert mk.mk_plan_simulate(plan, 200, 3) == mk.MK_OK
    finally:
        mk.mk_plan_destroy(plan)


def test_missing_wait_is_a_race():
    def m(descs):
        for d in descs:
            if d.op == mk.MK_OP_GATEUP and d.layer == 1:
                d.wait_event = -1
                return
    plan = _mutated(m)
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_ERR_PLAN
        assert mk.mk_plan_simulate(plan, 5, 1) == mk.MK_ERR_PLAN
    finally:
        mk.mk_plan_destroy(plan)


def test_wait_on_wrong_event_is_rejected():
    def m(descs):
        for d in descs:
            if d.op == mk.MK_OP_DOWN and d.layer == 0:
                # wait for the O-projection instead of gate/up: reads h too early
                d.wait_event = d.wait_event - 1
                return
    plan = _mutated(m)
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_ERR_PLAN
    finally:
        mk.mk_plan_destroy(plan)


def test_level_order_violation_is_rejected():
    def m(descs):
        # put a layer-1 QKV slice at the head of a CU list
        for d in descs:
            if d.op == mk.MK_OP_QKV and d.layer == 1:
                d.slot = -1
                return
    plan = _mutated(m)
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_ERR_PLAN
    finally:
        mk.mk_plan_destroy(plan)


def test_dropped_instruction_is_rejected():
    plan = _tiny_plan()
    try:
        descs = mk.mk_plan_export(plan)
        idx = next(i for i, d in enumerate(descs) if d.op == mk.MK_OP_OPROJ)
        del descs[idx]
        assert mk.mk_plan_set_instructions(plan, descs) == mk.MK_OK
        assert mk.mk_plan_validate(plan) == mk.MK_ERR_PLAN
    finally:
        mk.mk_plan_destroy(plan)


def test_trigger_in_wrong_event_is_rejected():
    def m(descs):
        for d in descs:
            if d.op == mk.MK_OP_OPROJ and d.layer == 0:
                d.signal_event = d.signal_event + 1  # counts toward gate/up's event instead
                return
    plan = _mutated(m)
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_ERR_PLAN
    finally:
        mk.mk_plan_destroy(plan)


def test_bad_shapes_and_options():
    base = si.TINY
    bad = [dict(head_dim=96), dict(n_kv_heads=3), dict(hidden=300)]
    for kw in bad:
        d = dict(base.__dict__)
        d.update(kw)
        s = si.ModelShape(**d)
        with pytest.raises(mk.MkError) as e:
            mk.mk_plan_create(shape_struct(s), plan_opts(1, 128, num_cus=8))
        assert e.value.code == mk.MK_ERR_SHAPE
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_create(shape_struct(base), plan_opts(17, 128, num_cus=8))
    assert e.value.code == mk.MK_ERR_INVALID_ARG
    # attention keeps no per-position state in LDS: one split may span the whole context
    plan = mk.mk_plan_create(shape_struct(base), plan_opts(1, 4096, kv_splits=1, num_cus=8,
                                                           exec_mode=mk.MK_EXEC_FLAT))
    try:
        assert mk.mk_plan_get_info(plan).lds_bytes <= 160 * 1024
    finally:
        mk.mk_plan_destroy(plan)


def test_role_engine_limits():
    s16 = SHAPES["llama1b_b16"][0]
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_create(shape_struct(s16), plan_opts(16, 4160, num_cus=256))
    assert e.value.code == mk.MK_ERR_UNSUPPORTED
    # sentinel synchronisation exists only inside one persistent launch
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_create(shape_struct(si.TINY), plan_opts(1, 128, num_cus=8, sync_mode=mk.MK_SYNC_SENTINEL,
                                                            exec_mode=mk.MK_EXEC_MULTI))
    assert e.value.code == mk.MK_ERR_UNSUPPORTED
    for name in ("llama1b_pos1024", "llama8b_pos2048"):
        shape, batch, max_ctx = SHAPES[name]
        plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256,
                                                                sync_mode=mk.MK_SYNC_SENTINEL))
        try:
            info = mk.mk_plan_get_info(plan)
            assert info.lds_bytes == 160 * 1024
            ws_sent = mk.mk_plan_sizes(plan)[0]
        finally:
            mk.mk_plan_destroy(plan)
        plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256))
        try:
            assert mk.mk_plan_sizes(plan)[0] < ws_sent  # sentinel mode keeps two step parities
        finally:
            mk.mk_plan_destroy(plan)


def test_sizes_match_layouts():
    shape, batch, max_ctx = SHAPES["llama1b_pos1024"]
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256))
    try:
        ws, kv, lg, n = mk.mk_plan_sizes(plan)
        assert kv == 2 * 16 * 2 * 1 * 8 * max_ctx * 64
        assert lg == 4 * 128256
        assert ws < 64 << 20
    finally:
        mk.mk_plan_destroy(plan)


def test_misaligned_or_short_workspace_is_refused_before_any_device_call():
    # both checks come before the context touches a device, so no GPU is needed
    plan = mk.mk_plan(shape_struct(si.TINY), plan_opts(1, 128, exec_mode=mk.MK_EXEC_FLAT, num_cus=8))
    try:
        ws, _, _, _ = mk.mk_plan_sizes(plan)
        with pytest.raises(mk.MkError) as e:
            mk.mk_ctx_create(plan, 0x10000 + 16, ws, 0)
        assert e.value.code == mk.MK_ERR_ALIGN
        with pytest.raises(mk.MkError) as e:
            mk.mk_ctx_create(plan, 0x10000, ws - 256, 0)
        assert e.value.code == mk.MK_ERR_CTX_OVERFLOW
    finally:
        mk.mk_plan_destroy(plan)


def test_mk_plan_and_mk_plan_create_build_the_same_plan():
    opts = plan_opts(1, 1152, exec_mode=mk.MK_EXEC_FLAT, sync_mode=mk.MK_SYNC_FLAG, num_cus=256)
    a = mk.mk_plan(shape_struct(si.LLAMA_1B), opts)
    b = mk.mk_plan_create(shape_struct(si.LLAMA_1B), opts)
    try:
        da, db = mk.mk_plan_export(a), mk.mk_plan_export(b)
        assert len(da) == len(db)
        fields = [f for f, _ in mk.mk_instr_desc._fields_]
        assert all(getattr(x, f) == getattr(y, f) for x, y in zip(da, db) for f in fields)
    finally:
        mk.mk_plan_destroy(a)
        mk.mk_plan_destroy(b)


@pytest.mark.parametrize("name", ["tiny", "llama1b_pos1024", "llama1b_pos8192", "llama8b_pos2048"])
@pytest.mark.parametrize("sync_mode", [mk.MK_SYNC_COUNTER, mk.MK_SYNC_FLAG])
def test_stream_engine_plans(name, sync_mode):
    # one sequence per step; its LDS holds the widest input vector, the row
    # results and the attention instruction's own layout
    shape, batch, max_ctx = SHAPES[name]
    plan = mk.mk_plan(shape_struct(shape), plan_opts(1, max_ctx, num_cus=256, exec_mode=mk.MK_EXEC_STREAM,
                                                       sync_mode=sync_mode))
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_OK
        info = mk.mk_plan_get_info(plan)
        kmax = max(shape.hidden, shape.n_q_heads * shape.head_dim, shape.ffn)
        assert kmax * 4 < info.lds_bytes <= 160 * 1024
        assert mk.mk_plan_simulate(plan, 3, 7) == mk.MK_OK
    finally:
        mk.mk_plan_destroy(plan)


def test_stream_engine_limits():
    s = si.WORKLOADS["llama1b_pos1024"].shape
    with pytest.raises(mk.MkError) as e:  # one sequence per step only
        mk.mk_plan(shape_struct(s), plan_opts(2, 1152, num_cus=256, exec_mode=mk.MK_EXEC_STREAM))
    assert e.value.code == mk.MK_ERR_UNSUPPORTED
    with pytest.raises(mk.MkError) as e:  # data sentinels: role engine and one-sequence homogeneous engine
        mk.mk_plan(shape_struct(s), plan_opts(1, 1152, num_cus=256, exec_mode=mk.MK_EXEC_STREAM,
                                              sync_mode=mk.MK_SYNC_SENTINEL))
    assert e.value.code == mk.MK_ERR_UNSUPPORTED
    with pytest.raises(mk.MkError) as e:  # the batched (MFMA) projections do not poll
        mk.mk_plan(shape_struct(s), plan_opts(2, 1152, num_cus=256, exec_mode=mk.MK_EXEC_FLAT,
                                              sync_mode=mk.MK_SYNC_SENTINEL))
    assert e.value.code == mk.MK_ERR_UNSUPPORTED
    plan = mk.mk_plan(shape_struct(s), plan_opts(1, 1152, num_cus=256, exec_mode=mk.MK_EXEC_FLAT,
                                                 sync_mode=mk.MK_SYNC_SENTINEL))
    try:
        lay = mk.mk_plan_get_layout(plan)
        assert lay[7] == lay[5] - lay[0] > 0  # a second activation copy, one per step parity
    finally:
        mk.mk_plan_destroy(plan)


def test_batched_down_projection_split_by_input_columns():
    """Batched plans of the homogeneous engine cut each down-projection slice
    (whole 16-row tiles) into I / 2048 parts of one staged input chunk; the
    parts of a slice share its output rows and its event (the last part to
    finish merges and triggers), every CU gets one part per layer at
    Llama-1B batch 16, and one-sequence plans keep whole slices."""
    shape, batch, max_ctx = SHAPES["llama1b_b16"]
    plan = mk.mk_plan_create(shape_struct(shape), plan_opts(batch, max_ctx, num_cus=256, exec_mode=mk.MK_EXEC_FLAT))
    try:
        descs = mk.mk_plan_export(plan)
        parts = {}
        for d in descs:
            if d.op == mk.MK_OP_DOWN:
                assert d.n_splits == shape.ffn // 2048 == 4
                assert d.r0 % 16 == 0 and d.r1 - d.r0 == 32
                parts.setdefault((d.layer, d.r0), []).append(d)
        assert len(parts) == shape.n_layers * shape.hidden // 32
        for ps in parts.values():
            assert sorted(p.split for p in ps) == [0, 1, 2, 3]
            assert len({(p.r1, p.signal_event, p.wait_event) for p in ps}) == 1
        for l in range(shape.n_layers):
            cus = [d.cu for d in descs if d.op == mk.MK_OP_DOWN and d.layer == l]
            assert len(cus) == 256 and len(set(cus)) == 256
        assert mk.mk_plan_validate(plan) == mk.MK_OK
        assert mk.mk_plan_simulate(plan, 3, 11) == mk.MK_OK
    finally:
        mk.mk_plan_destroy(plan)
    shape1, batch1, max_ctx1 = SHAPES["llama1b_pos1024"]
    plan = mk.mk_plan_create(shape_struct(shape1), plan_opts(batch1, max_ctx1, num_cus=256, exec_mode=mk.MK_EXEC_FLAT))
    try:
        assert all(d.n_splits == 1 for d in mk.mk_plan_export(plan) if d.op == mk.MK_OP_DOWN)
    finally:
        mk.mk_plan_destroy(plan)


def test_down_slice_missing_a_part_is_rejected():
    # FFN 6144 at batch 3: three parts per down slice; one part relabelled as
    # its neighbour leaves the slice's partial sums incomplete
    s = si.ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=6144, vocab=4096)
    plan = mk.mk_plan_create(shape_struct(s), plan_opts(3, 128, num_cus=8, exec_mode=mk.MK_EXEC_FLAT))
    try:
        assert mk.mk_plan_validate(plan) == mk.MK_OK
        assert mk.mk_plan_simulate(plan, 50, 5) == mk.MK_OK
        descs = mk.mk_plan_export(plan)
        d = next(x for x in descs if x.op == mk.MK_OP_DOWN and x.layer == 1 and x.split == 2)
        d.split = 1
        assert mk.mk_plan_set_instructions(plan, descs) == mk.MK_OK
        assert mk.mk_plan_validate(plan) == mk.MK_ERR_PLAN
    finally:
        mk.mk_plan_destroy(plan)
