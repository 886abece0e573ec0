"""ctypes binding of libmk.so: the C ABI of include/mk.h under the same names.

Argument marshalling only: every step of the decode pass runs in the HIP
kernels of libmk.so.  PyTorch is used by callers for device memory and
streams; there is no CPU fallback -- if libmk.so is missing, loading fails
with an error naming the build step.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmk.so")

MK_OK = 0
MK_ERR_INVALID_ARG = -1
MK_ERR_SHAPE = -2
MK_ERR_ALIGN = -3
MK_ERR_NOT_RESIDENT = -4
MK_ERR_CTX_OVERFLOW = -5
MK_ERR_HIP = -6
MK_ERR_TIMEOUT = -7
MK_ERR_INPUT = -8
MK_ERR_PLAN = -9
MK_ERR_STATE = -10
MK_ERR_UNSUPPORTED = -11
MK_ERR_SCRATCH = -12

MK_SYNC_COUNTER, MK_SYNC_FLAG, MK_SYNC_SENTINEL = 0, 1, 2
MK_EXEC_MEGA, MK_EXEC_MULTI, MK_EXEC_FLAT, MK_EXEC_STREAM, MK_EXEC_FLAT_MULTI, MK_EXEC_QUEUE = 0, 1, 2, 3, 4, 5
MK_ADVANCE = 1
MK_MAX_STEPS = 65536
MK_OP_QKV, MK_OP_ATTN, MK_OP_OPROJ, MK_OP_GATEUP, MK_OP_DOWN, MK_OP_LMHEAD = 1, 2, 3, 4, 5, 6

GRIDSYNC_VARIANTS = {0: "cooperative_grid_sync", 1: "counter_release_acquire", 2: "counter_write_through",
                     3: "epoch_flags", 4: "nan_sentinel_payload", 5: "xcd_two_level_flags"}


class MkError(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        self.code = code
        super().__init__(f"{where}: {mk_strerror(code)} ({code})" if where else f"{mk_strerror(code)} ({code})")


class mk_model_shape(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("rms_eps", C.c_double), ("rope_theta", C.c_double), ("tie_embeddings", C.c_int32)]


class mk_plan_opts(C.Structure):
    _fields_ = [("max_batch", C.c_int32), ("max_ctx", C.c_int32), ("kv_splits", C.c_int32),
                ("sync_mode", C.c_int32), ("exec_mode", C.c_int32), ("num_cus", C.c_int32), ("flags", C.c_int32)]


class mk_plan_info(C.Structure):
    _fields_ = [("num_cus", C.c_int32), ("n_instructions", C.c_int32), ("n_levels", C.c_int32),
                ("n_counters", C.c_int32), ("kv_splits", C.c_int32), ("max_instr_per_cu", C.c_int32),
                ("block_threads", C.c_int32), ("lds_bytes", C.c_int32), ("sync_mode", C.c_int32),
                ("exec_mode", C.c_int32), ("max_batch", C.c_int32), ("max_ctx", C.c_int32),
                ("weight_bytes", C.c_double)]


class mk_instr_desc(C.Structure):
    _fields_ = [("cu", C.c_int32), ("slot", C.c_int32), ("op", C.c_int32), ("layer", C.c_int32),
                ("level", C.c_int32), ("r0", C.c_int32), ("r1", C.c_int32), ("split", C.c_int32),
                ("n_splits", C.c_int32), ("wait_event", C.c_int32), ("wait_count", C.c_int32),
                ("signal_event", C.c_int32)]


_PPV = C.POINTER(C.c_void_p)


class mk_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("final_norm", C.c_void_p),
                ("attn_norm", _PPV), ("wq", _PPV), ("wk", _PPV), ("wv", _PPV), ("wo", _PPV),
                ("mlp_norm", _PPV), ("wg", _PPV), ("wu", _PPV), ("wd", _PPV)]


class mk_device_info(C.Structure):
    _fields_ = [("num_cus", C.c_int32), ("lds_per_block", C.c_int32), ("lds_per_cu", C.c_int32),
                ("warp_size", C.c_int32), ("clock_khz", C.c_int32), ("mem_clock_khz", C.c_int32),
                ("mem_bus_bits", C.c_int32), ("max_threads_per_block", C.c_int32),
                ("mega_blocks_per_cu", C.c_int32), ("arch", C.c_char * 64)]


_lib = None

# name -> (restype, argtypes) for every symbol include/mk.h declares
SIGNATURES = {
    "mk_strerror": (C.c_char_p, [C.c_int]),
    "mk_plan": (C.c_int, [C.POINTER(mk_model_shape), C.POINTER(mk_plan_opts), C.POINTER(C.c_void_p)]),
    "mk_plan_create": (C.c_int, [C.POINTER(mk_model_shape), C.POINTER(mk_plan_opts), C.POINTER(C.c_void_p)]),
    "mk_plan_validate": (C.c_int, [C.c_void_p]),
    "mk_plan_sizes": (C.c_int, [C.c_void_p, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t),
                                C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "mk_plan_get_info": (C.c_int, [C.c_void_p, C.POINTER(mk_plan_info)]),
    "mk_plan_export": (C.c_int, [C.c_void_p, C.POINTER(mk_instr_desc), C.c_size_t, C.POINTER(C.c_size_t)]),
    "mk_plan_simulate": (C.c_int, [C.c_void_p, C.c_int32, C.c_uint64]),
    "mk_plan_destroy": (None, [C.c_void_p]),
    "mk_plan_get_queue": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_size_t, C.POINTER(C.c_size_t)]),
    "mk_events_normalize": (C.c_int, [C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int64),
                                      C.c_uint32, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                      C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "mk_plan_set_instructions": (C.c_int, [C.c_void_p, C.POINTER(mk_instr_desc), C.c_size_t]),
    "mk_ctx_create": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p)]),
    "mk_ctx_create_scratch": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(C.c_void_p)]),
    "mk_load_weights": (C.c_int, [C.c_void_p, C.POINTER(mk_weights), C.c_void_p]),
    "mk_decode_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_uint32, C.c_void_p]),
    "mk_decode_steps": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_int32, C.c_void_p]),
    "mk_graph_create": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_uint32, C.c_void_p, C.POINTER(C.c_void_p)]),
    "mk_graph_launch": (C.c_int, [C.c_void_p, C.c_void_p]),
    "mk_graph_destroy": (None, [C.c_void_p]),
    "mk_get_device_error": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(C.c_int32)]),
    "mk_ctx_reset": (C.c_int, [C.c_void_p, C.c_void_p]),
    "mk_ctx_epoch": (C.c_int64, [C.c_void_p]),
    "mk_ctx_destroy": (None, [C.c_void_p]),
    "mk_ctx_set_watchdog_us": (C.c_int, [C.c_void_p, C.c_uint32, C.c_void_p]),
    "mk_plan_get_layout": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint64)]),
    "mk_ctx_set_trace": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "mk_ctx_set_epoch": (C.c_int, [C.c_void_p, C.c_int64]),
    "mk_device_query": (C.c_int, [C.c_int32, C.POINTER(mk_device_info)]),
    "mk_gridsync_scratch_bytes": (C.c_size_t, [C.c_int32]),
    "mk_gridsync_bench": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "mk_lds_stream_read": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]),
    "mk_stream_read": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32, C.c_void_p]),
}


def load_library(path: str = LIB_PATH):
    """Load libmk.so (built by __graft_entry__.build() or build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = C.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int, where: str):
    if rc != MK_OK:
        raise MkError(rc, where)


def mk_strerror(code: int) -> str:
    return load_library().mk_strerror(code).decode()


# ------------------------------------------------------------------ plans

def mk_plan(shape: mk_model_shape, opts: mk_plan_opts) -> C.c_void_p:
    out = C.c_void_p()
    _check(load_library().mk_plan(C.byref(shape), C.byref(opts), C.byref(out)), "mk_plan")
    return out


def mk_plan_create(shape: mk_model_shape, opts: mk_plan_opts) -> C.c_void_p:
    out = C.c_void_p()
    _check(load_library().mk_plan_create(C.byref(shape), C.byref(opts), C.byref(out)), "mk_plan_create")
    return out


def mk_plan_validate(plan) -> int:
    return load_library().mk_plan_validate(plan)


def mk_plan_simulate(plan, n_trials: int, seed: int) -> int:
    return load_library().mk_plan_simulate(plan, n_trials, seed)


def mk_plan_sizes(plan):
    ws, kv, lg, ni = C.c_size_t(), C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(load_library().mk_plan_sizes(plan, C.byref(ws), C.byref(kv), C.byref(lg), C.byref(ni)), "mk_plan_sizes")
    return ws.value, kv.value, lg.value, ni.value


def mk_plan_get_info(plan) -> mk_plan_info:
    info = mk_plan_info()
    _check(load_library().mk_plan_get_info(plan, C.byref(info)), "mk_plan_get_info")
    return info


def mk_plan_get_queue(plan) -> List[int]:
    lib = load_library()
    n = C.c_size_t()
    _check(lib.mk_plan_get_queue(plan, None, 0, C.byref(n)), "mk_plan_get_queue")
    arr = (C.c_int32 * max(n.value, 1))()
    _check(lib.mk_plan_get_queue(plan, arr, n.value, C.byref(n)), "mk_plan_get_queue")
    return list(arr[:n.value])


MK_NORM_NO_REDUCTION = 1


def mk_events_normalize(preds: List[List[int]], rank: Optional[List[int]] = None, flags: int = 0):
    """Normalise a task graph given as predecessor lists.  Returns (rc, dict
    with wait, trigger, slot, count, order, n_events)."""
    nt = len(preds)
    begin = (C.c_int32 * (nt + 1))()
    flat = [q for ps in preds for q in ps]
    lst = (C.c_int32 * max(len(flat), 1))(*flat)
    acc = 0
    for t, ps in enumerate(preds):
        begin[t] = acc
        acc += len(ps)
    begin[nt] = acc
    rk = (C.c_int64 * nt)(*rank) if rank is not None else None
    outs = [(C.c_int32 * max(nt, 1))() for _ in range(5)]
    ne = C.c_int32()
    rc = load_library().mk_events_normalize(nt, begin, lst, rk, flags, *outs, C.byref(ne))
    wait, trig, slot, count, order = (list(o[:nt]) for o in outs)
    return rc, {"wait": wait, "trigger": trig, "slot": slot, "count": count[:ne.value], "order": order,
                "n_events": ne.value}


def mk_plan_export(plan) -> List[mk_instr_desc]:
    lib = load_library()
    n = C.c_size_t()
    _check(lib.mk_plan_export(plan, None, 0, C.byref(n)), "mk_plan_export")
    arr = (mk_instr_desc * n.value)()
    _check(lib.mk_plan_export(plan, arr, n.value, C.byref(n)), "mk_plan_export")
    return list(arr)


def mk_plan_set_instructions(plan, descs: Sequence[mk_instr_desc]) -> int:
    arr = (mk_instr_desc * len(descs))(*descs)
    return load_library().mk_plan_set_instructions(plan, arr, len(descs))


def mk_plan_get_layout(plan):
    out = (C.c_uint64 * 8)()
    _check(load_library().mk_plan_get_layout(plan, out), "mk_plan_get_layout")
    return list(out)


def mk_plan_destroy(plan):
    if plan:
        load_library().mk_plan_destroy(plan)


# ------------------------------------------------------------------ contexts

def mk_ctx_create(plan, d_workspace: int, workspace_bytes: int, stream: int) -> C.c_void_p:
    out = C.c_void_p()
    _check(load_library().mk_ctx_create(plan, C.c_void_p(d_workspace), workspace_bytes, C.c_void_p(stream),
                                        C.byref(out)), "mk_ctx_create")
    return out


def mk_ctx_create_scratch(plan, stream: int) -> C.c_void_p:
    out = C.c_void_p()
    _check(load_library().mk_ctx_create_scratch(plan, C.c_void_p(stream), C.byref(out)), "mk_ctx_create_scratch")
    return out


def mk_load_weights(ctx, weights: mk_weights, stream: int):
    _check(load_library().mk_load_weights(ctx, C.byref(weights), C.c_void_p(stream)), "mk_load_weights")


def mk_decode_step(ctx, d_tokens: int, d_positions: int, batch: int, d_kv: int, d_logits: int,
                   d_next: Optional[int], flags: int, stream: int) -> int:
    return load_library().mk_decode_step(ctx, C.c_void_p(d_tokens), C.c_void_p(d_positions), batch,
                                         C.c_void_p(d_kv), C.c_void_p(d_logits),
                                         C.c_void_p(d_next) if d_next else None, flags, C.c_void_p(stream))


def mk_decode_steps(ctx, d_tokens: int, d_positions: int, batch: int, d_kv: int, d_logits: int,
                    d_next: Optional[int], n_steps: int, stream: int) -> int:
    return load_library().mk_decode_steps(ctx, C.c_void_p(d_tokens), C.c_void_p(d_positions), batch,
                                          C.c_void_p(d_kv), C.c_void_p(d_logits),
                                          C.c_void_p(d_next) if d_next else None, n_steps, C.c_void_p(stream))


def mk_graph_create(ctx, d_tokens: int, d_positions: int, batch: int, d_kv: int, d_logits: int,
                    d_next: Optional[int], flags: int, stream: int):
    out = C.c_void_p()
    _check(load_library().mk_graph_create(ctx, C.c_void_p(d_tokens), C.c_void_p(d_positions), batch,
                                          C.c_void_p(d_kv), C.c_void_p(d_logits),
                                          C.c_void_p(d_next) if d_next else None, flags, C.c_void_p(stream),
                                          C.byref(out)), "mk_graph_create")
    return out


def mk_graph_launch(graph, stream: int) -> int:
    return load_library().mk_graph_launch(graph, C.c_void_p(stream))


def mk_graph_destroy(graph):
    load_library().mk_graph_destroy(graph)


def mk_get_device_error(ctx, stream: int):
    detail = C.c_int32()
    rc = load_library().mk_get_device_error(ctx, C.c_void_p(stream), C.byref(detail))
    return rc, detail.value


def mk_ctx_reset(ctx, stream: int):
    _check(load_library().mk_ctx_reset(ctx, C.c_void_p(stream)), "mk_ctx_reset")


def mk_ctx_epoch(ctx) -> int:
    return load_library().mk_ctx_epoch(ctx)


def mk_ctx_set_watchdog_us(ctx, us: int, stream: int):
    _check(load_library().mk_ctx_set_watchdog_us(ctx, us, C.c_void_p(stream)), "mk_ctx_set_watchdog_us")


def mk_ctx_set_trace(ctx, d_trace: Optional[int], n_records: int, stream: int):
    _check(load_library().mk_ctx_set_trace(ctx, C.c_void_p(d_trace) if d_trace else None, n_records,
                                           C.c_void_p(stream)), "mk_ctx_set_trace")


def mk_ctx_set_epoch(ctx, epoch: int):
    _check(load_library().mk_ctx_set_epoch(ctx, epoch), "mk_ctx_set_epoch")


def mk_ctx_destroy(ctx):
    if ctx:
        load_library().mk_ctx_destroy(ctx)


def mk_device_query(device: int = 0) -> mk_device_info:
    info = mk_device_info()
    _check(load_library().mk_device_query(device, C.byref(info)), "mk_device_query")
    return info


def mk_gridsync_scratch_bytes(n_blocks: int) -> int:
    return load_library().mk_gridsync_scratch_bytes(n_blocks)


def mk_gridsync_bench(variant: int, n_barriers: int, n_blocks: int, d_scratch: int, d_result: int, stream: int):
    _check(load_library().mk_gridsync_bench(variant, n_barriers, n_blocks, C.c_void_p(d_scratch),
                                            C.c_void_p(d_result), C.c_void_p(stream)), "mk_gridsync_bench")


def mk_lds_stream_read(d_buf: int, nbytes: int, d_out: int, n_blocks: int, n_waves: int, stream: int):
    _check(load_library().mk_lds_stream_read(C.c_void_p(d_buf), nbytes, C.c_void_p(d_out), n_blocks, n_waves,
                                             C.c_void_p(stream)), "mk_lds_stream_read")


def mk_stream_read(d_buf: int, nbytes: int, d_out: int, n_blocks: int, stream: int):
    _check(load_library().mk_stream_read(C.c_void_p(d_buf), nbytes, C.c_void_p(d_out), n_blocks,
                                         C.c_void_p(stream)), "mk_stream_read")
