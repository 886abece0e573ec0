"""Device-memory plumbing around the C ABI.

`Engine` owns one plan and one context: it allocates the workspace with
torch (the library never allocates), binds bf16 weight tensors that live on
the GPU, and enqueues decode steps on a torch stream.  Every call goes
through libmk.so (mk.py); nothing here computes any part of the pass.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional

import torch

from . import mk

_LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd")


def shape_struct(shape) -> mk.mk_model_shape:
    """mk_model_shape from any object with the ModelShape attributes."""
    return mk.mk_model_shape(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                             shape.ffn, shape.vocab, float(shape.rms_eps), float(shape.rope_theta),
                             1 if shape.tied else 0)


def plan_opts(max_batch: int, max_ctx: int, kv_splits: int = 0, sync_mode: int = mk.MK_SYNC_COUNTER,
              exec_mode: int = mk.MK_EXEC_MEGA, num_cus: int = 0) -> mk.mk_plan_opts:
    return mk.mk_plan_opts(max_batch, max_ctx, kv_splits, sync_mode, exec_mode, num_cus, 0)


class Engine:
    def __init__(self, shape, gpu_weights: Dict[str, object], max_batch: int, max_ctx: int, kv_splits: int = 0,
                 sync_mode: int = mk.MK_SYNC_COUNTER, exec_mode: int = mk.MK_EXEC_MEGA,
                 stream: Optional[torch.cuda.Stream] = None, device: str = "cuda:0", scratch: bool = False):
        """gpu_weights: {"embed", "lm_head" (None when tied), "final_norm",
        "layers": [{attn_norm, wq, wk, wv, wo, mlp_norm, wg, wu, wd}]}, every
        tensor bf16, contiguous, on `device`.  scratch: take the workspace
        from the library's static device array (mk_ctx_create_scratch)
        instead of allocating one."""
        self.shape = shape
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.plan = mk.mk_plan(shape_struct(shape), plan_opts(max_batch, max_ctx, kv_splits, sync_mode,
                                                                     exec_mode))
        self.info = mk.mk_plan_get_info(self.plan)
        ws, self.kv_bytes, self.logits_bytes, self.n_instr = mk.mk_plan_sizes(self.plan)
        self.ws_bytes = ws
        if scratch:
            self._ws = None
            self.ws_ptr = None
            self.ctx = mk.mk_ctx_create_scratch(self.plan, self.stream.cuda_stream)
        else:
            self._ws = torch.empty(ws + 256, dtype=torch.uint8, device=self.device)
            base = self._ws.data_ptr()
            self.ws_ptr = (base + 255) // 256 * 256
            self.ctx = mk.mk_ctx_create(self.plan, self.ws_ptr, ws, self.stream.cuda_stream)
        self._bind(gpu_weights)

    def _bind(self, w):
        L = self.shape.n_layers
        keep = []
        arrays = {}
        for k in _LAYER_KEYS:
            arr = (C.c_void_p * L)()
            for l in range(L):
                t = w["layers"][l][k]
                assert t.dtype == torch.bfloat16 and t.is_contiguous() and t.device == self.device, k
                arr[l] = t.data_ptr()
                keep.append(t)
            arrays[k] = arr
        lm = w.get("lm_head")
        ws = mk.mk_weights(w["embed"].data_ptr(), lm.data_ptr() if lm is not None else None,
                           w["final_norm"].data_ptr(), *[C.cast(arrays[k], mk._PPV) for k in _LAYER_KEYS])
        mk.mk_load_weights(self.ctx, ws, self.stream.cuda_stream)
        self._keep = (keep, arrays, w)

    def workspace_view(self, byte_offset: int, n_floats: int) -> torch.Tensor:
        """fp32 view of n_floats of the workspace at byte_offset (a layout
        offset from mk_plan_get_layout): lets tests read activations back."""
        assert self._ws is not None, "a scratch context's workspace is the library's own"
        start = self.ws_ptr - self._ws.data_ptr() + byte_offset
        assert start % 4 == 0 and start + 4 * n_floats <= self._ws.numel()
        return self._ws[start:start + 4 * n_floats].view(torch.float32)

    def kv_cache(self) -> torch.Tensor:
        s = self.shape
        return torch.zeros((s.n_layers, 2, self.info.max_batch, s.n_kv_heads, self.info.max_ctx, s.head_dim),
                           dtype=torch.bfloat16, device=self.device)

    def step(self, tokens: torch.Tensor, positions: torch.Tensor, kv: torch.Tensor, logits: torch.Tensor,
             next_tokens: Optional[torch.Tensor] = None, advance: bool = False):
        """Enqueue one decode step on the engine's stream (no host sync)."""
        assert tokens.dtype == torch.int32 and positions.dtype == torch.int32
        assert kv.dtype == torch.bfloat16 and logits.dtype == torch.float32
        assert kv.numel() * 2 == self.kv_bytes and kv.is_contiguous()
        b = tokens.numel()
        assert positions.numel() == b and logits.numel() >= b * self.shape.vocab
        rc = mk.mk_decode_step(self.ctx, tokens.data_ptr(), positions.data_ptr(), b, kv.data_ptr(),
                               logits.data_ptr(), next_tokens.data_ptr() if next_tokens is not None else None,
                               mk.MK_ADVANCE if advance else 0, self.stream.cuda_stream)
        if rc != mk.MK_OK:
            raise mk.MkError(rc, "mk_decode_step")

    def steps(self, tokens: torch.Tensor, positions: torch.Tensor, kv: torch.Tensor, logits: torch.Tensor,
              next_tokens: Optional[torch.Tensor], n_steps: int):
        """Enqueue n_steps greedy steps as one persistent launch (no host sync);
        logits [n_steps][batch][vocab], next_tokens [n_steps][batch]."""
        assert tokens.dtype == torch.int32 and positions.dtype == torch.int32
        assert kv.dtype == torch.bfloat16 and logits.dtype == torch.float32
        assert kv.numel() * 2 == self.kv_bytes and kv.is_contiguous()
        b = tokens.numel()
        assert positions.numel() == b and logits.numel() >= n_steps * b * self.shape.vocab
        assert next_tokens is None or next_tokens.numel() >= n_steps * b
        rc = mk.mk_decode_steps(self.ctx, tokens.data_ptr(), positions.data_ptr(), b, kv.data_ptr(),
                                logits.data_ptr(), next_tokens.data_ptr() if next_tokens is not None else None,
                                n_steps, self.stream.cuda_stream)
        if rc != mk.MK_OK:
            raise mk.MkError(rc, "mk_decode_steps")

    def graph(self, tokens: torch.Tensor, positions: torch.Tensor, kv: torch.Tensor, logits: torch.Tensor,
              next_tokens: Optional[torch.Tensor] = None, advance: bool = False):
        """Capture one step on these buffers as a hipGraph (MK_EXEC_FLAT_MULTI);
        returns an object with launch() and close()."""
        b = tokens.numel()
        g = mk.mk_graph_create(self.ctx, tokens.data_ptr(), positions.data_ptr(), b, kv.data_ptr(),
                               logits.data_ptr(), next_tokens.data_ptr() if next_tokens is not None else None,
                               mk.MK_ADVANCE if advance else 0, self.stream.cuda_stream)
        eng = self

        class _Graph:
            def launch(self):
                rc = mk.mk_graph_launch(g, eng.stream.cuda_stream)
                if rc != mk.MK_OK:
                    raise mk.MkError(rc, "mk_graph_launch")

            def close(self):
                torch.cuda.synchronize(eng.device)
                mk.mk_graph_destroy(g)

        return _Graph()

    def device_error(self):
        return mk.mk_get_device_error(self.ctx, self.stream.cuda_stream)

    def reset(self):
        mk.mk_ctx_reset(self.ctx, self.stream.cuda_stream)

    def close(self):
        if getattr(self, "ctx", None):
            torch.cuda.synchronize(self.device)
            mk.mk_ctx_destroy(self.ctx)
            self.ctx = None
        if getattr(self, "plan", None):
            mk.mk_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def to_gpu(weights: Dict[str, object], device: str = "cuda:0") -> Dict[str, object]:
    """Copy a CPU weight dict (synthetic generator layout) to the GPU."""
    out = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in weights.items() if k != "layers"}
    out["layers"] = [{k: v.to(device) for k, v in ld.items()} for ld in weights["layers"]]
    return out
