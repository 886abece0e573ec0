"""ctypes front end of the CPU oracle (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
import this module.  It never touches a GPU and shares no code with the HIP
library.  The arithmetic lives in mk_oracle.c; this file only marshals
numpy arrays into it.

Parity status: every piece (bf16 rounding, matvec, RMSNorm, RoPE, attention,
SiLU, argmax, cache indexing) and the composed step are pinned by tests under
tests/ against closed forms, invariants, numpy/torch library routines and a
third-party Llama implementation; no function here is unpinned.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from typing import Dict, List, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liborc.so")
SRC_PATH = os.path.join(HERE, "mk_oracle.c")

KV_BF16 = 0
KV_F64 = 1

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile mk_oracle.c into liborc.so with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        tmp = LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Shape(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_double), ("rope_theta", C.c_double),
                ("tied", C.c_int32)]


_PP = C.POINTER(C.c_void_p)


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("final_norm", C.c_void_p),
                ("attn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP),
                ("mlp_norm", _PP), ("wg", _PP), ("wu", _PP), ("wd", _PP)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = C.CDLL(LIB_PATH)
            dp = C.POINTER(C.c_double)
            L.orc_bf16_to_f64.restype = C.c_double
            L.orc_bf16_to_f64.argtypes = [C.c_uint16]
            L.orc_f64_to_bf16.restype = C.c_uint16
            L.orc_f64_to_bf16.argtypes = [C.c_double]
            L.orc_matvec.restype = None
            L.orc_matvec.argtypes = [C.c_void_p, C.c_int64, C.c_int64, dp, dp]
            L.orc_rmsnorm.restype = None
            L.orc_rmsnorm.argtypes = [dp, C.c_void_p, C.c_int64, C.c_double, dp]
            L.orc_rope.restype = None
            L.orc_rope.argtypes = [dp, C.c_int, C.c_int64, C.c_double]
            L.orc_silu.restype = C.c_double
            L.orc_silu.argtypes = [C.c_double]
            L.orc_attend.restype = None
            L.orc_attend.argtypes = [dp, C.c_void_p, C.c_void_p, C.c_int, C.c_int64, C.c_int, C.c_double, dp, dp]
            L.orc_argmax_f32.restype = C.c_int64
            L.orc_argmax_f32.argtypes = [dp, C.c_int64]
            L.orc_kv_index.restype = C.c_int64
            L.orc_kv_index.argtypes = [C.POINTER(Shape), C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                       C.c_int64, C.c_int64, C.c_int64]
            L.orc_decode_step.restype = C.c_int
            L.orc_decode_step.argtypes = [C.POINTER(Shape), C.POINTER(Weights), C.c_int32, C.c_void_p,
                                          C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, dp, C.c_void_p,
                                          dp]
            L.orc_num_threads.restype = C.c_int
            _lib = L
    return _lib


def _dptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


# ------------------------------------------------------------------ pieces

def bf16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_bf16_to_f64(int(x)) for x in b], dtype=np.float64)


def f64_to_bf16(vals) -> np.ndarray:
    L = lib()
    v = np.asarray(vals, dtype=np.float64).ravel()
    return np.array([L.orc_f64_to_bf16(float(x)) for x in v], dtype=np.uint16)


def matvec(W_bits: np.ndarray, x: np.ndarray) -> np.ndarray:
    W = _u16(W_bits)
    rows, cols = W.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(rows, dtype=np.float64)
    lib().orc_matvec(W.ctypes.data, rows, cols, _dptr(x), _dptr(y))
    return y


def rmsnorm(x: np.ndarray, gain_bits: Optional[np.ndarray], eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    g = None if gain_bits is None else _u16(gain_bits)
    lib().orc_rmsnorm(_dptr(x), None if g is None else g.ctypes.data, x.size, eps, _dptr(out))
    return out


def rope(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    u = np.array(u, dtype=np.float64, copy=True)
    lib().orc_rope(_dptr(u), u.size, pos, theta)
    return u


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """K, V: [n_pos][d] as uint16 (bf16 bits) or float64.  Returns (out, weights)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    if K.dtype == np.uint16:
        mode = KV_BF16
    else:
        mode = KV_F64
        K = np.ascontiguousarray(K, dtype=np.float64)
        V = np.ascontiguousarray(V, dtype=np.float64)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    n, d = K.shape
    out = np.empty(d, dtype=np.float64)
    w = np.empty(max(n, 1), dtype=np.float64)
    lib().orc_attend(_dptr(q), K.ctypes.data, V.ctypes.data, mode, n, d, scale, _dptr(out), _dptr(w))
    return out, w[:n]


def argmax_f32(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, dtype=np.float64)
    return int(lib().orc_argmax_f32(_dptr(v), v.size))


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ------------------------------------------------------------------ model

class Model:
    """Holds numpy views of one model's bf16 weights and runs oracle steps."""

    def __init__(self, shape, weights: Dict[str, object]):
        """shape: synth_inputs.ModelShape; weights: synth_inputs.make_weights()
        output, or the same structure with numpy uint16 arrays."""
        self.shape = shape
        s = shape
        self.cshape = Shape(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                            float(s.rms_eps), float(s.rope_theta), 1 if s.tied else 0)
        conv = _to_bits
        self._keep: List[np.ndarray] = []
        self.embed = conv(weights["embed"])
        self.lm_head = conv(weights["lm_head"]) if weights.get("lm_head") is not None else None
        self.final_norm = conv(weights["final_norm"])
        self._keep += [self.embed, self.final_norm] + ([self.lm_head] if self.lm_head is not None else [])
        L = s.n_layers
        self.layers = [{k: conv(v) for k, v in ld.items()} for ld in weights["layers"]]
        arrs = {}
        for name in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd"):
            ptrs = (C.c_void_p * max(L, 1))()
            for l in range(L):
                a = self.layers[l][name]
                self._keep.append(a)
                ptrs[l] = a.ctypes.data
            arrs[name] = ptrs
        self._ptr_arrays = arrs
        if s.tied:
            lm = None
        else:
            if self.lm_head is None:
                raise ValueError("untied shape needs an lm_head tensor")
            lm = self.lm_head.ctypes.data
        self.cweights = Weights(self.embed.ctypes.data, lm, self.final_norm.ctypes.data,
                                *[C.cast(arrs[n], _PP) for n in ("attn_norm", "wq", "wk", "wv", "wo",
                                                                  "mlp_norm", "wg", "wu", "wd")])

    def step(self, tokens, positions, kv: np.ndarray, b_max: int, max_ctx: int, probe: Optional[np.ndarray] = None):
        """One decode step.  kv: numpy uint16 (bf16 cache) or float64 array laid
        out [L][2][b_max][n_kv][max_ctx][d]; updated in place.  Returns
        (logits float64 [B][V], next tokens int32 [B]).  probe (optional,
        float64 [B][L][3][n_kv][d]) receives the appended keys before and
        after the rotation and the appended values, unrounded."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        B = tok.size
        if kv.dtype == np.uint16:
            mode = KV_BF16
        elif kv.dtype == np.float64:
            mode = KV_F64
        else:
            raise TypeError("kv cache must be uint16 (bf16 bits) or float64")
        assert kv.flags["C_CONTIGUOUS"]
        logits = np.empty((B, self.shape.vocab), dtype=np.float64)
        nxt = np.empty(B, dtype=np.int32)
        rc = lib().orc_decode_step(C.byref(self.cshape), C.byref(self.cweights), B, tok.ctypes.data,
                                   pos.ctypes.data, kv.ctypes.data, mode, b_max, max_ctx, _dptr(logits),
                                   nxt.ctypes.data, None if probe is None else _dptr(probe))
        if rc != 0:
            raise ValueError(f"oracle step failed with code {rc}")
        return logits, nxt

    def kv_index(self, b_max, max_ctx, l, plane, b, g, t) -> int:
        return int(lib().orc_kv_index(C.byref(self.cshape), b_max, max_ctx, l, plane, b, g, t))


def _to_bits(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return _u16(t)
    # torch bf16 tensor
    import torch
    assert t.dtype == torch.bfloat16
    return np.ascontiguousarray(t.contiguous().view(torch.int16).numpy().view(np.uint16))
