"""Seeded synthetic inputs for the decode path (workload shapes + generators).

This module is the only code shared by the CPU oracle side and the GPU side:
it draws random numbers and lays out the workload recipes; it holds none of
the decoder arithmetic.  Every tensor comes from its own torch CPU generator
whose seed is derived from (master seed, tensor name) with SHA-256, so any
tensor is reproducible on its own.

Recipes (all seeded from master seed 0 unless a caller says otherwise):
  * projection / embedding / LM-head weights: N(0, 0.02) drawn in fp32,
    rounded to bf16 (round-to-nearest-even, torch's conversion);
  * norm gains: 1.0 in bf16;
  * KV-cache prefill: N(0, 1) rounded to bf16 for every slot below the first
    decode position of its sequence; slots at or above it hold zeros;
  * token ids: uniform integers in [0, vocab);
  * batched lengths: uniform integers in [lo, hi] inclusive.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 1e4
    tied: bool = False


@dataclasses.dataclass(frozen=True)
class Workload:
    """A decode workload: model shape plus the decode recipe."""
    name: str
    shape: ModelShape
    batch: int
    steps: int              # decode passes
    start_pos: int          # first decode position (prefilled slots below it); -1: per-sequence lengths
    prompt_len: int = 0     # tiny model: prompt tokens fed one per step from position 0
    len_lo: int = 0         # batched decode: per-sequence KV length range (inclusive)
    len_hi: int = 0
    max_ctx: int = 0

    def positions0(self, seed: int = 0) -> List[int]:
        """First decode position of each sequence."""
        if self.start_pos >= 0:
            return [self.start_pos] * self.batch
        g = _gen(seed, self.name + "/lengths")
        return torch.randint(self.len_lo, self.len_hi + 1, (self.batch,), generator=g).tolist()


TINY = ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768, vocab=4096)
LLAMA_1B = ModelShape(n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64, ffn=8192,
                      vocab=128256, tied=True)
LLAMA_8B = ModelShape(n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                      vocab=128256, tied=False)

WORKLOADS: Dict[str, Workload] = {
    # 16 random prompt tokens fed one per step at positions 0..15, then greedy: 47 passes.
    "tiny": Workload("tiny", TINY, batch=1, steps=47, start_pos=0, prompt_len=16, max_ctx=128),
    "llama1b_pos1024": Workload("llama1b_pos1024", LLAMA_1B, batch=1, steps=128, start_pos=1024,
                                max_ctx=1024 + 128),
    "llama1b_pos8192": Workload("llama1b_pos8192", LLAMA_1B, batch=1, steps=64, start_pos=8192,
                                max_ctx=8192 + 64),
    "llama1b_b16": Workload("llama1b_b16", LLAMA_1B, batch=16, steps=64, start_pos=-1, len_lo=512,
                            len_hi=4096, max_ctx=4096 + 64),
    "llama8b_pos2048": Workload("llama8b_pos2048", LLAMA_8B, batch=1, steps=64, start_pos=2048,
                                max_ctx=2048 + 64),
}


def _seed_of(master: int, name: str) -> int:
    h = hashlib.sha256(f"{master}:{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(master: int, name: str) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed_of(master, name))
    return g


def normal_bf16(shape, std: float, master: int, name: str) -> torch.Tensor:
    """bf16 CPU tensor of N(0, std^2) values (drawn in fp32, rounded RNE)."""
    g = _gen(master, name)
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def uniform_ints(n: int, lo: int, hi_exclusive: int, master: int, name: str) -> List[int]:
    g = _gen(master, name)
    return torch.randint(lo, hi_exclusive, (n,), generator=g).tolist()


LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd")


def layer_tensor_shapes(s: ModelShape) -> Dict[str, tuple]:
    d = s.head_dim
    return {
        "attn_norm": (s.hidden,),
        "wq": (s.n_q_heads * d, s.hidden),
        "wk": (s.n_kv_heads * d, s.hidden),
        "wv": (s.n_kv_heads * d, s.hidden),
        "wo": (s.hidden, s.n_q_heads * d),
        "mlp_norm": (s.hidden,),
        "wg": (s.ffn, s.hidden),
        "wu": (s.ffn, s.hidden),
        "wd": (s.hidden, s.ffn),
    }


def make_weights(s: ModelShape, master: int = 0, std: float = 0.02, gain_std: float = 0.0,
                 prefix: str = "") -> Dict[str, object]:
    """Seeded bf16 CPU weights for shape `s`.

    Returns {"embed", "lm_head" (None when tied), "final_norm", "layers": [dict]}.
    gain_std > 0 draws norm gains as 1 + N(0, gain_std^2) (used by tests that
    want the gains to matter); 0 gives the workloads' gains of exactly 1.
    """
    def gain(name):
        if gain_std == 0.0:
            return torch.ones(s.hidden, dtype=torch.bfloat16)
        return (1.0 + normal_bf16((s.hidden,), gain_std, master, prefix + name).float()).to(torch.bfloat16)

    w: Dict[str, object] = {}
    w["embed"] = normal_bf16((s.vocab, s.hidden), std, master, prefix + "embed")
    w["lm_head"] = None if s.tied else normal_bf16((s.vocab, s.hidden), std, master, prefix + "lm_head")
    w["final_norm"] = gain("final_norm")
    layers = []
    for l in range(s.n_layers):
        shapes = layer_tensor_shapes(s)
        ld = {}
        for name in LAYER_TENSORS:
            key = f"{prefix}layers.{l}.{name}"
            if name.endswith("norm"):
                ld[name] = gain(key)
            else:
                ld[name] = normal_bf16(shapes[name], std, master, key)
        layers.append(ld)
    w["layers"] = layers
    return w


def kv_cache_shape(s: ModelShape, b_max: int, max_ctx: int) -> tuple:
    """[L][2 (keys, values)][B_max][n_kv][max_ctx][head_dim], bf16."""
    return (s.n_layers, 2, b_max, s.n_kv_heads, max_ctx, s.head_dim)


def make_kv_cache(s: ModelShape, b_max: int, max_ctx: int, prefill_lens: List[int], master: int = 0,
                  name: str = "kv_prefill") -> torch.Tensor:
    """bf16 CPU cache with N(0,1) values in slots [0, prefill_lens[b]) of sequence b."""
    kv = torch.zeros(kv_cache_shape(s, b_max, max_ctx), dtype=torch.bfloat16)
    for b, n in enumerate(prefill_lens):
        if n <= 0:
            continue
        vals = normal_bf16((s.n_layers, 2, s.n_kv_heads, n, s.head_dim), 1.0, master, f"{name}/seq{b}")
        kv[:, :, b, :, :n, :] = vals
    return kv


def workload_tokens(wl: Workload, master: int = 0) -> List[int]:
    """First tokens of each sequence (tiny model: the whole prompt)."""
    if wl.prompt_len:
        return uniform_ints(wl.prompt_len, 0, wl.shape.vocab, master, wl.name + "/prompt")
    return uniform_ints(wl.batch, 0, wl.shape.vocab, master, wl.name + "/tokens")


def bf16_bits(t: Optional[torch.Tensor]):
    """numpy uint16 view of a bf16 CPU tensor (None passes through)."""
    if t is None:
        return None
    return t.contiguous().view(torch.int16).numpy().view("uint16")
