"""Seeded synthetic workloads for the MLA forward hot path.

This module only draws and rounds random numbers; it holds none of the
attention arithmetic.  Both the HIP path (through the binding) and the fp64
oracle consume the arrays it returns, so the two sides always see the same
rounded values.

Shapes follow the pages' setting: DeepSeek-V2-Lite / DeepSeek-V3 MLA dims
(latent d_kv = 512, decoupled RoPE band d_rope = 64, per-head d_nope = 128 and
d_v = 128), a 4096-token causal forward, one sequence-parallel rank's share of
a 16384-token sequence (SP = 8), and a 32K-context absorbed decode.  See
"A Training-Memory Regression in MLA Sequence Parallelism ... LAGA" (Pith
review), sections "The pith" and "What carries the argument", and "TPLA:
Tensor Parallel Latent Attention ..." (Pith review), "If this is right".

Recipe (fixed draw order, numpy PCG64, one generator per workload):
  explicit: q_nope, q_pe, c_kv, k_pe, w_kv_b as fp64 standard normals;
            w_kv_b scaled by 1/sqrt(d_kv); every c_kv row divided by its own
            root-mean-square (fp64, no epsilon, no gain); then rounded to the
            storage dtype (bf16 round-to-nearest-even, or fp32).
  decode:   q_nope, q_pe (fp64 normals), then the latent cache one sequence at
            a time as fp32 normals (the k_pe band is taken as already rotated),
            then w_kv_b as for explicit.

bf16 tensors are returned as uint16 bit patterns (``*_bits``) and, for the
small ones, also as float32 arrays holding exactly the rounded values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "ExplicitConfig", "DecodeConfig", "EXPLICIT_CONFIGS", "DECODE_CONFIGS",
    "round_to_bf16_bits", "bf16_bits_to_f32", "make_explicit_inputs",
    "make_decode_inputs",
]


@dataclasses.dataclass(frozen=True)
class ExplicitConfig:
    name: str
    batch: int
    s_q: int
    s_kv: int
    n_heads: int
    d_kv: int
    d_nope: int
    d_rope: int
    d_v: int
    q_pos0: int
    kv_pos0: int
    causal: bool
    dtype: str          # "bf16" or "fp32": storage dtype of every input
    seed: int
    rope_base: float = 10000.0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_nope + self.d_rope))

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the causal mask lets through, per
        head and batch element."""
        if not self.causal:
            return self.s_q * self.s_kv
        total = 0
        # key j visible to query i iff kv_pos0 + j <= q_pos0 + i
        for i in range(self.s_q):
            n = self.q_pos0 + i - self.kv_pos0 + 1
            total += min(max(n, 0), self.s_kv)
        return total

    def visible_keys(self) -> int:
        """Rows of the latent that at least one query can see."""
        if not self.causal:
            return self.s_kv
        n = self.q_pos0 + self.s_q - 1 - self.kv_pos0 + 1
        return min(max(n, 0), self.s_kv)

    def flops(self) -> dict:
        """Algorithmic FLOPs of one forward call: the up-projection over the
        visible latent rows plus 2*(d_qk + d_v) per visible pair and head."""
        up = 2 * self.batch * self.visible_keys() * self.d_kv * self.n_heads * (self.d_nope + self.d_v)
        attn = 2 * self.batch * self.n_heads * self.visible_pairs() * (self.d_nope + self.d_rope + self.d_v)
        return {"up_proj": up, "attention": attn, "total": up + attn}


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    cache_len: int      # rows per sequence, including the new token's own row
    n_heads: int
    d_kv: int
    d_nope: int
    d_rope: int
    d_v: int
    n_splits: int
    seed: int
    rope_base: float = 10000.0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_nope + self.d_rope))

    def algorithmic_bytes(self) -> dict:
        """Bytes the decode step must move at least once (bf16 storage, fp32
        output): the latent cache rows, the W_UK/W_UV weights, the queries and
        the output."""
        cache = self.batch * self.cache_len * (self.d_kv + self.d_rope) * 2
        w = self.n_heads * (self.d_nope + self.d_v) * self.d_kv * 2
        q = self.batch * self.n_heads * (self.d_nope + self.d_rope) * 2
        out = self.batch * self.n_heads * self.d_v * 4
        return {"cache": cache, "weights": w, "queries": q, "out": out,
                "total": cache + w + q + out}

    def flops(self) -> dict:
        d_lat = self.d_kv + self.d_rope
        absorb = 2 * self.batch * self.n_heads * self.d_nope * self.d_kv
        attn = 2 * self.batch * self.n_heads * self.cache_len * (d_lat + self.d_kv)
        unabsorb = 2 * self.batch * self.n_heads * self.d_kv * self.d_v
        return {"absorb": absorb, "attention": attn, "unabsorb": unabsorb,
                "total": absorb + attn + unabsorb}


EXPLICIT_CONFIGS = {
    c.name: c for c in [
        ExplicitConfig("tiny_fp32", 1, 64, 64, 4, 32, 16, 8, 16, 0, 0, True, "fp32", 1001),
        ExplicitConfig("v2lite_bf16", 1, 4096, 4096, 16, 512, 128, 64, 128, 0, 0, True, "bf16", 1002),
        ExplicitConfig("v3_bf16", 1, 4096, 4096, 128, 512, 128, 64, 128, 0, 0, True, "bf16", 1003),
        ExplicitConfig("v3_sp8_rank3", 1, 2048, 16384, 128, 512, 128, 64, 128, 6144, 0, True, "bf16", 1004),
        # longer sequences at V3 dims for the explicit-vs-absorbed memory and
        # time comparison (the LAGA page's 4K / 8K / 16K range)
        ExplicitConfig("v3_s8k_bf16", 1, 8192, 8192, 128, 512, 128, 64, 128, 0, 0, True, "bf16", 1006),
        ExplicitConfig("v3_s16k_bf16", 1, 16384, 16384, 128, 512, 128, 64, 128, 0, 0, True, "bf16", 1007),
        # one rank's share after LAGA's all-to-all at S = 16384 over 8 ranks:
        # H/8 = 16 heads over the whole causal sequence (the head-shard shape
        # of the fused up-projection comparison)
        ExplicitConfig("v3_headshard_sp8", 1, 16384, 16384, 16, 512, 128, 64, 128, 0, 0, True, "bf16", 1008),
    ]
}

DECODE_CONFIGS = {
    c.name: c for c in [
        DecodeConfig("v3_decode_b64_32k", 64, 32768, 128, 512, 128, 64, 128, 16, 1005),
    ]
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (round-to-nearest-even) and return the uint16 bits.
    Inputs here are finite normals, so NaN/Inf handling is not needed."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp64 draw to the storage dtype; returns float32 values that are
    exactly representable in that dtype."""
    if dtype == "fp32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(round_to_bf16_bits(x))
    raise ValueError(dtype)


def make_explicit_inputs(cfg: ExplicitConfig, seed: Optional[int] = None) -> dict:
    """Inputs of one explicit-form forward call, as float32 arrays holding the
    rounded values (bf16-exact for bf16 configs).

    Layouts (row-major):
      q_nope [B, S_q, H, d_nope]    q_pe [B, S_q, H, d_rope] (un-rotated)
      c_kv   [B, S_kv, d_kv]        k_pe [B, S_kv, d_rope]   (un-rotated)
      w_kv_b [H*(d_nope+d_v), d_kv]: row h*(d_nope+d_v)+n holds the weights of
             output n of head h; n < d_nope are the K_nope outputs, the rest
             the V outputs.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, Sq, Skv, H = cfg.batch, cfg.s_q, cfg.s_kv, cfg.n_heads
    q_nope = rng.standard_normal((B, Sq, H, cfg.d_nope))
    q_pe = rng.standard_normal((B, Sq, H, cfg.d_rope))
    c_kv = rng.standard_normal((B, Skv, cfg.d_kv))
    k_pe = rng.standard_normal((B, Skv, cfg.d_rope))
    w = rng.standard_normal((H * (cfg.d_nope + cfg.d_v), cfg.d_kv)) * (1.0 / np.sqrt(cfg.d_kv))
    c_kv = c_kv / np.sqrt(np.mean(c_kv * c_kv, axis=-1, keepdims=True))
    return {
        "q_nope": _store(q_nope, cfg.dtype),
        "q_pe": _store(q_pe, cfg.dtype),
        "c_kv": _store(c_kv, cfg.dtype),
        "k_pe": _store(k_pe, cfg.dtype),
        "w_kv_b": _store(w, cfg.dtype),
    }


def make_decode_inputs(cfg: DecodeConfig, seed: Optional[int] = None,
                       cache_len: Optional[np.ndarray] = None) -> dict:
    """Inputs of one absorbed decode step.

      q_nope [B, H, d_nope], q_pe [B, H, d_rope] (un-rotated): float32, bf16-exact
      cache_bits [B, L, d_kv + d_rope] uint16 bf16 bits: latent c_kv then the
             already-rotated k_pe band, one row per cached token
      cache_len [B] int32: rows attended per sequence (default: all L)
      w_kv_b as for the explicit form, float32 bf16-exact
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, L, H = cfg.batch, cfg.cache_len, cfg.n_heads
    d_lat = cfg.d_kv + cfg.d_rope
    q_nope = _store(rng.standard_normal((B, H, cfg.d_nope)), "bf16")
    q_pe = _store(rng.standard_normal((B, H, cfg.d_rope)), "bf16")
    cache_bits = np.empty((B, L, d_lat), dtype=np.uint16)
    for b in range(B):
        cache_bits[b] = round_to_bf16_bits(rng.standard_normal((L, d_lat), dtype=np.float32))
    w = _store(rng.standard_normal((H * (cfg.d_nope + cfg.d_v), cfg.d_kv)) * (1.0 / np.sqrt(cfg.d_kv)), "bf16")
    if cache_len is None:
        cache_len = np.full((B,), L, dtype=np.int32)
    return {"q_nope": q_nope, "q_pe": q_pe, "cache_bits": cache_bits,
            "cache_len": np.asarray(cache_len, dtype=np.int32), "w_kv_b": w}


def small_explicit(name: str, *, batch=1, s_q=64, s_kv=None, n_heads=4, d_kv=32,
                   d_nope=16, d_rope=8, d_v=16, q_pos0=0, kv_pos0=0, causal=True,
                   dtype="fp32", seed=7) -> ExplicitConfig:
    """An ad-hoc explicit configuration for tests (same recipe, other sizes)."""
    return ExplicitConfig(name, batch, s_q, s_q if s_kv is None else s_kv, n_heads, d_kv,
                          d_nope, d_rope, d_v, q_pos0, kv_pos0, causal, dtype, seed)


def small_decode(name: str, *, batch=2, cache_len=300, n_heads=4, d_kv=512, d_nope=128,
                 d_rope=64, d_v=128, n_splits=4, seed=11) -> DecodeConfig:
    return DecodeConfig(name, batch, cache_len, n_heads, d_kv, d_nope, d_rope, d_v, n_splits, seed)
