"""fp64 CPU oracle for the MLA forward hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it.

What it computes, and where the pages state it:

  Pages cited (Pith review pages):
    [LAGA]  "A Training-Memory Regression in MLA Sequence Parallelism: Why
             Megatron-Core Forbids Absorption, and LAGA -- a
             Communication-Efficient Fix"
    [TPLA]  "TPLA: Tensor Parallel Latent Attention for Efficient
             Disaggregated Prefill and Decode Inference"
    [Helix] "Helix Parallelism: Rethinking Sharding Strategies for
             Interactive Multi-Million-Token LLM Decoding"

  * Explicit form (the form used for training and the per-rank compute of
    LAGA): per-head K_nope and V are the latent c_KV times the shared linear
    up-projection W_kv_b; a small RoPE band is carried beside the latent, once
    per token, and shared by all heads; causal softmax attention runs in head
    dimension.  [LAGA] "What carries the argument", Fig. 2 caption ("Explicit
    (B1)" and "LAGA" data flows), axiom ledger (the up-projection is linear and
    shared across heads; the latent is common to all heads).
  * Absorbed form: the query is moved into latent space through the transpose
    of W_kv_b's key part, attention runs against the latent plus RoPE band, and
    the post-attention latent accumulator is mapped back through W_kv_b's value
    part.  [LAGA] "What carries the argument", Fig. 2 caption ("Absorbed
    (B2)"); the 576-wide latent row per token: [TPLA] "If this is right".
  * Split-KV decode: each KV chunk yields a partial output and its
    log-sum-exp; the partials are rescaled by their LSE and summed, which
    reproduces the exact softmax.  [Helix] "What carries the argument" and
    "Core claim".

Readings where the pages leave a step open (each one is also listed in the
design notes of the repository):
  R1 W_kv_b layout: a linear map from d_kv to H*(d_nope+d_v), stored as
     [H*(d_nope+d_v), d_kv] (one row per output feature); head h owns rows
     h*(d_nope+d_v) .. (h+1)*(d_nope+d_v)-1, first d_nope of them K_nope, the
     rest V.  Then "W_kv_b transposed times q_nope" is literally W_UK[h]^T q.
  R2 RoPE: rotate-half pairing (m, m + d_r/2), theta_m = base^(-2m/d_r),
     angle = position * theta_m, base 10000.
  R3 Explicit inputs are un-rotated and rotated at absolute positions
     (q_pos0 + i, kv_pos0 + j).  In decode the cache holds k_pe already rotated
     and only q_pe is rotated, at position L_b - 1.
  R4 Softmax scale 1/sqrt(d_nope + d_rope) on the whole logit.
  R5 Causal: key j visible to query i iff kv_pos0 + j <= q_pos0 + i.  A query
     with no visible key gets O = 0 and LSE = -inf.
  R6 Decode chunks: c = ceil(L_b / n_s), chunk k = [k*c, min(L_b, (k+1)*c));
     an empty chunk has lse = -inf and a zero partial.
  R7 LSE is the natural log of the sum of exp of the scaled logits.
  R13 Backward: the gradient of sum(d_out * O) with respect to the five
     inputs of the explicit form (q_nope, q_pe, c_kv, k_pe, W_kv_b), all
     in the inputs' own (un-rotated) coordinates.

Everything is float64 on the exact input values.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "rope_theta", "rope_rotate", "weight_slices", "visibility_mask",
    "explicit_fwd", "absorbed_fwd", "decode_absorbed", "lse_merge",
    "brute_force_explicit", "explicit_bwd",
]


# --------------------------------------------------------------------------
# RoPE on the decoupled band (reading R2)
# --------------------------------------------------------------------------
def rope_theta(d_rope: int, base: float) -> np.ndarray:
    """theta_m = base^(-2m/d_rope), m = 0 .. d_rope/2 - 1 (reading R2)."""
    m = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * m / d_rope)


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE of the last axis of ``x`` at positions ``pos``.

    ``pos`` broadcasts against x[..., 0].  Pair (m, m+h) is rotated by the
    angle pos*theta_m:
        y[m]   = x[m] cos - x[m+h] sin
        y[m+h] = x[m+h] cos + x[m] sin
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def weight_slices(w_kv_b: np.ndarray, n_heads: int, d_nope: int, d_v: int):
    """Per-head W_UK [H, d_nope, d_kv] and W_UV [H, d_v, d_kv] (reading R1)."""
    w = np.asarray(w_kv_b, dtype=np.float64)
    d_kv = w.shape[1]
    w = w.reshape(n_heads, d_nope + d_v, d_kv)
    return w[:, :d_nope, :], w[:, d_nope:, :]


def visibility_mask(s_q: int, s_kv: int, q_pos0: int, kv_pos0: int, causal: bool) -> np.ndarray:
    """[s_q, s_kv] boolean: key j visible to query i (reading R5)."""
    if not causal:
        return np.ones((s_q, s_kv), dtype=bool)
    qp = q_pos0 + np.arange(s_q)[:, None]
    kp = kv_pos0 + np.arange(s_kv)[None, :]
    return kp <= qp


def _masked_softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Row softmax of s over the visible entries.  Returns (P, lse); rows with
    no visible entry get P = 0 and lse = -inf."""
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.where(vis, np.exp(s - m_safe), 0.0)
    l = np.sum(e, axis=-1, keepdims=True)
    p = np.where(has, e / np.where(has, l, 1.0), 0.0)
    lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return p, lse[..., 0]


def _positions(n: int, p0: int) -> np.ndarray:
    return p0 + np.arange(n, dtype=np.float64)


# --------------------------------------------------------------------------
# Explicit form (B1 / LAGA-local)
# --------------------------------------------------------------------------
def explicit_fwd(q_nope, q_pe, c_kv, k_pe, w_kv_b, *, q_pos0=0, kv_pos0=0, causal=True,
                 softmax_scale: Optional[float] = None, rope_base=10000.0,
                 heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None):
    """Explicit-form MLA forward.

    q_nope [B,S_q,H,d_n], q_pe [B,S_q,H,d_r], c_kv [B,S_kv,d_c], k_pe [B,S_kv,d_r],
    w_kv_b [H*(d_n+d_v), d_c].  Returns (O [B,S_q',H',d_v], LSE [B,H',S_q']) for
    the selected ``heads`` and query ``rows`` (all by default).

    K_nope[j,h] = W_UK[h] c_j and V[j,h] = W_UV[h] c_j; the logit is
    sigma*(q_nope.K_nope + R(q_pe, q_pos0+i).R(k_pe, kv_pos0+j)) with the
    rotated key band shared by every head; causal softmax; O = P V.
    [LAGA] "What carries the argument" and Fig. 2 (B1 / LAGA flows).
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    B, S_q, H, d_n = q_nope.shape
    S_kv = c_kv.shape[1]
    d_r = q_pe.shape[-1]
    d_v = w_kv_b.shape[0] // H - d_n
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_n + d_r)
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    w_uk, w_uv = weight_slices(w_kv_b, H, d_n, d_v)

    qpos = _positions(S_q, q_pos0)[rows]
    kpos = _positions(S_kv, kv_pos0)
    vis = visibility_mask(S_q, S_kv, q_pos0, kv_pos0, causal)[rows]
    out = np.zeros((B, len(rows), len(heads), d_v))
    lse = np.zeros((B, len(heads), len(rows)))
    for b in range(B):
        k_rot = rope_rotate(k_pe[b], kpos, rope_base)                     # [S_kv, d_r], shared by heads
        for hi, h in enumerate(heads):
            k_n = c_kv[b] @ w_uk[h].T                                      # [S_kv, d_n]
            v = c_kv[b] @ w_uv[h].T                                        # [S_kv, d_v]
            q_rot = rope_rotate(q_pe[b, rows, h], qpos, rope_base)         # [S_q', d_r]
            s = softmax_scale * (q_nope[b, rows, h] @ k_n.T + q_rot @ k_rot.T)
            p, l = _masked_softmax_rows(s, vis)
            out[b, :, hi] = p @ v
            lse[b, hi] = l
    return out, lse


# --------------------------------------------------------------------------
# Absorbed form (B2) on the same inputs
# --------------------------------------------------------------------------
def absorbed_fwd(q_nope, q_pe, c_kv, k_pe, w_kv_b, *, q_pos0=0, kv_pos0=0, causal=True,
                 softmax_scale: Optional[float] = None, rope_base=10000.0,
                 heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None):
    """Absorbed-form MLA forward on explicit-form inputs.

    q_lat = W_UK[h]^T q_nope (d_c wide); logit sigma*(q_lat.c_j + R(q_pe).R(k_pe));
    o_lat = sum_j P c_j (the post-attention latent accumulator); O = W_UV[h] o_lat.
    [LAGA] "What carries the argument" (q_absorbed and the latent accumulator)
    and Fig. 2 ("Absorbed (B2)": absorb -> latent attention -> un-absorb).
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    B, S_q, H, d_n = q_nope.shape
    S_kv = c_kv.shape[1]
    d_r = q_pe.shape[-1]
    d_v = w_kv_b.shape[0] // H - d_n
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_n + d_r)
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    w_uk, w_uv = weight_slices(w_kv_b, H, d_n, d_v)
    qpos = _positions(S_q, q_pos0)[rows]
    kpos = _positions(S_kv, kv_pos0)
    vis = visibility_mask(S_q, S_kv, q_pos0, kv_pos0, causal)[rows]
    out = np.zeros((B, len(rows), len(heads), d_v))
    lse = np.zeros((B, len(heads), len(rows)))
    for b in range(B):
        k_rot = rope_rotate(k_pe[b], kpos, rope_base)
        for hi, h in enumerate(heads):
            q_lat = q_nope[b, rows, h] @ w_uk[h]                           # [S_q', d_c]
            q_rot = rope_rotate(q_pe[b, rows, h], qpos, rope_base)
            s = softmax_scale * (q_lat @ c_kv[b].T + q_rot @ k_rot.T)
            p, l = _masked_softmax_rows(s, vis)
            o_lat = p @ c_kv[b]                                            # [S_q', d_c]
            out[b, :, hi] = o_lat @ w_uv[h].T
            lse[b, hi] = l
    return out, lse


# --------------------------------------------------------------------------
# Split-KV merge by log-sum-exp ([Helix] "What carries the argument")
# --------------------------------------------------------------------------
def lse_merge(o_part: np.ndarray, lse_part: np.ndarray):
    """Merge chunk partials along axis 0.

    o_part [n_s, ..., d] holds each chunk's output normalised within the
    chunk; lse_part [n_s, ...] its log-sum-exp.  lse = logsumexp_k lse_k and
    o = sum_k exp(lse_k - lse) o_k.  Chunks with lse_k = -inf weigh nothing;
    if every chunk is empty the result is o = 0, lse = -inf.
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    m = np.max(lse_part, axis=0)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    wgt = np.where(np.isfinite(lse_part), np.exp(lse_part - m_safe), 0.0)
    tot = np.sum(wgt, axis=0)
    lse = np.where(has, m_safe + np.log(np.where(has, tot, 1.0)), -np.inf)
    scale = np.where(has, 1.0 / np.where(has, tot, 1.0), 0.0)
    o = np.einsum("k...,k...d->...d", wgt * scale, o_part)
    return o, lse


def chunk_bounds(length: int, n_splits: int):
    """[start, end) of each of the n_splits chunks of a length-L sequence
    (reading R6)."""
    c = -(-length // n_splits) if length > 0 else 0
    return [(min(length, k * c), min(length, (k + 1) * c)) for k in range(n_splits)]


# --------------------------------------------------------------------------
# Absorbed split-KV decode
# --------------------------------------------------------------------------
def decode_absorbed(q_nope, q_pe, cache, cache_len, w_kv_b, *, n_splits, d_kv,
                    softmax_scale: Optional[float] = None, rope_base=10000.0,
                    batches: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None):
    """One decode step in absorbed form with the KV sequence split in chunks.

    q_nope [B,H,d_n], q_pe [B,H,d_r] (un-rotated), cache [B,L,d_kv+d_r] (latent
    then already-rotated k_pe; may be a callable b -> [L, d_kv+d_r] array so a
    large cache can be upcast one sequence at a time), cache_len [B],
    w_kv_b [H*(d_n+d_v), d_kv].

    Per sequence b with L_b rows: q~ = [W_UK[h]^T q_nope ; R(q_pe, L_b - 1)];
    logits sigma * q~ . row_t for t < L_b; per chunk a normalised partial
    latent output and its LSE; merged by lse_merge; O = W_UV[h] o_lat.
    Returns a dict with out [B',H',d_v], lse [B',H'], q_tilde [B',H',d_kv+d_r],
    o_part [B',n_s,H',d_kv], lse_part [B',n_s,H'] and o_lat [B',H',d_kv].
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    B, H, d_n = q_nope.shape
    d_r = q_pe.shape[-1]
    d_v = w_kv_b.shape[0] // H - d_n
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_n + d_r)
    batches = list(range(B)) if batches is None else list(batches)
    heads = list(range(H)) if heads is None else list(heads)
    w_uk, w_uv = weight_slices(w_kv_b, H, d_n, d_v)
    get = cache if callable(cache) else (lambda b: np.asarray(cache[b]))
    nb, nh = len(batches), len(heads)
    res = {
        "out": np.zeros((nb, nh, d_v)), "lse": np.zeros((nb, nh)),
        "q_tilde": np.zeros((nb, nh, d_kv + d_r)),
        "o_part": np.zeros((nb, n_splits, nh, d_kv)), "lse_part": np.zeros((nb, n_splits, nh)),
        "o_lat": np.zeros((nb, nh, d_kv)),
    }
    for bi, b in enumerate(batches):
        L = int(cache_len[b])
        rows = np.asarray(get(b)[:L], dtype=np.float64)                    # [L, d_kv+d_r]
        q_lat = np.stack([q_nope[b, h] @ w_uk[h] for h in heads])          # [H', d_kv]
        q_rot = rope_rotate(q_pe[b, heads], np.full(nh, L - 1, dtype=np.float64), rope_base)
        q_t = np.concatenate([q_lat, q_rot], axis=-1)                      # [H', d_kv+d_r]
        res["q_tilde"][bi] = q_t
        for k, (t0, t1) in enumerate(chunk_bounds(L, n_splits)):
            if t1 <= t0:
                res["lse_part"][bi, k] = -np.inf
                continue
            s = softmax_scale * (q_t @ rows[t0:t1].T)                      # [H', T]
            m = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - m)
            l = np.sum(e, axis=-1, keepdims=True)
            res["o_part"][bi, k] = (e / l) @ rows[t0:t1, :d_kv]
            res["lse_part"][bi, k] = (m + np.log(l))[:, 0]
        o_lat, lse = lse_merge(res["o_part"][bi], res["lse_part"][bi])
        res["o_lat"][bi] = o_lat
        res["lse"][bi] = lse
        res["out"][bi] = np.stack([w_uv[h] @ o_lat[hi] for hi, h in enumerate(heads)])
    return res


# --------------------------------------------------------------------------
# Backward of the explicit form (the training setting of [LAGA])
# --------------------------------------------------------------------------
def _softmax_bwd(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """Row softmax Jacobian applied to dP: dS = P * (dP - sum_j P dP) per row
    (rows with no visible key have P = 0 and get dS = 0)."""
    return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))


def explicit_bwd(q_nope, q_pe, c_kv, k_pe, w_kv_b, d_out, *, q_pos0=0, kv_pos0=0, causal=True,
                 softmax_scale: Optional[float] = None, rope_base=10000.0,
                 heads: Optional[Sequence[int]] = None):
    """Gradients of sum(d_out * O) through explicit_fwd, with respect to every
    input.  [LAGA] is about training: its "If this is right" section states
    that LAGA's parameter gradients equal the explicit form's, and the Fig. 5
    caption bounds their difference; this is the explicit form's gradient.

    Reverse mode through the forward's steps, per batch entry and head:
      O = P V                      -> dV = P^T dO, dP = dO V^T
      P = softmax(s) over visible  -> dS = P * (dP - rowsum(P * dP))
      s = sigma (q_n K^T + q_r k_r^T)
                                   -> dq_n = sigma dS K, dq_r = sigma dS k_r,
                                      dK = sigma dS^T q_n, dk_r = sigma dS^T q_r
      K = c W_UK^T, V = c W_UV^T   -> dc = dK W_UK + dV W_UV,
                                      dW_UK = dK^T c, dW_UV = dV^T c
      q_r = R(q_pe, p), k_r = R(k_pe, p')
                                   -> R is a rotation, so its transpose rotates
                                      back: dq_pe = R(dq_r, -p); the key band is
                                      shared by the heads, so
                                      dk_pe = R(sum_h dk_r, -p')
    Returns a dict with dq_nope [B,S_q,H,d_n], dq_pe [B,S_q,H,d_r],
    dc_kv [B,S_kv,d_c], dk_pe [B,S_kv,d_r] and dw_kv_b [H*(d_n+d_v), d_c].
    With ``heads`` only those heads are differentiated: their dq and W_kv_b
    rows are exact, other heads' entries are zero, and dc_kv / dk_pe hold
    only the selected heads' terms of their sums over heads.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    B, S_q, H, d_n = q_nope.shape
    S_kv = c_kv.shape[1]
    d_r = q_pe.shape[-1]
    d_v = w_kv_b.shape[0] // H - d_n
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_n + d_r)
    sig = softmax_scale
    w_uk, w_uv = weight_slices(w_kv_b, H, d_n, d_v)
    qpos = _positions(S_q, q_pos0)
    kpos = _positions(S_kv, kv_pos0)
    vis = visibility_mask(S_q, S_kv, q_pos0, kv_pos0, causal)
    g = {"dq_nope": np.zeros_like(q_nope), "dq_pe": np.zeros_like(q_pe), "dc_kv": np.zeros_like(c_kv),
         "dk_pe": np.zeros_like(k_pe)}
    dw_uk = np.zeros_like(w_uk)
    dw_uv = np.zeros_like(w_uv)
    heads = list(range(H)) if heads is None else list(heads)
    for b in range(B):
        k_rot = rope_rotate(k_pe[b], kpos, rope_base)
        dk_rot = np.zeros_like(k_rot)
        for h in heads:
            k_n = c_kv[b] @ w_uk[h].T
            v = c_kv[b] @ w_uv[h].T
            q_rot = rope_rotate(q_pe[b, :, h], qpos, rope_base)
            s = sig * (q_nope[b, :, h] @ k_n.T + q_rot @ k_rot.T)
            p, _ = _masked_softmax_rows(s, vis)
            do = d_out[b, :, h]
            dv = p.T @ do
            dp = do @ v.T
            ds = _softmax_bwd(p, dp)
            g["dq_nope"][b, :, h] = sig * (ds @ k_n)
            g["dq_pe"][b, :, h] = rope_rotate(sig * (ds @ k_rot), -qpos, rope_base)
            dk_n = sig * (ds.T @ q_nope[b, :, h])
            dk_rot += sig * (ds.T @ q_rot)
            g["dc_kv"][b] += dk_n @ w_uk[h] + dv @ w_uv[h]
            dw_uk[h] += dk_n.T @ c_kv[b]
            dw_uv[h] += dv.T @ c_kv[b]
        g["dk_pe"][b] = rope_rotate(dk_rot, -kpos, rope_base)
    g["dw_kv_b"] = _head_grads_to_w_layout(dw_uk, dw_uv)
    return g


def _head_grads_to_w_layout(dw_uk: np.ndarray, dw_uv: np.ndarray) -> np.ndarray:
    """[H, d_n, d_c] and [H, d_v, d_c] back to W_kv_b's row layout (reading R1):
    head h's rows are its d_n key rows, then its d_v value rows."""
    H = dw_uk.shape[0]
    return np.concatenate([dw_uk, dw_uv], axis=1).reshape(H * (dw_uk.shape[1] + dw_uv.shape[1]), -1)


# --------------------------------------------------------------------------
# Brute force (pure Python loops, no BLAS), tiny inputs only
# --------------------------------------------------------------------------
def brute_force_explicit(q_nope, q_pe, c_kv, k_pe, w_kv_b, *, q_pos0=0, kv_pos0=0, causal=True,
                         softmax_scale=None, rope_base=10000.0):
    """The explicit form written element by element with Python floats.
    Meant for inputs of a few thousand elements."""
    q_nope = np.asarray(q_nope, dtype=np.float64).tolist()
    q_pe = np.asarray(q_pe, dtype=np.float64).tolist()
    c_kv = np.asarray(c_kv, dtype=np.float64).tolist()
    k_pe = np.asarray(k_pe, dtype=np.float64).tolist()
    w = np.asarray(w_kv_b, dtype=np.float64).tolist()
    B, S_q, H, d_n = len(q_nope), len(q_nope[0]), len(q_nope[0][0]), len(q_nope[0][0][0])
    S_kv, d_c, d_r = len(c_kv[0]), len(c_kv[0][0]), len(q_pe[0][0][0])
    d_v = len(w) // H - d_n
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_n + d_r)
    half = d_r // 2

    def rot(x, p):
        y = [0.0] * d_r
        for m in range(half):
            th = p * float(rope_base) ** (-2.0 * m / d_r)
            y[m] = x[m] * math.cos(th) - x[m + half] * math.sin(th)
            y[m + half] = x[m + half] * math.cos(th) + x[m] * math.sin(th)
        return y

    out = [[[[0.0] * d_v for _ in range(H)] for _ in range(S_q)] for _ in range(B)]
    lse = [[[0.0] * S_q for _ in range(H)] for _ in range(B)]
    for b in range(B):
        krot = [rot(k_pe[b][j], kv_pos0 + j) for j in range(S_kv)]
        for h in range(H):
            base_row = h * (d_n + d_v)
            kn = [[sum(c_kv[b][j][c] * w[base_row + n][c] for c in range(d_c)) for n in range(d_n)]
                  for j in range(S_kv)]
            vv = [[sum(c_kv[b][j][c] * w[base_row + d_n + n][c] for c in range(d_c)) for n in range(d_v)]
                  for j in range(S_kv)]
            for i in range(S_q):
                qr = rot(q_pe[b][i][h], q_pos0 + i)
                logits = []
                for j in range(S_kv):
                    if causal and kv_pos0 + j > q_pos0 + i:
                        continue
                    dot = sum(q_nope[b][i][h][n] * kn[j][n] for n in range(d_n))
                    dot += sum(qr[m] * krot[j][m] for m in range(d_r))
                    logits.append((j, softmax_scale * dot))
                if not logits:
                    lse[b][h][i] = -math.inf
                    continue
                mx = max(s for _, s in logits)
                den = sum(math.exp(s - mx) for _, s in logits)
                lse[b][h][i] = mx + math.log(den)
                for j, s in logits:
                    p = math.exp(s - mx) / den
                    for n in range(d_v):
                        out[b][i][h][n] += p * vv[j][n]
    return np.array(out), np.array(lse)
