"""GPU parity of the explicit-form backward (mla_bwd_explicit) against the
fp64 oracle's explicit_bwd, on the same seeded inputs.

The backward is fed the oracle's forward output and LSE (rounded to fp32), so
each case tests the backward's own arithmetic; one case chains the GPU
forward into the GPU backward.  Gradients are not O(1) quantities, so the
max-abs bars are taken relative to the largest reference entry:
  * fp32 arithmetic (SIMT kernels): max|d| <= 1e-5 max(1, max|ref|) for the
    fp32 configuration (the spec fp32 bar, scaled), 1e-4 max(1, max|ref|)
    for bf16-stored inputs whose reductions run over up to 512 * 128 terms;
  * bf16 / fp16 operands (MFMA kernels): max|d| <= 1e-2 max(1, max|ref|) and
    rel-L2 <= 5e-3 (the spec bf16 bars, scaled).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from head_latent_attention_02_amd import inputs as I

pytestmark = pytest.mark.gpu

GRADS = ("dq_nope", "dq_pe", "dc_kv", "dk_pe", "dw_kv_b")


def _say(msg):
    print(f"[gpu-bwd] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_02_amd import mla as m
    m.library()
    return m


def _args(cfg):
    return dict(q_pos0=cfg.q_pos0, kv_pos0=cfg.kv_pos0, causal=cfg.causal, softmax_scale=cfg.softmax_scale,
                rope_base=cfg.rope_base)


def _case(cfg, seed):
    x = I.make_explicit_inputs(cfg)
    rng = np.random.default_rng(seed)
    do = rng.standard_normal((cfg.batch, cfg.s_q, cfg.n_heads, cfg.d_v)).astype(np.float32)
    ro, rl = O.explicit_fwd(**x, **_args(cfg))
    g = O.explicit_bwd(**x, d_out=do.astype(np.float64), **_args(cfg))
    return x, do, ro.astype(np.float32), rl.astype(np.float32), g


def _run(mla, cfg, x, out, lse, do, algo):
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(tdt).cuda() for k, v in x.items()}
    _say(f"backward {cfg.name}: B={cfg.batch} Sq={cfg.s_q} Skv={cfg.s_kv} H={cfg.n_heads} q_pos0={cfg.q_pos0} "
         f"kv_pos0={cfg.kv_pos0} causal={cfg.causal} algo={algo}")
    grads, ws = mla.mla_bwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"],
                                     torch.from_numpy(out).cuda(), torch.from_numpy(lse).cuda(),
                                     torch.from_numpy(do).cuda(), algo=algo, **_args(cfg))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in grads.items()}


def _compare(got, ref, what, rel_max, rel_l2=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all(), what
    scale = max(1.0, float(np.abs(ref).max()))
    err = float(np.abs(got - ref).max())
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    _say(f"{what}: max|d|={err:.3e} (max|ref| {float(np.abs(ref).max()):.3e}) rel-L2={rel:.3e}")
    assert err <= rel_max * scale, f"{what}: max|d| {err} > {rel_max} * {scale}"
    if rel_l2 is not None:
        assert rel <= rel_l2, f"{what}: rel-L2 {rel}"


def test_backward_tiny_fp32(mla):
    cfg = I.EXPLICIT_CONFIGS["tiny_fp32"]
    x, do, out, lse, g = _case(cfg, 901)
    got = _run(mla, cfg, x, out, lse, do, mla.MLA_ALGO_AUTO)
    for k in GRADS:
        _compare(got[k], g[k], f"tiny_fp32 {k}", 1e-5)


SIMT_CASES = [
    I.small_explicit("bwd_ragged", batch=2, s_q=70, s_kv=70, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     dtype="bf16", seed=911),
    I.small_explicit("bwd_offset_q", s_q=33, s_kv=90, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     q_pos0=57, dtype="bf16", seed=912),
    I.small_explicit("bwd_masked_rows", s_q=40, s_kv=40, n_heads=3, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     kv_pos0=17, dtype="bf16", seed=913),
    I.small_explicit("bwd_noncausal_sp", s_q=24, s_kv=50, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     q_pos0=10, causal=False, dtype="bf16", seed=914),
    I.small_explicit("bwd_small_dims", batch=2, s_q=30, s_kv=30, n_heads=3, d_kv=48, d_nope=24, d_rope=16, d_v=20,
                     q_pos0=5, kv_pos0=0, dtype="fp32", seed=915),
]


@pytest.mark.parametrize("cfg", SIMT_CASES, ids=lambda c: c.name)
def test_backward_simt(mla, cfg):
    x, do, out, lse, g = _case(cfg, cfg.seed)
    got = _run(mla, cfg, x, out, lse, do, mla.MLA_ALGO_SIMT)
    for k in GRADS:
        _compare(got[k], g[k], f"{cfg.name} {k}", 1e-4 if cfg.dtype == "bf16" else 1e-5)


MFMA_CASES = [
    I.small_explicit("mbwd_ragged", batch=2, s_q=300, s_kv=300, n_heads=3, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     dtype="bf16", seed=931),
    I.small_explicit("mbwd_offset_q", s_q=100, s_kv=612, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     q_pos0=512, dtype="bf16", seed=932),
    I.small_explicit("mbwd_masked_rows", s_q=96, s_kv=96, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     kv_pos0=40, dtype="bf16", seed=933),
    I.small_explicit("mbwd_noncausal", s_q=77, s_kv=131, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     causal=False, dtype="bf16", seed=934),
    # a sequence-parallel rank's rows: keys past the last visible one (and past
    # the padded tile) get zero gradients
    I.small_explicit("mbwd_sp_share", s_q=64, s_kv=1024, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     q_pos0=192, dtype="bf16", seed=935),
    I.small_explicit("mbwd_one_key", s_q=1, s_kv=1, n_heads=2, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     dtype="bf16", seed=936),
    I.small_explicit("mbwd_multi_tile", s_q=700, s_kv=700, n_heads=1, d_kv=512, d_nope=128, d_rope=64, d_v=128,
                     dtype="bf16", seed=937),
    # B*H a multiple of 8: the attention kernels deal the (batch, head) pairs
    # over the XCDs, here across two batch entries, with ragged last tiles
    I.small_explicit("mbwd_xcd_deal", batch=2, s_q=300, s_kv=300, n_heads=4, d_kv=512, d_nope=128, d_rope=64,
                     d_v=128, dtype="bf16", seed=938),
    I.small_explicit("mbwd_xcd_deal_offset", batch=2, s_q=150, s_kv=420, n_heads=8, d_kv=512, d_nope=128,
                     d_rope=64, d_v=128, q_pos0=270, dtype="bf16", seed=939),
]


@pytest.mark.parametrize("cfg", MFMA_CASES, ids=lambda c: c.name)
def test_backward_mfma(mla, cfg):
    x, do, out, lse, g = _case(cfg, cfg.seed)
    got = _run(mla, cfg, x, out, lse, do, mla.MLA_ALGO_MFMA)
    for k in GRADS:
        _compare(got[k], g[k], f"{cfg.name} {k}", 1e-2, 5e-3)


def test_backward_after_gpu_forward(mla):
    """The GPU forward's own output and LSE into the GPU backward: the
    forward's rounding (bf16 inputs, fp16 attention operands) enters the
    softmax-Jacobian term rowsum(d_out * out), so the bf16 bars apply."""
    cfg = SIMT_CASES[0]
    x = I.make_explicit_inputs(cfg)
    do = np.random.default_rng(921).standard_normal((cfg.batch, cfg.s_q, cfg.n_heads, cfg.d_v)).astype(np.float32)
    t = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    out, lse, _ = mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **_args(cfg))
    grads, _ = mla.mla_bwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out, lse,
                                    torch.from_numpy(do).cuda(), **_args(cfg))
    torch.cuda.synchronize()
    g = O.explicit_bwd(**x, d_out=do.astype(np.float64), **_args(cfg))
    for k in GRADS:
        _compare(grads[k].cpu().numpy(), g[k], f"chained {k}", 1e-2, 5e-3)


def _oracle_bwd_pooled(x, do, cfg, heads):
    """explicit_bwd over `heads`, one head per task on a thread pool (BLAS
    single-threaded inside), the per-head results summed: the head-subset
    results partition the full gradient (pinned in the oracle tests)."""
    import concurrent.futures as cf
    import os

    from threadpoolctl import threadpool_limits
    workers = max(1, min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))
    d64 = do.astype(np.float64)
    with threadpool_limits(limits=1, user_api="blas"), cf.ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda h: O.explicit_bwd(**x, d_out=d64, **_args(cfg), heads=[h]), heads))
    out = {k: sum(p[k] for p in parts) for k in GRADS}
    return out


def test_backward_v3_heads_full_compare(mla):
    """All 128 heads at 1024 tokens (several key and query tiles per head),
    every gradient compared whole."""
    cfg = I.small_explicit("mbwd_h128", s_q=1024, s_kv=1024, n_heads=128, d_kv=512, d_nope=128, d_rope=64,
                           d_v=128, dtype="bf16", seed=941)
    x = I.make_explicit_inputs(cfg)
    do = np.random.default_rng(942).standard_normal((1, 1024, 128, 128)).astype(np.float32)
    ro, rl = O.explicit_fwd(**x, **_args(cfg))
    got = _run(mla, cfg, x, ro.astype(np.float32), rl.astype(np.float32), do, mla.MLA_ALGO_MFMA)
    g = _oracle_bwd_pooled(x, do, cfg, list(range(128)))
    for k in GRADS:
        _compare(got[k], g[k], f"h128 {k}", 1e-2, 5e-3)


def test_backward_v3_full_size_sampled_heads(mla):
    """The timed V3 shape (4096 tokens, 128 heads): the query gradients and the
    W_kv_b rows of heads 0 and 127, whose oracle terms need only those heads;
    the other gradients must be finite.  The forward output and LSE fed to the
    backward are the oracle's on those heads and the GPU forward's elsewhere
    (they enter only their own heads' terms)."""
    cfg = I.EXPLICIT_CONFIGS["v3_bf16"]
    x = I.make_explicit_inputs(cfg)
    do = np.random.default_rng(943).standard_normal((1, 4096, 128, 128)).astype(np.float32)
    heads = [0, 127]
    t = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    out, lse, _ = mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **_args(cfg))
    ro, rl = O.explicit_fwd(**x, **_args(cfg), heads=heads)
    out[:, :, heads] = torch.from_numpy(ro.astype(np.float32)).cuda()
    lse[:, heads] = torch.from_numpy(rl.astype(np.float32)).cuda()
    _say("backward v3_bf16 full size: B=1 Sq=4096 H=128")
    grads, _ = mla.mla_bwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out.contiguous(),
                                    lse.contiguous(), torch.from_numpy(do).cuda(), **_args(cfg))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in grads.items()}
    for k in GRADS:
        assert np.isfinite(got[k]).all(), k
    g = _oracle_bwd_pooled(x, do, cfg, heads)
    hd = cfg.d_nope + cfg.d_v
    for h in heads:
        _compare(got["dq_nope"][:, :, h], g["dq_nope"][:, :, h], f"v3 dq_nope head {h}", 1e-2, 5e-3)
        _compare(got["dq_pe"][:, :, h], g["dq_pe"][:, :, h], f"v3 dq_pe head {h}", 1e-2, 5e-3)
        _compare(got["dw_kv_b"][h * hd:(h + 1) * hd], g["dw_kv_b"][h * hd:(h + 1) * hd], f"v3 dW rows head {h}",
                 1e-2, 5e-3)
