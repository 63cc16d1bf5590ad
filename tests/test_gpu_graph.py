"""Both entry points under HIP graph capture: a step captured once and replayed
gives the eager result bit for bit, on every replay, with eager calls on
other inputs and host synchronisations between the replays (the kernels hold
no state between launches and the library records no memset).
"""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_02_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-graph] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_02_amd import mla as m
    m.library()
    return m


def _explicit_tensors(cfg, seed):
    x = I.make_explicit_inputs(cfg, seed=seed)
    return {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}


def test_explicit_graph_replay(mla):
    cfg = I.small_explicit("graph_explicit", batch=2, s_q=300, s_kv=300, n_heads=3, d_kv=512, d_nope=128,
                           d_rope=64, d_v=128, dtype="bf16", seed=401)
    t = _explicit_tensors(cfg, 401)
    other = _explicit_tensors(cfg, 402)
    out = torch.empty((cfg.batch, cfg.s_q, cfg.n_heads, cfg.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.batch, cfg.n_heads, cfg.s_q), dtype=torch.float32, device="cuda")

    def call(src, o, l, ws):
        return mla.mla_fwd_explicit(src["q_nope"], src["q_pe"], src["c_kv"], src["k_pe"], src["w_kv_b"],
                                    causal=cfg.causal, softmax_scale=cfg.softmax_scale, out=o, lse=l,
                                    workspace=ws)

    _say(f"explicit eager reference: B={cfg.batch} S={cfg.s_q} H={cfg.n_heads}")
    _, _, ws = call(t, out, lse, None)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(t, out, lse, ws)                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _say("capturing the explicit step")
    with torch.cuda.graph(g):
        call(t, out, lse, ws)
    torch.cuda.synchronize()

    o2 = torch.empty_like(out)
    l2 = torch.empty_like(lse)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"explicit replay {rep}")
        assert torch.equal(out, ref_o), f"explicit replay {rep}: output differs from the eager call"
        assert torch.equal(lse, ref_l), f"explicit replay {rep}: lse differs from the eager call"
        # eager work on other inputs (and its own buffers) between replays
        call(other, o2, l2, None)
        torch.cuda.synchronize()


def test_decode_graph_replay(mla):
    cfg = I.small_decode("graph_decode", batch=5, cache_len=700, n_heads=16, n_splits=16, seed=403)
    lens = np.array([700, 1, 0, 17, 333], dtype=np.int32)

    def tensors(seed):
        x = I.make_decode_inputs(cfg, seed=seed, cache_len=lens)
        return (torch.from_numpy(x["q_nope"]).to(torch.bfloat16).cuda(),
                torch.from_numpy(x["q_pe"]).to(torch.bfloat16).cuda(),
                torch.from_numpy(x["cache_bits"].view(np.int16)).cuda().view(torch.bfloat16),
                torch.from_numpy(x["cache_len"]).cuda(),
                torch.from_numpy(x["w_kv_b"]).to(torch.bfloat16).cuda())

    a, b = tensors(403), tensors(404)
    out = torch.empty((cfg.batch, cfg.n_heads, cfg.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.batch, cfg.n_heads), dtype=torch.float32, device="cuda")

    def call(src, o, l, ws):
        qn, qp, cache, cl, w = src
        return mla.mla_decode_absorbed(qn, qp, cache, cl, w, n_splits=cfg.n_splits,
                                       softmax_scale=cfg.softmax_scale, out=o, lse=l, workspace=ws)

    _say(f"decode eager reference: B={cfg.batch} L={cfg.cache_len} H={cfg.n_heads} lens={lens.tolist()}")
    _, _, ws = call(a, out, lse, None)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(a, out, lse, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _say("capturing the decode step")
    with torch.cuda.graph(g):
        call(a, out, lse, ws)
    torch.cuda.synchronize()

    o2 = torch.empty_like(out)
    l2 = torch.empty_like(lse)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"decode replay {rep}")
        assert torch.equal(out, ref_o), f"decode replay {rep}: output differs from the eager call"
        assert torch.equal(torch.nan_to_num(lse, neginf=-1e30), torch.nan_to_num(ref_l, neginf=-1e30)), \
            f"decode replay {rep}: lse differs from the eager call"
        call(b, o2, l2, None)
        torch.cuda.synchronize()
