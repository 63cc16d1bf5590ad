"""The allocation-free decode entry point (mla_decode_absorbed_noalloc)
against the workspace entry point (mla_decode_absorbed), through the C ABI.

Both run the same kernels on the same inputs, so their outputs must agree bit
for bit.  Cases: two calls in a row with the second smaller (the fixed scratch
keeps the first call's contents), a ragged batch with empty and one-row
sequences, and the largest 128-head batch whose intermediates fit the
scratch."""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_02_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_02_amd import mla as m
    m.library()
    return m


def _inputs(cfg, lens):
    x = I.make_decode_inputs(cfg, cache_len=np.array(lens, dtype=np.int32))
    cache = torch.from_numpy(x["cache_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    qn = torch.from_numpy(x["q_nope"]).to(torch.bfloat16).cuda()
    qp = torch.from_numpy(x["q_pe"]).to(torch.bfloat16).cuda()
    w = torch.from_numpy(x["w_kv_b"]).to(torch.bfloat16).cuda()
    cl = torch.from_numpy(x["cache_len"]).cuda()
    return qn, qp, cache, cl, w


def _check_same(mla, cfg, lens):
    qn, qp, cache, cl, w = _inputs(cfg, lens)
    d = mla.decode_desc(batch=cfg.batch, n_heads=cfg.n_heads, d_kv=cfg.d_kv, d_nope=cfg.d_nope,
                        d_rope=cfg.d_rope, d_v=cfg.d_v, max_cache_len=cfg.cache_len, n_splits=cfg.n_splits)
    need = mla.mla_decode_absorbed_workspace_size(d)
    _say(f"{cfg.name}: B={cfg.batch} L={cfg.cache_len} H={cfg.n_heads} splits={cfg.n_splits} "
         f"intermediates {need} of {mla.DECODE_NOALLOC_MAX_BYTES} bytes")
    assert 0 < need <= mla.DECODE_NOALLOC_MAX_BYTES
    ref_out, ref_lse, _ = mla.mla_decode_absorbed(qn, qp, cache, cl, w, n_splits=cfg.n_splits)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    mla.mla_decode_absorbed_noalloc(qn, qp, cache, cl, w, out, lse, n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), f"{cfg.name}: out differs, max|d| {(out - ref_out).abs().max().item()}"
    same_lse = torch.equal(torch.nan_to_num(lse, neginf=-1e30), torch.nan_to_num(ref_lse, neginf=-1e30))
    assert same_lse, f"{cfg.name}: lse differs"
    return out


def test_noalloc_two_calls_second_smaller(mla):
    big = I.small_decode("noalloc_big", batch=8, cache_len=4096, n_heads=128, n_splits=16, seed=601)
    small = I.small_decode("noalloc_small", batch=3, cache_len=700, n_heads=64, n_splits=5, seed=602)
    _check_same(mla, big, [4096, 4000, 17, 1, 2048, 4095, 333, 1024])
    _check_same(mla, small, [700, 1, 333])


def test_noalloc_largest_batch_that_fits(mla):
    per_seq = None
    cfg = None
    for b in range(64, 0, -1):
        cfg = I.small_decode("noalloc_max", batch=b, cache_len=512, n_heads=128, n_splits=16, seed=603)
        d = mla.decode_desc(batch=b, n_heads=128, d_kv=512, d_nope=128, d_rope=64, d_v=128, max_cache_len=512,
                            n_splits=16)
        per_seq = mla.mla_decode_absorbed_workspace_size(d)
        if per_seq <= mla.DECODE_NOALLOC_MAX_BYTES:
            break
    lens = [512 - 7 * i for i in range(cfg.batch)]
    _check_same(mla, cfg, lens)


def test_noalloc_oversize_is_refused(mla):
    cfg = I.small_decode("noalloc_over", batch=40, cache_len=64, n_heads=128, n_splits=16, seed=604)
    qn, qp, cache, cl, w = _inputs(cfg, [64] * 40)
    out = torch.zeros((40, 128, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_absorbed_noalloc(qn, qp, cache, cl, w, out, None, n_splits=16)
    assert e.value.status == mla.MLA_ERR_WORKSPACE_TOO_SMALL
