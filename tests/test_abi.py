"""C-ABI checks that need no GPU: the library loads, exports every function
include/mla.h declares, sizes workspaces, and rejects invalid calls on the host
before anything is enqueued (so fake device pointers are never touched)."""
import ctypes
import os
import re

import pytest

from head_latent_attention_02_amd import mla
from head_latent_attention_02_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mla.LIB_PATH),
                                reason="libmla.so not built (run __graft_entry__.build())")

FAKE = 0x10000          # never dereferenced: every call below fails validation first


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = mla.library()
    declared = _header_functions()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(mla.EXPORTED_SYMBOLS)


def test_status_strings_and_info():
    lib = mla.library()
    for code, name in [(0, "MLA_OK"), (1, "MLA_ERR_INVALID_ARGUMENT"), (2, "MLA_ERR_UNSUPPORTED"),
                       (3, "MLA_ERR_WORKSPACE_TOO_SMALL"), (4, "MLA_ERR_HIP")]:
        assert lib.mla_status_string(code).decode() == name
    assert "gfx950" in mla.build_info()


def test_struct_layout_matches_header(tmp_path):
    """ctypes field offsets equal what a C compiler makes of include/mla.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {"]
    for cname, py in [("mla_explicit_desc", mla.MlaExplicitDesc), ("mla_decode_desc", mla.MlaDecodeDesc)]:
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in [("mla_explicit_desc", mla.MlaExplicitDesc), ("mla_decode_desc", mla.MlaDecodeDesc)]:
        assert got[(cname, "size")] == ctypes.sizeof(py)
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def _v3_desc(**kw):
    base = dict(batch=1, s_q=4096, s_kv=4096, n_heads=128, d_kv=512, d_nope=128, d_rope=64, d_v=128)
    base.update(kw)
    return mla.explicit_desc(**base)


def test_explicit_workspace_sizes():
    d = _v3_desc()
    ws = mla.mla_fwd_explicit_workspace_size(d)
    # K_nope + V^T fp16 for 4096 padded rows x 128 heads x 256, plus small tables
    assert ws >= 2 * 128 * 4096 * 256
    assert ws < 2 * 128 * 4096 * 256 + (8 << 20)
    kn, vt, kr, s_pad = mla.mla_fwd_explicit_workspace_layout(d)
    assert s_pad == 4096 and kn < vt < kr < ws
    # one SP rank: only the 8192 visible latent rows are projected
    d2 = _v3_desc(s_q=2048, s_kv=16384, q_pos0=6144)
    assert mla.mla_fwd_explicit_workspace_layout(d2)[3] == 8192
    # fp32 inputs take the SIMT path, which has no MFMA layout
    d3 = _v3_desc(in_dtype=mla.MLA_FP32)
    assert mla.mla_fwd_explicit_workspace_size(d3) > 0
    with pytest.raises(mla.MlaError):
        mla.mla_fwd_explicit_workspace_layout(d3)


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("n_heads", 0), ("s_q", -1), ("d_rope", 63), ("d_rope", 0), ("d_kv", 0),
    ("causal", 2), ("in_dtype", 7), ("algo", 9), ("rope_base", -1.0), ("softmax_scale", float("nan")),
])
def test_explicit_rejects_bad_descriptor(field, value):
    d = _v3_desc()
    setattr(d, field, value)
    assert mla.mla_fwd_explicit_workspace_size(d) == 0
    st = mla.library().mla_fwd_explicit(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                        1 << 40, None)
    assert st == mla.MLA_ERR_INVALID_ARGUMENT


def test_explicit_null_pointers_and_workspace():
    lib = mla.library()
    d = _v3_desc()
    ws = mla.mla_fwd_explicit_workspace_size(d)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None]
    for i in range(6):
        a = list(args)
        a[i] = None
        assert lib.mla_fwd_explicit(ctypes.byref(d), *a) == mla.MLA_ERR_INVALID_ARGUMENT
    a = list(args)
    a[8] = ws - 1
    assert lib.mla_fwd_explicit(ctypes.byref(d), *a) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    a = list(args)
    a[7] = None
    assert lib.mla_fwd_explicit(ctypes.byref(d), *a) == mla.MLA_ERR_INVALID_ARGUMENT
    # misaligned operand on the MFMA path
    a = list(args)
    a[0] = FAKE + 2
    assert lib.mla_fwd_explicit(ctypes.byref(d), *a) == mla.MLA_ERR_INVALID_ARGUMENT
    # empty query set: valid and a no-op that touches nothing
    d0 = _v3_desc(s_q=0)
    assert lib.mla_fwd_explicit(ctypes.byref(d0), None, None, FAKE, FAKE, FAKE, None, None, FAKE,
                                mla.mla_fwd_explicit_workspace_size(d0), None) == mla.MLA_OK


def test_explicit_unsupported():
    lib = mla.library()
    d = _v3_desc(d_nope=96, algo=mla.MLA_ALGO_MFMA)
    assert mla.mla_fwd_explicit_workspace_size(d) == 0
    assert lib.mla_fwd_explicit(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                None) == mla.MLA_ERR_UNSUPPORTED
    # SIMT path limit on head widths
    d = _v3_desc(d_nope=256, d_rope=64, d_v=256, algo=mla.MLA_ALGO_SIMT)
    assert lib.mla_fwd_explicit(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                None) == mla.MLA_ERR_UNSUPPORTED


def test_fused_algo_workspace_and_scope():
    lib = mla.library()
    d = _v3_desc(algo=mla.MLA_ALGO_FUSED)
    ws = mla.mla_fwd_explicit_workspace_size(d)
    # the two fp32 (cos, sin) RoPE tables and the fp16 key band only: no K_nope / V^T
    assert 0 < ws <= 2 * (8 * 4096 * 32) + 2 * 4096 * 64 + 3 * 256
    assert ws + 2 * 128 * 4096 * 256 <= mla.mla_fwd_explicit_workspace_size(_v3_desc(algo=mla.MLA_ALGO_MFMA))
    with pytest.raises(mla.MlaError):
        mla.mla_fwd_explicit_workspace_layout(d)
    # shapes the MFMA kernels do not take are unsupported, not rerouted
    d1 = _v3_desc(d_nope=96, algo=mla.MLA_ALGO_FUSED)
    assert mla.mla_fwd_explicit_workspace_size(d1) == 0
    assert lib.mla_fwd_explicit(ctypes.byref(d1), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                None) == mla.MLA_ERR_UNSUPPORTED
    # misaligned operand on the fused path
    assert lib.mla_fwd_explicit(ctypes.byref(d), FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws,
                                None) == mla.MLA_ERR_INVALID_ARGUMENT
    # the fused algorithm names an explicit-forward kernel only
    assert mla.mla_fwd_absorbed_workspace_size(d) == 0
    assert mla.mla_bwd_explicit_workspace_size(d) == 0
    assert mla.mla_decode_absorbed_workspace_size(_dec_desc(algo=mla.MLA_ALGO_FUSED)) == 0


def _dec_desc(**kw):
    base = dict(batch=64, n_heads=128, d_kv=512, d_nope=128, d_rope=64, d_v=128, max_cache_len=32768,
                n_splits=16)
    base.update(kw)
    return mla.decode_desc(**base)


def test_decode_workspace_and_layout():
    d = _dec_desc()
    ws = mla.mla_decode_absorbed_workspace_size(d)
    q, l, o, esz = mla.mla_decode_absorbed_workspace_layout(d)
    assert esz == 2 and q < l < o < ws
    assert ws - o >= 64 * 16 * 128 * 512 * esz
    d2 = _dec_desc(in_dtype=mla.MLA_FP32)
    assert mla.mla_decode_absorbed_workspace_layout(d2)[3] == 4


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, mla.MLA_ERR_INVALID_ARGUMENT), ("n_splits", 0, mla.MLA_ERR_INVALID_ARGUMENT),
    ("max_cache_len", -1, mla.MLA_ERR_INVALID_ARGUMENT), ("cache_batch_stride", 100, mla.MLA_ERR_INVALID_ARGUMENT),
    ("d_rope", 3, mla.MLA_ERR_INVALID_ARGUMENT), ("n_splits", 65, mla.MLA_ERR_UNSUPPORTED),
    ("out_dtype", 5, mla.MLA_ERR_INVALID_ARGUMENT),
])
def test_decode_rejects(field, value, status):
    d = _dec_desc()
    setattr(d, field, value)
    st = mla.library().mla_decode_absorbed(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                           1 << 40, None)
    assert st == status


def test_decode_mfma_eligibility():
    lib = mla.library()
    for kw in [dict(n_heads=24), dict(n_heads=256), dict(cache_batch_stride=32768 * 576 + 4)]:
        d = _dec_desc(algo=mla.MLA_ALGO_MFMA, **kw)
        st = lib.mla_decode_absorbed(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                     None)
        assert st == mla.MLA_ERR_UNSUPPORTED, kw
    d = _dec_desc()
    ws = mla.mla_decode_absorbed_workspace_size(d)
    assert lib.mla_decode_absorbed(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws - 1,
                                   None) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    assert lib.mla_decode_absorbed(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, ws,
                                   None) == mla.MLA_ERR_INVALID_ARGUMENT


def test_flop_and_byte_accounting():
    v3 = I.EXPLICIT_CONFIGS["v3_bf16"].flops()
    assert v3["up_proj"] == 2 * 4096 * 512 * 128 * 256
    assert v3["attention"] == 2 * 128 * (4096 * 4097 // 2) * 320
    sp = I.EXPLICIT_CONFIGS["v3_sp8_rank3"]
    assert sp.visible_keys() == 8192
    assert sp.visible_pairs() == sum(6144 + i + 1 for i in range(2048))
    dec = I.DECODE_CONFIGS["v3_decode_b64_32k"].algorithmic_bytes()
    assert dec["cache"] == 64 * 32768 * 576 * 2


def test_absorbed_workspace_and_validation():
    lib = mla.library()
    d = _v3_desc()
    ws = mla.mla_fwd_absorbed_workspace_size(d)
    # q~ bf16 and the fp16 per-row latent outputs for 4096 rows x 128 heads,
    # plus the latent rows and small per-row arrays
    rows = 4096 * 128
    need = rows * 576 * 2 + rows * 512 * 2 + 4096 * 576 * 2
    assert need <= ws < need + (8 << 20)
    for field, value in [("batch", 0), ("d_rope", 63), ("causal", 2), ("in_dtype", 7), ("algo", 9)]:
        dd = _v3_desc()
        setattr(dd, field, value)
        assert mla.mla_fwd_absorbed_workspace_size(dd) == 0
        assert lib.mla_fwd_absorbed(ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                    None) == mla.MLA_ERR_INVALID_ARGUMENT
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None]
    for i in range(6):
        a = list(args)
        a[i] = None
        assert lib.mla_fwd_absorbed(ctypes.byref(d), *a) == mla.MLA_ERR_INVALID_ARGUMENT
    a = list(args)
    a[8] = ws - 1
    assert lib.mla_fwd_absorbed(ctypes.byref(d), *a) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    # the MFMA kernels need a multiple of 16 heads
    d2 = _v3_desc(n_heads=24, algo=mla.MLA_ALGO_MFMA)
    assert mla.mla_fwd_absorbed_workspace_size(d2) == 0
    assert lib.mla_fwd_absorbed(ctypes.byref(d2), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                None) == mla.MLA_ERR_UNSUPPORTED
    # empty query set: valid and a no-op that touches nothing
    d0 = _v3_desc(s_q=0)
    assert lib.mla_fwd_absorbed(ctypes.byref(d0), None, None, FAKE, FAKE, FAKE, None, None, FAKE,
                                mla.mla_fwd_absorbed_workspace_size(d0), None) == mla.MLA_OK


@pytest.mark.parametrize("scale", [0.0, -0.1, float("inf")])
def test_non_positive_scale_rejected_by_every_entry_point(scale):
    """The MFMA kernels subtract the row max of raw scores, which is the max
    of the scaled logits only for a positive scale; every entry point refuses
    other scales on the host."""
    lib = mla.library()
    d = _v3_desc(softmax_scale=scale)
    assert mla.mla_fwd_explicit_workspace_size(d) == 0
    assert mla.mla_fwd_absorbed_workspace_size(d) == 0
    for fn in (lib.mla_fwd_explicit, lib.mla_fwd_absorbed):
        assert fn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                  None) == mla.MLA_ERR_INVALID_ARGUMENT
    dd = _dec_desc(softmax_scale=scale)
    assert mla.mla_decode_absorbed_workspace_size(dd) == 0
    assert lib.mla_decode_absorbed(ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                   None) == mla.MLA_ERR_INVALID_ARGUMENT


# ---- the binding checks every tensor before it reaches the library --------
def _explicit_tensors(B=1, S=8, Skv=8, H=2, dn=128, dr=64, dv=128, dkv=512, dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    return dict(q_nope=torch.zeros(B, S, H, dn, dtype=dtype), q_pe=torch.zeros(B, S, H, dr, dtype=dtype),
                c_kv=torch.zeros(B, Skv, dkv, dtype=dtype), k_pe=torch.zeros(B, Skv, dr, dtype=dtype),
                w_kv_b=torch.zeros(H * (dn + dv), dkv, dtype=dtype))


def _call_explicit(t, **kw):
    return mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **kw)


def test_binding_explicit_valid_tensors_only_fail_on_device():
    # well-formed host tensors pass every shape / dtype / layout check and are
    # refused only because they are not on a GPU
    with pytest.raises(ValueError, match="GPU device"):
        _call_explicit(_explicit_tensors())


def _explicit_mutations():
    import torch
    base = _explicit_tensors
    yield "q_pe shape", dict(base(), q_pe=torch.zeros(1, 8, 3, 64, dtype=torch.bfloat16)), {}, "q_pe"
    yield "k_pe shape", dict(base(), k_pe=torch.zeros(1, 7, 64, dtype=torch.bfloat16)), {}, "k_pe"
    yield "c_kv batch", dict(base(), c_kv=torch.zeros(2, 8, 512, dtype=torch.bfloat16)), {}, "c_kv"
    yield "w_kv_b cols", dict(base(), w_kv_b=torch.zeros(512, 256, dtype=torch.bfloat16)), {}, "w_kv_b"
    yield "w_kv_b rows", dict(base(), w_kv_b=torch.zeros(511, 512, dtype=torch.bfloat16)), {}, "w_kv_b"
    yield "dtype mix", dict(base(), c_kv=torch.zeros(1, 8, 512, dtype=torch.float32)), {}, "c_kv"
    t = base()
    t["q_nope"] = torch.zeros(1, 8, 128, 2, dtype=torch.bfloat16).transpose(2, 3)
    yield "q_nope strided", t, {}, "q_nope"
    yield "out shape", base(), dict(out=torch.zeros(1, 8, 2, 64)), "out"
    yield "out dtype", base(), dict(out=torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16)), "out"
    yield "lse shape", base(), dict(lse=torch.zeros(1, 8, 2)), "lse"
    yield "workspace dtype", base(), dict(workspace=torch.zeros(16, dtype=torch.float32)), "workspace"


@pytest.mark.parametrize("case", list(_explicit_mutations()), ids=lambda c: c[0])
def test_binding_explicit_rejects(case):
    _, t, kw, what = case
    with pytest.raises(ValueError, match=what):
        _call_explicit(t, **kw)


def _decode_tensors(B=2, H=16, L=8, dn=128, dr=64, dv=128, dkv=512):
    import torch
    bf = torch.bfloat16
    return dict(q_nope=torch.zeros(B, H, dn, dtype=bf), q_pe=torch.zeros(B, H, dr, dtype=bf),
                kv_cache=torch.zeros(B, L, dkv + dr, dtype=bf), cache_len=torch.full((B,), L, dtype=torch.int32),
                w_kv_b=torch.zeros(H * (dn + dv), dkv, dtype=bf))


def _call_decode(t, **kw):
    return mla.mla_decode_absorbed(t["q_nope"], t["q_pe"], t["kv_cache"], t["cache_len"], t["w_kv_b"], **kw)


def test_binding_decode_valid_tensors_only_fail_on_device():
    with pytest.raises(ValueError, match="GPU device"):
        _call_decode(_decode_tensors())


def _decode_mutations():
    import torch
    bf = torch.bfloat16
    base = _decode_tensors
    yield "cache_len dtype", dict(base(), cache_len=torch.full((2,), 8, dtype=torch.int64)), {}, "cache_len"
    yield "cache_len shape", dict(base(), cache_len=torch.full((3,), 8, dtype=torch.int32)), {}, "cache_len"
    yield "cache batch", dict(base(), kv_cache=torch.zeros(3, 8, 576, dtype=bf)), {}, "kv_cache"
    yield "cache dtype", dict(base(), kv_cache=torch.zeros(2, 8, 576)), {}, "kv_cache"
    yield "cache row", dict(base(), kv_cache=torch.zeros(2, 8, 600, dtype=bf)[:, :, :576]), {}, "kv_cache"
    yield "q_pe shape", dict(base(), q_pe=torch.zeros(2, 8, 64, dtype=bf)), {}, "q_pe"
    yield "w_kv_b rows", dict(base(), w_kv_b=torch.zeros(16 * 256 + 1, 512, dtype=bf)), {}, "w_kv_b"
    t = base()
    t["q_nope"] = torch.zeros(2, 128, 16, dtype=bf).transpose(1, 2)
    yield "q_nope strided", t, {}, "q_nope"
    yield "out shape", base(), dict(out=torch.zeros(2, 16, 64)), "out"
    yield "lse dtype", base(), dict(lse=torch.zeros(2, 16, dtype=bf)), "lse"


@pytest.mark.parametrize("case", list(_decode_mutations()), ids=lambda c: c[0])
def test_binding_decode_rejects(case):
    _, t, kw, what = case
    with pytest.raises(ValueError, match=what):
        _call_decode(t, **kw)


def test_noalloc_decode_rejects_on_the_host():
    """The allocation-free decode step refuses, before touching any device, a
    step whose intermediates exceed the fixed scratch, and invalid
    descriptors."""
    lib = mla.library()
    big = _dec_desc()                      # 64 x 128 heads x 16 splits: ~144 MB of intermediates
    assert mla.mla_decode_absorbed_workspace_size(big) > mla.DECODE_NOALLOC_MAX_BYTES
    st = lib.mla_decode_absorbed_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in lib.mla_last_error().decode()
    for field, value in [("batch", 0), ("n_splits", 0), ("softmax_scale", 0.0), ("d_rope", 3)]:
        d = _dec_desc(batch=4)
        setattr(d, field, value)
        assert lib.mla_decode_absorbed_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                               None) == mla.MLA_ERR_INVALID_ARGUMENT
    d = _dec_desc(batch=4)
    assert lib.mla_decode_absorbed_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                                           None) == mla.MLA_ERR_INVALID_ARGUMENT


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MLA_DECODE_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mla.DECODE_NOALLOC_MAX_BYTES


def _header_arity():
    """Number of parameters of every function include/mla.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(mla_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argtypes_match_header_arity():
    """Every ctypes prototype has exactly as many parameters as the C
    declaration, so no call can pass a pointer where a size is expected."""
    lib = mla.library()
    arity = _header_arity()
    assert set(arity) == set(mla.EXPORTED_SYMBOLS)
    for name, n in arity.items():
        assert len(getattr(lib, name).argtypes) == n, (name, len(getattr(lib, name).argtypes), n)
