"""Benchmark of the MLA forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * explicit (LAGA-local) forward at DeepSeek-V3 dims: B=1, S=4096, n_h=128,
    d_kv=512, d_nope=128, d_rope=64, d_v=128, causal (latent up-projection,
    RoPE, causal attention);
  * absorbed split-KV decode: B=64 sequences of 32768 cached tokens, n_h=128,
    16 KV chunks merged by log-sum-exp, up-projected to d_v=128.

Prints ONE JSON line.  `value` is the explicit forward's algorithmic TFLOP/s
(causally visible pairs plus the up-projection of the visible latent rows,
divided by the time of the explicit part of each step); the decode part is
reported as tokens/s and algorithmic HBM GB/s.

Two timed regions of K steps each follow the warm-up:
  1. eager calls, with HIP events that the library records around each of its
     launches on the stream the kernels run on (mla_timing_*): the per-kernel
     durations and roofline figures;
  2. the same step captured once as two HIP graphs (explicit, decode; checked
     bit-identical to the eager result) and replayed K times: the step time,
     `value`, tokens/s and GB/s, without per-launch host overhead between the
     kernels.  `--no-graph` reports the eager region's step time instead.
After the graph region each captured step replays back to back for about two
seconds while a side thread reads the graphics clock and the socket power
through amdsmi; the
matrix-unit fractions are also given against the peak scaled to that clock
(`clock`, `roofline.frac_at_clock`), since the quoted peak assumes 2.4 GHz.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--copy-calibration]

HBM traffic (`roofline.traffic`) comes from rocprofv3 FETCH_SIZE / WRITE_SIZE
passes over this same command, each divided by the factor the same counter
reads for a plain device copy of known size (`--copy-calibration` runs that
copy before the warm-up).  The figures sit in HBM_COUNTERS below together with
a digest of the kernel's sources; once those sources change, traffic is
reported as null until the counters are taken again.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16 / fp16
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_CLOCK_MHZ = 2400.0        # the shader clock the matrix peak is quoted at
METRIC = "MLA attn fwd TFLOP/s (+% MFMA peak) at V3 dims; absorbed decode tok/s (+% HBM)"
COPY_CALIBRATION_BYTES = 1 << 30   # bytes read (and written) by the calibration copy

CSRC = os.path.join(ROOT, "head_latent_attention_02_amd", "csrc")
# Kernel -> the sources its code comes from.
KERNEL_SOURCES = {
    "mfma_attention": ["mfma_attn.hip", "common.h", "kernels.h"],
    "mfma_up_projection": ["mfma_upproj.hip", "common.h", "kernels.h"],
    "mfma_split_kv": ["mfma_decode.hip", "common.h", "kernels.h"],
    "lse_combine": ["combine.hip", "common.h", "kernels.h"],
}
# rocprofv3 counter readings per launch at the default workloads, KiB as the
# counter reports them, and the copy-calibration factors (counter KiB * 1024
# per byte actually moved by the calibration copy).  "digest" is
# source_digest() of the kernel's sources when the counters were taken.
HBM_COUNTERS: dict = {
    # taken with the sources of digest below; see profiles/hbm_traffic_counters.md
    "mfma_attention": {"digest": "3d5f6139de14b62c", "fetch_kib": 400906.3, "write_kib": 264192.7,
                      "fetch_factor": 0.50002, "write_factor": 1.0},
    "mfma_up_projection": {"digest": "e5764d858299461f", "fetch_kib": 43514.0, "write_kib": 262475.5,
                          "fetch_factor": 0.50002, "write_factor": 1.0},
    "mfma_split_kv": {"digest": "07a5151308c08d0f", "fetch_kib": 1216703.3, "write_kib": 131584.0,
                     "fetch_factor": 0.50002, "write_factor": 1.0},
    "lse_combine": {"digest": "505b7a7a5042aa17", "fetch_kib": 75877.3, "write_kib": 4352.0,
                   "fetch_factor": 0.50002, "write_factor": 1.0},
}


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def hbm_traffic(kernel: str):
    """HBM bytes per launch from the recorded counters, or None if stale."""
    c = HBM_COUNTERS.get(kernel)
    if c is None or kernel not in KERNEL_SOURCES or source_digest(kernel) != c["digest"]:
        return None
    return c["fetch_kib"] * 1024 / c["fetch_factor"] + c["write_kib"] * 1024 / c["write_factor"]


# The pages' own figures, with the hardware and setting they were measured
# on.  Context only: none is a single-device MLA forward rate, and none was
# measured on this hardware.
CONTEXT = [
    {"page": "LAGA (Pith review)", "where": "abstract; Table 1",
     "figure": "collective bytes per layer, explicit 587.2 MB vs LAGA 296.0 MB (1.98x less)",
     "hardware": "8x Ascend 910B", "setting": "DeepSeek-V3 dims, S=16384, SP=8"},
    {"page": "LAGA (Pith review)", "where": "\"If this is right\"; Fig. 3",
     "figure": "communication ratio 1.88x (16 heads) to 1.98x (128 heads)",
     "hardware": "Ascend 910B", "setting": "SP 4-16, S 4K-16K"},
    {"page": "LAGA (Pith review)", "where": "abstract; \"If this is right\"",
     "figure": "attention-block throughput LAGA/explicit 1.04-1.06x in one node, 1.07-1.24x across nodes "
               "(fused kernel, rising with S)",
     "hardware": "8x / 16x Ascend 910B", "setting": "n_h=128, S 4K-16K"},
    {"page": "LAGA (Pith review)", "where": "abstract; referee report",
     "figure": "activation memory absorbed minus explicit: +9.2 GB eager, +19.2 GB fused",
     "hardware": "Ascend 910B (A100 cross-check)", "setting": "S=16384, SP=8"},
    {"page": "TPLA (Pith review)", "where": "\"If this is right\"; abstract",
     "figure": "decode throughput vs MLA: 1.79x (DeepSeek-V3), 1.93x (Kimi-K2)",
     "hardware": "GPU type not stated", "setting": "32K context, MoE layers removed"},
    {"page": "Helix (Pith review)", "where": "core claim; abstract",
     "figure": "up to 1.5x lower token-to-token latency (DeepSeek-R1) and up to 32x larger batch; "
               "1.13x lower latency, 4x batch for Llama-405B",
     "hardware": "simulated GB200 NVL72 (FP4)", "setting": "1M-token KV cache"},
]


def host_info() -> dict:
    """CPU model, visible CPUs and the BLAS build numpy uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')}, " \
                       f"{os.path.basename(i.get('filepath', ''))})"
                break
    except Exception:
        pass
    return {"cpu_model": model, "cpus_visible": len(os.sched_getaffinity(0)), "blas": blas}


def pool_size() -> int:
    """Worker threads for the oracle: the CPUs this process may run on, capped
    by the thread budget the environment sets (OMP_NUM_THREADS), 16 if unset."""
    cap = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(len(os.sched_getaffinity(0)), cap))


def explicit_case(mla, torch, cfg, args):
    """Time one explicit-form configuration on its own: the call as a HIP graph
    replay (checked bit-identical to the eager call), and per-kernel averages
    from the library's launch events over eager calls."""
    log(f"explicit configuration {cfg.name}: inputs, {args.steps} graph replays, {args.steps} eager calls")
    x = I_mod().make_explicit_inputs(cfg)
    t = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    del x
    out = torch.empty((cfg.batch, cfg.s_q, cfg.n_heads, cfg.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.batch, cfg.n_heads, cfg.s_q), dtype=torch.float32, device="cuda")
    kw = dict(q_pos0=cfg.q_pos0, kv_pos0=cfg.kv_pos0, causal=cfg.causal, softmax_scale=cfg.softmax_scale,
              out=out, lse=lse)
    _, _, ws = mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **kw)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], workspace=ws, **kw)
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    if not (torch.equal(out, ref[0]) and torch.equal(torch.nan_to_num(lse, neginf=-1e30),
                                                     torch.nan_to_num(ref[1], neginf=-1e30))):
        raise RuntimeError(f"{cfg.name}: graph replay differs from the eager call")
    for _ in range(args.warmup):
        g.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for _ in range(args.steps):
        ev[0].record()
        g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        ms.append(ev[0].elapsed_time(ev[1]))
    mla.mla_timing_reset()
    mla.mla_timing_begin()
    for _ in range(args.steps):
        mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], workspace=ws, **kw)
    torch.cuda.synchronize()
    mla.mla_timing_end()
    kt = mla.mla_timing_get()
    mla.mla_timing_reset()
    fl = cfg.flops()
    avg = float(np.mean(ms))
    kernels = {name: {"avg_ms": tot / max(n, 1), "launches_per_call": n / args.steps} for name, (tot, n) in kt.items()}
    for name, work in (("mfma_attention", fl["attention"]), ("mfma_up_projection", fl["up_proj"])):
        if name in kernels:
            a = work / (kernels[name]["avg_ms"] * 1e-3) / 1e12
            kernels[name].update({"achieved": a, "unit": "TFLOP/s", "frac": a / PEAK_MFMA_TFLOPS,
                                  "work_per_launch": work})
    tflops = fl["total"] / (avg * 1e-3) / 1e12
    del t, out, lse, ws, g
    torch.cuda.empty_cache()
    return {"workload": f"{cfg.name} explicit fwd (B={cfg.batch}, S_q={cfg.s_q} at q_pos0={cfg.q_pos0}, "
                        f"S_kv={cfg.s_kv}, n_h={cfg.n_heads}, causal)",
            "ms": avg, "algorithmic_flop": fl["total"], "tflops": tflops, "frac_mfma_peak": tflops / PEAK_MFMA_TFLOPS,
            "timing": "hip_graph_replay", "kernels": kernels}


def backward_case(mla, torch, cfg, args):
    """The explicit-form backward at the explicit workload: time per call
    (HIP events, eager, after one untimed call) and per-kernel averages.
    Algorithmic FLOPs: the up-projection recomputed for K and V, the five
    attention products per visible pair and head (S = Q K^T 192, dP = dO V^T
    128, dV = P^T dO 128, dK = dS^T Q 192, dQ = dS K 192), and the two
    latent-space GEMMs dc_kv = dKV W and dW = dKV^T c_kv."""
    log(f"backward of {cfg.name}: inputs, forward, {args.steps} timed calls")
    x = I_mod().make_explicit_inputs(cfg)
    t = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    del x
    kw = dict(q_pos0=cfg.q_pos0, kv_pos0=cfg.kv_pos0, causal=cfg.causal, softmax_scale=cfg.softmax_scale)
    out, lse, _ = mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **kw)
    g = torch.Generator(device="cuda").manual_seed(cfg.seed)
    d_out = torch.randn(out.shape, device="cuda", generator=g)
    grads, ws = mla.mla_bwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out, lse, d_out, **kw)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for _ in range(args.steps):
        ev[0].record()
        mla.mla_bwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out, lse, d_out, grads=grads,
                             workspace=ws, **kw)
        ev[1].record()
        torch.cuda.synchronize()
        ms.append(ev[0].elapsed_time(ev[1]))
    mla.mla_timing_reset()
    mla.mla_timing_begin()
    for _ in range(args.steps):
        mla.mla_bwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out, lse, d_out, grads=grads,
                             workspace=ws, **kw)
    torch.cuda.synchronize()
    mla.mla_timing_end()
    kt = mla.mla_timing_get()
    mla.mla_timing_reset()
    pairs, vk, H = cfg.visible_pairs() * cfg.batch, cfg.visible_keys() * cfg.batch, cfg.n_heads
    gemm = 2 * vk * H * (cfg.d_nope + cfg.d_v) * cfg.d_kv
    attn = 2 * H * pairs * (3 * (cfg.d_nope + cfg.d_rope) + 2 * cfg.d_v)
    work = {"mfma_up_projection": gemm, "bwd_kv": 2 * H * pairs * (2 * (cfg.d_nope + cfg.d_rope) + 2 * cfg.d_v),
            "bwd_dq": 2 * H * pairs * (cfg.d_nope + cfg.d_rope), "bwd_gemms": 2 * gemm}
    kernels = {}
    for name, (tot, n) in kt.items():
        ent = {"avg_ms": tot / max(n, 1), "launches_per_call": n / args.steps}
        if name in work:
            ach = work[name] / (ent["avg_ms"] * 1e-3) / 1e12
            ent.update({"algorithmic_flop": work[name], "achieved": ach, "unit": "TFLOP/s",
                        "frac": ach / PEAK_MFMA_TFLOPS})
        kernels[name] = ent
    total = gemm + attn + 2 * gemm
    avg = float(np.mean(ms))
    del t, out, lse, d_out, grads, ws
    torch.cuda.empty_cache()
    return {"workload": f"{cfg.name} explicit-form backward (B={cfg.batch}, S={cfg.s_q}, n_h={cfg.n_heads}, causal)",
            "ms": avg, "algorithmic_flop": total, "tflops": total / (avg * 1e-3) / 1e12,
            "frac_mfma_peak": total / (avg * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, "timing": "eager, HIP events",
            "kernels": kernels,
            "note": "bwd_kv recomputes S and dP, bwd_dq recomputes them again; counted once in algorithmic_flop"}


def I_mod():
    from head_latent_attention_02_amd import inputs as I
    return I


def fused_upproj_flop(cfg, qb=256, kt=128):
    """MFMA FLOPs of the up-projection as the fused kernel executes it: every
    256-query block up-projects each 128-key tile it reads (keys up to the
    causal limit of its last row), for every head."""
    total_tiles = 0
    for q0 in range(0, cfg.s_q, qb):
        last = min(q0 + qb, cfg.s_q) - 1
        kend = cfg.s_kv if not cfg.causal else min(max(cfg.q_pos0 + last - cfg.kv_pos0 + 1, 0), cfg.s_kv)
        total_tiles += -(-kend // kt)
    return 2 * cfg.batch * cfg.n_heads * total_tiles * kt * cfg.d_kv * (cfg.d_nope + cfg.d_v)


def fused_case(mla, torch, cfg, args):
    """The explicit forward with K_nope/V materialised in HBM (up-projection
    GEMM, then attention) against the fused kernel that recomputes them per
    query block, on one configuration: time per call (HIP events, eager, after
    one untimed call), per-kernel averages, and the device memory each call
    allocates (rise of torch.cuda.max_memory_allocated over the resident
    inputs)."""
    log(f"materialised vs fused up-projection at {cfg.name}: {args.form_calls + 2} calls of each")
    x = I_mod().make_explicit_inputs(cfg)
    t = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    del x
    fl = cfg.flops()
    res = {"workload": f"{cfg.name} explicit fwd (B={cfg.batch}, S={cfg.s_q}, n_h={cfg.n_heads}, causal): "
                       "one rank's heads after the all-to-all of S=16384 over 8 ranks",
           "algorithmic_flop": fl["total"]}
    outs = {}
    for name, algo in (("materialised", mla.MLA_ALGO_MFMA), ("fused", mla.MLA_ALGO_FUSED)):
        kw = dict(q_pos0=cfg.q_pos0, kv_pos0=cfg.kv_pos0, causal=cfg.causal, softmax_scale=cfg.softmax_scale,
                  algo=algo)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        out, lse, ws = mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **kw)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ms = []
        for _ in range(args.form_calls):
            ev[0].record()
            mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out=out, lse=lse,
                                 workspace=ws, **kw)
            ev[1].record()
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]))
        mla.mla_timing_reset()
        mla.mla_timing_begin()
        for _ in range(2):
            mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out=out, lse=lse,
                                 workspace=ws, **kw)
        torch.cuda.synchronize()
        mla.mla_timing_end()
        kt = mla.mla_timing_get()
        mla.mla_timing_reset()
        kernels = {k: {"avg_ms": tot / max(n, 1)} for k, (tot, n) in kt.items()}
        avg = float(np.mean(ms))
        res[name] = {"ms": avg, "tflops_algorithmic": fl["total"] / (avg * 1e-3) / 1e12,
                     "device_bytes": int(peak), "workspace_bytes": int(ws.numel()), "kernels": kernels}
        outs[name] = out
        del lse, ws
    f = res["fused"]
    executed = fl["attention"] + fused_upproj_flop(cfg)
    ka = f["kernels"].get("fused_attention")
    if ka:
        ach = executed / (ka["avg_ms"] * 1e-3) / 1e12
        ka.update({"executed_flop": executed, "achieved": ach, "unit": "TFLOP/s", "frac": ach / PEAK_MFMA_TFLOPS,
                   "note": "executed = attention + the up-projection repeated per 256-query block"})
    res["fused_over_materialised_time"] = f["ms"] / res["materialised"]["ms"]
    res["memory_saved_bytes"] = res["materialised"]["device_bytes"] - f["device_bytes"]
    res["max_abs_diff_fused_vs_materialised"] = float((outs["fused"] - outs["materialised"]).abs().max())
    del t, outs
    torch.cuda.empty_cache()
    return res


def forms_memory_and_time(mla, torch, names, args):
    """Explicit (K_nope/V materialised, and fused into the attention) and
    absorbed forms of the same V3 causal forward at several sequence lengths:
    time per call (HIP events, eager, after one untimed call)
    and the device memory each call allocates, measured as the rise of
    torch.cuda.max_memory_allocated over the resident inputs while the binding
    allocates the outputs and the workspace and the call runs."""
    I = I_mod()
    res = []
    for name in names:
        cfg = I.EXPLICIT_CONFIGS[name]
        log(f"explicit vs absorbed form at S={cfg.s_q}: inputs, then {args.form_calls} calls of each")
        x = I.make_explicit_inputs(cfg)
        t = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
        del x
        row = {"tokens": cfg.s_q, "n_heads": cfg.n_heads}
        forms = (("explicit", mla.mla_fwd_explicit, mla.MLA_ALGO_AUTO),
                 ("explicit_fused", mla.mla_fwd_explicit, mla.MLA_ALGO_FUSED),
                 ("absorbed", mla.mla_fwd_absorbed, mla.MLA_ALGO_AUTO))
        for form, fn, algo in forms:
            kw = dict(q_pos0=cfg.q_pos0, kv_pos0=cfg.kv_pos0, causal=cfg.causal, softmax_scale=cfg.softmax_scale,
                      algo=algo)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            out, lse, ws = fn(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **kw)
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated() - base
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ms = []
            for _ in range(args.form_calls):
                ev[0].record()
                fn(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], out=out, lse=lse, workspace=ws, **kw)
                ev[1].record()
                torch.cuda.synchronize()
                ms.append(ev[0].elapsed_time(ev[1]))
            row[form] = {"ms": float(np.mean(ms)), "device_bytes": int(peak), "workspace_bytes": int(ws.numel()),
                         "output_bytes": int(out.numel() * 4 + lse.numel() * 4)}
            del out, lse, ws
        row["gap_bytes"] = row["absorbed"]["device_bytes"] - row["explicit"]["device_bytes"]
        res.append(row)
        del t
        torch.cuda.empty_cache()
    slope = None
    if len(res) >= 2:
        slope = (res[-1]["gap_bytes"] - res[0]["gap_bytes"]) / (res[-1]["tokens"] - res[0]["tokens"])
    cfg0 = I.EXPLICIT_CONFIGS[names[0]]
    pages = cfg0.n_heads * (cfg0.d_kv - (cfg0.d_nope + cfg0.d_v)) * 2
    return {"rows": res, "measured_gap_slope_bytes_per_token": slope,
            "pages_slope_bytes_per_token_bf16": pages,
            "pages_slope": "n_h * (d_kv - (d_nope + d_v)) values per token, 2 bytes each"}


def absorbed_forward(mla, torch, ecfg, t, fl, args):
    """The explicit workload in absorbed form (mla_fwd_absorbed): time per call
    (eager, HIP events around each call, after one untimed call) and the
    workspace each form needs at 4K / 8K / 16K tokens (sizes from the library)."""
    log(f"absorbed-form forward: {args.steps} calls")
    out = torch.empty((ecfg.batch, ecfg.s_q, ecfg.n_heads, ecfg.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((ecfg.batch, ecfg.n_heads, ecfg.s_q), dtype=torch.float32, device="cuda")
    kw = dict(q_pos0=ecfg.q_pos0, kv_pos0=ecfg.kv_pos0, causal=ecfg.causal, softmax_scale=ecfg.softmax_scale,
              out=out, lse=lse)
    _, _, ws = mla.mla_fwd_absorbed(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], **kw)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for _ in range(args.steps):
        ev[0].record()
        mla.mla_fwd_absorbed(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"], workspace=ws, **kw)
        ev[1].record()
        torch.cuda.synchronize()
        ms.append(ev[0].elapsed_time(ev[1]))
    avg = float(np.mean(ms))
    H, S = ecfg.n_heads, ecfg.s_q
    pairs = fl["attention"] / (2 * H * (ecfg.d_nope + ecfg.d_rope + ecfg.d_v))
    flop = (2 * pairs * H * (ecfg.d_kv + ecfg.d_rope + ecfg.d_kv)
            + 2 * ecfg.batch * S * H * ecfg.d_nope * ecfg.d_kv + 2 * ecfg.batch * S * H * ecfg.d_kv * ecfg.d_v)
    mem = []
    for n in (4096, 8192, 16384):
        d = mla.explicit_desc(batch=ecfg.batch, s_q=n, s_kv=n, n_heads=H, d_kv=ecfg.d_kv, d_nope=ecfg.d_nope,
                              d_rope=ecfg.d_rope, d_v=ecfg.d_v, causal=ecfg.causal)
        mem.append({"tokens": n, "explicit_workspace_bytes": mla.mla_fwd_explicit_workspace_size(d),
                    "absorbed_workspace_bytes": mla.mla_fwd_absorbed_workspace_size(d)})
    slope = [(m["absorbed_workspace_bytes"] - m["explicit_workspace_bytes"]) / m["tokens"] for m in mem]
    return {"ms": avg, "algorithmic_flop": flop, "tflops": flop / (avg * 1e-3) / 1e12,
            "explicit_equivalent_tflops": fl["total"] / (avg * 1e-3) / 1e12,
            "workspace": mem, "gap_bytes_per_token": slope}


def summarise_clock(samples, power, limit):
    """Medians of the second half of the polled clock (MHz), socket power (W)
    and power cap: the power reading is a trailing average, and the clock
    settles once the load has run for a while.  amdsmi reports the cap in
    microwatts on some releases and in watts on others."""
    if not samples:
        return {"error": "no clock samples"}
    samples, power, limit = samples[len(samples) // 2:], power[len(power) // 2:], limit[len(limit) // 2:]
    r = {"sclk_mhz_median": float(np.median(samples)), "sclk_mhz_min": min(samples),
         "sclk_mhz_max": max(samples), "samples": len(samples)}
    if power:
        r["socket_power_w_median"] = float(np.median(power))
    if limit:
        lim = float(np.median(limit))
        r["power_limit_w"] = lim / 1e6 if lim > 1e5 else lim
    return r


def clock_under_load(torch, replay, seconds=2.0):
    """Median graphics (shader) clock in MHz while `replay` runs back to back
    for about `seconds`: amdsmi's current SYS clock polled every 10 ms from a
    side thread, with the socket power and its cap from the same polls (the
    medians of the second half of the samples).
    Returns the reason instead when amdsmi is unavailable."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:  # no amdsmi module or no access to the driver
        return {"error": f"amdsmi unavailable: {e}"}
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        dev = torch.cuda.current_device()
        if not handles:
            return {"error": "amdsmi lists no GPU"}
        h = handles[dev] if dev < len(handles) else handles[0]
        samples, power, limit, stop = [], [], [], threading.Event()

        def poll():
            while not stop.is_set():
                try:
                    clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.SYS)["clk"]
                    if isinstance(clk, (int, float)) and clk > 0:
                        samples.append(float(clk))
                    pw = amdsmi.amdsmi_get_power_info(h)
                    cur = pw.get("current_socket_power", "N/A")
                    if cur in ("N/A", 0):
                        cur = pw.get("socket_power", "N/A")
                    if isinstance(cur, (int, float)) and cur > 0:
                        power.append(float(cur))
                    if isinstance(pw.get("power_limit"), (int, float)) and pw["power_limit"] > 0:
                        limit.append(float(pw["power_limit"]))
                except Exception:
                    pass
                time.sleep(0.01)

        th = threading.Thread(target=poll, daemon=True)
        th.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                replay()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        return summarise_clock(samples, power, limit)
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--explicit-config", default="v3_bf16")
    p.add_argument("--decode-config", default="v3_decode_b64_32k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0,
                   help="approximate CPU seconds for the oracle baseline sample")
    p.add_argument("--no-absorbed", action="store_true",
                   help="skip the absorbed-form forward of the explicit workload")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the graphics-clock probe after the timed region (it replays each step for ~2 s)")
    p.add_argument("--no-graph", action="store_true",
                   help="time the step as eager calls (no HIP graph replay)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the timing of the V2-Lite and SP=8-rank explicit configurations")
    p.add_argument("--no-forms", action="store_true",
                   help="skip the explicit-vs-absorbed memory and time comparison at 4K/8K/16K tokens")
    p.add_argument("--no-backward", action="store_true", help="skip the explicit-form backward")
    p.add_argument("--no-fused", action="store_true",
                   help="skip the materialised-vs-fused up-projection comparison at the head-shard share")
    p.add_argument("--form-calls", type=int, default=3,
                   help="timed calls per form and length in the explicit-vs-absorbed comparison")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run a plain 1 GiB device copy (3 times) before the warm-up, as the "
                        "reference reading for HBM byte counters")
    return p.parse_args()


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(ecfg, x_host, out_gpu, dcfg, dx_host, dout_gpu, budget_s):
    """Time the fp64 oracle on a bounded sample of the same workload and, on
    the same sample, compare the GPU outputs with it."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    from oracle import mla_oracle as O

    workers = pool_size()

    def one_head(h):
        return O.explicit_fwd(x_host["q_nope"], x_host["q_pe"], x_host["c_kv"], x_host["k_pe"], x_host["w_kv_b"],
                              q_pos0=ecfg.q_pos0, kv_pos0=ecfg.kv_pos0, causal=ecfg.causal,
                              softmax_scale=ecfg.softmax_scale, heads=[h])[0]

    # explicit: a pool of single-threaded-BLAS workers, one head per task; the
    # sample is the first k heads (all query rows), k sized to the budget
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        one_head(0)
        t_one = time.perf_counter() - t0
        k = int(max(1, min(ecfg.n_heads, workers * (0.7 * budget_s) // max(t_one, 1e-3))))
        k = max(1, min(ecfg.n_heads, (k // workers) * workers or k))
        heads = list(range(k))
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(workers) as ex:
            parts = list(ex.map(one_head, heads))
        t_exp = time.perf_counter() - t0
    ro = np.concatenate(parts, axis=2)
    fl = ecfg.flops()
    flops_sample = fl["total"] * k / ecfg.n_heads
    got = out_gpu[:, :, :k]
    err = np.abs(got - ro)
    parity_exp = {"max_abs": float(err.max()), "rel_l2": float(np.linalg.norm(got - ro) / np.linalg.norm(ro)),
                  "sample": f"heads 0..{k - 1} of {ecfg.n_heads}, all {ecfg.s_q} query rows"}

    # decode: one sequence, all heads
    bits = dx_host["cache_bits"]
    from head_latent_attention_02_amd import inputs as I
    dec_threads = blas_threads()
    t0 = time.perf_counter()
    r = O.decode_absorbed(dx_host["q_nope"], dx_host["q_pe"], lambda b: I.bf16_bits_to_f32(bits[b]),
                          dx_host["cache_len"], dx_host["w_kv_b"], n_splits=dcfg.n_splits, d_kv=dcfg.d_kv,
                          softmax_scale=dcfg.softmax_scale, batches=[0])
    t_dec = time.perf_counter() - t0
    dg = dout_gpu[:1]
    derr = np.abs(dg - r["out"])
    parity_dec = {"max_abs": float(derr.max()),
                  "rel_l2": float(np.linalg.norm(dg - r["out"]) / np.linalg.norm(r["out"])),
                  "sample": f"sequence 0 of {dcfg.batch}, all {dcfg.n_heads} heads"}
    hi = host_info()
    return ({"value": flops_sample / t_exp / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
             "sample": f"explicit fwd at {ecfg.name} dims, heads 0..{k - 1} of {ecfg.n_heads} (all rows), "
                       f"{t_exp:.1f} s; fp64 numpy, {workers} worker threads over heads, BLAS single-threaded",
             **hi},
            {"value": 1.0 / t_dec, "unit": "tok/s", "cores": dec_threads, "kind": "oracle",
             "sample": f"absorbed decode, 1 of {dcfg.batch} sequences (L={dcfg.cache_len}, all heads), "
                       f"{t_dec:.1f} s; fp64 numpy, BLAS with {dec_threads} threads", **hi},
            {"explicit": parity_exp, "decode": parity_dec})


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs the MLA hot path on one GPU; the library has no "
                                   "multi-GPU path (--gpus must be 1)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from head_latent_attention_02_amd import inputs as I
    from head_latent_attention_02_amd import mla

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mla.library()

    ecfg = I.EXPLICIT_CONFIGS[args.explicit_config]
    dcfg = I.DECODE_CONFIGS[args.decode_config]
    log(f"generating inputs: {ecfg.name}, {dcfg.name}")
    x = I.make_explicit_inputs(ecfg)
    dx = I.make_decode_inputs(dcfg)
    t = {k: torch.from_numpy(v).to(torch.bfloat16).to(dev) for k, v in x.items()}
    cache = torch.from_numpy(dx["cache_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    dq_nope = torch.from_numpy(dx["q_nope"]).to(torch.bfloat16).to(dev)
    dq_pe = torch.from_numpy(dx["q_pe"]).to(torch.bfloat16).to(dev)
    dw = torch.from_numpy(dx["w_kv_b"]).to(torch.bfloat16).to(dev)
    dlen = torch.from_numpy(dx["cache_len"]).to(dev)

    out = torch.empty((ecfg.batch, ecfg.s_q, ecfg.n_heads, ecfg.d_v), dtype=torch.float32, device=dev)
    lse = torch.empty((ecfg.batch, ecfg.n_heads, ecfg.s_q), dtype=torch.float32, device=dev)
    dout = torch.empty((dcfg.batch, dcfg.n_heads, dcfg.d_v), dtype=torch.float32, device=dev)
    dlse = torch.empty((dcfg.batch, dcfg.n_heads), dtype=torch.float32, device=dev)
    ws = dws = None

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    exp_ms, dec_ms = [], []

    def step(record):
        nonlocal ws, dws
        if record:
            ev[0].record()
        _, _, ws = mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"],
                                        q_pos0=ecfg.q_pos0, kv_pos0=ecfg.kv_pos0, causal=ecfg.causal,
                                        softmax_scale=ecfg.softmax_scale, out=out, lse=lse, workspace=ws)
        if record:
            ev[1].record()
        _, _, dws = mla.mla_decode_absorbed(dq_nope, dq_pe, cache, dlen, dw, n_splits=dcfg.n_splits,
                                            softmax_scale=dcfg.softmax_scale, out=dout, lse=dlse, workspace=dws)
        if record:
            ev[2].record()

    if args.copy_calibration:
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {COPY_CALIBRATION_BYTES} bytes")
        del src, dst

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    mla.mla_timing_reset()
    mla.mla_timing_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        exp_ms.append(ev[0].elapsed_time(ev[1]))
        dec_ms.append(ev[1].elapsed_time(ev[2]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mla.mla_timing_end()
    kt = mla.mla_timing_get()
    log("timed region done")

    ms_step = (t1 - t0) * 1e3 / args.steps
    e_ms = float(np.mean(exp_ms))
    d_ms = float(np.mean(dec_ms))
    e_med, d_med = float(np.median(exp_ms)), float(np.median(dec_ms))
    eager = {"ms_per_step": ms_step, "explicit_ms": e_ms, "decode_ms": d_ms}
    graph = None
    clocks = None
    if not args.no_graph:
        # the reference outputs of one eager step
        step(False)
        torch.cuda.synchronize()
        ref = [out.clone(), lse.clone(), dout.clone(), dlse.clone()]
        g_exp, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(False)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        log("capturing the explicit and decode steps as HIP graphs")
        with torch.cuda.graph(g_exp):
            mla.mla_fwd_explicit(t["q_nope"], t["q_pe"], t["c_kv"], t["k_pe"], t["w_kv_b"],
                                 q_pos0=ecfg.q_pos0, kv_pos0=ecfg.kv_pos0, causal=ecfg.causal,
                                 softmax_scale=ecfg.softmax_scale, out=out, lse=lse, workspace=ws)
        with torch.cuda.graph(g_dec):
            mla.mla_decode_absorbed(dq_nope, dq_pe, cache, dlen, dw, n_splits=dcfg.n_splits,
                                    softmax_scale=dcfg.softmax_scale, out=dout, lse=dlse, workspace=dws)
        torch.cuda.synchronize()
        for buf in (out, lse, dout, dlse):
            buf.fill_(float("nan"))
        g_exp.replay()
        g_dec.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(torch.nan_to_num(a, neginf=-1e30), torch.nan_to_num(b, neginf=-1e30))
                   for a, b in zip((out, lse, dout, dlse), ref))
        if not same:
            raise RuntimeError("graph replay differs from the eager step")
        for _ in range(args.warmup):
            g_exp.replay()
            g_dec.replay()
        log(f"timing {args.steps} graph replays")
        g_exp_ms, g_dec_ms = [], []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            ev[0].record()
            g_exp.replay()
            ev[1].record()
            g_dec.replay()
            ev[2].record()
            torch.cuda.synchronize()
            g_exp_ms.append(ev[0].elapsed_time(ev[1]))
            g_dec_ms.append(ev[1].elapsed_time(ev[2]))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_step = (t1 - t0) * 1e3 / args.steps
        e_ms = float(np.mean(g_exp_ms))
        d_ms = float(np.mean(g_dec_ms))
        e_med, d_med = float(np.median(g_exp_ms)), float(np.median(g_dec_ms))
        graph = {"ms_per_step": ms_step, "explicit_ms": e_ms, "decode_ms": d_ms,
                 "check": "replay bit-identical to the eager step"}
    if graph is not None and not args.no_clock:
        log("graphics clock under each step's load (amdsmi, after the timed region)")
        clocks = {"explicit": clock_under_load(torch, g_exp.replay), "decode": clock_under_load(torch, g_dec.replay),
                  "source": "amdsmi_get_clock_info(SYS) and amdsmi_get_power_info polled every 10 ms while the "
                            "captured step replays back to back for about 2 s after the timed region; "
                            "medians of the second second",
                  "peak_clock_mhz": PEAK_CLOCK_MHZ}
    fl = ecfg.flops()
    dflops = dcfg.flops()
    dbytes = dcfg.algorithmic_bytes()
    explicit_tflops = fl["total"] / (e_ms * 1e-3) / 1e12
    decode_tok_s = dcfg.batch / (d_ms * 1e-3)
    decode_gbs = dbytes["total"] / (d_ms * 1e-3) / 1e9

    # per-kernel averages and their algorithmic rates
    B, H, L = dcfg.batch, dcfg.n_heads, dcfg.cache_len
    per_kernel_work = {
        "mfma_attention": ("TFLOP/s", fl["attention"]),
        "mfma_up_projection": ("TFLOP/s", fl["up_proj"]),
        "mfma_split_kv": ("GB/s", dbytes["cache"]),
        # the fp16 partials and fp32 chunk LSEs it reads, and W_UV (bf16)
        "lse_combine": ("GB/s", B * dcfg.n_splits * H * (dcfg.d_kv * 2 + 4) + H * dcfg.d_v * dcfg.d_kv * 2),
        "absorb": ("GB/s", H * dcfg.d_nope * dcfg.d_kv * 2 + B * H * (dcfg.d_kv + dcfg.d_rope) * 2),
    }
    kernels = {}
    for name, (ms_tot, n) in kt.items():
        avg = ms_tot / max(n, 1)
        ent = {"avg_ms": avg, "launches_per_step": n / args.steps}
        if name in per_kernel_work:
            unit, work = per_kernel_work[name]
            ent["achieved"] = work / (avg * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
            ent["unit"] = unit
        if name in KERNEL_SOURCES:
            ent["traffic"] = hbm_traffic(name)
        kernels[name] = ent

    def roof(name, bound, unit, work, peak):
        if name not in kt:
            return None
        avg = kt[name][0] / max(kt[name][1], 1)
        ach = work / (avg * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        return {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
                "traffic": hbm_traffic(name), "traffic_unit": "bytes per launch",
                "kernel": name, "avg_ms": avg, "work_per_launch": work,
                "source_digest": source_digest(name)}

    roofline = roof("mfma_attention", "mfma", "TFLOP/s", fl["attention"], PEAK_MFMA_TFLOPS)
    # the matrix peak scales with the shader clock: the same rate against the
    # peak at the clock measured under this step's load
    clk = (clocks or {}).get("explicit") or {}
    if roofline is not None and "sclk_mhz_median" in clk:
        pk = PEAK_MFMA_TFLOPS * clk["sclk_mhz_median"] / PEAK_CLOCK_MHZ
        roofline["peak_at_clock"] = pk
        roofline["frac_at_clock"] = roofline["achieved"] / pk
    roofline_decode = roof("mfma_split_kv", "hbm", "GB/s", dbytes["cache"], PEAK_HBM_GBS)

    res = {
        "metric": METRIC,
        "value": explicit_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{ecfg.name} explicit fwd (B={ecfg.batch}, S={ecfg.s_q}, n_h={ecfg.n_heads}, causal) + "
                        f"{dcfg.name} absorbed decode (B={dcfg.batch}, L={dcfg.cache_len}, n_h={dcfg.n_heads}, "
                        f"{dcfg.n_splits} splits)",
            "explicit": {"batch": ecfg.batch, "seq_len": ecfg.s_q, "n_heads": ecfg.n_heads, "d_kv": ecfg.d_kv,
                         "d_nope": ecfg.d_nope, "d_rope": ecfg.d_rope, "d_v": ecfg.d_v,
                         "algorithmic_flop": fl["total"]},
            "decode": {"batch": dcfg.batch, "cache_len": dcfg.cache_len, "n_heads": dcfg.n_heads,
                       "n_splits": dcfg.n_splits, "algorithmic_bytes": dbytes["total"],
                       "algorithmic_flop": dflops["total"]},
            "arithmetic": "bf16 inputs; up-projection bf16 MFMA; attention QK^T/PV fp16 MFMA; decode bf16 MFMA; "
                          "fp32 accumulate and fp32 outputs",
        },
        "explicit": {"ms": e_ms, "ms_median": e_med, "tflops": explicit_tflops,
                     "frac_mfma_peak": explicit_tflops / PEAK_MFMA_TFLOPS,
                     "frac_mfma_peak_at_clock": (explicit_tflops / (PEAK_MFMA_TFLOPS * clk["sclk_mhz_median"]
                                                                    / PEAK_CLOCK_MHZ)
                                                 if "sclk_mhz_median" in clk else None)},
        "decode": {"ms": d_ms, "ms_median": d_med, "tok_per_s": decode_tok_s, "algorithmic_gbs": decode_gbs,
                   "frac_hbm_peak": decode_gbs / PEAK_HBM_GBS},
        "roofline": roofline,
        "roofline_decode": roofline_decode,
        "kernels": kernels,
        "timing": {"step": "hip_graph_replay" if graph is not None else "eager", "eager": eager,
                   "graph": graph},
        "clock": clocks,
    }

    res["context"] = CONTEXT

    if not args.no_absorbed:
        res["absorbed_forward"] = absorbed_forward(mla, torch, ecfg, t, fl, args)

    if not args.no_configs:
        res["configs"] = {name: explicit_case(mla, torch, I.EXPLICIT_CONFIGS[name], args)
                          for name in ("v3_sp8_rank3", "v2lite_bf16")}

    if not args.no_backward:
        res["backward"] = backward_case(mla, torch, ecfg, args)

    if not args.no_fused:
        res["fused_headshard"] = fused_case(mla, torch, I.EXPLICIT_CONFIGS["v3_headshard_sp8"], args)

    if not args.no_cpu_baseline:
        log("oracle CPU baseline on a bounded sample")
        cb_e, cb_d, parity = cpu_baseline(ecfg, x, out.cpu().numpy(), dcfg, dx, dout.cpu().numpy(),
                                          args.cpu_budget_s)
        res["cpu_baseline"] = cb_e
        res["cpu_baseline_decode"] = cb_d
        res["parity_sample"] = parity

    if not args.no_forms:
        del t, cache, dq_nope, dq_pe, dw, dlen, ws, dws
        torch.cuda.empty_cache()
        res["forms_memory"] = forms_memory_and_time(mla, torch, ["v3_bf16", "v3_s8k_bf16", "v3_s16k_bf16"], args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
