#!/usr/bin/env python3
"""Benchmark of the GCA hot path on one MI355X.

One step = causal retrieval (Gumbel top-k) + grouped cross-attention forward + backward over one
batch of the 16K-token training workload (B=8, L=16384 = 256 chunks of 64, H=12, d=64, K=8, G=2,
bf16, synthetic N(0,1)/8 inputs).  Prints one JSON line: tokens/s with inputs resident in HBM,
the roofline position of the dominant kernel (HIP events around each kernel launch inside the
timed region), the CPU oracle timed on a bounded sample of the same workload, the per-chunk
retrieve+attend latency over 1M- and 16M-token histories held in HBM, and the rows beside the
step: landmark gradients, sliding-window attention, the window and GCA fused in one call, the
forward-only workload (one group, no Gumbel noise, no LSE) and the step at 4K/16K/64K contexts
with the same tokens per batch.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-inference] [--no-cpu-baseline]
                    [--no-scaling] [--copy-calibration]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GCA fwd+bwd tokens/s at 16K ctx; per-chunk retrieve+attend latency at 16M"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, TFLOP/s
UNIT_FLOPS = 2 * 64 * 64 * 64  # one 64x64x64 matrix product (one slot, one head)
# The third ceiling of the attention passes, the exponential pipe: every pass takes one v_exp_f32
# per score element (4,096 per tile).  A probe of independent v_exp_f32 chains measured 8.3 cycles
# per wave instruction per SIMD with two waves per SIMD (one wave: 8.7), i.e. 64 / 8.3 results per
# cycle per SIMD; over 1,024 SIMDs at the 2.4 GHz peak clock that is 1.89e13 per second.  Reported
# beside the HBM and matrix-core fractions, not used as the roofline denominator.
EXP_CYCLES_PER_WAVE_INSTR = 8.3
PEAK_EXP_PER_S = 1024 * 64 / EXP_CYCLES_PER_WAVE_INSTR * 2.4e9
EXPS_PER_TILE = 64 * 64


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def training_step_setup(seed=0):
    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    shape = I.TRAIN_16K_G2
    cfg = gca.Config(B=shape.B, G=shape.G, H=shape.H, n_q=shape.n_q, n_kv=shape.n_kv, topk=shape.topk,
                     dtype="bf16", use_gumbel=True, seed=1)
    log("generating inputs", shape)
    host = I.make_inputs(shape, "bf16", seed=seed, scale=0.125)
    dev = {k: v.cuda() for k, v in host.items()}
    G, B, H, nq, K = shape.G, shape.B, shape.H, shape.n_q, shape.topk
    bufs = {
        "idx": torch.empty((G, B, nq, K), dtype=torch.int32, device="cuda"),
        "score": torch.empty((G, B, nq, K), dtype=torch.float32, device="cuda"),
        "o": torch.empty_like(dev["q"]),
        "lse": torch.empty((G, B, H, nq, K, 64), dtype=torch.float32, device="cuda"),
        "dq": torch.empty_like(dev["q"]),
        "dk": torch.empty_like(dev["k"]),
        "dv": torch.empty_like(dev["v"]),
        "dscore": torch.empty((G, B, nq, K), dtype=torch.float32, device="cuda"),
    }
    ws_b = torch.empty(gca.workspace_size(gca.OP_BACKWARD, cfg), dtype=torch.uint8, device="cuda")
    assert gca.workspace_size(gca.OP_RETRIEVE, cfg) == 0

    def step():
        gca.retrieve(cfg, dev["lq"], dev["lk"], bufs["idx"], bufs["score"])
        gca.forward(cfg, dev["q"], dev["k"], dev["v"], bufs["idx"], bufs["score"], o=bufs["o"], lse=bufs["lse"])
        gca.backward(cfg, dev["q"], dev["k"], dev["v"], bufs["idx"], bufs["score"], bufs["lse"], dev["dout"],
                     ws=ws_b, out=(bufs["dq"], bufs["dk"], bufs["dv"], bufs["dscore"]))

    return shape, cfg, host, dev, bufs, step


def kernel_figures(shape, idx_cpu):
    """Algorithmic flops and HBM bytes per launch of each kernel (compulsory traffic)."""
    import numpy as np

    G, B, H, nq, nkv, K = shape.G, shape.B, shape.H, shape.n_q, shape.n_kv, shape.topk
    idx = np.asarray(idx_cpu)
    used = idx[:, :, : nq - 1] >= 0            # row r feeds query chunk r + 1
    tiles = int(used.sum()) * H                # (slot, head) pairs of 64x64 tiles
    tok = B * nq * 64
    T = tok * H * 64 * 2                       # one [B, H, L, 64] bf16 tensor
    lse = G * tok * H * K * 4
    lmk = G * B * (nq + nkv) * 64 * 2
    sel = G * B * nq * K * 8
    pairs = G * B * nq * (nq - 1) // 2
    ex = EXPS_PER_TILE * tiles                 # one exponential per score element and pass
    return {
        "score_topk": {"flops": 2 * 64 * pairs, "bytes": lmk + sel, "tiles": 0},
        # forward: S and PV per tile; reads Q, K, V, writes O and LSE
        "attend_fwd": {"flops": 2 * UNIT_FLOPS * tiles, "bytes": (G + 1 + 1 + G) * T + lse + sel, "tiles": tiles, "exps": ex},
        # query-major backward: dP' and dQ per tile; reads Q, dO, K, V, LSE, writes dQ
        "bwd_query": {"flops": 2 * UNIT_FLOPS * tiles, "bytes": (G + G + 1 + 1 + G) * T + lse + sel, "tiles": tiles, "exps": ex},
        # key-major backward: dK and dV per tile; reads Q, dO, K, V, LSE, writes dK, dV
        "bwd_key": {"flops": 2 * UNIT_FLOPS * tiles, "bytes": (G + G + 1 + 1 + 1 + 1) * T + lse, "tiles": tiles, "exps": ex},
        "inverse_index": {"flops": 0, "bytes": sel // 2, "tiles": 0},
        "score_grad": {"flops": 0, "bytes": sel, "tiles": 0},
    }


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it was taken on the
    current kernel sources (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's readings)."""
    from long_context_lm_amd import profiling

    path = os.path.join(ROOT, "profiles", "gca_train16k_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != profiling.source_hash() or kernel not in t.get("kernels", {}):
        return None
    return t["kernels"][kernel]["hbm_bytes"]


def step_roofline(shape, idx_cpu):
    """The step's algorithmic floor: forward and backward each at the larger of their matrix-core
    and HBM times.  Forward: two 64x64x64 products per (valid slot, head) tile; Q, K, V read, O
    and the LSE written.  Backward: four products per tile (dP', dV, dQ, dK, no recompute); Q,
    dO, K, V read, dQ, dK, dV written, LSE read.  At the 16K, G=2 shape (384,768 tiles) this is
    163.7 us (forward, HBM) + 322.8 us (backward, matrix cores) = 486.5 us."""
    import numpy as np

    G, B, H, nq, K = shape.G, shape.B, shape.H, shape.n_q, shape.topk
    tiles = int((np.asarray(idx_cpu)[:, :, : nq - 1] >= 0).sum()) * H
    T = B * nq * 64 * H * 64 * 2
    lse = G * B * nq * 64 * H * K * 4
    sel = G * B * nq * K * 8
    fwd = {"flops": 2 * UNIT_FLOPS * tiles, "bytes": (2 * G + 2) * T + lse + sel}
    bwd = {"flops": 4 * UNIT_FLOPS * tiles, "bytes": (3 * G + 4) * T + lse + sel}

    def t(f, pf, pb):
        return max(f["flops"] / pf, f["bytes"] / pb)

    return {"tiles": tiles, "forward": fwd, "backward": bwd,
            "floor_us": (t(fwd, PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9)
                         + t(bwd, PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9)) * 1e6,
            "t": t}


def measured_peaks():
    """Rates measured on this GPU in this run, beside the vendor peaks: a plain 1 GiB device copy
    (bytes read + written per second) and a bf16 8192^3 matrix product through torch (hipBLASLt),
    the rate a dense bf16 contraction reaches here."""
    import torch

    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    a.record()
    for _ in range(n):
        dst.copy_(src)
    b.record()
    b.synchronize()
    copy_gbs = 2 * src.numel() * n / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    m = 8192
    x = torch.randn((m, m), device="cuda", dtype=torch.bfloat16)
    y = torch.randn((m, m), device="cuda", dtype=torch.bfloat16)
    z = torch.empty((m, m), device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(x, y, out=z)
    a.record()
    for _ in range(n):
        torch.mm(x, y, out=z)
    b.record()
    b.synchronize()
    gemm_tflops = 2 * m ** 3 * n / (a.elapsed_time(b) * 1e-3) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": copy_gbs, "bf16_gemm_tflops": gemm_tflops,
            "how": "1 GiB device copy (read + write bytes / time); torch.mm bf16 8192x8192x8192"}


def both_ceilings(fig, ms, peaks):
    """A kernel's position against both ceilings, vendor and measured."""
    t = ms * 1e-3
    tb = fig["bytes"] / t / 1e9
    tf = fig["flops"] / t / 1e12
    out = {"avg_ms": ms, "hbm_gbs": tb, "hbm_frac": tb / PEAK_HBM_GBS, "mfma_tflops": tf,
           "mfma_frac": tf / PEAK_BF16_TFLOPS}
    if fig.get("exps"):
        out["exp_per_s"] = fig["exps"] / t
        out["exp_frac"] = out["exp_per_s"] / PEAK_EXP_PER_S
    if peaks:
        out["hbm_frac_measured_peak"] = tb / peaks["hbm_copy_gbs"]
        out["mfma_frac_measured_peak"] = tf / peaks["bf16_gemm_tflops"]
    return out


def roofline_for(name, fig, ms):
    t = ms * 1e-3
    t_mfma = fig["flops"] / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = fig["bytes"] / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(name)
    if t_mfma >= t_hbm:
        ach = fig["flops"] / t / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic,
                "algorithmic_flops": fig["flops"], "algorithmic_bytes": fig["bytes"], "avg_launch_ms": ms}
    ach = fig["bytes"] / t / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBS, "traffic": traffic,
            "algorithmic_flops": fig["flops"], "algorithmic_bytes": fig["bytes"], "avg_launch_ms": ms}


def cpu_baseline(shape, host, rows=3):
    """The oracle on a bounded sample: the first `rows` batch rows of the workload (both groups,
    all heads), about 10-15 s of host work."""
    from long_context_lm_amd import inputs as I
    from oracle import gca_oracle as O

    x = {k: I.as_f64(v[:, 0:rows] if k in ("lq", "lk", "q", "dout") else v[0:rows]) for k, v in host.items()}
    threads = 1
    try:
        from threadpoolctl import threadpool_info

        blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:
        pass
    c0 = time.process_time()
    t0 = time.perf_counter()
    idx, sc = O.retrieve(x["lq"], x["lk"], shape.topk, use_gumbel=True, seed=1)
    _o, _lse = O.forward(x["q"], x["k"], x["v"], idx, sc, shift=1)
    O.backward(x["q"], x["k"], x["v"], idx, sc, x["dout"], shift=1)
    dt = time.perf_counter() - t0
    cpu_s = time.process_time() - c0  # CPU time of all the process's threads
    tokens = rows * shape.n_q * 64
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    busy = cpu_s / dt if dt > 0 else 1.0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": max(1, round(busy)), "kind": "oracle",
            "sample": f"batch rows 0..{rows - 1} of the workload ({tokens} tokens, G=2, H=12): retrieve+fwd+bwd, "
                      f"{dt:.1f} s wall, {cpu_s:.1f} s CPU ({busy:.2f} cores busy) on {os.cpu_count()} host "
                      f"CPUs (BLAS pool {threads} threads)",
            "host": {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity": affinity,
                     "blas_threads": threads, "seconds": dt, "cpu_seconds": cpu_s, "busy_cores": busy}}


def landmark_timing(shape, cfg, dev, bufs, iters=50):
    """gca_landmark_backward on the step's own indices and d(score) (a row beyond the timed step:
    the gradients that reach the landmarks through the retrieval scores)."""
    import torch

    from long_context_lm_amd import gca

    ws = torch.empty(max(gca.workspace_size(gca.OP_LANDMARK_BACKWARD, cfg), 1), dtype=torch.uint8, device="cuda")
    out = (torch.empty_like(dev["lq"]), torch.empty_like(dev["lk"]))

    def one():
        gca.landmark_backward(cfg, dev["lq"], dev["lk"], bufs["idx"], bufs["dscore"], ws=ws, out=out)

    for _ in range(5):
        one()
    torch.cuda.synchronize()
    gca.profile_collect()
    gca.profile_enable(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        one()
    b.record()
    torch.cuda.synchronize()
    gca.profile_enable(False)
    kern = {k: v[0] / v[1] * 1e3 for k, v in gca.profile_collect().items()}
    us = a.elapsed_time(b) / iters * 1e3
    G, B, nq, nkv, K = shape.G, shape.B, shape.n_q, shape.n_kv, shape.topk
    # compulsory bytes: lq, lk read, dlq, dlk written (bf16), idx and d(score) read
    nbytes = 2 * G * B * (nq + nkv) * 64 * 2 + G * B * nq * K * 8
    return {"us_per_call": us, "kernels_us": kern, "algorithmic_bytes": nbytes,
            "hbm_bound_us": nbytes / (PEAK_HBM_GBS * 1e9) * 1e6}


def window_timing(B=8, H=12, n_c=256, window=512, iters=10):
    """Sliding-window self-attention beside GCA (W = 512) at the training shape: gca_sw_forward +
    gca_sw_backward on synthetic bf16 inputs, timed apart from the GCA step."""
    import torch

    from long_context_lm_amd import gca

    gen = torch.Generator(device="cuda").manual_seed(77)
    q, k, v, do = (torch.randn((B, H, 64 * n_c, 64), generator=gen, device="cuda", dtype=torch.bfloat16)
                   for _ in range(4))
    cfg = gca.sw_config(B, H, n_c)
    ws = torch.empty(gca.workspace_size(gca.OP_SW_BACKWARD, cfg), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))

    def one():
        gca.sw_forward(cfg, q, k, v, window, o=o, lse=lse)
        gca.sw_backward(cfg, q, k, v, o, lse, do, window, ws=ws, out=grads)

    for _ in range(3):
        one()
    torch.cuda.synchronize()
    gca.profile_collect()
    gca.profile_enable(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        one()
    b.record()
    torch.cuda.synchronize()
    gca.profile_enable(False)
    kern = {kk: vv[0] / vv[1] * 1e3 for kk, vv in gca.profile_collect().items()}
    us = a.elapsed_time(b) / iters * 1e3
    L = 64 * n_c
    pairs = sum(min(i + 1, window) for i in range(L))  # (query, key) pairs per (batch row, head)
    fwd_flops = 4 * 64 * pairs * B * H      # q.k and p.v
    bwd_flops = 8 * 64 * pairs * B * H      # dp, dq, dk, dv
    res = {"workload": f"B={B} L={L} H={H} d=64 W={window} bf16", "us_per_step": us, "kernels_us": kern,
           "tokens_per_s": B * L / (us * 1e-6), "algorithmic_flops_fwd": fwd_flops, "algorithmic_flops_bwd": bwd_flops}
    fwd_us = kern.get("sw_fwd", 0.0)
    bwd_us = kern.get("sw_bwd_query", 0.0) + kern.get("sw_bwd_key", 0.0)
    if fwd_us > 0:
        res["fwd_tflops"] = fwd_flops / (fwd_us * 1e-6) / 1e12
    if bwd_us > 0:
        res["bwd_tflops"] = bwd_flops / (bwd_us * 1e-6) / 1e12
    res["mfma_frac"] = (fwd_flops + bwd_flops) / (us * 1e-6) / (PEAK_BF16_TFLOPS * 1e12)
    del q, k, v, do, o, lse, grads, ws
    torch.cuda.empty_cache()
    return res


def fused_timing(B=8, H=12, n_c=256, window=512, K=8, iters=10):
    """The layer's sliding window and GCA over the same queries, summed (G = 1, W = 512, K = 8,
    bf16, N(0,1)/8 inputs at the training shape): gca_fused_forward + gca_fused_backward against
    the separate calls (gca_sw_forward + gca_forward, gca_sw_backward + gca_backward) plus the two
    sums a caller of the separate calls needs (o and dq).  The retrieval is not timed (the same
    indices serve both)."""
    import torch

    from long_context_lm_amd import gca

    gen = torch.Generator(device="cuda").manual_seed(91)
    L = 64 * n_c

    def mk(shape):
        return (torch.randn(shape, generator=gen, device="cuda") / 8).to(torch.bfloat16)

    q, k_sw, v_sw, k, v, do = (mk((B, H, L, 64)) for _ in range(6))
    cfg = gca.Config(B=B, G=1, H=H, n_q=n_c, n_kv=n_c, topk=K, dtype="bf16", use_gumbel=True, seed=1)
    idx, sc = gca.retrieve(cfg, mk((1, B, n_c, 64)), mk((1, B, n_c, 64)))
    o = torch.empty_like(q)
    lse_sw = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    lse = torch.empty(cfg.shape("lse"), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
             torch.empty(idx.shape, dtype=torch.float32, device="cuda"))
    ws = torch.empty(gca.workspace_size(gca.OP_FUSED_BACKWARD, cfg), dtype=torch.uint8, device="cuda")

    def fused():
        gca.fused_forward(cfg, q, k_sw, v_sw, k, v, idx, sc, window, o=o, lse_sw=lse_sw, lse=lse)
        gca.fused_backward(cfg, q, k_sw, v_sw, k, v, idx, sc, o, lse_sw, lse, do, window, ws=ws, out=grads)

    swc = gca.sw_config(B, H, n_c)
    ws_sw = torch.empty(gca.workspace_size(gca.OP_SW_BACKWARD, swc), dtype=torch.uint8, device="cuda")
    ws_g = torch.empty(gca.workspace_size(gca.OP_BACKWARD, cfg), dtype=torch.uint8, device="cuda")
    o_sw, o_g = torch.empty_like(q), torch.empty_like(q)
    g_sw = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    g_g = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), grads[5])
    q1, do1, o_g1 = q[None], do[None], o_g[None]

    def separate():
        gca.sw_forward(swc, q, k_sw, v_sw, window, o=o_sw, lse=lse_sw)
        gca.forward(cfg, q1, k, v, idx, sc, o=o_g1, lse=lse)
        torch.add(o_sw, o_g, out=o)
        gca.sw_backward(swc, q, k_sw, v_sw, o_sw, lse_sw, do, window, ws=ws_sw, out=g_sw)
        gca.backward(cfg, q1, k, v, idx, sc, lse, do1, ws=ws_g, out=(g_g[0][None], g_g[1], g_g[2], g_g[3]))
        torch.add(g_sw[0], g_g[0], out=grads[0])

    ms_f, kern_f = _timed(fused, iters)
    ms_s, kern_s = _timed(separate, iters)
    res = {"workload": f"sliding window (W={window}) + GCA (K={K}, G=1) over the same queries, summed; B={B} L={L} "
                       f"H={H} d=64 bf16, inputs N(0,1)/8; forward + backward",
           "fused_us": ms_f * 1e3, "separate_us": ms_s * 1e3, "tokens_per_s_fused": B * L / (ms_f * 1e-3),
           "kernels_us_fused": kern_f, "kernels_us_separate": kern_s}
    del q, k_sw, v_sw, k, v, do, o, lse_sw, lse, grads, ws, ws_sw, ws_g, o_sw, o_g, g_sw, g_g
    torch.cuda.empty_cache()
    return res


def skewed_retrieval_timing(shape, dev, bufs, step, iters=10):
    """The training step (retrieve + forward + backward, G=2, K=8, Gumbel, bf16) with a hub
    chunk: every query landmark of a (group, batch row) shares a direction with key landmark 0,
    which then enters nearly every row's top-k (about 500 of the 512 (group, row) entries of a
    batch row).  Same q, k, v, dout as the headline step; the step's landmarks are overwritten.
    The hub's list is split into segments that helper workgroups of the key-major pass walk."""
    import numpy as np

    from long_context_lm_amd import inputs as I

    lq, lk = I.hub_landmarks(shape, seed=5)
    dev["lq"].copy_(I.to_dtype(lq, "bf16"))
    dev["lk"].copy_(I.to_dtype(lk, "bf16"))
    ms, kern = _timed(step, iters)
    idx = bufs["idx"].cpu().numpy()[:, :, : shape.n_q - 1]
    per_b = [int(np.bincount(idx[:, b][idx[:, b] >= 0], minlength=shape.n_kv).max()) for b in range(shape.B)]
    res = {"workload": "GCA retrieve+fwd+bwd, B=8 L=16384 H=12 d=64 K=8 G=2, Gumbel, bf16; landmarks with a hub "
                       "chunk (chunk 0 in nearly every row's top-k)",
           "ms_per_step": ms, "tokens_per_s": shape.B * shape.n_q * 64 / (ms * 1e-3), "kernels_us": kern,
           "max_entries_per_chunk": max(per_b), "mean_entries_per_chunk": float((idx >= 0).sum() / (shape.B * shape.n_kv))}
    return res


def _device_inputs(shape, seed, scale=0.125):
    """Seeded N(0, scale^2) bf16 inputs drawn on the device (timing runs only: their values
    change no launch shape, and host generation of several GiB would dominate the run)."""
    import torch

    from long_context_lm_amd import inputs as I

    gen = torch.Generator(device="cuda").manual_seed(seed)
    out = {}
    for name in I.STREAMS:
        x = torch.randn(shape.tensor_shape(name), generator=gen, device="cuda", dtype=torch.float32)
        out[name] = x.mul_(scale).to(torch.bfloat16)
        del x
    return out


def _timed(fn, iters, warmup=3):
    """Average event time (ms) of fn over iters calls, and the per-kernel averages (us)."""
    import torch

    from long_context_lm_amd import gca

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    gca.profile_collect()
    gca.profile_enable(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    gca.profile_enable(False)
    kern = {k: v[0] / v[1] * 1e3 for k, v in gca.profile_collect().items()}
    return a.elapsed_time(b) / iters, kern


def tiny_forward_latency(iters=50):
    """The tiny fp32 problem (B=1, L=1024 in 16 chunks, H=2, K=4, one group, no Gumbel): retrieve +
    forward with the LSE, per call.  At this size the call is launch- and latency-bound; warm is
    queued behind a spin kernel (GPU time), warm_host_launch submitted to an idle GPU."""
    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    shape = I.TINY_FP32
    cfg = gca.Config(B=shape.B, G=shape.G, H=shape.H, n_q=shape.n_q, n_kv=shape.n_kv, topk=shape.topk,
                     dtype="f32", q_chunk_base=shape.q_chunk_base, shift=shape.shift)
    host = I.make_inputs(shape, "f32", seed=0, names=("lq", "lk", "q", "k", "v"))
    d = {n: t.cuda() for n, t in host.items()}
    idx = torch.empty((shape.G, shape.B, shape.n_q, shape.topk), dtype=torch.int32, device="cuda")
    sc = torch.empty_like(idx, dtype=torch.float32)

    def one():
        gca.retrieve(cfg, d["lq"], d["lk"], idx, sc)
        gca.forward(cfg, d["q"], d["k"], d["v"], idx, sc)

    for _ in range(5):
        one()
    torch.cuda.synchronize()
    return {"workload": "GCA retrieve+fwd (with LSE), B=1 L=1024 (16 chunks) H=2 d=64 K=4 G=1, no Gumbel, fp32",
            "warm": _latency(one, iters, _queue_ahead), "warm_host_launch": _latency(one, iters)}


def forward_timing(iters=20):
    """The bf16 forward at the training shape with one retrieval group and no Gumbel noise
    (B=8, L=16384, H=12, K=8, G=1, inputs N(0,1)/8): gca_retrieve + gca_forward without the
    log-sum-exp output, as a forward-only layer call runs it."""
    import numpy as np
    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    shape = I.TRAIN_16K
    cfg = gca.Config(B=shape.B, G=shape.G, H=shape.H, n_q=shape.n_q, n_kv=shape.n_kv, topk=shape.topk,
                     dtype="bf16")
    dev = _device_inputs(shape, seed=11)
    G, B, H, nq, K = shape.G, shape.B, shape.H, shape.n_q, shape.topk
    idx = torch.empty((G, B, nq, K), dtype=torch.int32, device="cuda")
    score = torch.empty((G, B, nq, K), dtype=torch.float32, device="cuda")
    o = torch.empty_like(dev["q"])

    def one():
        gca.retrieve(cfg, dev["lq"], dev["lk"], idx, score)
        gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx, score, need_lse=False, o=o)

    ms, kern = _timed(one, iters)
    used = int((idx.cpu().numpy()[:, :, : nq - 1] >= 0).sum()) * H
    tok = B * nq * 64
    T = tok * H * 64 * 2
    flops = 2 * UNIT_FLOPS * used + 2 * 64 * G * B * nq * (nq - 1) // 2
    # Q, K, V read, O written; landmarks read; indices and scores written then read
    nbytes = 4 * T + G * B * 2 * nq * 64 * 2 + 2 * G * B * nq * K * 8
    floor = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
    res = {"workload": "GCA retrieve+fwd (no LSE), B=8 L=16384 H=12 d=64 K=8 G=1, no Gumbel, bf16, inputs N(0,1)/8",
           "us_per_call": ms * 1e3, "tokens_per_s": tok / (ms * 1e-3), "kernels_us": kern,
           "algorithmic_flops": flops, "algorithmic_bytes": nbytes, "floor_us": floor * 1e6,
           "frac": floor / (ms * 1e-3), "bound": "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (PEAK_BF16_TFLOPS * 1e12) else "mfma"}
    del dev, idx, score, o
    torch.cuda.empty_cache()
    return res


def length_scaling(lengths=(4096, 16384, 65536), tokens=131072, iters=10):
    """Tokens/s of the training step (retrieve + forward + backward, G=2, K=8, Gumbel, bf16) at
    several context lengths with the tokens per batch fixed (B = tokens / L).  The attention work
    per token is at most K chunks whatever L is; the landmark scores grow with the number of
    earlier chunks.  [Notes, Loss / training strategy] states near-linear training cost in the
    context length; this shows how far the step stays linear in L."""
    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    out = {}
    for L in lengths:
        B, C = tokens // L, L // 64
        shape = I.Shape(B=B, G=2, H=12, n_q=C, n_kv=C, topk=8)
        cfg = gca.Config(B=B, G=2, H=12, n_q=C, n_kv=C, topk=8, dtype="bf16", use_gumbel=True, seed=1)
        dev = _device_inputs(shape, seed=21)
        G, H, K = 2, 12, 8
        idx = torch.empty((G, B, C, K), dtype=torch.int32, device="cuda")
        score = torch.empty((G, B, C, K), dtype=torch.float32, device="cuda")
        o = torch.empty_like(dev["q"])
        lse = torch.empty((G, B, H, C, K, 64), dtype=torch.float32, device="cuda")
        grads = (torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"]),
                 torch.empty((G, B, C, K), dtype=torch.float32, device="cuda"))
        n_r = gca.workspace_size(gca.OP_RETRIEVE, cfg)
        ws_r = torch.empty(n_r, dtype=torch.uint8, device="cuda") if n_r else None
        ws_b = torch.empty(gca.workspace_size(gca.OP_BACKWARD, cfg), dtype=torch.uint8, device="cuda")

        def step():
            gca.retrieve(cfg, dev["lq"], dev["lk"], idx, score, ws=ws_r)
            gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx, score, o=o, lse=lse)
            gca.backward(cfg, dev["q"], dev["k"], dev["v"], idx, score, lse, dev["dout"], ws=ws_b, out=grads)

        ms, kern = _timed(step, iters)
        out[str(L)] = {"B": B, "ms_per_step": ms, "tokens_per_s": tokens / (ms * 1e-3), "kernels_us": kern}
        del dev, idx, score, o, lse, grads, ws_r, ws_b
        torch.cuda.empty_cache()
    return out


# Cycles of the spin kernel that holds the GPU before a warm timed step (about 0.2 ms at the
# shader clock): long enough for the host to submit every launch of the step behind it.
QUEUE_AHEAD_CYCLES = 400_000


def _latency(step, iters, before=None):
    """Median, p10 and p90 (us) of `step` between two events on the current stream.  `before`
    runs ahead of each repetition: the 1 GiB flush for cold runs, a short spin kernel for warm
    runs (so the step is queued before the GPU reaches it and the span is GPU time), or nothing,
    which times a step submitted to an idle GPU, host launch time included."""
    import torch

    times = []
    for _ in range(iters):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    times.sort()
    return {"median_us": statistics.median(times), "p10_us": times[len(times) // 10],
            "p90_us": times[(9 * len(times)) // 10]}


def _queue_ahead():
    import torch

    torch.cuda._sleep(QUEUE_AHEAD_CYCLES)


def inference_latency(shape, iters=50):
    """Per-chunk retrieve + attend latency over a long history held in HBM (warm and cold)."""
    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    cfg = gca.Config(B=shape.B, G=shape.G, H=shape.H, n_q=shape.n_q, n_kv=shape.n_kv, topk=shape.topk,
                     dtype="bf16", q_chunk_base=shape.q_chunk_base, shift=shape.shift)
    host = I.make_inputs(shape, "bf16", seed=0, names=("lq", "lk", "q"))
    lq, lk, q = (host[n].cuda() for n in ("lq", "lk", "q"))
    gen = torch.Generator(device="cuda").manual_seed(1234)
    k = torch.randn(shape.tensor_shape("k"), generator=gen, device="cuda", dtype=torch.bfloat16)
    v = torch.randn(shape.tensor_shape("v"), generator=gen, device="cuda", dtype=torch.bfloat16)
    idx = torch.empty((shape.G, shape.B, shape.n_q, shape.topk), dtype=torch.int32, device="cuda")
    sc = torch.empty_like(idx, dtype=torch.float32)
    o = torch.empty_like(q)
    nws = gca.workspace_size(gca.OP_RETRIEVE, cfg)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    # cold runs first read 1 GiB (> the 256 MB MALL): the history leaves the caches, which keep
    # only clean lines (a write would leave dirty lines whose write-back the next step would pay)
    flush = torch.zeros(1 << 27, dtype=torch.int64, device="cuda")

    def one():
        gca.retrieve(cfg, lq, lk, idx, sc, ws=ws if nws else None)
        gca.forward(cfg, q, k, v, idx, sc, need_lse=False, o=o)

    for _ in range(5):
        one()
    torch.cuda.synchronize()
    res = {}
    gca.profile_collect()
    gca.profile_enable(True)
    for _ in range(iters):
        one()
    torch.cuda.synchronize()
    gca.profile_enable(False)
    res["kernels_us"] = {k: v[0] / v[1] * 1e3 for k, v in gca.profile_collect().items()}
    # the same step captured once in a HIP graph and replayed (a serving loop's launch pattern)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        one()
    torch.cuda.synchronize()
    res["warm"] = _latency(one, iters, _queue_ahead)
    res["cold"] = _latency(one, iters, lambda: flush.max())
    res["warm_host_launch"] = _latency(one, iters)
    res["graph_warm"] = _latency(graph.replay, iters, _queue_ahead)
    res["graph_cold"] = _latency(graph.replay, iters, lambda: flush.max())
    # a plain streaming read of the same landmark bytes (torch's max over them as int32 words),
    # warm and cold: what a one-pass read of this size takes on this GPU, launch and drain included
    lk32 = lk.view(torch.int32)
    res["plain_landmark_read"] = {"bytes": lk32.numel() * 4,
                                  "warm": _latency(lambda: lk32.max(), iters, _queue_ahead),
                                  "cold": _latency(lambda: lk32.max(), iters, lambda: flush.max())}
    lmk_bytes = shape.G * shape.B * shape.n_kv * 64 * 2
    gather = shape.G * shape.B * shape.topk * shape.H * 2 * 64 * 64 * 2
    res["hbm_bytes"] = lmk_bytes + gather
    res["hbm_bound_us"] = res["hbm_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e6
    del k, v, flush, graph
    torch.cuda.empty_cache()
    return res


def token_decode_latency(shape, iters=100):
    """Per-token latency of autoregressive decode over a long history held in HBM: one new token
    attends (gca_decode_tokens) to the chunks retrieved once for its chunk; the retrieval itself
    runs once per 64 tokens, so its cost per token is a 64th of the chunk step's."""
    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    cfg = gca.Config(B=shape.B, G=shape.G, H=shape.H, n_q=shape.n_q, n_kv=shape.n_kv, topk=shape.topk,
                     dtype="bf16", q_chunk_base=shape.q_chunk_base, shift=shape.shift)
    host = I.make_inputs(shape, "bf16", seed=0, names=("lq", "lk", "q"))
    lq, lk = host["lq"].cuda(), host["lk"].cuda()
    q1 = host["q"][:, :, :, :1].contiguous().cuda()
    gen = torch.Generator(device="cuda").manual_seed(1234)
    k = torch.randn(shape.tensor_shape("k"), generator=gen, device="cuda", dtype=torch.bfloat16)
    v = torch.randn(shape.tensor_shape("v"), generator=gen, device="cuda", dtype=torch.bfloat16)
    nws = gca.workspace_size(gca.OP_RETRIEVE, cfg)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    idx, sc = gca.retrieve(cfg, lq, lk, ws=ws if nws else None)
    o1 = torch.empty_like(q1)
    flush = torch.zeros(1 << 27, dtype=torch.int64, device="cuda")
    for _ in range(5):
        gca.decode_tokens(cfg, q1, k, v, idx, sc, o=o1)
    torch.cuda.synchronize()
    res = {}
    def tok():
        gca.decode_tokens(cfg, q1, k, v, idx, sc, o=o1)

    res["warm"] = _latency(tok, iters, _queue_ahead)
    res["cold"] = _latency(tok, iters, lambda: flush.max())
    res["warm_host_launch"] = _latency(tok, iters)
    # GPU time per call with the launches queued back to back
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush.max()
    a.record()
    for _ in range(iters):
        gca.decode_tokens(cfg, q1, k, v, idx, sc, o=o1)
    b.record()
    b.synchronize()
    res["back_to_back_us"] = a.elapsed_time(b) * 1e3 / iters
    res["hbm_bytes"] = shape.G * shape.B * shape.topk * shape.H * 2 * 64 * 64 * 2
    res["hbm_bound_us"] = res["hbm_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e6
    del k, v, flush
    torch.cuda.empty_cache()
    return res


def offload_latency(shape, iters=50):
    """Per-chunk latency with the K/V history in pinned host memory (the pages' memory-offload
    inference): retrieve over the device-resident landmarks, fetch the retrieved tiles over the
    host link (gca_fetch_chunks), attend to the fetched tiles."""
    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    cfg = gca.Config(B=shape.B, G=shape.G, H=shape.H, n_q=shape.n_q, n_kv=shape.n_kv, topk=shape.topk,
                     dtype="bf16", q_chunk_base=shape.q_chunk_base, shift=shape.shift)
    fcfg = gca.fetched_config(cfg)
    host = I.make_inputs(shape, "bf16", seed=0, names=("lq", "lk", "q"))
    lq, lk, q = (host[n].cuda() for n in ("lq", "lk", "q"))
    # K/V history in pinned host memory (hipHostMalloc of the exact size: torch's caching pinned
    # allocator rounds a 25.8 GB request up to 32 GiB and keeps it), filled by repeating a seeded
    # 32 MiB random block
    import ctypes

    import numpy as np

    hip = ctypes.CDLL("libamdhip64.so")
    blk = torch.randn(1 << 24, generator=torch.Generator().manual_seed(1234)).to(torch.bfloat16)
    kv, ptrs = [], []
    numel = 1
    for dim in shape.tensor_shape("k"):
        numel *= dim
    for _ in range(2):
        ptr = ctypes.c_void_p()
        if hip.hipHostMalloc(ctypes.byref(ptr), ctypes.c_size_t(2 * numel), ctypes.c_uint(0)) != 0:
            raise RuntimeError(f"hipHostMalloc of {2 * numel} bytes failed")
        ptrs.append(ptr)
        raw = np.ctypeslib.as_array((ctypes.c_int16 * numel).from_address(ptr.value))
        t = torch.from_numpy(raw).view(torch.bfloat16).view(shape.tensor_shape("k"))
        flat = t.view(-1)
        for i in range(0, flat.numel(), blk.numel()):
            n = min(blk.numel(), flat.numel() - i)
            flat[i:i + n].copy_(blk[:n])
        kv.append(t)
    k, v = kv
    idx = torch.empty((shape.G, shape.B, shape.n_q, shape.topk), dtype=torch.int32, device="cuda")
    sc = torch.empty_like(idx, dtype=torch.float32)
    n_c = fcfg.n_kv
    k_c = torch.empty((shape.B, shape.H, n_c * 64, 64), dtype=torch.bfloat16, device="cuda")
    v_c = torch.empty_like(k_c)
    idx_c = torch.empty_like(idx)
    o = torch.empty_like(q)
    nws = gca.workspace_size(gca.OP_RETRIEVE, cfg)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    flush = torch.zeros(1 << 27, dtype=torch.int64, device="cuda")

    def one():
        gca.retrieve(cfg, lq, lk, idx, sc, ws=ws if nws else None)
        gca.fetch_chunks(cfg, idx, k, v, out=(k_c, v_c, idx_c))
        gca.forward(fcfg, q, k_c, v_c, idx_c, sc, need_lse=False, o=o)

    for _ in range(5):
        one()
    torch.cuda.synchronize()
    res = {}
    gca.profile_collect()
    gca.profile_enable(True)
    for _ in range(iters):
        one()
    torch.cuda.synchronize()
    gca.profile_enable(False)
    res["kernels_us"] = {kk: vv[0] / vv[1] * 1e3 for kk, vv in gca.profile_collect().items()}
    res["warm"] = _latency(one, iters, _queue_ahead)
    res["cold"] = _latency(one, iters, lambda: flush.max())
    res["warm_host_launch"] = _latency(one, iters)
    # the host link's rate for a plain 1 GiB DMA copy out of the same pinned history
    dst = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(k.view(-1)[: 1 << 29], non_blocking=True)
    a.record()
    dst.copy_(k.view(-1)[: 1 << 29], non_blocking=True)
    b.record()
    b.synchronize()
    res["host_link_copy_gbs"] = (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9
    res["host_link_bytes"] = shape.G * shape.B * shape.n_q * shape.topk * shape.H * 2 * 64 * 64 * 2
    res["host_link_bound_us"] = res["host_link_bytes"] / (res["host_link_copy_gbs"] * 1e9) * 1e6
    res["hbm_bytes"] = shape.G * shape.B * shape.n_kv * 64 * 2 + 2 * res["host_link_bytes"]
    torch.cuda.synchronize()
    del k, v, kv, t, flat, raw, flush, dst
    for ptr in ptrs:
        hip.hipHostFree(ptr)
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-inference", action="store_true", help="skip the 1M/16M-history latency runs")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-scaling", action="store_true", help="skip the context-length scaling runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the GCA path here runs on a single MI355X with no "
              "sharding or collectives; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_lm_amd import gca
    from long_context_lm_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gca.load()
    shape, cfg, host, dev, bufs, step = training_step_setup()
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the headline: K steps between two events, no per-launch events inside
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tokens = shape.B * shape.n_q * 64
    log(f"step {ms:.3f} ms -> {tokens / (ms * 1e-3) / 1e6:.2f} M tokens/s")
    # per-kernel durations: the same K steps again, each launch between events on its stream
    gca.profile_collect()
    gca.profile_enable(True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    gca.profile_enable(False)
    kern = gca.profile_collect()
    ms_bracketed = start.elapsed_time(end) / args.steps
    log(f"  with per-launch events: {ms_bracketed:.3f} ms per step")
    # spread of single steps (after the timed region, one event pair per step)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in evs)
    spread = None
    if each:
        spread = {"median_ms": statistics.median(each), "p10_ms": each[len(each) // 10],
                  "p90_ms": each[(9 * len(each)) // 10], "steps": len(each)}
        log(f"  single steps: median {spread['median_ms']:.3f} ms, p10 {spread['p10_ms']:.3f}, "
            f"p90 {spread['p90_ms']:.3f}")

    figs = kernel_figures(shape, bufs["idx"].cpu().numpy())
    kernels = {}
    for name, (tot, n) in kern.items():
        avg = tot / max(n, 1)
        kernels[name] = {"avg_ms": avg, "launches": n}
        if name in figs and figs[name]["flops"] + figs[name]["bytes"] > 0:
            r = roofline_for(name, figs[name], avg)
            kernels[name].update({"bound": r["bound"], "frac": r["frac"], "achieved": r["achieved"], "unit": r["unit"]})
    dominant = max(kern.items(), key=lambda kv: kv[1][0])[0]
    roof = roofline_for(dominant, figs[dominant], kern[dominant][0] / kern[dominant][1])
    for k, v in kernels.items():
        log(f"  {k:12s} {v['avg_ms'] * 1e3:9.1f} us  x{v['launches']}"
            + (f"  {v['bound']} {v['frac'] * 100:5.1f}%" if "frac" in v else ""))

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log("measured peaks: plain device copy, bf16 matrix product")
    peaks = measured_peaks()
    log(f"  copy {peaks['hbm_copy_gbs']:.0f} GB/s, bf16 GEMM {peaks['bf16_gemm_tflops']:.0f} TFLOP/s")
    # whole-step position: the forward's and the backward's algorithmic floors against the step
    sr = step_roofline(shape, bufs["idx"].cpu().numpy())
    fl = sr["t"]
    step_floor_us = sr["floor_us"]
    step_floor_measured_us = (fl(sr["forward"], peaks["bf16_gemm_tflops"] * 1e12, peaks["hbm_copy_gbs"] * 1e9)
                              + fl(sr["backward"], peaks["bf16_gemm_tflops"] * 1e12, peaks["hbm_copy_gbs"] * 1e9)) * 1e6
    roof["step_floor_us"] = step_floor_us
    roof["step_frac"] = step_floor_us / (ms * 1e3)
    roof["step_floor_measured_peaks_us"] = step_floor_measured_us
    roof["step_frac_measured_peaks"] = step_floor_measured_us / (ms * 1e3)
    roof["measured_peaks"] = peaks
    if roof["unit"] == "GB/s":
        roof["frac_measured_peak"] = roof["achieved"] / peaks["hbm_copy_gbs"]
    else:
        roof["frac_measured_peak"] = roof["achieved"] / peaks["bf16_gemm_tflops"]
    log(f"  step floor {step_floor_us:.1f} us (vendor peaks) -> step_frac {roof['step_frac']:.3f}; "
        f"{step_floor_measured_us:.1f} us (measured peaks) -> {roof['step_frac_measured_peaks']:.3f}")
    backward_kernels = {}
    for name in ("attend_fwd", "bwd_query", "bwd_key"):
        if name in kern and name in figs:
            backward_kernels[name] = both_ceilings(figs[name], kern[name][0] / kern[name][1], peaks)
            c = backward_kernels[name]
            log(f"  {name:12s} HBM {c['hbm_gbs']:.0f} GB/s ({c['hbm_frac']:.3f}), matrix cores "
                f"{c['mfma_tflops']:.0f} TFLOP/s ({c['mfma_frac']:.3f}), exponentials "
                f"{c.get('exp_per_s', 0) / 1e12:.2f} T/s ({c.get('exp_frac', 0):.3f})")
    # the step against the exponential pipe alone: three passes of one exponential per element
    step_exps = 3 * EXPS_PER_TILE * sr["tiles"]
    roof["step_exps"] = step_exps
    roof["step_exp_floor_us"] = step_exps / PEAK_EXP_PER_S * 1e6
    roof["step_exp_frac"] = roof["step_exp_floor_us"] / (ms * 1e3)
    log(f"  exponentials: {step_exps / 1e9:.2f} G per step, {roof['step_exp_floor_us']:.1f} us at the pipe's "
        f"rate -> {roof['step_exp_frac']:.3f} of the step")

    log("landmark gradients (gca_landmark_backward) on the step's indices and d(score)")
    lmk = landmark_timing(shape, cfg, dev, bufs)
    log(f"  {lmk['us_per_call']:.1f} us per call " + ", ".join(f"{k} {v:.1f}" for k, v in lmk["kernels_us"].items()))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(shape, host)
        log(f"  oracle {cpu['value']:.0f} tokens/s")

    log("training step with a hub chunk in nearly every row's top-k (skewed retrieval)")
    skew = skewed_retrieval_timing(shape, dev, bufs, step)
    log(f"  {skew['ms_per_step']:.3f} ms per step ({skew['tokens_per_s'] / 1e6:.1f} M tokens/s), at most "
        f"{skew['max_entries_per_chunk']} entries per chunk; "
        + ", ".join(f"{k} {v:.1f}" for k, v in skew["kernels_us"].items()))

    infer = None
    del dev, bufs
    torch.cuda.empty_cache()
    log("sliding-window attention beside GCA (W = 512), forward + backward at the training shape")
    sw = window_timing()
    log(f"  {sw['us_per_step']:.1f} us per fwd+bwd ({sw['tokens_per_s'] / 1e6:.1f} M tokens/s); "
        + ", ".join(f"{k} {v:.1f}" for k, v in sw["kernels_us"].items())
        + f"; fwd {sw.get('fwd_tflops', 0):.0f} TFLOP/s, bwd {sw.get('bwd_tflops', 0):.0f} TFLOP/s, "
        f"matrix-core fraction {sw['mfma_frac']:.3f}")
    log("sliding window + GCA in one call (fused) against the separate calls, at the training shape")
    fz = fused_timing()
    log(f"  fused {fz['fused_us']:.1f} us, separate {fz['separate_us']:.1f} us per fwd+bwd; fused: "
        + ", ".join(f"{k} {v:.1f}" for k, v in fz["kernels_us_fused"].items()))
    log("tiny fp32 problem (B=1, L=1024, H=2, K=4): retrieve + forward per call")
    tiny = tiny_forward_latency()
    log(f"  {tiny['warm']['median_us']:.1f} us warm, {tiny['warm_host_launch']['median_us']:.1f} us with the "
        "host's launch")
    log("forward only at the training shape (G=1, no Gumbel, no LSE)")
    fwd = forward_timing()
    log(f"  {fwd['us_per_call']:.1f} us per call ({fwd['tokens_per_s'] / 1e6:.1f} M tokens/s), "
        + ", ".join(f"{k} {v:.1f}" for k, v in fwd["kernels_us"].items())
        + f"; floor {fwd['floor_us']:.1f} us ({fwd['bound']}), frac {fwd['frac']:.3f}")
    scaling = None
    if not args.no_scaling:
        log("context-length scaling of the training step at 131,072 tokens per batch")
        scaling = length_scaling()
        for L, r in scaling.items():
            log(f"  L={L:>6} B={r['B']:>2}: {r['ms_per_step']:.3f} ms, {r['tokens_per_s'] / 1e6:.2f} M tokens/s; "
                + ", ".join(f"{k} {v:.0f}" for k, v in r["kernels_us"].items()))
    if not args.no_inference:
        infer = {}
        for label, shp in (("1M", I.INFER_1M), ("16M", I.INFER_16M)):
            log("inference latency", label)
            infer[label] = inference_latency(shp)
            r = infer[label]
            log(f"  {label}: warm {r['warm']['median_us']:.1f} us, "
                f"cold {r['cold']['median_us']:.1f} us (host launch included: "
                f"{r['warm_host_launch']['median_us']:.1f} us); graph replay warm "
                f"{r['graph_warm']['median_us']:.1f} us, cold {r['graph_cold']['median_us']:.1f} us; "
                + ", ".join(f"{k} {v:.1f}" for k, v in r["kernels_us"].items())
                + f"; plain read of the {r['plain_landmark_read']['bytes'] / 2**20:.0f} MiB of landmarks: warm "
                f"{r['plain_landmark_read']['warm']['median_us']:.1f} us, cold "
                f"{r['plain_landmark_read']['cold']['median_us']:.1f} us")
        log("per-token decode over the 16M history (one token, retrieval reused for the chunk)")
        r = token_decode_latency(I.INFER_16M)
        infer["16M_token"] = r
        tok = r["warm"]["median_us"] + infer["16M"]["warm"]["median_us"] / 64
        r["per_token_with_amortised_chunk_step_us"] = tok
        log(f"  16M_token: warm {r['warm']['median_us']:.1f} us, cold {r['cold']['median_us']:.1f} us, "
            f"back to back {r['back_to_back_us']:.1f} us per call; "
            f"with the chunk step amortised over 64 tokens {tok:.1f} us per token")
        for label, shp in (("1M_host_kv", I.INFER_1M), ("16M_host_kv", I.INFER_16M)):
            log("inference latency, K/V history in pinned host memory", label)
            r = offload_latency(shp)
            infer[label] = r
            log(f"  {label}: warm {r['warm']['median_us']:.1f} us, cold {r['cold']['median_us']:.1f} us; fetch "
                f"{r['kernels_us'].get('fetch_chunks', 0):.1f} us for {r['host_link_bytes'] / 2**20:.1f} MiB "
                f"(host-link copy rate {r['host_link_copy_gbs']:.1f} GB/s -> bound {r['host_link_bound_us']:.1f} us)")

    out = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_with_launch_events": ms_bracketed,
        "step_spread": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GCA retrieve+fwd+bwd, Gumbel top-k, B=8 L=16384 (256 chunks of 64) "
                               "H=12 d=64 K=8 G=2, inputs N(0,1)/8", "global_batch": shape.B,
                   "seq_len": shape.n_q * 64, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "kernel_ceilings": backward_kernels,
        "inference_latency": infer,
        "landmark_backward": lmk,
        "sliding_window": sw,
        "fused_window_gca": fz,
        "skewed_retrieval": skew,
        "forward_only": fwd,
        "tiny_fp32_forward": tiny,
        "length_scaling": scaling,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
