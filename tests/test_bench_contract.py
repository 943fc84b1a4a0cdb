"""The benchmark's command-line contract, checked on the CPU (no GPU needed).

bench.py measures one GPU: asked for more it must exit with an explanation before touching a
device, and its helpers that compute the reported algorithmic figures must count what the
method does (valid slots of the causal retrieval, the 64x64x64 products per slot).
"""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_kernel_figures_count_valid_slots():
    sys.path.insert(0, ROOT)
    import bench
    from long_context_lm_amd import inputs as I

    shape = I.Shape(B=2, G=2, H=3, n_q=16, n_kv=16, topk=4)
    # row r has min(r, K) valid slots (strictly earlier chunks); rows feed query chunk r + 1
    idx = np.full((2, 2, 16, 4), -1, dtype=np.int32)
    for r in range(16):
        idx[:, :, r, : min(r, 4)] = 0
    figs = bench.kernel_figures(shape, idx)
    per_row = sum(min(r, 4) for r in range(15))  # the last row feeds no query chunk
    tiles = 2 * 2 * per_row * 3
    assert figs["attend_fwd"]["tiles"] == tiles
    assert figs["attend_fwd"]["flops"] == 2 * 2 * 64 ** 3 * tiles
    assert figs["bwd_key"]["flops"] == figs["bwd_query"]["flops"] == figs["attend_fwd"]["flops"]
    # causal landmark pairs: G * B * sum_i i
    assert figs["score_topk"]["flops"] == 2 * 64 * 2 * 2 * (16 * 15 // 2)


def test_step_roofline_at_the_16k_training_shape():
    """The step floor: forward at its HBM time (Q, K, V, O, LSE) plus backward at its matrix-core
    time (four 64x64x64 products per tile) = 163.6 + 322.8 us at the 16K, G=2 shape, where every
    (group, batch row) has sum_c min(c - 1, 8) = 2004 valid (chunk, slot) pairs."""
    sys.path.insert(0, ROOT)
    import bench
    from long_context_lm_amd import inputs as I

    shape = I.TRAIN_16K_G2
    idx = np.full((2, 8, 256, 8), -1, dtype=np.int32)
    for r in range(256):
        idx[:, :, r, : min(r, 8)] = 0
    sr = bench.step_roofline(shape, idx)
    assert sr["tiles"] == 2 * 8 * 2004 * 12 == 384_768
    T = 8 * 16384 * 12 * 64 * 2
    lse = 2 * 8 * 16384 * 12 * 8 * 4
    assert sr["forward"]["bytes"] == 6 * T + lse + 2 * 8 * 256 * 8 * 8
    assert sr["backward"]["flops"] == 4 * 2 * 64 ** 3 * 384_768
    fwd_us = sr["forward"]["bytes"] / 8e12 * 1e6
    bwd_us = sr["backward"]["flops"] / 2.5e15 * 1e6
    assert abs(fwd_us - 163.6) < 0.1 and abs(bwd_us - 322.8) < 0.1
    assert abs(sr["floor_us"] - (fwd_us + bwd_us)) < 1e-6


def test_profile_hash_ignores_comments_but_not_code():
    """The profiles record a hash of the kernel sources; the bench reports their HBM traffic only
    while it matches.  Comments and layout do not change the kernels, so they must not change the
    hash; any code change must."""
    from long_context_lm_amd import profiling as P

    src = "int f(int a) {  // the sum\n  return a + 1; /* one\n more */\n}\n"
    assert P.code_text(src) == P.code_text("int f(int a) {\n return a + 1;  // changed note\n}")
    assert P.code_text(src) != P.code_text("int f(int a) { return a + 2; }")
    assert "//" not in P.code_text(src) and "/*" not in P.code_text(src)
    h = P.source_hash()
    assert len(h) == 16 and h == P.source_hash()
    for f in P.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(P.HERE, f)), f
