"""GPU parity of sliding-window attention (gca_sw_forward / gca_sw_backward) against the oracle.

Bars: fp32 max-abs <= 1e-4, bf16 relative L2 <= 1e-2 for o, lse and the gradients.  Sizes:
sequences of 1, 3 and 11 chunks with windows of one chunk, two chunks, 512 tokens and longer than
the sequence (causal attention), then the 16K training shape (B=8, L=16384, H=12, W=512) on
sampled tokens the oracle computes one by one.
"""

import dataclasses

import numpy as np
import pytest
import torch

from long_context_lm_amd import gca
from oracle import gca_oracle as O
from tests.gpu_util import assert_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gca.load()
    yield
    torch.cuda.synchronize()


def _inputs(B, H, n_c, seed, scale=1.0, dtype="bf16"):
    g = torch.Generator().manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [(scale * torch.randn((B, H, 64 * n_c, 64), generator=g)).to(tdt) for _ in range(4)]


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_c", [1, 3, 11])
@pytest.mark.parametrize("window", [64, 128, 512, 4096])
def test_sw_forward_matches_oracle(n_c, window, dtype):
    say("case sw forward", n_c, window, dtype)
    q, k, v, _ = _inputs(2, 3, n_c, seed=n_c * 7 + window, dtype=dtype)
    cfg = dataclasses.replace(gca.sw_config(2, 3, n_c), dtype=dtype)
    o, lse = gca.sw_forward(cfg, q.cuda(), k.cuda(), v.cuda(), window)
    torch.cuda.synchronize()
    ro, rl = O.sw_attention(_f64(q), _f64(k), _f64(v), window)
    e1 = assert_close("o", _f64(o), ro, dtype)
    e2 = assert_close("lse", _f64(lse), rl, dtype)
    assert np.max(np.abs(_f64(lse) - rl)) < (2e-3 if dtype == "bf16" else 1e-4)
    say("  errors", f"o {e1:.2e} lse {e2:.2e}")


def test_sw_forward_training_shape_sampled():
    B, H, n_c, W = 8, 12, 256, 512
    say("case sw forward 16K", B, H, n_c, W)
    q, k, v, _ = _inputs(B, H, n_c, seed=3)
    cfg = gca.sw_config(B, H, n_c)
    o, lse = gca.sw_forward(cfg, q.cuda(), k.cuda(), v.cuda(), W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    toks = np.concatenate([[0, 1, 63, 64, 511, 512, 513, 16383], rng.integers(0, 64 * n_c, 24)])
    got, ref = [], []
    for i in toks:
        b, h = rng.integers(0, B), rng.integers(0, H)
        lo = max(0, i - W + 1)
        ro, rl = O.sw_attention(_f64(q[b:b + 1, h:h + 1, lo:i + 1]), _f64(k[b:b + 1, h:h + 1, lo:i + 1]),
                                _f64(v[b:b + 1, h:h + 1, lo:i + 1]), W)
        got.append(_f64(o[b, h, i]))
        ref.append(ro[0, 0, -1])
        assert abs(float(lse[b, h, i]) - rl[0, 0, -1]) < 2e-3
    assert_close("o sampled", np.array(got), np.array(ref), "bf16")


def _sw_grads(B, H, n_c, window, seed, dtype="bf16"):
    q, k, v, do = _inputs(B, H, n_c, seed=seed, dtype=dtype)
    dev = [t.cuda() for t in (q, k, v, do)]
    cfg = dataclasses.replace(gca.sw_config(B, H, n_c), dtype=dtype)
    o, lse = gca.sw_forward(cfg, *dev[:3], window)
    dq, dk, dv = gca.sw_backward(cfg, *dev[:3], o, lse, dev[3], window)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_c", [1, 3, 11])
@pytest.mark.parametrize("window", [64, 128, 512, 4096])
def test_sw_backward_matches_oracle(n_c, window, dtype):
    say("case sw backward", n_c, window, dtype)
    (q, k, v, do), got = _sw_grads(2, 3, n_c, window, seed=n_c * 5 + window, dtype=dtype)
    ref = O.sw_attention_backward(_f64(q), _f64(k), _f64(v), _f64(do), window)
    errs = [assert_close(name, _f64(g), r, dtype) for name, g, r in zip(("dq", "dk", "dv"), got, ref)]
    say("  errors", " ".join(f"{e:.2e}" for e in errs))


def test_sw_backward_is_deterministic():
    _, a = _sw_grads(2, 2, 12, 512, seed=1)
    _, b = _sw_grads(2, 2, 12, 512, seed=1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_sw_backward_training_shape_sampled():
    B, H, n_c, W = 8, 12, 256, 512
    say("case sw backward 16K", B, H, n_c, W)
    (q, k, v, do), (dq, dk, dv) = _sw_grads(B, H, n_c, W, seed=4)
    rng = np.random.default_rng(1)
    L = 64 * n_c
    got, ref = {n: [] for n in ("dq", "dk", "dv")}, {n: [] for n in ("dq", "dk", "dv")}
    for pos in np.concatenate([[0, 63, 64, 511, 512, L - 1], rng.integers(0, L, 6)]):
        b, h = rng.integers(0, B), rng.integers(0, H)
        lo, hi = max(0, pos - W + 1), min(L, pos + W)  # every query and key that reaches pos
        sl = (slice(b, b + 1), slice(h, h + 1), slice(lo, hi))
        r = O.sw_attention_backward(_f64(q[sl]), _f64(k[sl]), _f64(v[sl]), _f64(do[sl]), W)
        for n, g, rr in zip(("dq", "dk", "dv"), (dq, dk, dv), r):
            got[n].append(_f64(g[b, h, pos]))
            ref[n].append(rr[0, 0, pos - lo])
    for n in got:
        assert_close(n + " sampled", np.array(got[n]), np.array(ref[n]), "bf16")


def _membership_inputs(B, H, n_c):
    """k = 0 makes every score 0, so P is uniform over each token's window; v[j] = one-hot of
    j mod 64 then makes o[i] the histogram (by residue) of the keys in token i's window."""
    L = 64 * n_c
    q = torch.randn((B, H, L, 64), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    k = torch.zeros((B, H, L, 64), dtype=torch.bfloat16)
    v = torch.zeros((B, H, L, 64), dtype=torch.bfloat16)
    v[:, :, torch.arange(L), torch.arange(L) % 64] = 1.0
    return q, k, v


@pytest.mark.parametrize("window", [64, 128, 512])
def test_sw_window_membership_is_exact(window):
    """Which keys every token attends to, checked bit for bit: for tokens with a full window,
    P = 1/W is exact in bf16 and o[i, d] = #{j in (i - W, i] : j = d mod 64} / W; in the backward
    with dO one-hot, dq is exactly 0 (k = 0) and dv[j, d] = #{i in [j, j + W) : i = d mod 64,
    i < L} / W for keys whose covering queries all have full windows."""
    B, H, n_c = 1, 2, 11
    L = 64 * n_c
    say("case window membership", window)
    q, k, v = _membership_inputs(B, H, n_c)
    cfg = gca.sw_config(B, H, n_c)
    o, lse = gca.sw_forward(cfg, q.cuda(), k.cuda(), v.cuda(), window)
    dout = torch.zeros((B, H, L, 64), dtype=torch.bfloat16)
    dout[:, :, torch.arange(L), torch.arange(L) % 64] = float(window)
    dq, dk, dv = gca.sw_backward(cfg, q.cuda(), k.cuda(), v.cuda(), o, lse, dout.cuda(), window)
    torch.cuda.synchronize()
    o, dq, dv = _f64(o), _f64(dq), _f64(dv)
    i = np.arange(L)
    for tok in range(window - 1, L):
        keys = np.arange(tok - window + 1, tok + 1)
        expect = np.bincount(keys % 64, minlength=64) / window
        assert np.array_equal(o[0, 0, tok], expect) and np.array_equal(o[0, 1, tok], expect), f"o, token {tok}"
    assert not dq.any(), "dq must be exactly zero when k = 0"
    for j in range(window - 1, L):
        qs = i[(i >= j) & (i < j + window)]
        expect = np.bincount(qs % 64, minlength=64).astype(np.float64)
        assert np.array_equal(dv[0, 0, j], expect), f"dv, key {j}"
