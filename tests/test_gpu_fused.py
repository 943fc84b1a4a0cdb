"""GPU parity of the fused layer attention: sliding window + GCA over the same queries, summed
(gca_fused_forward / gca_fused_backward), against the oracle's fused_attention.

Bars: fp32 max-abs 1e-4, bf16 relative L2 1e-2 (and per 64x64 tile); retrieved indices come from
gca_retrieve and are compared with the oracle's bit for bit.
"""

import numpy as np
import pytest
import torch

from long_context_lm_amd import gca
from long_context_lm_amd import inputs as I
from oracle import gca_oracle as O
from tests.gpu_util import assert_close, assert_tiles_close, config_for, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gca.load()
    yield
    torch.cuda.synchronize()


def _case(shape, dtype, window, seed, scale=1.0, alias=False, hub=False):
    say("case fused", shape, dtype, "window", window, "alias", alias, "hub", hub)
    cfg = config_for(shape, dtype, use_gumbel=True, seed=seed)
    host = I.make_inputs(shape, dtype, seed=seed, scale=scale)
    if hub:
        lq, lk = I.hub_landmarks(shape, seed)
        host["lq"], host["lk"] = I.to_dtype(lq, dtype), I.to_dtype(lk, dtype)
    extra = I.make_inputs(shape, dtype, seed=seed + 1000, scale=scale, names=("k", "v"))
    q = host["q"][0]  # [B, H, L, 64]: the layer's queries (one group)
    dout = host["dout"][0]
    k_sw, v_sw = (host["k"], host["v"]) if alias else (extra["k"], extra["v"])
    d = {n: t.cuda() for n, t in (("q", q), ("k_sw", k_sw), ("v_sw", v_sw), ("k", host["k"]), ("v", host["v"]),
                                  ("dout", dout), ("lq", host["lq"]), ("lk", host["lk"]))}
    idx, sc = gca.retrieve(cfg, d["lq"], d["lk"])
    o, lse_sw, lse = gca.fused_forward(cfg, d["q"], d["k_sw"], d["v_sw"], d["k"], d["v"], idx, sc, window)
    grads = gca.fused_backward(cfg, d["q"], d["k_sw"], d["v_sw"], d["k"], d["v"], idx, sc, o, lse_sw, lse,
                               d["dout"], window)
    torch.cuda.synchronize()
    x = {n: I.as_f64(t) for n, t in (("q", q), ("k_sw", k_sw), ("v_sw", v_sw), ("k", host["k"]), ("v", host["v"]),
                                     ("dout", dout))}
    r_idx, r_sc = O.retrieve(I.as_f64(host["lq"]), I.as_f64(host["lk"]), shape.topk, use_gumbel=True, seed=seed)
    np.testing.assert_array_equal(idx.cpu().numpy(), r_idx)
    np.testing.assert_array_equal(sc.cpu().numpy(), r_sc)
    return cfg, d, (idx, sc), (o, lse_sw, lse, grads), x, (r_idx, r_sc)


def _compare(dtype, got, x, ref_sel, window):
    o, lse_sw, lse, grads = got
    r_idx, r_sc = ref_sel
    r_o, r_lse_sw, r_lse = O.fused_attention(x["q"], x["k_sw"], x["v_sw"], x["k"], x["v"], r_idx, r_sc, window)
    r_g = O.fused_attention_backward(x["q"], x["k_sw"], x["v_sw"], x["k"], x["v"], r_idx, r_sc, x["dout"], window)
    errs = {"o": assert_close("o", I.as_f64(o), r_o, dtype),
            "lse_sw": assert_close("lse_sw", lse_sw.cpu().numpy(), r_lse_sw, dtype)}
    from tests.gpu_util import lse_compare
    errs["lse"] = lse_compare("lse", lse, r_lse, dtype)
    for name, g, r in zip(("dq", "dk_sw", "dv_sw", "dk", "dv", "dscore"), grads, r_g):
        errs[name] = assert_close(name, I.as_f64(g), r, dtype)
        if dtype == "bf16" and name != "dscore":
            assert_tiles_close(name, I.as_f64(g), r)
    if dtype == "bf16":
        assert_tiles_close("o", I.as_f64(o), r_o)
    say("  errors", {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("window,n", [(64, 5), (128, 9), (512, 12), (4096, 7)])
def test_fused_matches_oracle(dtype, window, n):
    """Window shorter than, equal to and longer than the sequence; K = 4 with Gumbel top-k; chunks
    with no retrieval (the first two) and rows with fewer candidates than K."""
    shape = I.Shape(B=2, G=1, H=2, n_q=n, n_kv=n, topk=4)
    _, _, _, got, x, ref_sel = _case(shape, dtype, window, seed=window + n)
    _compare(dtype, got, x, ref_sel, window)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_with_aliased_keys(dtype):
    """k_sw, v_sw the same tensors as the history k, v: the gradient of each is dk_sw + dk."""
    shape = I.Shape(B=1, G=1, H=2, n_q=10, n_kv=10, topk=8)
    _, _, _, got, x, ref_sel = _case(shape, dtype, 192, seed=3, alias=True)
    _compare(dtype, got, x, ref_sel, 192)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_hub_chunk_splits_its_list(dtype):
    """A hub chunk (every query landmark shares the direction of key landmark 0) at n_q = 200, K = 8,
    window 128: chunk 0 is named by nearly all 199 rows that feed a query chunk, so the fused
    backward's key-major pass splits its list into segments of 64.  Against the oracle's fused
    backward, and a second call must give the same bits (the segments' partials are summed in
    segment order whatever order the helper workgroups take them in)."""
    shape = I.Shape(B=1, G=1, H=2, n_q=200, n_kv=200, topk=8)
    cfg, d, (idx, sc), got, x, ref_sel = _case(shape, dtype, 128, seed=23, scale=0.5, hub=True)
    o, lse_sw, lse, grads = got
    again = gca.fused_backward(cfg, d["q"], d["k_sw"], d["v_sw"], d["k"], d["v"], idx, sc, o, lse_sw, lse,
                               d["dout"], 128)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk_sw", "dv_sw", "dk", "dv", "dscore"), grads, again):
        assert torch.equal(a, b), f"{name}: second call differs"
    feeds = ref_sel[0][:, :, : shape.n_q - 1]
    n_hub = int((feeds == 0).sum())
    say(f"  chunk 0 named by {n_hub} backward entries")
    assert n_hub > 128, "the hub list must be split"
    _compare(dtype, got, x, ref_sel, 128)


def test_fused_equals_the_two_separate_calls():
    """The fused forward against gca_sw_forward + gca_forward summed (fp32: within rounding of the
    two sums), the fused backward against gca_sw_backward + gca_backward."""
    shape = I.Shape(B=2, G=1, H=3, n_q=11, n_kv=11, topk=8)
    cfg, d, (idx, sc), (o, lse_sw, lse, grads), x, _ = _case(shape, "f32", 256, seed=9)
    swc = gca.Config(B=2, G=1, H=3, n_q=11, n_kv=11, topk=1, dtype="f32")
    o_sw, l_sw = gca.sw_forward(swc, d["q"], d["k_sw"], d["v_sw"], 256)
    o_g, l_g = gca.forward(cfg, d["q"][None].contiguous(), d["k"], d["v"], idx, sc)
    g_sw = gca.sw_backward(swc, d["q"], d["k_sw"], d["v_sw"], o_sw, l_sw, d["dout"], 256)
    g_g = gca.backward(cfg, d["q"][None].contiguous(), d["k"], d["v"], idx, sc, l_g, d["dout"][None].contiguous())
    torch.cuda.synchronize()
    torch.testing.assert_close(o, o_sw + o_g[0], rtol=0, atol=2e-6)
    assert torch.equal(lse_sw, l_sw)
    # (at this size gca_forward runs its decode-size kernel, which sums in another order)
    torch.testing.assert_close(lse, l_g, rtol=0, atol=1e-6)
    torch.testing.assert_close(grads[0], g_sw[0] + g_g[0][0], rtol=0, atol=2e-5)
    for a, b in ((grads[1], g_sw[1]), (grads[2], g_sw[2]), (grads[3], g_g[1]), (grads[4], g_g[2])):
        torch.testing.assert_close(a, b, rtol=0, atol=2e-5)
    torch.testing.assert_close(grads[5], g_g[3], rtol=0, atol=1e-5)


def test_fused_is_deterministic():
    shape = I.Shape(B=1, G=1, H=2, n_q=9, n_kv=9, topk=4)
    cfg, d, (idx, sc), first, _, _ = _case(shape, "bf16", 128, seed=4)
    o, lse_sw, lse = gca.fused_forward(cfg, d["q"], d["k_sw"], d["v_sw"], d["k"], d["v"], idx, sc, 128)
    g = gca.fused_backward(cfg, d["q"], d["k_sw"], d["v_sw"], d["k"], d["v"], idx, sc, o, lse_sw, lse, d["dout"], 128)
    torch.cuda.synchronize()
    for a, b in zip((o, lse_sw, lse, *g), (first[0], first[1], first[2], *first[3])):
        assert torch.equal(a, b)


@pytest.mark.timeout(600)
def test_fused_training_shape_against_separate_calls():
    """B=8, L=16384, H=12, W=512, K=8, one group, bf16 inputs N(0,1)/8 (the layer at the training
    shape): the fused calls against the two separate calls, which the other parity tests pin to the
    oracle; relative L2 1e-2 per tensor and per tile."""
    shape = I.Shape(B=8, G=1, H=12, n_q=256, n_kv=256, topk=8)
    cfg = config_for(shape, "bf16", use_gumbel=True, seed=1)
    gen = torch.Generator(device="cuda").manual_seed(5)
    mk = lambda s: (torch.randn(s, generator=gen, device="cuda") / 8).to(torch.bfloat16)
    L = 256 * 64
    q, k_sw, v_sw, k, v, dout = (mk((8, 12, L, 64)) for _ in range(6))
    lq, lk = mk((1, 8, 256, 64)), mk((1, 8, 256, 64))
    idx, sc = gca.retrieve(cfg, lq, lk)
    o, lse_sw, lse = gca.fused_forward(cfg, q, k_sw, v_sw, k, v, idx, sc, 512)
    grads = gca.fused_backward(cfg, q, k_sw, v_sw, k, v, idx, sc, o, lse_sw, lse, dout, 512)
    swc = gca.Config(B=8, G=1, H=12, n_q=256, n_kv=256, topk=1, dtype="bf16")
    o_sw, l_sw = gca.sw_forward(swc, q, k_sw, v_sw, 512)
    o_g, l_g = gca.forward(cfg, q[None], k, v, idx, sc)
    g_sw = gca.sw_backward(swc, q, k_sw, v_sw, o_sw, l_sw, dout, 512)
    g_g = gca.backward(cfg, q[None], k, v, idx, sc, l_g, dout[None])
    torch.cuda.synchronize()
    refs = {"o": o_sw.double() + o_g[0].double(), "dq": g_sw[0].double() + g_g[0][0].double(),
            "dk_sw": g_sw[1].double(), "dv_sw": g_sw[2].double(), "dk": g_g[1].double(), "dv": g_g[2].double()}
    gots = {"o": o, "dq": grads[0], "dk_sw": grads[1], "dv_sw": grads[2], "dk": grads[3], "dv": grads[4]}
    for name in refs:
        for b in (0, 7):
            g = gots[name][b].double().cpu().numpy()
            r = refs[name][b].cpu().numpy()
            assert_close(f"{name}[b={b}]", g, r, "bf16")
            assert_tiles_close(f"{name}[b={b}]", g, r)
    assert torch.equal(lse_sw, l_sw)
    torch.testing.assert_close(grads[5], g_g[3], rtol=2e-2, atol=2e-3)
