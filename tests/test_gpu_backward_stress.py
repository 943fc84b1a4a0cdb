"""GPU parity of the backward under retrieval skew and with caller-built indices.

A hub chunk: when every retrieval row's query landmark shares a direction with one key landmark,
that chunk enters the top-k of nearly every row [Notes, Key designs: causal retrieval: the top-k
runs over all earlier chunks, so one salient chunk can be selected by many rows].  Its key-side
sums then run over the longest entry lists the inverse retrieval index can hold: here more than
512 (group, row, slot) entries, which the landmark key pass walks in more than eight 64-entry
pieces.

The key-major pass splits a list longer than 128 entries into segments of 64 that separate
workgroups walk (here more than eight), and sums their partials in segment order; the hub's list
takes that path, and its result must not change from one call to the next.

Caller-built indices: gca_forward and gca_backward count every slot with 0 <= idx < n_kv, also
chunks at or after the row's own chunk (a caller's own selection, or the compact buffers of
gca_fetch_chunks).  The key-major pass must then include the same slots as the query-major pass.
"""

import numpy as np
import pytest
import torch

from long_context_lm_amd import gca
from long_context_lm_amd import inputs as I
from oracle import gca_oracle as O
from tests.gpu_util import assert_close, assert_tiles_close, config_for, lse_compare, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gca.load()
    yield
    torch.cuda.synchronize()


def _hub_inputs(shape, dtype, seed):
    """Seeded inputs with key landmark 0 of every (group, batch row) pointing along a direction
    that every query landmark shares: s_i0 is about 8 against about N(0, 1) for the rest.  q and k
    are N(0, 1) (sharp per-chunk softmaxes); v and dout are N(0, 1)/4, so that the hub's dk and
    dv, sums over about 600 entries, stay near 1 and 6 and the absolute float32 bar of 1e-4 sits
    above float32 resolution at their magnitude (with unit v and dout |dv| reaches about 24)."""
    host = I.make_inputs(shape, dtype, seed=seed, scale=1.0)
    quarter = I.make_inputs(shape, dtype, seed=seed, scale=0.25, names=("v", "dout"))
    host["v"], host["dout"] = quarter["v"], quarter["dout"]
    lq, lk = I.hub_landmarks(shape, seed)
    host["lq"] = I.to_dtype(lq, dtype)
    host["lk"] = I.to_dtype(lk, dtype)
    return host


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hub_chunk_backward_and_landmarks(dtype):
    """G=2, n_q=n_kv=300, K=8, Gumbel: chunk 0 is named by more than 512 entries of its batch row's
    inverse index.  dq, dk, dv, d(score) against the oracle backward and the landmark gradients
    against the oracle's; fp32 within max-abs 1e-4, bf16 within relative L2 1e-2 (and per tile)."""
    shape = I.Shape(B=1, G=2, H=2, n_q=300, n_kv=300, topk=8)
    cfg = config_for(shape, dtype, use_gumbel=True, seed=21)
    say("case hub", shape, dtype)
    host = _hub_inputs(shape, dtype, seed=13)
    x = {k: I.as_f64(v) for k, v in host.items()}
    dev = upload(host)
    idx, sc = gca.retrieve(cfg, dev["lq"], dev["lk"])
    o, lse = gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx, sc)
    dq, dk, dv, ds = gca.backward(cfg, dev["q"], dev["k"], dev["v"], idx, sc, lse, dev["dout"])
    dlq, dlk = gca.landmark_backward(cfg, dev["lq"], dev["lk"], idx, ds)
    # the hub's list is split over several key-major workgroups (segments placed by an atomic
    # counter whose order varies): a second call must still give the same bits
    again = gca.backward(cfg, dev["q"], dev["k"], dev["v"], idx, sc, lse, dev["dout"])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dscore"), (dq, dk, dv, ds), again):
        assert torch.equal(a, b), f"{name}: second call differs"
    say("  gpu done; running oracle")
    r_idx, r_sc = O.retrieve(x["lq"], x["lk"], 8, use_gumbel=True, seed=21)
    np.testing.assert_array_equal(idx.cpu().numpy(), r_idx)
    np.testing.assert_array_equal(sc.cpu().numpy(), r_sc)
    # entries of chunk 0 in the backward's index (rows that feed a query chunk) and the landmark one
    feeds = r_idx[:, :, : shape.n_q - 1]
    n_bwd, n_lmk = int((feeds == 0).sum()), int((r_idx == 0).sum())
    say(f"  chunk 0 named by {n_bwd} backward entries, {n_lmk} landmark entries")
    assert n_bwd > 512 and n_lmk > 512, "the hub list must exceed eight segments and eight landmark pieces"
    r_o, r_lse = O.forward(x["q"], x["k"], x["v"], r_idx, r_sc)
    r_g = O.backward(x["q"], x["k"], x["v"], r_idx, r_sc, x["dout"])
    errs = {"o": assert_close("o", I.as_f64(o), r_o, dtype), "lse": lse_compare("lse", lse, r_lse, dtype)}
    for name, got, ref in zip(("dq", "dk", "dv", "dscore"), (dq, dk, dv, ds), r_g):
        errs[name] = assert_close(name, I.as_f64(got), ref, dtype)
        if dtype == "bf16" and name != "dscore":
            assert_tiles_close(name, I.as_f64(got), ref)
    # the hub tile itself, on its own (it is one tile of 300 per head)
    for name, got, ref in (("dk", dk, r_g[1]), ("dv", dv, r_g[2])):
        assert_close(f"{name}[chunk 0]", I.as_f64(got)[:, :, :64], ref[:, :, :64], dtype)
    r_dlq, r_dlk = O.landmark_backward(x["lq"], x["lk"], r_idx, ds.cpu().numpy().astype(np.float64))
    errs["dlq"] = assert_close("dlq", I.as_f64(dlq), r_dlq, dtype)
    errs["dlk"] = assert_close("dlk", I.as_f64(dlk), r_dlk, dtype)
    errs["dlk0"] = assert_close("dlk[chunk 0]", I.as_f64(dlk)[:, :, 0], r_dlk[:, :, 0], dtype)
    say("  errors", {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_caller_indices_at_or_after_the_row(dtype):
    """idx chosen by the caller, not by gca_retrieve: distinct chunks drawn from all of [0, n_kv),
    so rows name chunks at or after their own (and, with n_kv = 100, chunks of the second 64-chunk
    block from rows below 64), plus invalid slots.  The forward uses every slot with
    0 <= idx < n_kv; the backward's dq, dk, dv and d(score) must count exactly those slots."""
    shape = I.Shape(B=2, G=2, H=2, n_q=80, n_kv=100, topk=4)
    cfg = config_for(shape, dtype)
    say("case caller idx", shape, dtype)
    host = I.make_inputs(shape, dtype, seed=31, scale=1.0, names=("q", "k", "v", "dout"))
    rng = np.random.default_rng(31)
    idx = np.full((2, 2, 80, 4), -1, dtype=np.int32)
    for g in range(2):
        for b in range(2):
            for r in range(80):
                n = int(rng.integers(0, 5))  # 0..4 valid slots
                idx[g, b, r, :n] = rng.choice(100, size=n, replace=False)
    idx[0, 0, 5] = [99, 64, 70, -1]  # row 5 (global chunk 5) naming only later chunks
    score = np.where(idx >= 0, rng.standard_normal(idx.shape), -np.inf).astype(np.float32)
    x = {k: I.as_f64(v) for k, v in host.items()}
    dev = upload(host)
    idx_t = torch.from_numpy(idx).cuda()
    sc_t = torch.from_numpy(score).cuda()
    o, lse = gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx_t, sc_t)
    grads = gca.backward(cfg, dev["q"], dev["k"], dev["v"], idx_t, sc_t, lse, dev["dout"])
    torch.cuda.synchronize()
    r_o, r_lse = O.forward(x["q"], x["k"], x["v"], idx, score)
    r_g = O.backward(x["q"], x["k"], x["v"], idx, score, x["dout"])
    assert_close("o", I.as_f64(o), r_o, dtype)
    lse_compare("lse", lse, r_lse, dtype)
    for name, got, ref in zip(("dq", "dk", "dv", "dscore"), grads, r_g):
        assert_close(name, I.as_f64(got), ref, dtype)
    # chunks 64..99 are only reachable through rows below 64 and through later rows alike
    assert_close("dk[chunks 64..99]", I.as_f64(grads[1])[:, :, 64 * 64:], r_g[1][:, :, 64 * 64:], dtype)
    assert_close("dv[chunks 64..99]", I.as_f64(grads[2])[:, :, 64 * 64:], r_g[2][:, :, 64 * 64:], dtype)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_lists_odd_shapes(dtype):
    """Three groups, three batch rows, K = 16, a history longer than the query chunks, and a hub
    chunk named by more than 128 entries (G (n_q - 1) = 147): its list is split into three
    segments of at most 64, while the other chunks' lists are walked whole.  Against the oracle
    backward, and a second call must give the same bits."""
    shape = I.Shape(B=3, G=3, H=2, n_q=50, n_kv=60, topk=16)
    cfg = config_for(shape, dtype, use_gumbel=True, seed=7)
    say("case split lists", shape, dtype)
    host = _hub_inputs(shape, dtype, seed=17)
    x = {k: I.as_f64(v) for k, v in host.items()}
    dev = upload(host)
    idx, sc = gca.retrieve(cfg, dev["lq"], dev["lk"])
    o, lse = gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx, sc)
    grads = gca.backward(cfg, dev["q"], dev["k"], dev["v"], idx, sc, lse, dev["dout"])
    again = gca.backward(cfg, dev["q"], dev["k"], dev["v"], idx, sc, lse, dev["dout"])
    torch.cuda.synchronize()
    r_idx, r_sc = O.retrieve(x["lq"], x["lk"], 16, use_gumbel=True, seed=7)
    np.testing.assert_array_equal(idx.cpu().numpy(), r_idx)
    feeds = r_idx[:, :, : shape.n_q - 1]
    longest = max(int((feeds[:, b] == j).sum()) for b in range(shape.B) for j in range(shape.n_kv))
    say(f"  longest list {longest} entries")
    assert longest > 128, "a list must be split"
    r_g = O.backward(x["q"], x["k"], x["v"], r_idx, r_sc, x["dout"])
    for name, got, ref, rep in zip(("dq", "dk", "dv", "dscore"), grads, r_g, again):
        assert torch.equal(got, rep), f"{name}: second call differs"
        assert_close(name, I.as_f64(got), ref, dtype)
        if dtype == "bf16" and name in ("dk", "dv"):
            assert_tiles_close(name, I.as_f64(got), ref)
