"""GPU parity of the landmark gradients (gca_landmark_backward) against the CPU oracle.

Bars: fp32 max-abs <= 1e-4, bf16 relative L2 <= 1e-2; bit-identical results from run to run;
exact zeros for chunks no slot selected.  Indices come from the oracle's retrieval (so the kernel
is tested on its own) and, in the chained case, from the GPU path itself.
"""

import numpy as np
import pytest
import torch

from long_context_lm_amd import gca
from long_context_lm_amd import inputs as I
from oracle import gca_oracle as O
from tests.gpu_util import assert_close, config_for, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gca.load()
    yield
    torch.cuda.synchronize()


def _case(shape, dtype, seed):
    host = I.make_inputs(shape, dtype, seed=seed, scale=0.125, names=("lq", "lk"))
    lq, lk = I.as_f64(host["lq"]), I.as_f64(host["lk"])
    idx, _ = O.retrieve(lq, lk, shape.topk, q_chunk_base=shape.q_chunk_base, n_kv=shape.n_kv)
    rng = np.random.default_rng(seed + 7)
    ds = np.where(idx >= 0, rng.standard_normal(idx.shape), 0.0).astype(np.float32)
    return host, lq, lk, idx, ds


def _run(shape, dtype, seed):
    say("case", shape, dtype)
    host, lq, lk, idx, ds = _case(shape, dtype, seed)
    cfg = config_for(shape, dtype)
    dev = upload(host)
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda()
    ds_d = torch.from_numpy(ds).cuda()
    dlq, dlk = gca.landmark_backward(cfg, dev["lq"], dev["lk"], idx_d, ds_d)
    torch.cuda.synchronize()
    r_dlq, r_dlk = O.landmark_backward(lq, lk, idx, ds, q_chunk_base=shape.q_chunk_base, n_kv=shape.n_kv)
    e1 = assert_close("dlq", I.as_f64(dlq), r_dlq, dtype)
    e2 = assert_close("dlk", I.as_f64(dlk), r_dlk, dtype)
    # chunks that no slot selected get exact zeros
    got = I.as_f64(dlk)
    for g, b in np.ndindex(shape.G, shape.B):
        used = np.zeros(shape.n_kv, dtype=bool)
        sel = idx[g, b][idx[g, b] >= 0]
        used[sel] = True
        assert np.all(got[g, b][~used] == 0), "unselected chunks must get zero gradients"
    say("  errors", f"dlq {e1:.2e} dlk {e2:.2e}")
    return cfg, dev, idx_d, ds_d, dlq, dlk


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_landmark_gradients_small(dtype):
    _run(I.Shape(B=2, G=2, H=1, n_q=37, n_kv=37, topk=8), dtype, seed=1)


def test_landmark_gradients_offsets_and_topk16():
    _run(I.Shape(B=1, G=3, H=1, n_q=20, n_kv=30, topk=16, q_chunk_base=12, shift=0), "f32", seed=2)


def test_landmark_gradients_16k_training_shape():
    """B=8, 256 chunks of 64, G=2, K=8: every output row compared."""
    _run(I.Shape(B=8, G=2, H=12, n_q=256, n_kv=256, topk=8), "bf16", seed=3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_landmark_gradients_64k_context(dtype):
    """1,024 chunks per sequence (the 64K step of the context-length sweep, B=2, G=2): rows of up
    to 1,023 candidates and early key chunks named by many rows (long inverse-index walks)."""
    _run(I.Shape(B=2, G=2, H=12, n_q=1024, n_kv=1024, topk=8), dtype, seed=6)


def test_landmark_gradients_decode_long_history():
    """One retrieval row over a 5,000-chunk history: nearly every key chunk gets zero."""
    _run(I.Shape(B=1, G=2, H=12, n_q=1, n_kv=5000, topk=8, q_chunk_base=5000, shift=0), "bf16", seed=4)


def test_landmark_gradients_deterministic():
    cfg, dev, idx_d, ds_d, dlq, dlk = _run(I.Shape(B=2, G=2, H=1, n_q=64, n_kv=64, topk=8), "bf16", seed=5)
    dlq2, dlk2 = gca.landmark_backward(cfg, dev["lq"], dev["lk"], idx_d, ds_d)
    torch.cuda.synchronize()
    assert torch.equal(dlq, dlq2) and torch.equal(dlk, dlk2)


def test_landmark_gradients_empty_sides():
    # no retrieval rows: every key landmark gets zero
    shape = I.Shape(B=1, G=2, H=1, n_q=0, n_kv=9, topk=4)
    cfg = config_for(shape, "f32")
    lk = torch.randn(2, 1, 9, 64, device="cuda")
    dlk = torch.full_like(lk, 7.0)
    empty = torch.empty(2, 1, 0, 64, device="cuda")
    gca.landmark_backward(cfg, empty, lk, torch.empty(2, 1, 0, 4, dtype=torch.int32, device="cuda"),
                          torch.empty(2, 1, 0, 4, device="cuda"), out=(torch.empty_like(empty), dlk))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dlk).item() == 0
    # no history: every query landmark gets zero
    shape = I.Shape(B=1, G=1, H=1, n_q=3, n_kv=0, topk=4)
    cfg = config_for(shape, "f32")
    lq = torch.randn(1, 1, 3, 64, device="cuda")
    dlq = torch.full_like(lq, 7.0)
    idx = torch.full((1, 1, 3, 4), -1, dtype=torch.int32, device="cuda")
    gca.landmark_backward(cfg, lq, torch.empty(1, 1, 0, 64, device="cuda"), idx, torch.zeros(1, 1, 3, 4, device="cuda"),
                          out=(dlq, torch.empty(1, 1, 0, 64, device="cuda")))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dlq).item() == 0


def test_landmark_gradients_chained_with_the_gpu_backward():
    """retrieve -> forward -> backward -> landmark gradients on the GPU, against the oracle chain."""
    shape = I.Shape(B=2, G=2, H=3, n_q=21, n_kv=21, topk=8)
    cfg = config_for(shape, "bf16", use_gumbel=True, seed=5)
    host = I.make_inputs(shape, "bf16", seed=8, scale=0.125)
    x = {k: I.as_f64(v) for k, v in host.items()}
    dev = upload(host)
    idx, sc = gca.retrieve(cfg, dev["lq"], dev["lk"])
    o, lse = gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx, sc)
    _, _, _, ds = gca.backward(cfg, dev["q"], dev["k"], dev["v"], idx, sc, lse, dev["dout"])
    dlq, dlk = gca.landmark_backward(cfg, dev["lq"], dev["lk"], idx, ds)
    torch.cuda.synchronize()
    r_idx, r_sc = O.retrieve(x["lq"], x["lk"], 8, use_gumbel=True, seed=5)
    np.testing.assert_array_equal(idx.cpu().numpy(), r_idx)
    _, _, _, r_ds = O.backward(x["q"], x["k"], x["v"], r_idx, r_sc, x["dout"], shift=1)
    r_dlq, r_dlk = O.landmark_backward(x["lq"], x["lk"], r_idx, r_ds)
    assert_close("dlq", I.as_f64(dlq), r_dlq, "bf16")
    assert_close("dlk", I.as_f64(dlk), r_dlk, "bf16")
