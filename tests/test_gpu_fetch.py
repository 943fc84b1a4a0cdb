"""GPU parity of the fetch of retrieved chunks (gca_fetch_chunks) against the CPU oracle.

The fetch is byte work: tiles and remapped indices must match the oracle's gather exactly, from
device memory and from pinned host memory alike.  Attention over the fetched tiles must be
bit-identical to attention over the whole history (the same kernels see the same tile values).
Indices come from the GPU retrieval of seeded inputs; out-of-range slots come from chunk counts
below K.
"""

import numpy as np
import pytest
import torch

from long_context_lm_amd import gca
from long_context_lm_amd import inputs as I
from oracle import gca_oracle as O
from tests.gpu_util import config_for, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gca.load()
    yield
    torch.cuda.synchronize()


def _pinned(t):
    out = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    out.copy_(t)
    return out


def _retrieved(shape, dtype, seed):
    host = I.make_inputs(shape, dtype, seed=seed, scale=0.125)
    cfg = config_for(shape, dtype)
    dev = upload(host)
    idx, sc = gca.retrieve(cfg, dev["lq"], dev["lk"])
    return cfg, host, dev, idx, sc


def _check_against_oracle(name, got, idx, k_host, v_host, n_kv):
    k_c, v_c, idx_c = got
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    r_k, r_v, r_idx = O.fetch_chunks(idx_np, I.as_f64(k_host), I.as_f64(v_host), n_kv=n_kv)
    assert np.array_equal(idx_c.cpu().numpy(), r_idx), f"{name}: remapped indices differ"
    valid = r_idx >= 0
    got_k, got_v = I.as_f64(k_c), I.as_f64(v_c)
    G, B, n_q, K = idx_np.shape
    for g, b, r, s in zip(*np.nonzero(valid)):  # only slots in range are written
        c = (g * n_q + r) * K + s
        rows = slice(64 * c, 64 * c + 64)
        assert np.array_equal(got_k[b, :, rows], r_k[b, :, rows]), f"{name}: K tile of slot {(g, b, r, s)}"
        assert np.array_equal(got_v[b, :, rows], r_v[b, :, rows]), f"{name}: V tile of slot {(g, b, r, s)}"


SHAPES = [
    # training-like rows (short histories, out-of-range slots in the first rows)
    I.Shape(B=2, G=2, H=3, n_q=6, n_kv=6, topk=4, q_chunk_base=0, shift=1),
    # decode over a history: one row, every slot in range
    I.Shape(B=1, G=2, H=4, n_q=1, n_kv=700, topk=8, q_chunk_base=700, shift=0),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=["rows", "decode"])
def test_fetch_matches_oracle_device_and_pinned(shape, dtype):
    say("case fetch", shape, dtype)
    cfg, host, dev, idx, sc = _retrieved(shape, dtype, seed=5)
    got = gca.fetch_chunks(cfg, idx, dev["k"], dev["v"])
    _check_against_oracle("device source", got, idx, host["k"], host["v"], shape.n_kv)
    pk, pv = _pinned(host["k"]), _pinned(host["v"])
    got_h = gca.fetch_chunks(cfg, idx, pk, pv)
    _check_against_oracle("pinned host source", got_h, idx, host["k"], host["v"], shape.n_kv)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_over_fetched_chunks_is_bit_identical(dtype):
    shape = I.Shape(B=1, G=2, H=4, n_q=1, n_kv=700, topk=8, q_chunk_base=700, shift=0)
    say("case fetched attention", shape, dtype)
    cfg, host, dev, idx, sc = _retrieved(shape, dtype, seed=11)
    o_full, lse_full = gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx, sc)
    k_c, v_c, idx_c = gca.fetch_chunks(cfg, idx, _pinned(host["k"]), _pinned(host["v"]))
    o_c, lse_c = gca.forward(gca.fetched_config(cfg), dev["q"], k_c, v_c, idx_c, sc)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_full)
    assert torch.equal(lse_c, lse_full)


def test_fetch_from_a_view_inside_a_pinned_allocation():
    shape = I.Shape(B=2, G=2, H=3, n_q=4, n_kv=9, topk=3, q_chunk_base=5, shift=0)
    say("case pinned view", shape)
    cfg, host, dev, idx, sc = _retrieved(shape, "bf16", seed=2)
    big_k = _pinned(torch.cat([torch.zeros_like(host["k"][:1]), host["k"]]))
    big_v = _pinned(torch.cat([torch.zeros_like(host["v"][:1]), host["v"]]))
    got = gca.fetch_chunks(cfg, idx, big_k[1:], big_v[1:])
    _check_against_oracle("pinned view", got, idx, host["k"], host["v"], shape.n_kv)


def test_pageable_host_memory_is_refused():
    shape = I.Shape(B=1, G=1, H=2, n_q=2, n_kv=4, topk=2, q_chunk_base=4, shift=0)
    cfg, host, dev, idx, sc = _retrieved(shape, "bf16", seed=1)
    with pytest.raises(gca.GcaError):
        gca.fetch_chunks(cfg, idx, host["k"], host["v"])  # ordinary (pageable) CPU tensors
    torch.cuda.synchronize()
