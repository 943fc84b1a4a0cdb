"""GPU parity of token-level decode (gca_decode_tokens) against the CPU oracle.

Bars: fp32 max-abs <= 1e-4, bf16 relative L2 <= 1e-2 (the kernel computes in fp32 throughout).
Cases: one token and partial chunks (ragged over the four-token batches), K = 8 and K = 16 (two
rounds of slots per wave), invalid slots, shift = 1 (no retrieval row: zeros), compact K/V from
gca_fetch_chunks, and agreement with the chunk forward's first rows.
"""

import dataclasses

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


def _case(shape, dtype, n_tok, seed):
    host = I.make_inputs(shape, dtype, seed=seed, scale=0.125)
    cfg = config_for(shape, dtype)
    dev = upload(host)
    idx, sc = gca.retrieve(cfg, dev["lq"], dev["lk"])
    q_tok = dev["q"][:, :, :, :n_tok].contiguous()
    return cfg, host, dev, idx, sc, q_tok


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_tok", [1, 3, 6, 64])
@pytest.mark.parametrize("topk", [8, 16])
def test_decode_tokens_matches_oracle(dtype, n_tok, topk):
    shape = I.Shape(B=2, G=2, H=3, n_q=1, n_kv=40, topk=topk, q_chunk_base=40, shift=0)
    say("case decode", shape, dtype, n_tok)
    cfg, host, dev, idx, sc, q_tok = _case(shape, dtype, n_tok, seed=n_tok + topk)
    o = gca.decode_tokens(cfg, q_tok, dev["k"], dev["v"], idx, sc)
    torch.cuda.synchronize()
    ref = O.decode_tokens(I.as_f64(q_tok), I.as_f64(host["k"]), I.as_f64(host["v"]), idx.cpu().numpy(),
                          sc.cpu().numpy(), shift=0)
    err = assert_close("o", I.as_f64(o), ref, dtype)
    say("  error", f"{err:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_tokens_invalid_slots_and_no_row(dtype):
    # 5 past chunks and K = 8: three slots are invalid
    shape = I.Shape(B=1, G=2, H=2, n_q=1, n_kv=5, topk=8, q_chunk_base=5, shift=0)
    cfg, host, dev, idx, sc, q_tok = _case(shape, dtype, 2, seed=3)
    assert int((idx < 0).sum()) == 2 * 3
    o = gca.decode_tokens(cfg, q_tok, dev["k"], dev["v"], idx, sc)
    torch.cuda.synchronize()
    ref = O.decode_tokens(I.as_f64(q_tok), I.as_f64(host["k"]), I.as_f64(host["v"]), idx.cpu().numpy(),
                          sc.cpu().numpy(), shift=0)
    assert_close("o", I.as_f64(o), ref, dtype)
    # shift = 1: the single query chunk has no retrieval row, so every output is zero
    cfg1 = dataclasses.replace(cfg, shift=1)
    o1 = gca.decode_tokens(cfg1, q_tok, dev["k"], dev["v"], idx, sc, o=torch.full_like(q_tok, 7.0))
    torch.cuda.synchronize()
    assert not o1.any()


def test_decode_tokens_agrees_with_chunk_forward_and_fetched_chunks():
    shape = I.Shape(B=1, G=2, H=4, n_q=1, n_kv=300, topk=8, q_chunk_base=300, shift=0)
    cfg, host, dev, idx, sc, q_tok = _case(shape, "f32", 5, seed=21)
    o_chunk, _ = gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx, sc)
    o_tok = gca.decode_tokens(cfg, q_tok, dev["k"], dev["v"], idx, sc)
    torch.cuda.synchronize()
    np.testing.assert_allclose(I.as_f64(o_tok), I.as_f64(o_chunk[:, :, :, :5]), rtol=0, atol=1e-5)
    # over the compact buffers of gca_fetch_chunks: the same tile values, so the same bits
    k_c, v_c, idx_c = gca.fetch_chunks(cfg, idx, dev["k"], dev["v"])
    o_c = gca.decode_tokens(gca.fetched_config(cfg), q_tok, k_c, v_c, idx_c, sc)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_tok)
