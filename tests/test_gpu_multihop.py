"""Chained (multi-hop) retrieval through the C ABI.

A higher retrieval group may retrieve on the basis of what the previous group retrieved
[Notes, Key designs: causal retrieval; the 2-hop needle task of Notes, Experiments: key findings
uses G = 2].  The kernels treat each group as an independent problem, so a chain is two calls:
hop 1 (retrieve + GCA forward) gives the fused output o1; the query landmark of chunk r for hop 2
is a fixed projection of o1 averaged over chunk r's tokens and heads,
    lq2[b, r] = W^T mean_{h, u in chunk r} o1[b, h, 64 r + u, :],
computed here by the test (float64, rounded to the problem dtype); hop 2 retrieves with lq2 over
its own key landmarks and attends.  Hop 1 is compared with the oracle, and hop 2 is compared with
the oracle run on the same lq2: indices bit-exact, outputs within the parity bars.
"""

import numpy as np
import pytest
import torch

from long_context_lm_amd import gca
from long_context_lm_amd import inputs as I
from oracle import gca_oracle as O
from tests.gpu_util import assert_close, config_for, say, upload

pytestmark = pytest.mark.gpu


def _hop2_landmarks(o1, H, W, dtype):
    """o1 [1, B, H, n_q*64, 64] (float64) -> lq2 [1, B, n_q, 64] in the problem dtype."""
    _, B, _, L, d = o1.shape
    per_chunk = o1.reshape(1, B, H, L // 64, 64, d).mean(axis=(2, 4))  # [1, B, n_q, d]
    lq2 = per_chunk @ W
    t = torch.from_numpy(lq2.astype(np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_two_hop_chain_matches_the_oracle_chain(dtype):
    shape = I.Shape(B=2, G=1, H=2, n_q=24, n_kv=24, topk=4)
    cfg = config_for(shape, dtype)
    say("case two-hop", shape, dtype)
    hop1 = I.make_inputs(shape, dtype, seed=41, scale=1.0)
    hop2 = I.make_inputs(shape, dtype, seed=42, scale=1.0, names=("lk", "q"))
    W = np.random.default_rng([42, 7]).standard_normal((64, 64)) * 2.0  # the fixed projection
    x1 = {k: I.as_f64(v) for k, v in hop1.items()}
    dev = upload(hop1)
    # hop 1
    idx1, sc1 = gca.retrieve(cfg, dev["lq"], dev["lk"])
    o1, _ = gca.forward(cfg, dev["q"], dev["k"], dev["v"], idx1, sc1, need_lse=False)
    torch.cuda.synchronize()
    r_idx1, r_sc1 = O.retrieve(x1["lq"], x1["lk"], 4)
    np.testing.assert_array_equal(idx1.cpu().numpy(), r_idx1)
    np.testing.assert_array_equal(sc1.cpu().numpy(), r_sc1)
    r_o1, _ = O.forward(x1["q"], x1["k"], x1["v"], r_idx1, r_sc1)
    assert_close("o1", I.as_f64(o1), r_o1, dtype)
    # hop 2: its query landmarks come from hop 1's output (the GPU's, so both sides see one lq2)
    lq2 = _hop2_landmarks(I.as_f64(o1), shape.H, W, dtype)
    idx2, sc2 = gca.retrieve(cfg, lq2.cuda(), hop2["lk"].cuda())
    o2, _ = gca.forward(cfg, hop2["q"].cuda(), dev["k"], dev["v"], idx2, sc2, need_lse=False)
    torch.cuda.synchronize()
    r_idx2, r_sc2 = O.retrieve(I.as_f64(lq2), I.as_f64(hop2["lk"]), 4)
    np.testing.assert_array_equal(idx2.cpu().numpy(), r_idx2)
    np.testing.assert_array_equal(sc2.cpu().numpy(), r_sc2)
    r_o2, _ = O.forward(I.as_f64(hop2["q"]), x1["k"], x1["v"], r_idx2, r_sc2)
    assert_close("o2", I.as_f64(o2), r_o2, dtype)
    # the second hop depends on the first: hop 2 with hop 1's landmarks selects other chunks
    direct, _ = O.retrieve(x1["lq"], I.as_f64(hop2["lk"]), 4)
    changed = float((direct != r_idx2).any(axis=-1).mean())
    say(f"  rows whose hop-2 selection differs from a retrieval with hop 1's landmarks: {changed:.0%}")
    assert changed > 0.5
