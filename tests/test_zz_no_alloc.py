"""The retrieval entry point that allocates nothing (gca_retrieve_static), through the C ABI.

It must return exactly what gca_retrieve returns with a caller workspace, on problems whose long
rows use the library's scratch array (several scan blocks per row, merged) and on problems that
need none, and keep doing so on the next call: two calls in a row, the second with a smaller
input, each compared with gca_retrieve bit for bit.
"""

import ctypes

import numpy as np
import pytest
import torch

from long_context_lm_amd import gca
from long_context_lm_amd import inputs as I
from tests.gpu_util import config_for, say

pytestmark = pytest.mark.gpu


def _static(cfg, lq, lk):
    lib = gca.load()
    shp = (cfg.G, cfg.B, cfg.n_q, cfg.topk)
    idx = torch.full(shp, 123, dtype=torch.int32, device="cuda")
    sc = torch.full(shp, 7.0, dtype=torch.float32, device="cuda")
    prob = cfg.problem()
    st = lib.gca_retrieve_static(ctypes.byref(prob), ctypes.c_void_p(lq.data_ptr()),
                                 ctypes.c_void_p(lk.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                 ctypes.c_void_p(sc.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, f"gca_retrieve_static returned status {st}"
    return idx, sc


def _compare(shape, dtype, gumbel, seed):
    say("case", shape, dtype, "gumbel", gumbel)
    cfg = config_for(shape, dtype, use_gumbel=gumbel, seed=seed)
    host = I.make_inputs(shape, dtype, seed=seed, scale=0.125, names=("lq", "lk"))
    lq, lk = host["lq"].cuda(), host["lk"].cuda()
    needs = gca.workspace_size(gca.OP_RETRIEVE, cfg)
    say("  workspace of gca_retrieve:", needs, "bytes")
    s_idx, s_sc = _static(cfg, lq, lk)
    r_idx, r_sc = gca.retrieve(cfg, lq, lk)
    torch.cuda.synchronize()
    assert torch.equal(s_idx, r_idx), "indices differ from gca_retrieve"
    assert torch.equal(s_sc, r_sc), "scores differ from gca_retrieve"
    return needs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_retrieve_matches_workspace_retrieve_twice(dtype):
    """First a long history (the scan splits each row over many blocks and merges their lists in
    the scratch array), then a smaller one on the same array, then a problem needing no scratch."""
    big = I.Shape(B=1, G=2, H=1, n_q=2, n_kv=300_000, topk=8, q_chunk_base=300_000, shift=0)
    small = I.Shape(B=1, G=2, H=1, n_q=3, n_kv=5_000, topk=16, q_chunk_base=4_999, shift=0)
    rows = I.Shape(B=2, G=2, H=1, n_q=40, n_kv=40, topk=8)
    assert _compare(big, dtype, True, 5) > 0
    assert _compare(small, dtype, False, 6) > 0
    assert _compare(rows, dtype, True, 7) == 0


def test_static_retrieve_empty_and_refusals():
    """Zero rows: validated, nothing launched.  Invalid arguments: the documented status, before
    any launch."""
    lib = gca.load()
    cfg = gca.Config(B=1, G=1, H=1, n_q=0, n_kv=4, topk=4)
    prob = cfg.problem()
    assert lib.gca_retrieve_static(ctypes.byref(prob), None, None, None, None, None) == 0
    bad = gca.Config(B=1, G=1, H=1, n_q=2, n_kv=4, topk=17).problem()
    z = torch.zeros(1024, device="cuda")
    p = ctypes.c_void_p(z.data_ptr())
    assert lib.gca_retrieve_static(ctypes.byref(bad), p, p, p, p, None) == 2  # topk > 16
    assert lib.gca_retrieve_static(None, p, p, p, p, None) == 1
    torch.cuda.synchronize()
