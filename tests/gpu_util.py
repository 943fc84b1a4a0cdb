"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path, compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

from long_context_lm_amd import gca
from long_context_lm_amd import inputs as I


def say(*args):
    print("[gpu-test]", *args, flush=True)
    sys.stdout.flush()


def config_for(shape: I.Shape, dtype: str, **kw) -> gca.Config:
    return gca.Config(B=shape.B, G=shape.G, H=shape.H, n_q=shape.n_q, n_kv=shape.n_kv, topk=shape.topk,
                      dtype=dtype, q_chunk_base=shape.q_chunk_base, shift=shape.shift, **kw)


def upload(tensors: dict, device="cuda") -> dict:
    return {k: v.to(device) for k, v in tensors.items()}


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def assert_close(name: str, got, ref, dtype: str):
    """fp32: max-abs <= 1e-4; bf16: relative L2 <= 1e-2 (the stated parity bars)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if dtype == "f32":
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        assert err <= 1e-4, f"{name}: max-abs {err:.3e} > 1e-4"
    else:
        err = rel_l2(got, ref)
        assert err <= 1e-2, f"{name}: rel-L2 {err:.3e} > 1e-2"
    return err


def lse_tokens(lse) -> np.ndarray:
    """Library lse [G, B, H, n_q, K, 64] -> the oracle's token-major [G, B, H, n_q * 64, K]."""
    a = lse.detach().cpu().numpy() if hasattr(lse, "detach") else np.asarray(lse)
    G, B, H, nq, K, S = a.shape
    return a.transpose(0, 1, 2, 3, 5, 4).reshape(G, B, H, nq * S, K)


def lse_compare(name: str, got, ref, dtype: str):
    got = lse_tokens(got).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_g, inf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(inf_g, inf_r), f"{name}: -inf pattern differs"
    return assert_close(name, got[~inf_r], ref[~inf_r], dtype)


def assert_tiles_close(name: str, got, ref, bar: float = 1e-2):
    """bf16 parity per 64x64 tile: the last two axes are (tokens, 64) with tokens a multiple of 64;
    every (leading index, chunk) tile must be within relative L2 `bar` of the reference, and a tile
    whose reference is exactly zero (no retrieval reaches it) must be exactly zero.  One wrong slot
    in one tile of a large tensor moves the whole-tensor norm by little; this catches it."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    L, d = ref.shape[-2:]
    assert L % 64 == 0, (name, ref.shape)
    g = got.reshape(-1, L // 64, 64, d)
    r = ref.reshape(-1, L // 64, 64, d)
    num = np.sqrt(((g - r) ** 2).sum(axis=(-1, -2)))
    den = np.sqrt((r ** 2).sum(axis=(-1, -2)))
    zero = den == 0
    assert np.all(num[zero] == 0), f"{name}: {int((num[zero] != 0).sum())} tiles nonzero where the reference is 0"
    rel = num[~zero] / den[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= bar, f"{name}: worst tile rel-L2 {worst:.3e} > {bar} ({int((rel > bar).sum())} tiles)"
    return worst
