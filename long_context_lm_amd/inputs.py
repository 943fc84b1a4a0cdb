"""Seeded synthetic inputs for the GCA path.

Shared by the tests, the smoke check and the benchmark.  It only draws numbers and
casts them; it holds none of the method's arithmetic.

Recipe: ``numpy.random.default_rng([seed, stream])`` with one stream per tensor in the
order lq, lk, q, k, v, dout; standard normal float32 values, multiplied by ``scale``
(exact for powers of two) and rounded to the working dtype (round-to-nearest-even for
bf16).  Shapes follow the pages' workloads: chunks of S = 64 tokens, head dim 64,
landmark dim 64, top-k 8, 16K-token training contexts and histories up to 16M tokens.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

STREAMS = ("lq", "lk", "q", "k", "v", "dout")


@dataclass(frozen=True)
class Shape:
    """Sizes of one GCA problem (chunk size S = 64, head and landmark dims 64)."""

    B: int
    G: int
    H: int
    n_q: int          # retrieval rows / query chunks in this call
    n_kv: int         # history chunks holding K, V and key landmarks
    topk: int
    q_chunk_base: int = 0
    shift: int = 1
    d: int = 64
    dl: int = 64

    @property
    def Lq(self) -> int:
        return self.n_q * 64

    @property
    def Lk(self) -> int:
        return self.n_kv * 64

    def tensor_shape(self, name: str):
        return {
            "lq": (self.G, self.B, self.n_q, self.dl),
            "lk": (self.G, self.B, self.n_kv, self.dl),
            "q": (self.G, self.B, self.H, self.Lq, self.d),
            "k": (self.B, self.H, self.Lk, self.d),
            "v": (self.B, self.H, self.Lk, self.d),
            "dout": (self.G, self.B, self.H, self.Lq, self.d),
        }[name]


# The workloads the pages describe (S=64, K=8, 16K training context, up to 16M history).
TINY_FP32 = Shape(B=1, G=1, H=2, n_q=16, n_kv=16, topk=4)
TRAIN_16K = Shape(B=8, G=1, H=12, n_q=256, n_kv=256, topk=8)
TRAIN_16K_G2 = Shape(B=8, G=2, H=12, n_q=256, n_kv=256, topk=8)
INFER_1M = Shape(B=1, G=2, H=12, n_q=1, n_kv=16384, topk=8, q_chunk_base=16384, shift=0)
INFER_16M = Shape(B=1, G=2, H=12, n_q=1, n_kv=262144, topk=8, q_chunk_base=262144, shift=0)


def normal(shape, seed: int, stream: str, scale: float = 1.0) -> np.ndarray:
    """float32 N(0, scale^2) draws for one named tensor stream."""
    rng = np.random.default_rng([seed, STREAMS.index(stream)])
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def to_dtype(x: np.ndarray, dtype: str):
    """Round a float32 array to the working dtype; returns a CPU torch tensor."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(shape: Shape, dtype: str, seed: int = 0, scale: float = 1.0,
                names=STREAMS):
    """CPU torch tensors (working dtype) for the named streams."""
    return {n: to_dtype(normal(shape.tensor_shape(n), seed, n, scale), dtype) for n in names}


def hub_landmarks(shape: Shape, seed: int, hub: int = 0):
    """Landmarks with a hub chunk: every query landmark shares a direction u of its (group,
    batch row), lq = 0.5 u + sqrt(0.75) z (unit variance), and key landmark `hub` is 2 u, so its
    score is about 8 against about N(0, 1) for the other chunks and it enters nearly every row's
    top-k.  float32 arrays lq [G, B, n_q, dl] and lk [G, B, n_kv, dl] (N(0, 1) elsewhere)."""
    rng = np.random.default_rng([seed, 99])
    G, B = shape.G, shape.B
    u = rng.standard_normal((G, B, 1, shape.dl))
    lq = 0.5 * u + np.sqrt(0.75) * rng.standard_normal((G, B, shape.n_q, shape.dl))
    lk = rng.standard_normal((G, B, shape.n_kv, shape.dl))
    lk[:, :, hub] = 2.0 * u[:, :, 0]
    return lq.astype(np.float32), lk.astype(np.float32)


def as_f64(t) -> np.ndarray:
    """Exact float64 copy of a CPU/GPU tensor (bf16 and fp32 values are exact in fp64)."""
    import torch

    return t.detach().to("cpu", torch.float64).numpy()
