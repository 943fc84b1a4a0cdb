"""Thin ctypes binding of the GCA C ABI (include/gca.h).

Argument marshalling only: every step of retrieval, attention, fusion and backward runs in the
HIP kernels of libgca.so.  PyTorch provides device memory and the current stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgca.so")

GCA_OK = 0
OP_RETRIEVE, OP_FORWARD, OP_BACKWARD, OP_LANDMARK_BACKWARD, OP_SW_BACKWARD, OP_FUSED_BACKWARD = 0, 1, 2, 3, 4, 5
DTYPES = {"bf16": 0, "f32": 1}


class Problem(ctypes.Structure):
    """Mirror of gca_problem (natural C alignment, 88 bytes)."""

    _fields_ = [
        ("B", ctypes.c_int32),
        ("G", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("S", ctypes.c_int32),
        ("n_q_chunks", ctypes.c_int64),
        ("q_chunk_base", ctypes.c_int64),
        ("n_kv_chunks", ctypes.c_int64),
        ("d_head", ctypes.c_int32),
        ("d_lmk", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("attn_scale", ctypes.c_float),
        ("score_scale", ctypes.c_float),
        ("use_gumbel", ctypes.c_int32),
        ("shift", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("gumbel_tau", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


EXPORTS = (
    "gca_workspace_size",
    "gca_retrieve",
    "gca_retrieve_static",
    "gca_forward",
    "gca_backward",
    "gca_status_string",
    "gca_last_hip_error",
    "gca_profile_enable",
    "gca_profile_collect",
    "gca_landmark_backward",
    "gca_fetch_chunks",
    "gca_decode_tokens",
    "gca_sw_forward",
    "gca_sw_backward",
    "gca_fused_forward",
    "gca_fused_backward",
)

_lib = None


class GcaError(RuntimeError):
    def __init__(self, call: str, status: int):
        lib = load()
        text = lib.gca_status_string(status).decode()
        hip = lib.gca_last_hip_error() if status == 5 else 0
        super().__init__(f"{call} failed: {text} (status {status}{', hip error %d' % hip if hip else ''})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libgca.so (built by long_context_lm_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run `python -m long_context_lm_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(Problem)
    lib.gca_workspace_size.argtypes = [ctypes.c_int, P, ctypes.POINTER(sz)]
    lib.gca_retrieve.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.gca_retrieve_static.argtypes = [P, vp, vp, vp, vp, vp]
    lib.gca_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gca_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gca_landmark_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gca_fetch_chunks.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.gca_decode_tokens.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp]
    lib.gca_sw_forward.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp]
    lib.gca_sw_backward.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gca_fused_forward.argtypes = [P, ctypes.c_int32] + [vp] * 10 + [vp]
    lib.gca_fused_backward.argtypes = [P, ctypes.c_int32] + [vp] * 18 + [sz, vp]
    for f in ("gca_fused_forward", "gca_fused_backward", "gca_workspace_size", "gca_retrieve", "gca_retrieve_static",
              "gca_forward", "gca_backward", "gca_landmark_backward",
              "gca_profile_enable", "gca_profile_collect"):
        getattr(lib, f).restype = ctypes.c_int
    lib.gca_status_string.argtypes = [ctypes.c_int]
    lib.gca_status_string.restype = ctypes.c_char_p
    lib.gca_last_hip_error.argtypes = []
    lib.gca_last_hip_error.restype = ctypes.c_int
    lib.gca_profile_enable.argtypes = [ctypes.c_int]
    lib.gca_profile_collect.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int)]
    _lib = lib
    return lib


@dataclass
class Config:
    """Problem options of one GCA layer call (see gca_problem in include/gca.h)."""

    B: int
    G: int
    H: int
    n_q: int
    n_kv: int
    topk: int = 8
    dtype: str = "bf16"
    q_chunk_base: int = 0
    shift: int = 1
    use_gumbel: bool = False
    seed: int = 0
    tau: float = 1.0
    attn_scale: float = 1.0 / math.sqrt(64)
    score_scale: float = 1.0 / math.sqrt(64)

    def shape(self, name: str):
        """The tensor shape include/gca.h states for `name` under this problem."""
        G, B, H, nq, nkv, K = self.G, self.B, self.H, self.n_q, self.n_kv, self.topk
        return {
            "lq": (G, B, nq, 64), "lk": (G, B, nkv, 64),
            "q": (G, B, H, nq * 64, 64), "kv": (B, H, nkv * 64, 64),
            "sel": (G, B, nq, K), "lse": (G, B, H, nq, K, 64),
        }[name]

    def problem(self) -> Problem:
        return Problem(B=self.B, G=self.G, H=self.H, S=64, n_q_chunks=self.n_q,
                       q_chunk_base=self.q_chunk_base, n_kv_chunks=self.n_kv, d_head=64,
                       d_lmk=64, topk=self.topk, dtype=DTYPES[self.dtype],
                       attn_scale=self.attn_scale, score_scale=self.score_scale,
                       use_gumbel=int(self.use_gumbel), shift=self.shift,
                       seed=self.seed & ((1 << 64) - 1), gumbel_tau=self.tau, reserved=0)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _expect(name: str, t, shape, dtype, device=None, host_ok: bool = False):
    """Refuse a tensor the C ABI would misread: the library sees only a pointer, so the shape,
    dtype, layout and device that include/gca.h states are checked here, before the call."""
    import torch

    if t is None:
        raise ValueError(f"{name}: tensor required")
    # any row-major view of the stated shape is the same memory (e.g. k as [B,H,n_kv*64,64] or
    # [B,H,n_kv,64,64]); what the library would misread is a different element count
    want = 1
    for x in shape:
        want *= int(x)
    if t.numel() != want:
        raise ValueError(f"{name}: shape {tuple(t.shape)} ({t.numel()} elements), expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (row-major)")
    if t.device.type != "cuda":
        # host sources of gca_fetch_chunks: the library itself tells pinned from pageable memory
        if not host_ok:
            raise ValueError(f"{name}: must be a GPU tensor")
    elif device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(call: str, status: int):
    if status != GCA_OK:
        raise GcaError(call, status)


def workspace_size(op: int, cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    prob = cfg.problem()
    _check("gca_workspace_size", load().gca_workspace_size(op, ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def _ws_bytes(ws, device) -> int:
    """Byte size of a caller-provided workspace (a contiguous tensor on the call's device)."""
    if not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"workspace: must be a contiguous tensor on {device}")
    return ws.numel() * ws.element_size()


def _workspace(op: int, cfg: Config, device):
    import torch

    n = workspace_size(op, cfg)
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def _torch_dtype(cfg: Config):
    import torch

    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def retrieve(cfg: Config, lq, lk, idx=None, score=None, ws=None):
    """gca_retrieve: returns (idx int32 [G,B,n_q,K], score fp32 [G,B,n_q,K])."""
    import torch

    dev = lq.device
    shp = (cfg.G, cfg.B, cfg.n_q, cfg.topk)
    idx = torch.empty(shp, dtype=torch.int32, device=dev) if idx is None else idx
    score = torch.empty(shp, dtype=torch.float32, device=dev) if score is None else score
    ft = _torch_dtype(cfg)
    _expect("lq", lq, cfg.shape("lq"), ft, dev)
    _expect("lk", lk, cfg.shape("lk"), ft, dev)
    _expect("idx", idx, shp, torch.int32, dev)
    _expect("score", score, shp, torch.float32, dev)
    if ws is None:
        ws, n = _workspace(OP_RETRIEVE, cfg, dev)
    else:
        n = _ws_bytes(ws, dev)
    prob = cfg.problem()
    _check("gca_retrieve", load().gca_retrieve(ctypes.byref(prob), _ptr(lq), _ptr(lk), _ptr(idx),
                                               _ptr(score), _ptr(ws), n, _stream()))
    return idx, score


def _check_attend(cfg: Config, q, k, v, idx, score, dev):
    import torch

    ft = _torch_dtype(cfg)
    _expect("q", q, cfg.shape("q"), ft, dev)
    _expect("k", k, cfg.shape("kv"), ft, dev)
    _expect("v", v, cfg.shape("kv"), ft, dev)
    _expect("idx", idx, cfg.shape("sel"), torch.int32, dev)
    _expect("score", score, cfg.shape("sel"), torch.float32, dev)


def retrieve_static(cfg: Config, lq, lk, idx=None, score=None):
    """gca_retrieve_static (no workspace, no allocation inside the library):
    returns (idx int32 [G,B,n_q,K], score fp32 [G,B,n_q,K])."""
    import torch

    dev = lq.device
    shp = (cfg.G, cfg.B, cfg.n_q, cfg.topk)
    idx = torch.empty(shp, dtype=torch.int32, device=dev) if idx is None else idx
    score = torch.empty(shp, dtype=torch.float32, device=dev) if score is None else score
    ft = _torch_dtype(cfg)
    _expect("lq", lq, cfg.shape("lq"), ft, dev)
    _expect("lk", lk, cfg.shape("lk"), ft, dev)
    _expect("idx", idx, shp, torch.int32, dev)
    _expect("score", score, shp, torch.float32, dev)
    prob = cfg.problem()
    _check("gca_retrieve_static", load().gca_retrieve_static(ctypes.byref(prob), _ptr(lq), _ptr(lk), _ptr(idx),
                                                             _ptr(score), _stream()))
    return idx, score


def forward(cfg: Config, q, k, v, idx, score, need_lse: bool = True, o=None, lse=None):
    """gca_forward: returns (o [G,B,H,n_q*64,64], lse fp32 [G,B,H,n_q,K,64] or None)."""
    import torch

    dev = q.device
    o = torch.empty_like(q) if o is None else o
    if need_lse and lse is None:
        lse = torch.empty((cfg.G, cfg.B, cfg.H, cfg.n_q, cfg.topk, 64), dtype=torch.float32, device=dev)
    _check_attend(cfg, q, k, v, idx, score, dev)
    _expect("o", o, cfg.shape("q"), _torch_dtype(cfg), dev)
    if need_lse:
        _expect("lse", lse, cfg.shape("lse"), torch.float32, dev)
    prob = cfg.problem()
    _check("gca_forward", load().gca_forward(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                             _ptr(score), _ptr(o), _ptr(lse) if need_lse else None,
                                             None, 0, _stream()))
    return o, (lse if need_lse else None)


def backward(cfg: Config, q, k, v, idx, score, lse, dout, ws=None, out=None):
    """gca_backward: returns (dq, dk, dv, dscore)."""
    import torch

    dev = q.device
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        dscore = torch.empty(idx.shape, dtype=torch.float32, device=dev)
    else:
        dq, dk, dv, dscore = out
    ft = _torch_dtype(cfg)
    _check_attend(cfg, q, k, v, idx, score, dev)
    _expect("lse", lse, cfg.shape("lse"), torch.float32, dev)
    _expect("dout", dout, cfg.shape("q"), ft, dev)
    _expect("dq", dq, cfg.shape("q"), ft, dev)
    _expect("dk", dk, cfg.shape("kv"), ft, dev)
    _expect("dv", dv, cfg.shape("kv"), ft, dev)
    _expect("dscore", dscore, cfg.shape("sel"), torch.float32, dev)
    if ws is None:
        ws, n = _workspace(OP_BACKWARD, cfg, dev)
    else:
        n = _ws_bytes(ws, dev)
    prob = cfg.problem()
    _check("gca_backward", load().gca_backward(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                               _ptr(score), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                               _ptr(dv), _ptr(dscore), _ptr(ws), n, _stream()))
    return dq, dk, dv, dscore


def landmark_backward(cfg: Config, lq, lk, idx, dscore, ws=None, out=None):
    """gca_landmark_backward: returns (dlq like lq, dlk like lk)."""
    import torch

    dlq, dlk = (torch.empty_like(lq), torch.empty_like(lk)) if out is None else out
    dev, ft = lq.device, _torch_dtype(cfg)
    for name, t, shp in (("lq", lq, "lq"), ("lk", lk, "lk"), ("dlq", dlq, "lq"), ("dlk", dlk, "lk")):
        _expect(name, t, cfg.shape(shp), ft, dev)
    _expect("idx", idx, cfg.shape("sel"), torch.int32, dev)
    _expect("dscore", dscore, cfg.shape("sel"), torch.float32, dev)
    if ws is None:
        ws, n = _workspace(OP_LANDMARK_BACKWARD, cfg, lq.device)
    else:
        n = _ws_bytes(ws, lq.device)
    prob = cfg.problem()
    _check("gca_landmark_backward", load().gca_landmark_backward(ctypes.byref(prob), _ptr(lq), _ptr(lk), _ptr(idx),
                                                                 _ptr(dscore), _ptr(dlq), _ptr(dlk), _ptr(ws), n,
                                                                 _stream()))
    return dlq, dlk


def decode_tokens(cfg: Config, q, k, v, idx, score, o=None):
    """gca_decode_tokens: q [G,B,H,n_tokens,64] of the call's single query chunk -> o like q."""
    import torch

    o = torch.empty_like(q) if o is None else o
    dev, ft = q.device, _torch_dtype(cfg)
    n_tok = int(q.shape[-2]) if q.dim() == 5 else 0
    _expect("q", q, (cfg.G, cfg.B, cfg.H, n_tok, 64), ft, dev)
    _expect("o", o, (cfg.G, cfg.B, cfg.H, n_tok, 64), ft, dev)
    _expect("k", k, cfg.shape("kv"), ft, dev)
    _expect("v", v, cfg.shape("kv"), ft, dev)
    _expect("idx", idx, cfg.shape("sel"), torch.int32, dev)
    _expect("score", score, cfg.shape("sel"), torch.float32, dev)
    prob = cfg.problem()
    _check("gca_decode_tokens", load().gca_decode_tokens(ctypes.byref(prob), int(q.shape[-2]), _ptr(q), _ptr(k),
                                                         _ptr(v), _ptr(idx), _ptr(score), _ptr(o), _stream()))
    return o


def sw_config(B: int, H: int, n_chunks: int, attn_scale: float = 1.0 / math.sqrt(64)) -> Config:
    """The problem of a sliding-window attention call over one sequence of n_chunks chunks."""
    return Config(B=B, G=1, H=H, n_q=n_chunks, n_kv=n_chunks, topk=1, dtype="bf16", attn_scale=attn_scale)


def sw_forward(cfg: Config, q, k, v, window: int = 512, need_lse: bool = True, o=None, lse=None):
    """gca_sw_forward: q, k, v [B,H,L,64] bf16 -> (o like q, lse fp32 [B,H,L] or None)."""
    import torch

    o = torch.empty_like(q) if o is None else o
    if need_lse and lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    seq = (cfg.B, cfg.H, cfg.n_q * 64, 64)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _expect(name, t, seq, _torch_dtype(cfg), q.device)
    if need_lse:
        _expect("lse", lse, seq[:-1], torch.float32, q.device)
    prob = cfg.problem()
    _check("gca_sw_forward", load().gca_sw_forward(ctypes.byref(prob), int(window), _ptr(q), _ptr(k), _ptr(v),
                                                   _ptr(o), _ptr(lse) if need_lse else None, _stream()))
    return o, (lse if need_lse else None)


def sw_backward(cfg: Config, q, k, v, o, lse, dout, window: int = 512, ws=None, out=None):
    """gca_sw_backward: returns (dq, dk, dv) like q."""
    import torch

    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if out is None else out
    seq = (cfg.B, cfg.H, cfg.n_q * 64, 64)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(name, t, seq, _torch_dtype(cfg), q.device)
    _expect("lse", lse, seq[:-1], torch.float32, q.device)
    if ws is None:
        ws, n = _workspace(OP_SW_BACKWARD, cfg, q.device)
    else:
        n = _ws_bytes(ws, q.device)
    prob = cfg.problem()
    _check("gca_sw_backward", load().gca_sw_backward(ctypes.byref(prob), int(window), _ptr(q), _ptr(k), _ptr(v),
                                                     _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                                     _ptr(ws), n, _stream()))
    return dq, dk, dv


def fused_forward(cfg: Config, q, k_sw, v_sw, k, v, idx, score, window: int = 512, need_lse: bool = True,
                  o=None, lse_sw=None, lse=None):
    """gca_fused_forward (G = 1): o = SW(q, k_sw, v_sw; window) + GCA(q, k, v, idx, score).
    q, k_sw, v_sw [B,H,L,64]; k, v [B,H,n_kv*64,64]; returns (o like q, lse_sw [B,H,L] or None,
    lse [1,B,H,n_q,K,64] or None)."""
    import torch

    dev, ft = q.device, _torch_dtype(cfg)
    if cfg.G != 1:
        raise ValueError("the fused layer attention has one retrieval group (G = 1)")
    seq = (cfg.B, cfg.H, cfg.n_q * 64, 64)
    o = torch.empty_like(q) if o is None else o
    if need_lse:
        lse_sw = torch.empty(seq[:-1], dtype=torch.float32, device=dev) if lse_sw is None else lse_sw
        lse = torch.empty(cfg.shape("lse"), dtype=torch.float32, device=dev) if lse is None else lse
    for name, t in (("q", q), ("k_sw", k_sw), ("v_sw", v_sw), ("o", o)):
        _expect(name, t, seq, ft, dev)
    _expect("k", k, cfg.shape("kv"), ft, dev)
    _expect("v", v, cfg.shape("kv"), ft, dev)
    _expect("idx", idx, cfg.shape("sel"), torch.int32, dev)
    _expect("score", score, cfg.shape("sel"), torch.float32, dev)
    if need_lse:
        _expect("lse_sw", lse_sw, seq[:-1], torch.float32, dev)
        _expect("lse", lse, cfg.shape("lse"), torch.float32, dev)
    prob = cfg.problem()
    _check("gca_fused_forward", load().gca_fused_forward(
        ctypes.byref(prob), int(window), _ptr(q), _ptr(k_sw), _ptr(v_sw), _ptr(k), _ptr(v), _ptr(idx), _ptr(score),
        _ptr(o), _ptr(lse_sw) if need_lse else None, _ptr(lse) if need_lse else None, _stream()))
    return o, (lse_sw if need_lse else None), (lse if need_lse else None)


def fused_backward(cfg: Config, q, k_sw, v_sw, k, v, idx, score, o, lse_sw, lse, dout, window: int = 512,
                   ws=None, out=None):
    """gca_fused_backward: returns (dq, dk_sw, dv_sw, dk, dv, dscore)."""
    import torch

    dev, ft = q.device, _torch_dtype(cfg)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k_sw), torch.empty_like(v_sw), torch.empty_like(k),
               torch.empty_like(v), torch.empty(idx.shape, dtype=torch.float32, device=dev))
    dq, dk_sw, dv_sw, dk, dv, dscore = out
    seq = (cfg.B, cfg.H, cfg.n_q * 64, 64)
    for name, t in (("q", q), ("k_sw", k_sw), ("v_sw", v_sw), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk_sw", dk_sw), ("dv_sw", dv_sw)):
        _expect(name, t, seq, ft, dev)
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _expect(name, t, cfg.shape("kv"), ft, dev)
    _expect("idx", idx, cfg.shape("sel"), torch.int32, dev)
    _expect("score", score, cfg.shape("sel"), torch.float32, dev)
    _expect("dscore", dscore, cfg.shape("sel"), torch.float32, dev)
    _expect("lse_sw", lse_sw, seq[:-1], torch.float32, dev)
    _expect("lse", lse, cfg.shape("lse"), torch.float32, dev)
    if ws is None:
        ws, n = _workspace(OP_FUSED_BACKWARD, cfg, dev)
    else:
        n = _ws_bytes(ws, dev)
    prob = cfg.problem()
    _check("gca_fused_backward", load().gca_fused_backward(
        ctypes.byref(prob), int(window), _ptr(q), _ptr(k_sw), _ptr(v_sw), _ptr(k), _ptr(v), _ptr(idx), _ptr(score),
        _ptr(o), _ptr(lse_sw), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk_sw), _ptr(dv_sw), _ptr(dk), _ptr(dv),
        _ptr(dscore), _ptr(ws), n, _stream()))
    return dq, dk_sw, dv_sw, dk, dv, dscore


def fetched_config(cfg: Config) -> Config:
    """The problem over the chunks gca_fetch_chunks gathered: n_kv = G * n_q * K."""
    return dataclasses.replace(cfg, n_kv=cfg.G * cfg.n_q * cfg.topk)


def fetch_chunks(cfg: Config, idx, k, v, out=None):
    """gca_fetch_chunks: returns (k_out, v_out [B,H,G*n_q*K*64,64] on idx's device, idx_out).

    k, v may be device tensors or pinned host tensors (torch pin_memory)."""
    import torch

    n_c = cfg.G * cfg.n_q * cfg.topk
    dev = idx.device
    if out is None:
        shape = (cfg.B, cfg.H, n_c * 64, 64)
        out = (torch.empty(shape, dtype=k.dtype, device=dev), torch.empty(shape, dtype=v.dtype, device=dev),
               torch.empty_like(idx))
    k_out, v_out, idx_out = out
    ft = _torch_dtype(cfg)
    _expect("idx", idx, cfg.shape("sel"), torch.int32, dev)
    _expect("k", k, cfg.shape("kv"), ft, host_ok=True)
    _expect("v", v, cfg.shape("kv"), ft, host_ok=True)
    _expect("k_out", k_out, (cfg.B, cfg.H, n_c * 64, 64), ft, dev)
    _expect("v_out", v_out, (cfg.B, cfg.H, n_c * 64, 64), ft, dev)
    _expect("idx_out", idx_out, cfg.shape("sel"), torch.int32, dev)
    prob = cfg.problem()
    _check("gca_fetch_chunks", load().gca_fetch_chunks(ctypes.byref(prob), _ptr(idx), _ptr(k), _ptr(v), _ptr(k_out),
                                                       _ptr(v_out), _ptr(idx_out), _stream()))
    return k_out, v_out, idx_out


def profile_enable(on: bool = True):
    _check("gca_profile_enable", load().gca_profile_enable(1 if on else 0))


def profile_collect() -> dict:
    """{kernel name: (total ms, launches)} for launches since the last collect."""
    lib = load()
    cap = 16
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int64 * cap)()
    n = ctypes.c_int(0)
    _check("gca_profile_collect", lib.gca_profile_collect(cap, names, ms, cnt, ctypes.byref(n)))
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n.value, cap))}
