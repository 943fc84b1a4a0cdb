"""Plain CPU oracle for Grouped Cross-Attention (GCA) with causal chunk retrieval.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this module.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this module imports nothing
from the product path.

Sources (pages on "Efficient Length-Generalizable Attention via Causal Retrieval for
Long-Context Language Modeling", ICML 2025):
  [Notes]  zhaoyang97.github.io Paper-Notes page on the paper.
  [Card]   paperdance.org card for arXiv 2410.01651 (English abstract).
  [Forum]  openreview.net forum page of the paper (abstract).
Sections of [Notes] are cited by their heading, e.g. [Notes, Key designs: GCA].

What is computed (all arithmetic in IEEE float64 unless a step says float32):
  * chunking: S = 64 tokens per chunk            [Notes, Overall framework]
  * causal retrieval: the landmark of chunk i is scored against the landmark of every
    strictly earlier chunk j; the top-k are kept   [Notes, Key designs: causal retrieval]
  * Gumbel top-k (training): noise is added to the scores before the top-k and only
    changes which chunks are selected              [Notes, Key designs: Gumbel top-k]
  * GCA: every token of the next chunk attends to each retrieved chunk with its own
    softmax; the k outputs are fused with a softmax of the retrieval scores, so the
    scores receive gradients                       [Notes, Key designs: GCA],
                                                   [Notes, Background: entry point]
  * K/V are shared by all retrieval groups         [Notes, Key designs: GCA, last item]
  * the retrieved chunks' K/V may be kept in host memory and loaded back at retrieval
    (fetch_chunks)                                 [Notes, Key designs: memory-offload inference]
  * tokens generated one at a time attend to the chunks retrieved once for their chunk
    (decode_tokens)                                same
  * sliding-window self-attention, W = 512, beside the retrieval
    (sw_attention, sw_attention_backward)          [Notes, Loss / training strategy]
  * the layer's two attentions summed (fused_attention, fused_attention_backward)     same

Readings taken where the pages leave a step open (each is listed in the design doc):
  R1  score s_ij = fl32(fl32(sum_d lq[i,d]*lk[j,d]) * score_scale) + 0.0f, the sum taken in
      float64 sequentially over d = 0..63 (every product of bf16/fp32 values is exact in
      float64, so this fixes one bit pattern per score).
  R2  one retrieval per (group, batch) shared by every head.
  R3  candidates of row i are j < min(i, n_kv); Q chunk t uses row t - shift.
  R4  ties are broken toward the lower chunk index; -0 is canonicalised to +0.
  R5  Gumbel noise g = -ln_s(-ln_s(u)), u from Philox4x64-10 (Salmon et al., SC'11) with
      key (seed, 0) and counter (j, i, (g << 32) | b, 0); ln_s is the fixed atanh-series
      logarithm below.  Perturbed r = fl32(s + fl32(tau * g)).
  R6  fusion weights are softmax over the valid slots of the clean scores; invalid slots
      carry idx = -1 and score = -inf; a token with no valid slot gets output 0.
  R7  attention inside a retrieved chunk is full (non-causal) over its 64 tokens, with
      z = attn_scale * <q, k>, no positional bias.
  R8  the fetched chunks form a compact buffer, slot (g, b, r, s) -> chunk (g n_q + r) K + s.
  R9  decoding the first n tokens of a chunk gives the chunk forward's first n rows.
  R10 the sliding window of token i is tokens max(0, i - W + 1) .. i (causal, itself included),
      one softmax of attn_scale <q, k>, no positional bias.
  R11 in a layer that runs both, the window and GCA (one retrieval group) read the same queries
      and their outputs are summed.

Parity pins: every function here is pinned in tests/test_oracle_pins.py against brute force,
library routines, closed forms, invariants and finite differences.
"""

from __future__ import annotations

import numpy as np

CHUNK = 64  # S, [Notes, Overall framework]

# ---------------------------------------------------------------------------------------
# Counter-based random numbers: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel
# Random Numbers: As Easy as 1, 2, 3", SC'11).  Written from the published definition:
# 10 rounds of two 64x64->128 multiplications, with the key bumped by the two Weyl
# constants between rounds.
# ---------------------------------------------------------------------------------------
_PHILOX_M0 = np.uint64(0xD2E7470EE14C6C93)
_PHILOX_M1 = np.uint64(0xCA5A826395121157)
_PHILOX_W0 = np.uint64(0x9E3779B97F4A7C15)  # golden ratio
_PHILOX_W1 = np.uint64(0xBB67AE8584CAA73B)  # sqrt(3) - 1
_LO32 = np.uint64(0xFFFFFFFF)
_SH32 = np.uint64(32)


def _mulhilo64(a: np.ndarray, b: np.uint64):
    """Full 128-bit product of uint64 arrays, returned as (hi, lo), via 32-bit limbs."""
    a0, a1 = a & _LO32, a >> _SH32
    b0, b1 = np.uint64(b) & _LO32, np.uint64(b) >> _SH32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _SH32) + (p01 & _LO32) + (p10 & _LO32)
    lo = (p00 & _LO32) | (mid << _SH32)
    hi = p11 + (p01 >> _SH32) + (p10 >> _SH32) + (mid >> _SH32)
    return hi, lo


def philox4x64_10(counter: np.ndarray, key) -> np.ndarray:
    """Philox4x64 with 10 rounds.  counter: uint64 [..., 4]; key: two uint64.  -> [..., 4]."""
    x = np.array(counter, dtype=np.uint64, copy=True)
    x0, x1, x2, x3 = x[..., 0], x[..., 1], x[..., 2], x[..., 3]
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    with np.errstate(over="ignore"):
        for rnd in range(10):
            hi0, lo0 = _mulhilo64(x0, _PHILOX_M0)
            hi1, lo1 = _mulhilo64(x2, _PHILOX_M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
            if rnd != 9:
                k0 = k0 + _PHILOX_W0
                k1 = k1 + _PHILOX_W1
    return np.stack([x0, x1, x2, x3], axis=-1)


# ---------------------------------------------------------------------------------------
# ln_s: a logarithm defined by a fixed sequence of IEEE float64 operations (no fused
# multiply-add), so that two faithful implementations agree bit for bit.  Textbook
# identity ln(m) = 2 atanh((m-1)/(m+1)) = 2 f (1 + f^2/3 + f^4/5 + ...), with m reduced
# to [sqrt(1/2), sqrt(2)) so that |f| <= 0.1716 and 12 terms reach float64 precision.
# ---------------------------------------------------------------------------------------
_LN2 = float.fromhex("0x1.62e42fefa39efp-1")        # ln 2 rounded to float64
_SQRT_HALF = float.fromhex("0x1.6a09e667f3bcdp-1")  # sqrt(1/2) rounded to float64
_ATANH_C = [1.0 / (2 * n + 1) for n in range(12)]   # c_n = fl64(1 / (2n + 1))


def ln_s(x: np.ndarray) -> np.ndarray:
    """ln_s(x) for finite x > 0, float64, evaluated in the fixed order stated above."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, m in [0.5, 1)
    small = m < _SQRT_HALF
    m = np.where(small, m * 2.0, m)          # exact
    e = np.where(small, e - 1, e).astype(np.float64)
    f = (m - 1.0) / (m + 1.0)
    z = f * f
    p = np.full_like(f, _ATANH_C[11])
    for n in range(10, -1, -1):
        p = p * z + _ATANH_C[n]              # two roundings: multiply, then add
    return e * _LN2 + (2.0 * f) * p


def gumbel_noise(seed: int, g: int, b: int, i, j) -> np.ndarray:
    """Standard Gumbel noise for the (g, b, row i, candidate j) pairs, rounded to float32.

    u = ((x >> 12) + 1/2) * 2^-52 with x the first Philox output word, so u is exact and in
    (0, 1); g = -ln_s(-ln_s(u)) (inverse-CDF sampling of the standard Gumbel law).
    """
    i = np.asarray(i, dtype=np.uint64)
    j = np.asarray(j, dtype=np.uint64)
    i, j = np.broadcast_arrays(i, j)
    ctr = np.zeros(i.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = j
    ctr[..., 1] = i
    ctr[..., 2] = (np.uint64(g) << _SH32) | np.uint64(b)
    x = philox4x64_10(ctr, (np.uint64(seed), np.uint64(0)))[..., 0]
    u = ((x >> np.uint64(12)).astype(np.float64) + 0.5) * (2.0 ** -52)
    return (-ln_s(-ln_s(u))).astype(np.float32)


# ---------------------------------------------------------------------------------------
# Causal retrieval  [Notes, Key designs: causal retrieval; Gumbel top-k]
# ---------------------------------------------------------------------------------------
def canonical_scores(lq_rows: np.ndarray, lk_rows: np.ndarray, score_scale: float) -> np.ndarray:
    """Reading R1.  lq_rows [n, dl], lk_rows [m, dl] (values exactly representable in
    float64) -> float32 [n, m]: fl32(fl32(sequential float64 dot) * fl32(score_scale)) + 0."""
    lq_rows = np.asarray(lq_rows, dtype=np.float64)
    lk_rows = np.asarray(lk_rows, dtype=np.float64)
    acc = np.zeros((lq_rows.shape[0], lk_rows.shape[0]), dtype=np.float64)
    for d in range(lq_rows.shape[1]):
        acc = acc + lq_rows[:, d, None] * lk_rows[None, :, d]
    s = acc.astype(np.float32) * np.float32(score_scale)
    return (s + np.float32(0.0)).astype(np.float32)


def retrieve(lq, lk, topk, *, score_scale=0.125, use_gumbel=False, seed=0, tau=1.0,
             q_chunk_base=0, n_kv=None):
    """Top-k past chunks per retrieval row.

    lq [G, B, n_q, dl], lk [G, B, n_kv, dl] -> idx int32 [G, B, n_q, K] (descending by the
    possibly-perturbed score r, ties toward lower j, padded with -1) and score float32
    [G, B, n_q, K] (the clean score s of each slot, padded with -inf).
    Row r is global chunk i = q_chunk_base + r and scores j < min(i, n_kv)  (R3).
    """
    lq = np.asarray(lq, dtype=np.float64)
    lk = np.asarray(lk, dtype=np.float64)
    G, B, n_q, _ = lq.shape
    if n_kv is None:
        n_kv = lk.shape[2]
    idx = np.full((G, B, n_q, topk), -1, dtype=np.int32)
    score = np.full((G, B, n_q, topk), -np.inf, dtype=np.float32)
    tau32 = np.float32(tau)
    for g in range(G):
        for b in range(B):
            if n_q == 0:
                continue
            top_i = q_chunk_base + n_q - 1
            m = min(top_i, n_kv)
            s_all = canonical_scores(lq[g, b], lk[g, b, :m], score_scale) if m > 0 else None
            for r in range(n_q):
                i = q_chunk_base + r
                nc = min(i, n_kv)
                if nc <= 0:
                    continue
                j = np.arange(nc)
                s = s_all[r, :nc]
                if use_gumbel:
                    noise = gumbel_noise(seed, g, b, i, j)
                    key = (s + (tau32 * noise).astype(np.float32)).astype(np.float32)
                    key = key + np.float32(0.0)
                else:
                    key = s
                order = np.lexsort((j, -key.astype(np.float64)))  # r descending, j ascending
                take = order[: min(topk, nc)]
                idx[g, b, r, : take.size] = j[take]
                score[g, b, r, : take.size] = s[take]
    return idx, score


# ---------------------------------------------------------------------------------------
# Grouped cross-attention forward / backward  [Notes, Key designs: GCA]
# ---------------------------------------------------------------------------------------
def _fusion_weights(score_row: np.ndarray, idx_row: np.ndarray):
    """Softmax over the valid slots of one row's clean scores (reading R6)."""
    valid = idx_row >= 0
    w = np.zeros(score_row.shape, dtype=np.float64)
    if valid.any():
        s = score_row[valid].astype(np.float64)
        e = np.exp(s - s.max())
        w[valid] = e / e.sum()
    return w, valid


def forward(q, k, v, idx, score, *, shift=1, attn_scale=0.125, return_slots=False):
    """O = sum_k w_k softmax(attn_scale Q K_jk^T) V_jk per query chunk.

    q [G, B, H, n_q*64, d]; k, v [B, H, n_kv*64, d]; idx/score [G, B, n_q, K].
    Returns o [G, B, H, n_q*64, d] (float64), lse [G, B, H, n_q*64, K] (float64, -inf on
    invalid slots) and, if return_slots, the per-slot outputs [G, B, H, n_q*64, K, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    G, B, H, Lq, d = q.shape
    n_q = Lq // CHUNK
    K = idx.shape[-1]
    sc = float(np.float32(attn_scale))
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.full((G, B, H, Lq, K), -np.inf, dtype=np.float64)
    slots = np.zeros((G, B, H, Lq, K, d), dtype=np.float64) if return_slots else None
    for g in range(G):
        for b in range(B):
            for t in range(n_q):
                row = t - shift
                if row < 0:
                    continue
                w, valid = _fusion_weights(score[g, b, row], idx[g, b, row])
                rows = slice(t * CHUNK, (t + 1) * CHUNK)
                qt = q[g, b, :, rows, :]                          # [H, 64, d]
                for kk in range(K):
                    if not valid[kk]:
                        continue
                    j = int(idx[g, b, row, kk])
                    keys = slice(j * CHUNK, (j + 1) * CHUNK)
                    z = sc * np.matmul(qt, np.swapaxes(k[b, :, keys, :], -1, -2))  # [H,64,64]
                    zmax = z.max(axis=-1, keepdims=True)
                    ez = np.exp(z - zmax)
                    den = ez.sum(axis=-1, keepdims=True)
                    a = ez / den
                    ok = np.matmul(a, v[b, :, keys, :])           # [H, 64, d]
                    lse[g, b, :, rows, kk] = (zmax + np.log(den))[..., 0]
                    o[g, b, :, rows, :] += w[kk] * ok
                    if return_slots:
                        slots[g, b, :, rows, kk, :] = ok
    if return_slots:
        return o, lse, slots
    return o, lse


def backward(q, k, v, idx, score, dout, *, shift=1, attn_scale=0.125):
    """Gradients of sum(dout * O) with the retrieved indices held fixed.

    Returns dq [G,B,H,Lq,d], dk, dv [B,H,Lk,d] (summed over groups and over every
    (token, slot) that retrieved a chunk) and dscore [G,B,n_q,K] (0 on invalid slots and on
    rows that feed no query chunk), all float64.
      e_{t,k}   = <dO_t, O_{t,k}>,       dw_k = sum over the chunk's tokens and heads of e,
      dscore_k  = w_k (dw_k - sum_k' w_k' dw_k'),
      dz_u      = w_k a_u (<dO_t, v_u> - e_{t,k}),
      dq_t     += attn_scale sum_u dz_u k_u,  dk_u += attn_scale dz_u q_t,
      dv_u     += w_k a_u dO_t.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    G, B, H, Lq, d = q.shape
    n_q = Lq // CHUNK
    K = idx.shape[-1]
    sc = float(np.float32(attn_scale))
    dq = np.zeros_like(q)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    dscore = np.zeros(idx.shape, dtype=np.float64)
    for g in range(G):
        for b in range(B):
            for t in range(n_q):
                row = t - shift
                if row < 0:
                    continue
                w, valid = _fusion_weights(score[g, b, row], idx[g, b, row])
                if not valid.any():
                    continue
                rows = slice(t * CHUNK, (t + 1) * CHUNK)
                qt = q[g, b, :, rows, :]
                dot = dout[g, b, :, rows, :]
                dw = np.zeros(K, dtype=np.float64)
                for kk in range(K):
                    if not valid[kk]:
                        continue
                    j = int(idx[g, b, row, kk])
                    keys = slice(j * CHUNK, (j + 1) * CHUNK)
                    kj, vj = k[b, :, keys, :], v[b, :, keys, :]
                    z = sc * np.matmul(qt, np.swapaxes(kj, -1, -2))
                    ez = np.exp(z - z.max(axis=-1, keepdims=True))
                    a = ez / ez.sum(axis=-1, keepdims=True)            # [H, 64, 64]
                    dpp = np.matmul(dot, np.swapaxes(vj, -1, -2))       # <dO_t, v_u>
                    e = (a * dpp).sum(axis=-1, keepdims=True)          # <dO_t, O_{t,k}>
                    dw[kk] = e.sum()
                    dz = w[kk] * a * (dpp - e)
                    dq[g, b, :, rows, :] += sc * np.matmul(dz, kj)
                    dk[b, :, keys, :] += sc * np.matmul(np.swapaxes(dz, -1, -2), qt)
                    dv[b, :, keys, :] += w[kk] * np.matmul(np.swapaxes(a, -1, -2), dot)
                wdw = float((w * dw).sum())
                dscore[g, b, row] = np.where(valid, w * (dw - wdw), 0.0)
    return dq, dk, dv, dscore


# ---------------------------------------------------------------------------------------
# Landmark gradients
# ---------------------------------------------------------------------------------------
def landmark_backward(lq, lk, idx, dscore, *, score_scale=0.125, q_chunk_base=0, n_kv=None):
    """Gradients that reach the landmarks through the retrieval scores, selection held fixed.

    The retrieval scores weight the fused outputs, so the language-model loss differentiates
    them [Notes, Key designs: GCA]; a score relates the landmark of a chunk to the landmark of
    an earlier chunk [Notes, Key designs: causal retrieval].  With s_ij = score_scale <lq_i, lk_j>
    (reading R1 without its float32 roundings, which carry no gradient) and dscore the gradient of
    the loss with respect to the clean score of each slot:
      dlq[g,b,r] = score_scale * sum_k dscore[g,b,r,k] lk[g,b,idx[g,b,r,k]]
      dlk[g,b,j] = score_scale * sum over (r, k) with idx[g,b,r,k] = j of dscore[g,b,r,k] lq[g,b,r]
    Slots count when 0 <= idx < min(q_chunk_base + r, n_kv) (the candidates of reading R3).
    Returns float64 arrays shaped like lq and lk.
    """
    lq = np.asarray(lq, dtype=np.float64)
    lk = np.asarray(lk, dtype=np.float64)
    dscore = np.asarray(dscore, dtype=np.float64)
    G, B, n_q, _ = lq.shape
    if n_kv is None:
        n_kv = lk.shape[2]
    K = idx.shape[-1]
    scale = float(np.float32(score_scale))
    dlq = np.zeros_like(lq)
    dlk = np.zeros_like(lk)
    for g in range(G):
        for b in range(B):
            for r in range(n_q):
                limit = min(q_chunk_base + r, n_kv)
                for kk in range(K):
                    j = int(idx[g, b, r, kk])
                    if 0 <= j < limit:
                        dlq[g, b, r] += dscore[g, b, r, kk] * lk[g, b, j]
                        dlk[g, b, j] += dscore[g, b, r, kk] * lq[g, b, r]
    return scale * dlq, scale * dlk


def fetch_chunks(idx, k, v, n_kv=None):
    """The retrieved chunks' K/V tiles, gathered for the chunk that attends to them.

    In inference the K/V of past chunks may be kept in host memory and the chunks a retrieval
    selects are loaded back before the next chunk attends to them [Notes, Key designs:
    memory-offload inference].  k, v [B, H, n_kv*64, d]; idx [G, B, n_q, K].  Slot (g, b, r, s)
    with 0 <= j = idx[g,b,r,s] < n_kv gets compact chunk c = (g*n_q + r)*K + s:
      k_out[b, h, c] = k[b, h, j],  v_out[b, h, c] = v[b, h, j],  idx_out[g, b, r, s] = c,
    and idx_out = -1 elsewhere (those tiles stay zero).  Returns (k_out, v_out, idx_out) with
    k_out, v_out [B, H, G*n_q*K*64, d] in the input dtype and idx_out int32.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    G, B, n_q, K = idx.shape
    _, H, L, d = k.shape
    if n_kv is None:
        n_kv = L // CHUNK
    n_c = G * n_q * K
    k_out = np.zeros((B, H, n_c * CHUNK, d), dtype=k.dtype)
    v_out = np.zeros((B, H, n_c * CHUNK, d), dtype=v.dtype)
    idx_out = np.full(idx.shape, -1, dtype=np.int32)
    for g in range(G):
        for b in range(B):
            for r in range(n_q):
                for s in range(K):
                    j = int(idx[g, b, r, s])
                    if not 0 <= j < n_kv:
                        continue
                    c = (g * n_q + r) * K + s
                    idx_out[g, b, r, s] = c
                    k_out[b, :, c * CHUNK:(c + 1) * CHUNK] = k[b, :, j * CHUNK:(j + 1) * CHUNK]
                    v_out[b, :, c * CHUNK:(c + 1) * CHUNK] = v[b, :, j * CHUNK:(j + 1) * CHUNK]
    return k_out, v_out, idx_out


def decode_tokens(q_tok, k, v, idx, score, *, shift=0, attn_scale=0.125):
    """Token-level decode: the first n tokens of a query chunk attend to its retrieved chunks.

    While a chunk's tokens are generated one at a time, each new token attends to the chunks
    retrieved once for the chunk [Notes, Key designs: GCA; Key designs: memory-offload
    inference].  Attention is per query token, so these are the first n rows of the chunk forward
    of a chunk whose first n tokens are q_tok: q_tok [G, B, H, n, d] (n <= 64) with
    idx/score [G, B, 1, K] -> o [G, B, H, n, d] (float64).
    """
    q_tok = np.asarray(q_tok, dtype=np.float64)
    G, B, H, n, d = q_tok.shape
    q = np.zeros((G, B, H, CHUNK, d))
    q[:, :, :, :n] = q_tok
    o, _ = forward(q, k, v, idx, score, shift=shift, attn_scale=attn_scale)
    return o[:, :, :, :n]


def sw_attention(q, k, v, window, *, attn_scale=0.125):
    """Sliding-window causal self-attention, the local attention beside GCA.

    [Notes, Loss / training strategy]: sliding-window self-attention with W = 512 beside the top-k
    retrieval.  Token i attends to tokens max(0, i - W + 1) .. i under one softmax of
    z = attn_scale <q_i, k_j>.  q, k, v [B, H, L, d] -> o [B, H, L, d] and the natural
    log-sum-exp lse [B, H, L], both float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    o = np.zeros((B, H, L, d))
    lse = np.zeros((B, H, L))
    for i in range(L):
        lo = max(0, i - window + 1)
        z = attn_scale * np.einsum("bhd,bhjd->bhj", q[:, :, i], k[:, :, lo:i + 1])
        m = z.max(axis=-1, keepdims=True)
        e = np.exp(z - m)
        s = e.sum(axis=-1, keepdims=True)
        o[:, :, i] = np.einsum("bhj,bhjd->bhd", e / s, v[:, :, lo:i + 1])
        lse[:, :, i] = (m + np.log(s))[..., 0]
    return o, lse


def sw_attention_backward(q, k, v, dout, window, *, attn_scale=0.125):
    """Gradients of sw_attention: with P the window softmax of token i, dP_ij = <dout_i, v_j> and
    D_i = sum_j P_ij dP_ij = <dout_i, o_i>,
      dS_ij = P_ij (dP_ij - D_i),  dq_i = attn_scale sum_j dS_ij k_j,
      dk_j = attn_scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i.
    All float64; returns (dq, dk, dv) shaped like q."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, L, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i in range(L):
        lo = max(0, i - window + 1)
        z = attn_scale * np.einsum("bhd,bhjd->bhj", q[:, :, i], k[:, :, lo:i + 1])
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        P = e / e.sum(axis=-1, keepdims=True)
        dP = np.einsum("bhd,bhjd->bhj", dout[:, :, i], v[:, :, lo:i + 1])
        D = (P * dP).sum(axis=-1, keepdims=True)
        dS = P * (dP - D)
        dq[:, :, i] = attn_scale * np.einsum("bhj,bhjd->bhd", dS, k[:, :, lo:i + 1])
        dk[:, :, lo:i + 1] += attn_scale * dS[..., None] * q[:, :, i][:, :, None, :]
        dv[:, :, lo:i + 1] += P[..., None] * dout[:, :, i][:, :, None, :]
    return dq, dk, dv


def fused_attention(q, k_sw, v_sw, k, v, idx, score, window, *, shift=1, attn_scale=0.125):
    """A layer's local window and GCA summed (reading R11): the layers that run GCA also run
    sliding-window self-attention beside the retrieval [Notes, Loss / training strategy].
      o = sw_attention(q, k_sw, v_sw, window) + forward(q, k, v, idx, score) (one group)
    q, k_sw, v_sw [B, H, L, d]; k, v [B, H, n_kv*64, d]; idx, score [1, B, n_q, K].
    Returns o [B, H, L, d], the window's lse [B, H, L] and the GCA lse [1, B, H, L, K] (float64)."""
    o_sw, lse_sw = sw_attention(q, k_sw, v_sw, window, attn_scale=attn_scale)
    o_g, lse = forward(np.asarray(q)[None], k, v, idx, score, shift=shift, attn_scale=attn_scale)
    return o_sw + o_g[0], lse_sw, lse


def fused_attention_backward(q, k_sw, v_sw, k, v, idx, score, dout, window, *, shift=1, attn_scale=0.125):
    """Gradients of sum(dout * fused_attention(...)): the gradient of a sum of the two maps.
    Returns dq (both parts), dk_sw, dv_sw (the window's), dk, dv, dscore (GCA's), float64."""
    dq_sw, dk_sw, dv_sw = sw_attention_backward(q, k_sw, v_sw, dout, window, attn_scale=attn_scale)
    dq_g, dk, dv, dscore = backward(np.asarray(q)[None], k, v, idx, score, np.asarray(dout)[None], shift=shift,
                                    attn_scale=attn_scale)
    return dq_sw + dq_g[0], dk_sw, dv_sw, dk, dv, dscore
