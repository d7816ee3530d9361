"""Plain, slow, obviously correct scaled-dot-product attention on the CPU in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never calls this.

What is computed is the plain definition of attention, with the full score matrix
materialised, because the tiled method reaches exactly the same result in real arithmetic:
the FlashAttention-T commentary (ai-stack.site, "FlashAttention-T：张量化注意力机制优化方案",
learning points) states the tiled algorithm keeps numerically the same result as standard
attention, and the xxqk.cn article ("Attention算子实战：从CUDA优化到昇腾/CANN部署",
section 2.2) describes it as the same QK^T -> softmax -> PV computed block by block.

Definition followed, per batch b and query head hq, with G = Hq / Hkv and hk = hq // G:

    S[i, j] = scale * sum_k Q[b, hq, i, k] * K[b, hk, j, k]
    S[i, j] = -inf               where causal and j > i
    P[i, j] = exp(S[i, j] - max_j S[i, j])
    O[b, hq, i, :] = sum_j P[i, j] * V[b, hk, j, :] / sum_j P[i, j]

Sources for each step:
  * max-subtracted exponent, row sum, then the product with V: the "fused attention"
    example on the FlashAttention-T page (code example 2) and the stable-softmax remark in
    section 2.2 of the xxqk.cn article;
  * ``(q * scale) @ k^T -> softmax -> @ v``: the ``raw_attention`` helper of the ewbang.com
    article (PyTorch FlashAttention for Turing, verification script);
  * tensor shapes [batch, heads, seq, head_dim], the causal flag and the default scale
    1/sqrt(head_dim): the API bullets of the jeff.news Aule-Attention article;
  * heads_q a multiple of heads_kv (grouped-query attention): same bullets, and the GQA /
    MQA examples of the jdon.com Aule-Attention article. The reading taken is that query
    head hq uses key/value head hq // G, i.e. K/V expanded with repeat_interleave;
  * varlen over packed ``qkv[total_tokens, 3, heads, head_dim]`` with cumulative
    ``cu_seqlens`` (``[0, 5, 12]`` means qkv[0:5] and qkv[5:12]), attention within each
    sequence only, output ``[total_tokens, heads, head_dim]``: the docstring of the
    varlen function in the ewbang.com article.

Readings where the pages are silent:
  * causal masking is top-left (key j is visible to query i iff j <= i) and needs
    seqlen_q == seqlen_k; the pages only show equal lengths;
  * decoding against a KV cache (FlashAttention-T commentary, FAQ 4, inference bullet:
    the KV cache is processed in blocks) is attention of Nq <= Nk new queries against all
    Nk cached keys; under causal masking the new queries are the last Nq positions of the
    sequence (bottom-right alignment: query i sees keys j <= i + Nk - Nq), so decoding them
    reproduces the last Nq rows of causal attention over the whole sequence;
  * the score modifiers of the varlen signature (window_size, softcap, alibi_slopes), which
    the ewbang.com varlen docstring names as parameters (sliding window (left, right), -1 for
    unbounded; a soft-capping value; ALiBi slopes of shape [heads] or [batch, heads]) without
    defining them, take their usual reading: with x = scale * q_i . k_j,
        x <- softcap * tanh(x / softcap)          if softcap > 0
        x <- x - slope[s, h] * |i - j|            if slopes are given (s = sequence, h = head)
    and key j is visible to query i iff it is inside the sequence, j <= i when causal,
    j >= i - left when left >= 0 and j <= i + right when right >= 0 (positions counted from
    the sequence start; causal with right = -1 or 0 is the same mask);
  * the scale is applied to the float64 dot product as the exact float32 value the
    library receives;
  * inputs are the values already rounded to the storage dtype (the generators do that);
    they are upcast exactly to float64 here.

Library primitives used as steps: numpy matmul (the dot products), numpy exp and sums.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _scale64(scale) -> float:
    # the library takes the scale as a C float: the oracle uses that exact value
    return float(np.float32(scale))


def _check_dense(q, k, v, causal):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [batch, heads, seq, head_dim]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("k and v must be [batch, heads_kv, seqlen_k, head_dim]")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("heads_q must be a multiple of heads_kv")
    if causal and Nq != Nk:
        raise ValueError("causal attention needs seqlen_q == seqlen_k")
    return B, Hq, Hkv, Nq, Nk, d


def _kv_head(hq: int, group: int) -> int:
    """Key/value head read by query head hq when ``group`` query heads share one."""
    return hq // group


def _causal_masked(rows: np.ndarray, n_keys: int) -> np.ndarray:
    """Boolean [len(rows), n_keys]: True where key j is in the future of query row i."""
    return np.arange(n_keys)[None, :] > np.asarray(rows)[:, None]


def _softmax_rows_times_v(S: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Row-wise max-subtracted softmax of S (float64, -inf = masked) times V."""
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    l = P.sum(axis=1, keepdims=True)
    return (P @ V) / l


def attention_ref(q, k, v, *, causal: bool, scale: float) -> np.ndarray:
    """Dense / GQA attention. q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d]. Returns float64
    [B,Hq,Nq,d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, Nq, Nk, d = _check_dense(q, k, v, causal)
    G = Hq // Hkv
    sc = _scale64(scale)
    out = np.empty((B, Hq, Nq, d), dtype=np.float64)
    if causal:
        masked = _causal_masked(np.arange(Nq), Nk)
    for b in range(B):
        for hq in range(Hq):
            hk = _kv_head(hq, G)
            S = sc * (q[b, hq] @ k[b, hk].T)
            if causal:
                S[masked] = -np.inf
            out[b, hq] = _softmax_rows_times_v(S, v[b, hk])
    return out


def attention_ref_rows(q, k, v, rows, *, causal: bool, scale: float) -> np.ndarray:
    """The same attention, for the query rows listed in ``rows`` only (the same rows for
    every batch and head). Returns float64 [B,Hq,len(rows),d]. Under causal masking row i
    sees keys 0..i."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, Nq, Nk, d = _check_dense(q, k, v, causal)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= Nq):
        raise ValueError("row index out of range")
    G = Hq // Hkv
    sc = _scale64(scale)
    out = np.empty((B, Hq, rows.size, d), dtype=np.float64)
    if causal:
        masked = _causal_masked(rows, Nk)
    for b in range(B):
        for hq in range(Hq):
            hk = _kv_head(hq, G)
            S = sc * (q[b, hq, rows] @ k[b, hk].T)
            if causal:
                S[masked] = -np.inf
            out[b, hq] = _softmax_rows_times_v(S, v[b, hk])
    return out


def _check_varlen(qkv, cu_seqlens):
    qkv = _f64(qkv)
    if qkv.ndim != 4 or qkv.shape[1] != 3:
        raise ValueError("qkv must be [total_tokens, 3, heads, head_dim]")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing, start at 0, length batch+1")
    if cu[-1] != qkv.shape[0]:
        raise ValueError("cu_seqlens[-1] must equal total_tokens")
    return qkv, cu


def _seq_as_dense(qkv, a, e):
    # [L, 3, H, d] slice -> three [1, H, L, d] tensors
    seg = qkv[a:e]
    return tuple(np.ascontiguousarray(seg[:, c].transpose(1, 0, 2))[None] for c in range(3))


def attention_ref_varlen(qkv, cu_seqlens, *, causal: bool, scale: float) -> np.ndarray:
    """Varlen attention over packed qkv [T,3,H,d]: each sequence cu[s]:cu[s+1] attends
    only within itself, with causal positions counted from the sequence start.
    Returns float64 [T,H,d]."""
    qkv, cu = _check_varlen(qkv, cu_seqlens)
    T, _, H, d = qkv.shape
    out = np.empty((T, H, d), dtype=np.float64)
    for s in range(cu.size - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        q, k, v = _seq_as_dense(qkv, a, e)
        out[a:e] = attention_ref(q, k, v, causal=causal, scale=scale)[0].transpose(1, 0, 2)
    return out


def attention_ref_varlen_rows(qkv, cu_seqlens, tokens, *, causal: bool,
                              scale: float) -> np.ndarray:
    """Varlen attention for the listed global token indices only. Returns float64
    [len(tokens),H,d] in the order given."""
    qkv, cu = _check_varlen(qkv, cu_seqlens)
    T, _, H, d = qkv.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size and (tokens.min() < 0 or tokens.max() >= T):
        raise ValueError("token index out of range")
    out = np.empty((tokens.size, H, d), dtype=np.float64)
    seq_of = np.searchsorted(cu, tokens, side="right") - 1
    for s in np.unique(seq_of):
        a, e = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero(seq_of == s)[0]
        local = tokens[sel] - a
        q, k, v = _seq_as_dense(qkv, a, e)
        res = attention_ref_rows(q, k, v, local, causal=causal, scale=scale)[0]
        out[sel] = res.transpose(1, 0, 2)
    return out


def _window_masked(rows, n_keys: int, left: int, right: int) -> np.ndarray:
    """Boolean [len(rows), n_keys]: True where key j lies outside the sliding window of
    query row i (before i - left when left >= 0, after i + right when right >= 0)."""
    rows = np.asarray(rows)[:, None]
    j = np.arange(n_keys)[None, :]
    out = np.zeros((rows.shape[0], n_keys), dtype=bool)
    if left >= 0:
        out |= j < rows - left
    if right >= 0:
        out |= j > rows + right
    return out


def _softcap(S: np.ndarray, cap: float) -> np.ndarray:
    """Soft capping of scaled scores: cap * tanh(S / cap), odd, slope 1 at 0, |.| < cap."""
    return cap * np.tanh(S / cap)


def _alibi_bias(rows, n_keys: int, slope: float) -> np.ndarray:
    """ALiBi: a penalty growing linearly with the distance between query i and key j."""
    return -slope * np.abs(np.asarray(rows)[:, None] - np.arange(n_keys)[None, :]).astype(np.float64)


def _check_mods(window, softcap, alibi_slopes, n_seqs, heads):
    left, right = (int(window[0]), int(window[1]))
    if left < -1 or right < -1:
        raise ValueError("window sizes must be >= -1")
    cap = float(np.float32(softcap))
    if not np.isfinite(cap) or cap < 0:
        raise ValueError("softcap must be finite and >= 0")
    slopes = None
    if alibi_slopes is not None:
        a = np.asarray(alibi_slopes, dtype=np.float32).astype(np.float64)
        if a.shape == (heads,):
            slopes = np.broadcast_to(a, (n_seqs, heads))
        elif a.shape == (n_seqs, heads):
            slopes = a
        else:
            raise ValueError("alibi_slopes must be [heads] or [batch, heads]")
    return left, right, cap, slopes


def attention_ref_varlen_mods(qkv, cu_seqlens, *, causal: bool, scale: float,
                              window=(-1, -1), softcap: float = 0.0, alibi_slopes=None,
                              tokens=None) -> np.ndarray:
    """Varlen attention with the score modifiers (sliding window, soft cap, ALiBi) in the
    order: scaled dot product, soft cap, ALiBi bias, masks (causal, window), softmax, times V.
    ``tokens`` limits the result to those global token indices (in the order given);
    otherwise every token. Returns float64 [T or len(tokens), H, d]."""
    qkv, cu = _check_varlen(qkv, cu_seqlens)
    T, _, H, d = qkv.shape
    left, right, cap, slopes = _check_mods(window, softcap, alibi_slopes, cu.size - 1, H)
    sc = _scale64(scale)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    if tok.size and (tok.min() < 0 or tok.max() >= T):
        raise ValueError("token index out of range")
    out = np.empty((tok.size, H, d), dtype=np.float64)
    seq_of = np.searchsorted(cu, tok, side="right") - 1
    for s in np.unique(seq_of):
        a, e = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero(seq_of == s)[0]
        rows = tok[sel] - a
        L = e - a
        masked = _window_masked(rows, L, left, right)
        if causal:
            masked |= _causal_masked(rows, L)
        for h in range(H):
            S = sc * (qkv[a + rows, 0, h] @ qkv[a:e, 1, h].T)
            if cap > 0:
                S = _softcap(S, cap)
            if slopes is not None:
                S = S + _alibi_bias(rows, L, slopes[s, h])
            S[masked] = -np.inf
            out[sel, h] = _softmax_rows_times_v(S, qkv[a:e, 2, h])
    return out


def _decode_masked(n_queries: int, n_keys: int) -> np.ndarray:
    """Boolean [n_queries, n_keys]: True where key j lies after query i, the queries being
    the last n_queries positions of an n_keys-long sequence."""
    shift = n_keys - n_queries
    return np.arange(n_keys)[None, :] > (np.arange(n_queries) + shift)[:, None]


def attention_ref_decode(q, k, v, *, causal: bool, scale: float) -> np.ndarray:
    """Attention of Nq new queries against an Nk-long key/value cache, q: [B,Hq,Nq,d],
    k, v: [B,Hkv,Nk,d], Nq <= Nk when causal, with bottom-right causal alignment (query i
    is sequence position Nk - Nq + i). Without masking it is attention_ref. Returns float64
    [B,Hq,Nq,d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, Nq, Nk, d = _check_dense(q, k, v, False)
    if causal and Nq > Nk:
        raise ValueError("causal decoding needs seqlen_q <= seqlen_k")
    G = Hq // Hkv
    sc = _scale64(scale)
    out = np.empty((B, Hq, Nq, d), dtype=np.float64)
    if causal:
        masked = _decode_masked(Nq, Nk)
    for b in range(B):
        for hq in range(Hq):
            hk = _kv_head(hq, G)
            S = sc * (q[b, hq] @ k[b, hk].T)
            if causal:
                S[masked] = -np.inf
            out[b, hq] = _softmax_rows_times_v(S, v[b, hk])
    return out


# ---------------------------------------------------------------- log-sum-exp and gradients
#
# Training through the tiled forward (FlashAttention-T commentary, FAQ 4, training bullet:
# the forward keeps no score matrix and the backward recomputes it) needs, per query row,
# the log-sum-exp of the scaled scores, and the gradients of O with respect to Q, K and V.
# Both have plain definitions, written out here:
#
#   LSE[i]  = log sum_j exp(S[i, j])                      (S scaled and masked as above)
#   P       = exp(S - LSE)                                (= softmax(S))
#   dV      = P^T dO
#   dP      = dO V^T
#   dS      = P * (dP - rowsum(dP * P))                   (softmax Jacobian, rowwise)
#   dQ      = scale * dS K,     dK = scale * dS^T Q
#
# With grouped-query attention, the gradient of a shared key/value head is the sum over the
# query heads that read it.

def _lse_rows(S: np.ndarray) -> np.ndarray:
    m = S.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]


def attention_ref_lse(q, k, v, *, causal: bool, scale: float) -> np.ndarray:
    """Per-row log-sum-exp (natural log) of the scaled, masked scores, float64 [B,Hq,Nq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, Nq, Nk, d = _check_dense(q, k, v, causal)
    G = Hq // Hkv
    sc = _scale64(scale)
    out = np.empty((B, Hq, Nq), dtype=np.float64)
    if causal:
        masked = _causal_masked(np.arange(Nq), Nk)
    for b in range(B):
        for hq in range(Hq):
            S = sc * (q[b, hq] @ k[b, _kv_head(hq, G)].T)
            if causal:
                S[masked] = -np.inf
            out[b, hq] = _lse_rows(S)
    return out


def _softmax_backward(P: np.ndarray, dP: np.ndarray) -> np.ndarray:
    """dS = P * (dP - rowsum(dP * P)): the gradient through a row-wise softmax."""
    return P * (dP - (dP * P).sum(axis=1, keepdims=True))


def attention_ref_bwd(q, k, v, do, *, causal: bool, scale: float):
    """Gradients of O = attention(q, k, v) for the output gradient ``do`` [B,Hq,Nq,d].
    Returns float64 (dq [B,Hq,Nq,d], dk [B,Hkv,Nk,d], dv [B,Hkv,Nk,d])."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Hkv, Nq, Nk, d = _check_dense(q, k, v, causal)
    if do.shape != q.shape:
        raise ValueError("do must have the shape of q")
    G = Hq // Hkv
    sc = _scale64(scale)
    dq = np.zeros((B, Hq, Nq, d))
    dk = np.zeros((B, Hkv, Nk, d))
    dv = np.zeros((B, Hkv, Nk, d))
    if causal:
        masked = _causal_masked(np.arange(Nq), Nk)
    for b in range(B):
        for hq in range(Hq):
            hk = _kv_head(hq, G)
            S = sc * (q[b, hq] @ k[b, hk].T)
            if causal:
                S[masked] = -np.inf
            P = np.exp(S - _lse_rows(S)[:, None])
            dv[b, hk] += P.T @ do[b, hq]
            dP = do[b, hq] @ v[b, hk].T
            dS = _softmax_backward(P, dP)
            dq[b, hq] = sc * (dS @ k[b, hk])
            dk[b, hk] += sc * (dS.T @ q[b, hq])
    return dq, dk, dv
