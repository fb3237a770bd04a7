"""Brute-force dense-matrix attention for tiny inputs (NumPy/SciPy, float64).

TEST INFRASTRUCTURE ONLY.  A second, independently written reference used to
pin the C oracle on tiny problems: it first un-pages every request into a
dense ``[kv_len, H_kv, D]`` array by walking the page table, then builds the
full ``[qo_len, kv_len]`` boolean visibility matrix (bottom-right aligned
causal band of width W+1, as the sliding-window convention of AMD-Ecosystem
flashinfer PR 234, "Why each fix" 1, defines it) and evaluates the softmax and
log-sum-exp with ``scipy.special``.  It shares no code with ``oracle.c``.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp, softmax


def _to_f64(t) -> np.ndarray:
    import torch

    return t.detach().cpu().to(torch.float64).numpy()


def unpage(cache: np.ndarray, kv_indptr, kv_indices, kv_last_page_len, b: int) -> np.ndarray:
    """Dense [kv_len, H_kv, D] keys (or values) of request ``b``."""
    pages = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
    if len(pages) == 0:
        return cache[:0].reshape(0, *cache.shape[2:])
    full = np.concatenate([cache[p] for p in pages], axis=0)  # [npages*P, H_kv, D]
    n = (len(pages) - 1) * cache.shape[1] + kv_last_page_len[b]
    return full[:n]


def visibility(qo_len: int, kv_len: int, causal: bool, window_left: int) -> np.ndarray:
    """Boolean [qo_len, kv_len]: row i (position kv_len-qo_len+i) sees column j."""
    pos = np.arange(kv_len - qo_len, kv_len)[:, None]
    key = np.arange(kv_len)[None, :]
    vis = np.ones((qo_len, kv_len), dtype=bool)
    if causal:
        vis &= key <= pos
    if window_left >= 0:
        vis &= key >= pos - window_left
    return vis


def attention(case, window_left=None):
    """(O [nnz_qo,H_q,D], LSE [nnz_qo,H_q]) for a ``synth.Case``, float64.
    A positive ``case.logits_soft_cap`` c replaces each scaled logit x by
    c * tanh(x / c) (numpy's tanh)."""
    W = case.window_left if window_left is None else window_left
    cap = case.logits_soft_cap
    q = _to_f64(case.q)
    kc = _to_f64(case.k_cache)
    vc = _to_f64(case.v_cache)
    qo = case.qo_indptr.cpu().numpy()
    kvp = case.kv_indptr.cpu().numpy()
    kvi = case.kv_indices.cpu().numpy()
    last = case.kv_last_page_len.cpu().numpy()
    G = case.num_qo_heads // case.num_kv_heads
    o = np.zeros_like(q)
    lse = np.full(q.shape[:2], -np.inf)
    for b in range(len(kvp) - 1):
        K = unpage(kc, kvp, kvi, last, b)
        V = unpage(vc, kvp, kvi, last, b)
        qb = q[qo[b]:qo[b + 1]]
        vis = visibility(len(qb), len(K), case.causal, W)
        for h in range(case.num_qo_heads):
            logits = case.sm_scale * (qb[:, h, :] @ K[:, h // G, :].T)  # [qo, kv]
            if cap > 0:
                logits = cap * np.tanh(logits / cap)
            for i in range(len(qb)):
                if not vis[i].any():
                    continue
                lse[qo[b] + i, h] = logsumexp(logits[i][vis[i]])
                w = softmax(logits[i][vis[i]])
                o[qo[b] + i, h] = w @ V[vis[i], h // G, :]
    return o, lse
