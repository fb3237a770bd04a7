"""Helpers for the GPU parity tests: run a synth.Case through the C ABI and
compare against the CPU oracle with the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_sliding_amd import pkvs as P
from paged_kv_sliding_amd.synth import Case

# Tolerances (compared in fp32): |O - O_ref| <= 2e-2, |LSE - LSE_ref| <= 1e-3.
O_TOL = 2e-2
LSE_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)


def kv_dtype_of(case: Case):
    """The 8-bit cache type of a case, or None when the cache is in its dtype."""
    return case.k_cache.dtype if case.k_cache.dtype in (torch.float8_e4m3fn,
                                                        torch.float8_e5m2) else None


def make_attention(case: Case, window_left=None, fixed_split_size=None, disable_split_kv=False,
                   batch_capacity=None, kv_capacity=None, qo_capacity=None, prefill_variant=0,
                   decode_waves=0):
    W = case.window_left if window_left is None else window_left
    kind = P.PKVS_DECODE if case.is_decode else P.PKVS_PREFILL
    split = case.fixed_split_size if fixed_split_size is None else fixed_split_size
    return P.BatchAttention(
        kind, num_qo_heads=case.num_qo_heads, num_kv_heads=case.num_kv_heads,
        head_dim=case.head_dim, page_size=case.page_size, dtype=case.dtype, window_left=W,
        causal=case.causal, fixed_split_size=split, disable_split_kv=disable_split_kv,
        batch_capacity=batch_capacity or max(case.batch_size, 1),
        qo_capacity=qo_capacity or max(int(case.qo_indptr[-1]), 1),
        kv_capacity=kv_capacity or max(max(case.kv_lens, default=1), 1),
        prefill_variant=prefill_variant, logits_soft_cap=case.logits_soft_cap,
        kv_dtype=kv_dtype_of(case), decode_waves=decode_waves)


def poisoned_outputs(q: torch.Tensor):
    """O and LSE buffers for a run, filled with NaN, so that any output element
    the kernels leave unwritten fails the comparison."""
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32,
                     device=q.device)
    return o, lse


def gpu_run(case: Case, window_left=None, att=None, return_lse=True, **kw):
    """plan() + run() of `case` through the C ABI into NaN-filled outputs."""
    W = case.window_left if window_left is None else window_left
    if att is None:
        att = make_attention(case, window_left=W, **kw)
    att.plan(qo_indptr=case.qo_indptr.cpu(), kv_indptr=case.kv_indptr.cpu(),
             kv_last_page_len=case.kv_last_page_len.cpu())
    o, lse = poisoned_outputs(case.q)
    res = att.run(case.q, case.k_cache, case.v_cache, case.kv_indices, sm_scale=case.sm_scale,
                  window_left=W, causal=case.causal, return_lse=return_lse,
                  k_scale=case.k_scale, v_scale=case.v_scale, out=o,
                  lse=lse if return_lse else None)
    torch.cuda.synchronize()
    return res


def assert_all_written(case: Case, o: torch.Tensor, lse: torch.Tensor, tag=""):
    """Every output row of a run into NaN-filled buffers was written: O finite
    everywhere, LSE finite for every query with a visible key, and (O = 0,
    LSE = -inf) for the queries of requests without keys."""
    keyless = torch.zeros(o.shape[0], dtype=torch.bool)
    qop = case.qo_indptr.cpu()
    for b, kv in enumerate(case.kv_lens):
        if kv == 0:
            keyless[int(qop[b]):int(qop[b + 1])] = True
    of = torch.isfinite(o.float()).all(dim=2).all(dim=1).cpu()
    bad_o = int((~of).sum())
    assert bad_o == 0, f"{tag}: {bad_o} query rows of O hold non-finite values"
    if lse is None:
        return
    lc = lse.cpu()
    lf = torch.isfinite(lc).all(dim=1)
    bad_l = int((~lf & ~keyless).sum())
    assert bad_l == 0, f"{tag}: {bad_l} query rows with keys have a non-finite LSE"
    if keyless.any():
        assert torch.isneginf(lc[keyless]).all(), f"{tag}: keyless rows must have LSE = -inf"
        assert (o[keyless.to(o.device)] == 0).all(), f"{tag}: keyless rows must have O = 0"
    log(f"  {tag}: all {o.shape[0]} query rows written ({int(keyless.sum())} keyless)")


def compare(o, lse, o_ref, lse_ref, rows=None, tag="", o_tol=O_TOL, lse_tol=LSE_TOL):
    """Element-wise check; reports max/mean abs diff and the mismatch share."""
    o = o.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:  # the oracle was run on these rows only (compact)
        o = o[rows]
    assert np.isfinite(o_ref).all(), f"{tag}: oracle produced non-finite O"
    d = np.abs(o - o_ref)
    bad = ~(d <= o_tol)  # NaN counts as bad
    msg = (f"{tag}: O max|d|={np.nanmax(d) if d.size else 0:.3e} mean={np.nanmean(d) if d.size else 0:.2e} "
           f"mismatch={bad.mean() if d.size else 0:.4%} (tol {o_tol})")
    if lse is not None:
        l = lse.detach().float().cpu().numpy().astype(np.float64)
        lr = lse_ref
        if rows is not None:
            l = l[rows]
        both_inf = np.isneginf(l) & np.isneginf(lr)
        # (-inf) - (-inf) is never evaluated: equal infinities count as 0 apart
        dl = np.zeros(l.shape, dtype=np.float64)
        np.subtract(l, lr, out=dl, where=~both_inf)
        dl = np.abs(dl)
        badl = ~(dl <= lse_tol)
        msg += (f"; LSE max|d|={np.nanmax(dl) if dl.size else 0:.3e} "
                f"mismatch={badl.mean() if dl.size else 0:.4%} (tol {lse_tol})")
        assert not badl.any(), msg
    assert not bad.any(), msg
    log("  " + msg)
    return msg


def oracle_for(case: Case, window_left=None, rows=None):
    return oracle.case_attention(case, rows=rows, window_left=window_left)


def sub_case(case: Case, requests) -> Case:
    """The listed requests of a decode batch as a compact host-side case (their
    pages gathered into a fresh cache), for the oracle."""
    kvp = case.kv_indptr.cpu()
    idx = case.kv_indices.cpu()
    pages, npg, lens, last = [], [], [], []
    for b in requests:
        pg = idx[kvp[b]:kvp[b + 1]]
        pages.append(pg)
        npg.append(len(pg))
        lens.append(case.kv_lens[b])
        last.append(int(case.kv_last_page_len[b]))
    pages = torch.cat(pages).long()
    kc = case.k_cache.index_select(0, pages.to(case.k_cache.device)).cpu()
    vc = case.v_cache.index_select(0, pages.to(case.v_cache.device)).cpu()
    new_kvp = torch.zeros(len(requests) + 1, dtype=torch.int32)
    new_kvp[1:] = torch.tensor(npg).cumsum(0)
    q = case.q[torch.tensor(list(requests), device=case.q.device)].cpu()
    return Case(
        name=case.name + "_sub", num_qo_heads=case.num_qo_heads, num_kv_heads=case.num_kv_heads,
        head_dim=case.head_dim, page_size=case.page_size, window_left=case.window_left,
        causal=case.causal, sm_scale=case.sm_scale, dtype=case.dtype, qo_lens=[1] * len(requests),
        kv_lens=lens, q=q, k_cache=kc, v_cache=vc,
        qo_indptr=torch.arange(len(requests) + 1, dtype=torch.int32), kv_indptr=new_kvp,
        kv_indices=torch.arange(len(pages), dtype=torch.int32),
        kv_last_page_len=torch.tensor(last, dtype=torch.int32), is_decode=True)
