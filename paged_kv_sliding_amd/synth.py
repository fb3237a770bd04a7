"""Seeded synthetic inputs for paged sliding-window attention.

This module only draws data: request lengths, CSR page tables over a shuffled
page pool, and N(0,1) query / key / value tensors.  It holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can consume
exactly the same bits from it.

Layouts follow the paged KV-cache convention of sglang's FlashInfer backend
(``flashinfer_backend.py``: the "NHD" wrappers built in
``FlashInferAttnBackend.__init__`` and the CSR arrays handed to
``fast_prefill_plan``):

* ``q``        ``[nnz_qo, H_q, D]``
* ``k_cache``, ``v_cache``  ``[num_pages, P, H_kv, D]`` (separate tensors)
* ``qo_indptr`` ``[B+1]``, ``kv_indptr`` ``[B+1]`` (in pages),
  ``kv_indices`` ``[nnz_pages]``, ``kv_last_page_len`` ``[B]``; all int32.

A request with ``n`` keys occupies ``ceil(n/P)`` pages and its last page holds
``n - (ceil(n/P)-1)*P`` valid slots (an empty request has no pages and a
last-page length of 0).  Slots past that length, and pool pages that no request
uses, are filled with NaN so that any read of them poisons the result.

The five workloads are the ones the sliding-window attention benchmark is
quoted on (tiny fp32 prefill, batched prefill with a cached prefix, a decode
window sweep, one 32k-token prefill, and a large split-KV decode).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

__all__ = [
    "CascadeInputs",
    "Case",
    "WORKLOADS",
    "build_case",
    "cascade_inputs",
    "case_from_lengths",
    "workload_lengths",
]


@dataclasses.dataclass
class Case:
    """One batch of paged attention input (all tensors on ``device``)."""

    name: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    window_left: int
    causal: bool
    sm_scale: float
    dtype: torch.dtype
    qo_lens: List[int]
    kv_lens: List[int]
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    qo_indptr: torch.Tensor
    kv_indptr: torch.Tensor
    kv_indices: torch.Tensor
    kv_last_page_len: torch.Tensor
    fixed_split_size: int = -1
    is_decode: bool = False
    logits_soft_cap: float = 0.0  # 0: no cap
    k_scale: float = 1.0          # the cache holds K / k_scale and V / v_scale
    v_scale: float = 1.0

    @property
    def batch_size(self) -> int:
        return len(self.kv_lens)

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    def host_layout(self):
        """Host int32 copies of the CSR arrays (what a planner consumes)."""
        return (self.qo_indptr.cpu(), self.kv_indptr.cpu(), self.kv_last_page_len.cpu())

    def with_window(self, window_left: int) -> "Case":
        return dataclasses.replace(self, window_left=window_left)


# name -> (B, H_q, H_kv, D, P, dtype, default W, seed, causal, decode)
WORKLOADS = {
    "tiny_prefill": dict(H_q=2, H_kv=1, D=64, P=4, dtype=torch.float32, W=4, seed=0, decode=False),
    "prefix_prefill": dict(H_q=4, H_kv=1, D=256, P=16, dtype=torch.bfloat16, W=511, seed=2, decode=False),
    "decode_sweep": dict(H_q=32, H_kv=8, D=128, P=16, dtype=torch.bfloat16, W=1023, seed=3, decode=True),
    "long_prefill": dict(H_q=32, H_kv=8, D=128, P=16, dtype=torch.bfloat16, W=4095, seed=4, decode=False),
    "split_decode": dict(H_q=64, H_kv=8, D=128, P=16, dtype=torch.bfloat16, W=4095, seed=5, decode=True,
                         split=2048),
}


def workload_lengths(name: str, gen: torch.Generator, extend_len: Optional[int] = None):
    """Draw (qo_lens, kv_lens) for a named workload from ``gen`` (CPU)."""
    if name == "tiny_prefill":
        e = int(extend_len)
        return [e], [e]
    if name == "prefix_prefill":
        prefix = torch.randint(0, 1024 + 1, (8,), generator=gen).tolist()
        ext = torch.randint(1, 512 + 1, (8,), generator=gen).tolist()
        return ext, [p + e for p, e in zip(prefix, ext)]
    if name == "decode_sweep":
        kv = torch.randint(1, 4096 + 1, (64,), generator=gen).tolist()
        return [1] * 64, kv
    if name == "long_prefill":
        return [32768], [32768]
    if name == "split_decode":
        kv = torch.randint(1024, 32768 + 1, (256,), generator=gen).tolist()
        return [1] * 256, kv
    raise KeyError(name)


def _fill_normal(t: torch.Tensor, gen: torch.Generator, chunk: int = 1 << 26) -> None:
    """Fill ``t`` with N(0,1) drawn in fp32 and rounded (RNE) to ``t.dtype``."""
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        tmp = torch.randn(e - s, generator=gen, device=t.device, dtype=torch.float32)
        flat[s:e].copy_(tmp)


def case_from_lengths(
    name: str,
    qo_lens: Sequence[int],
    kv_lens: Sequence[int],
    *,
    num_qo_heads: int,
    num_kv_heads: int,
    head_dim: int,
    page_size: int,
    dtype: torch.dtype,
    window_left: int,
    seed: int,
    causal: bool = True,
    sm_scale: Optional[float] = None,
    spare_pages: int = 0,
    device: str = "cpu",
    poison: bool = True,
    is_decode: bool = False,
    fixed_split_size: int = -1,
    value_gen: Optional[torch.Generator] = None,
    perm_gen: Optional[torch.Generator] = None,
    logits_soft_cap: float = 0.0,
    kv_dtype: Optional[torch.dtype] = None,
    k_scale: float = 1.0,
    v_scale: float = 1.0,
) -> Case:
    """Build a paged batch for explicit lengths.

    Page placement and values are drawn from generators seeded with ``seed``
    (page permutation on the CPU, values on ``device``).  ``spare_pages``
    extra pool pages are allocated and left unused (NaN-poisoned).  With an
    8-bit ``kv_dtype`` the caches hold the N(0,1) keys and values divided by
    ``k_scale`` / ``v_scale``, rounded to that type (torch's conversion).
    """
    B = len(kv_lens)
    assert len(qo_lens) == B
    P = page_size
    npages = [(n + P - 1) // P for n in kv_lens]
    nnz_pages = sum(npages)
    pool = nnz_pages + spare_pages
    if perm_gen is None:
        perm_gen = torch.Generator().manual_seed(seed)
    perm = torch.randperm(max(pool, 1), generator=perm_gen)[:nnz_pages].to(torch.int32)

    kv_indptr = torch.zeros(B + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.tensor(npages, dtype=torch.int64).cumsum(0).to(torch.int32)
    qo_indptr = torch.zeros(B + 1, dtype=torch.int32)
    qo_indptr[1:] = torch.tensor(list(qo_lens), dtype=torch.int64).cumsum(0).to(torch.int32)
    last = torch.tensor([0 if n == 0 else n - (np_ - 1) * P for n, np_ in zip(kv_lens, npages)],
                        dtype=torch.int32)
    nnz_qo = int(qo_indptr[-1])

    if value_gen is None:
        value_gen = torch.Generator(device=device).manual_seed(seed + 1_000_003)
    q = torch.empty(nnz_qo, num_qo_heads, head_dim, dtype=dtype, device=device)
    cache_dtype = dtype if kv_dtype is None else torch.float32
    k_cache = torch.empty(max(pool, 1), P, num_kv_heads, head_dim, dtype=cache_dtype,
                          device=device)
    v_cache = torch.empty_like(k_cache)
    _fill_normal(q, value_gen)
    _fill_normal(k_cache, value_gen)
    _fill_normal(v_cache, value_gen)

    if poison:
        # Unused pool pages and the slots after the last valid one of each
        # request are never part of any sequence: make stray reads visible.
        used = torch.zeros(max(pool, 1), dtype=torch.bool)
        used[perm.long()] = True
        unused = (~used).nonzero().flatten()
        if unused.numel():
            idx = unused.to(device)
            k_cache.index_fill_(0, idx, float("nan"))
            v_cache.index_fill_(0, idx, float("nan"))
        for b in range(B):
            if npages[b] and last[b] < P:
                pg = int(perm[int(kv_indptr[b + 1]) - 1])
                k_cache[pg, int(last[b]):].fill_(float("nan"))
                v_cache[pg, int(last[b]):].fill_(float("nan"))

    if kv_dtype is not None:
        k_cache = (k_cache / k_scale).to(kv_dtype)
        v_cache = (v_cache / v_scale).to(kv_dtype)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return Case(
        name=name,
        num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        page_size=P,
        window_left=window_left,
        causal=causal,
        sm_scale=float(sm_scale),
        dtype=dtype,
        qo_lens=list(qo_lens),
        kv_lens=list(kv_lens),
        q=q,
        k_cache=k_cache,
        v_cache=v_cache,
        qo_indptr=qo_indptr.to(device),
        kv_indptr=kv_indptr.to(device),
        kv_indices=perm.to(device),
        kv_last_page_len=last.to(device),
        fixed_split_size=fixed_split_size,
        is_decode=is_decode,
        logits_soft_cap=float(logits_soft_cap),
        k_scale=float(k_scale),
        v_scale=float(v_scale),
    )


def build_case(name: str, *, device: str = "cpu", window_left: Optional[int] = None,
               extend_len: int = 12, poison: bool = True) -> Case:
    """Build one of the five named workloads with its documented seed."""
    w = WORKLOADS[name]
    gen = torch.Generator().manual_seed(w["seed"])
    qo, kv = workload_lengths(name, gen, extend_len)
    spare = 0
    if name == "tiny_prefill":
        # pool of twice the pages needed, placed by a random permutation
        spare = (kv[0] + w["P"] - 1) // w["P"]
    return case_from_lengths(
        name if name != "tiny_prefill" else f"tiny_prefill_e{extend_len}",
        qo,
        kv,
        num_qo_heads=w["H_q"],
        num_kv_heads=w["H_kv"],
        head_dim=w["D"],
        page_size=w["P"],
        dtype=w["dtype"],
        window_left=w["W"] if window_left is None else window_left,
        seed=w["seed"] * 1000 + (extend_len if name == "tiny_prefill" else 0),
        causal=True,
        spare_pages=spare,
        device=device,
        poison=poison,
        is_decode=w["decode"],
        fixed_split_size=w.get("split", -1),
        perm_gen=gen,
    )


@dataclasses.dataclass
class CascadeInputs:
    """A paged batch rearranged the way a cascade prefill receives it: the
    keys / values of each request's query tokens in contiguous arrays, and a
    page table over the cached keys before them."""

    k_extend: torch.Tensor        # [nnz_qo, H_kv, D], row r = key of query token r
    v_extend: torch.Tensor
    k_cache: torch.Tensor         # copy of the pool, NaN outside the prefix tables
    v_cache: torch.Tensor
    kv_indptr: torch.Tensor       # [B+1] int32 (host)
    kv_indices: torch.Tensor      # int32, on the case's device
    kv_last_page_len: torch.Tensor  # [B] int32 (host)
    table_lens: List[int]         # cached keys each request's table holds


def cascade_inputs(case: Case, trim_to: Optional[int] = None) -> CascadeInputs:
    """Rearrange a paged prefill case (whose query tokens' keys already sit in
    the cache, after each request's prefix) into cascade inputs.

    The last ``qo_len`` keys of each request are gathered into ``k_extend`` /
    ``v_extend``.  The page table keeps the request's pages up to its prefix
    end; with ``trim_to`` = n >= 0 it starts at the page holding key
    ``max(0, prefix - n)`` (the pages before it are dropped, the way a
    sliding-window pool trims a prefix to the window).  Every slot of the pool
    that no table covers is NaN in the returned caches, so a read of it shows.
    """
    P = case.page_size
    B = len(case.kv_lens)
    kvp = case.kv_indptr.cpu().tolist()
    idx = case.kv_indices.cpu()
    dev = case.k_cache.device
    rows_pg, rows_slot = [], []
    new_kvp, new_idx, last, tlen = [0], [], [], []
    keep = torch.zeros(case.k_cache.shape[0], P, dtype=torch.bool)
    for b in range(B):
        pages = idx[kvp[b]:kvp[b + 1]]
        prefix = case.kv_lens[b] - case.qo_lens[b]
        for pos in range(prefix, case.kv_lens[b]):
            rows_pg.append(int(pages[pos // P]))
            rows_slot.append(pos % P)
        start = 0
        if trim_to is not None and trim_to >= 0:
            start = max(0, prefix - trim_to) // P * P
        n = prefix - start
        np_ = (n + P - 1) // P
        tab = pages[start // P:start // P + np_]
        new_idx.append(tab)
        new_kvp.append(new_kvp[-1] + np_)
        last.append(0 if n == 0 else n - (np_ - 1) * P)
        tlen.append(n)
        for i, pg in enumerate(tab.tolist()):
            keep[pg, : (P if i + 1 < np_ else last[-1])] = True
    pg_t = torch.tensor(rows_pg, dtype=torch.long, device=dev)
    sl_t = torch.tensor(rows_slot, dtype=torch.long, device=dev)
    drop = (~keep).to(dev)
    eight_bit = case.k_cache.element_size() == 1
    caches = []
    for cache in (case.k_cache, case.v_cache):
        if eight_bit:
            # 8-bit floats: move raw bytes; 0x7f is NaN in both e4m3 and e5m2
            raw = cache.view(torch.uint8)
            ext = raw[pg_t, sl_t].contiguous().view(cache.dtype)
            poisoned = raw.clone()
            poisoned[drop] = 0x7F
            caches.append((ext, poisoned.view(cache.dtype)))
        else:
            poisoned = cache.clone()
            poisoned[drop] = float("nan")
            caches.append((cache[pg_t, sl_t].contiguous(), poisoned))
    (k_ext, k_cache), (v_ext, v_cache) = caches
    kv_indices = torch.cat(new_idx).to(torch.int32) if new_idx else torch.zeros(0, dtype=torch.int32)
    return CascadeInputs(
        k_extend=k_ext, v_extend=v_ext, k_cache=k_cache, v_cache=v_cache,
        kv_indptr=torch.tensor(new_kvp, dtype=torch.int32), kv_indices=kv_indices.to(dev),
        kv_last_page_len=torch.tensor(last, dtype=torch.int32), table_lens=tlen)

