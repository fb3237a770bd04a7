"""Property tests of the planner (dry plans, no GPU): random batches, windows,
page sizes, head groups, kernel variants and split sizes, drawn by
hypothesis, against the invariants the kernels rely on.

Prefill: every (request, kv head, query) in exactly one query tile; a tile's
key range starts at a multiple of its kernel's key tile at or before the first
visible key of every query in it and reaches the last query's position; a tile
cut by the key split is a run of chunk items whose key ranges partition its
range at key-tile boundaries, with consecutive partial slots per token and one
merge entry per token; items are ordered by decreasing key count.  Decode: each (request, kv head)'s chunks
partition [window start rounded down to 32, kv_len) with the visible bound set
to the window start, and split pairs own consecutive partial slots, one merge
entry each.  Cascade: the one-pass plan covers every new token once over the
request's cached keys followed by its new tokens, split at the cached count."""
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from paged_kv_sliding_amd import pkvs as P

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])
INT32_MAX = 2**31 - 1


def csr(qo_lens, kv_lens, page):
    npages = [(n + page - 1) // page for n in kv_lens]
    kvp, qop = [0], [0]
    for n in npages:
        kvp.append(kvp[-1] + n)
    for n in qo_lens:
        qop.append(qop[-1] + n)
    last = [0 if n == 0 else n - (m - 1) * page for n, m in zip(kv_lens, npages)]
    return qop, kvp, last


def make(kind, **kw):
    base = dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                dtype=torch.bfloat16, window_left=31, causal=True, batch_capacity=8,
                qo_capacity=4096, kv_capacity=4096)
    base.update(kw)
    return P.pkvs_plan_create(P.make_desc(kind, **base))


@st.composite
def prefill_batches(draw):
    B = draw(st.integers(1, 6))
    qo = draw(st.lists(st.integers(0, 300), min_size=B, max_size=B))
    prefix = draw(st.lists(st.integers(0, 500), min_size=B, max_size=B))
    W = draw(st.sampled_from([-1, 0, 1, 31, 63, 64, 200, 900]))
    page = draw(st.sampled_from([1, 4, 16]))
    G = draw(st.sampled_from([1, 4, 8]))
    variant = draw(st.sampled_from([0, 1, 2, 4, 5]))
    return qo, [q + p for q, p in zip(qo, prefix)], W, page, G, variant


@SETTINGS
@given(prefill_batches())
def test_prefill_plan_invariants(batch):
    qo, kv, W, page, G, variant = batch
    h = make(P.PKVS_PREFILL, num_qo_heads=2 * G, num_kv_heads=2, page_size=page, window_left=W,
             prefill_variant=variant, batch_capacity=len(kv), qo_capacity=max(1, sum(qo)),
             kv_capacity=max(1, max(kv)))
    try:
        qop, kvp, last = csr(qo, kv, page)
        P.pkvs_prefill_plan(h, qop, kvp, last, len(kv), None, None)
        info = P.pkvs_plan_get_info(h)
        kt = 64 if info.prefill_variant in (5, 6) else 32
        items = P.pkvs_plan_copy_items(h).tolist()
        assert len(items) == info.num_items
        costs = [it[9] - it[7] for it in items]
        assert costs == sorted(costs, reverse=True)
        seen = check_tiles(items, kt, W, lambda b: kv[b] - qo[b], lambda b: kv[b],
                           lambda b: INT32_MAX, kvp, qop, info)
        expect = {(b, hk, t) for b in range(len(kv)) for hk in range(2)
                  for t in range(qop[b], qop[b + 1])}
        assert set(seen) == expect and set(seen.values()) <= {1}
    finally:
        P.pkvs_plan_destroy(h)


def check_tiles(items, kt, W, prefix_of, kv_len_of, split_of, kvp, qop, info):
    """Group the items by query tile, check each tile's key range and its
    chunks (see the module docstring); return the (request, kv head, token)
    coverage counts."""
    tiles, seen, slots = {}, {}, set()
    for it in items:
        b, hk, q0, qn, pos0, kv_len, pbase, kvb, split, kv_end, slot, stride = it[:12]
        assert kv_len == kv_len_of(b) and pbase == kvp[b] and split == split_of(b)
        assert 1 <= qn <= info.query_tile and pos0 == prefix_of(b) + (q0 - qop[b])
        tiles.setdefault((b, hk, q0, qn, pos0), []).append((kvb, kv_end, slot, stride))
    merges = 0
    for (b, hk, q0, qn, pos0), ch in tiles.items():
        ch.sort()
        kve = min(kv_len_of(b), pos0 + qn)
        assert kve == pos0 + qn  # causal: the last query sees its own key
        assert ch[0][0] % kt == 0 and ch[0][0] <= max(0, pos0 - W if W >= 0 else 0)
        assert ch[-1][1] == kve
        for (_, e0, _, _), (b1, _, _, _) in zip(ch, ch[1:]):
            assert e0 == b1 and b1 % kt == 0
        if len(ch) == 1:
            assert ch[0][2] == -1
        else:
            n = len(ch)
            assert info.key_chunks >= n and all(c[3] == n for c in ch)
            base = ch[0][2]
            assert [c[2] for c in ch] == list(range(base, base + n))
            mine = set(range(base, base + qn * n))
            assert not (mine & slots)
            slots |= mine
            merges += qn
        for t in range(q0, q0 + qn):
            seen[(b, hk, t)] = seen.get((b, hk, t), 0) + 1
    assert info.num_merges == merges
    return seen


@st.composite
def decode_batches(draw):
    B = draw(st.integers(1, 40))
    kv = draw(st.lists(st.integers(0, 3000), min_size=B, max_size=B))
    W = draw(st.sampled_from([-1, 0, 31, 127, 1023, 5000]))
    page = draw(st.sampled_from([1, 16, 64]))
    split = draw(st.sampled_from([-1, 32, 96, 512, 2048]))
    disable = draw(st.booleans())
    nw = draw(st.sampled_from([0, 1, 4]))
    return kv, W, page, split, disable, nw


@SETTINGS
@given(decode_batches())
def test_decode_plan_invariants(batch):
    kv, W, page, split, disable, nw = batch
    h = make(P.PKVS_DECODE, num_qo_heads=16, num_kv_heads=4, page_size=page, window_left=W,
             fixed_split_size=split, disable_split_kv=disable, decode_waves=nw,
             batch_capacity=len(kv), kv_capacity=max(1, max(kv)))
    try:
        _, kvp, last = csr([1] * len(kv), kv, page)
        P.pkvs_decode_plan(h, kvp, last, len(kv), None, None)
        info = P.pkvs_plan_get_info(h)
        items = P.pkvs_plan_copy_items(h).tolist()
        assert len(items) == info.num_items
        by = {}
        for b, hk, t0, t1, lo, pbase, slot, kv_len in items:
            assert kv_len == kv[b] and pbase == kvp[b]
            by.setdefault((b, hk), []).append((t0, t1, lo, slot))
        n_split = 0
        for b, n in enumerate(kv):
            ws = max(0, n - 1 - W) if W >= 0 else 0
            for hk in range(4):
                ch = sorted(by[(b, hk)])
                if n == 0:
                    assert ch == [(0, 0, 0, -1)]
                    continue
                assert ch[0][0] == ws // 32 * 32 and ch[-1][1] == n
                for (a0, a1, _, _), (b0, _, _, _) in zip(ch, ch[1:]):
                    assert a1 == b0
                for t0, t1, lo, _ in ch:
                    assert t0 % 32 == 0 and t0 < t1 and lo == max(ws, t0) and lo < t1
                if disable:
                    assert len(ch) == 1
                if len(ch) == 1:
                    assert ch[0][3] == -1
                else:
                    sl = [c[3] for c in ch]
                    assert sl == list(range(sl[0], sl[0] + len(sl)))
                    n_split += 1
        assert info.num_merges == n_split
    finally:
        P.pkvs_plan_destroy(h)


@st.composite
def cascade_batches(draw):
    B = draw(st.integers(1, 5))
    qo = draw(st.lists(st.integers(0, 300), min_size=B, max_size=B))
    tab = draw(st.lists(st.integers(0, 400), min_size=B, max_size=B))
    W = draw(st.sampled_from([-1, 0, 5, 100, 511]))
    page = draw(st.sampled_from([1, 16]))
    variant = draw(st.sampled_from([1, 2, 5]))
    return qo, tab, W, page, variant


@SETTINGS
@given(cascade_batches())
def test_one_pass_cascade_plan_invariants(batch):
    qo, tab, W, page, variant = batch
    h = make(P.PKVS_CASCADE, num_qo_heads=8, num_kv_heads=2, page_size=page, window_left=W,
             prefill_variant=variant, batch_capacity=len(qo), qo_capacity=max(1, sum(qo)),
             kv_capacity=max(1, max(tab)))
    try:
        assert P.pkvs_plan_get_info(h).cascade_passes == 1
        qop, kvp, last = csr(qo, tab, page)
        P.pkvs_cascade_plan(h, qop, kvp, last, len(qo), None, None)
        info = P.pkvs_plan_get_info(h)
        kt = 64 if info.prefill_variant in (5, 6) else 32
        items = P.pkvs_plan_copy_items(h).tolist()
        seen = check_tiles(items, kt, W, lambda b: tab[b], lambda b: tab[b] + qo[b],
                           lambda b: tab[b], kvp, qop, info)
        expect = {(b, hk, t) for b in range(len(qo)) for hk in range(2)
                  for t in range(qop[b], qop[b + 1])}
        assert set(seen) == expect and set(seen.values()) <= {1}
    finally:
        P.pkvs_plan_destroy(h)

