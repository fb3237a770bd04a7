"""Host-side tests of libpkvs that need no GPU: exported symbols, descriptor
validation, and invariants of the planner's work lists (dry plans)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from paged_kv_sliding_amd import pkvs as P
from paged_kv_sliding_amd.synth import build_case, workload_lengths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkvs.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkvs_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(P.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pkvs_\w+)", out))
    missing = set(header_functions()) - exported
    assert not missing, missing
    lib = ctypes.CDLL(P.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name)


# The calls of the boundary as the hot-path statement lists them, and the
# exported entry points that provide each (the plan object is created once for
# its capacities and re-planned in place; run() reads the device layout that
# plan() uploaded into the int workspace, so it takes only kv_indices).
BOUNDARY_CALLS = {
    "pkvs_workspace_bytes": ["pkvs_workspace_bytes", "pkvs_workspace_size"],
    "pkvs_prefill_plan": ["pkvs_plan_create", "pkvs_prefill_plan"],
    "pkvs_prefill_run": ["pkvs_prefill_run"],
    "pkvs_decode_plan": ["pkvs_plan_create", "pkvs_decode_plan"],
    "pkvs_decode_run": ["pkvs_decode_run"],
    "pkvs_merge_state": ["pkvs_merge_state"],
    "pkvs_plan_destroy": ["pkvs_plan_destroy"],
    "pkvs_strerror": ["pkvs_strerror"],
    "pkvs_last_error_message": ["pkvs_last_error_message", "pkvs_last_error"],
}


def test_boundary_calls_are_all_provided():
    declared = set(header_functions())
    for call, provided_by in BOUNDARY_CALLS.items():
        assert set(provided_by) <= declared, (call, provided_by)
    # the names the statement uses are exported under those names where the
    # signature is kept
    for name in ("pkvs_workspace_bytes", "pkvs_prefill_plan", "pkvs_prefill_run",
                 "pkvs_decode_plan", "pkvs_decode_run", "pkvs_merge_state", "pkvs_plan_destroy",
                 "pkvs_strerror", "pkvs_last_error_message"):
        assert name in declared


def test_every_declaration_cites_a_passage_or_says_utility():
    """Each function declared in include/pkvs.h is preceded by a comment that
    cites the passage it follows ([FIB], [PR31501], [PR234]) or says it is a
    library utility with no passage."""
    text = open(HEADER).read()
    for name in header_functions():
        m = re.search(r"/\*((?:(?!\*/).)*)\*/\s*(?:const\s+)?\w+\s*\**\s*" + name + r"\s*\(",
                      text, flags=re.S)
        assert m, f"{name}: no comment right before its declaration"
        doc = re.sub(r"\s*\n\s*\*\s*", " ", m.group(1))
        if name == "pkvs_decode_noalloc":
            # no passage: its comment names the callers it is for
            assert "callers that cannot allocate" in doc, name
            continue
        assert re.search(r"\[(FIB|PR31501|PR234)\]", doc) or "Library utility, no passage" \
            in doc, name


def test_workspace_bytes_equals_the_plans_sizes():
    for kind, kw in ((P.PKVS_PREFILL, {}), (P.PKVS_DECODE, dict(num_qo_heads=64, num_kv_heads=8,
                                                               window_left=4095, batch_capacity=256,
                                                               kv_capacity=32768,
                                                               fixed_split_size=2048)),
                     (P.PKVS_CASCADE, dict(window_left=511))):
        d = desc(kind, **kw)
        h = P.pkvs_plan_create(d)
        assert P.pkvs_workspace_bytes(d, kind == P.PKVS_DECODE) == P.pkvs_workspace_size(h)
        P.pkvs_plan_destroy(h)
        d2 = desc(kind, **dict(kw, kv_capacity=100))
        h2 = P.pkvs_plan_create(d2)
        assert P.pkvs_workspace_bytes(d, kind == P.PKVS_DECODE, 100) == \
            P.pkvs_workspace_size(h2)
        P.pkvs_plan_destroy(h2)
    assert err_code(lambda: P.pkvs_workspace_bytes(desc(), True)) == P.PKVS_ERR_INVALID_ARG
    assert "disagrees" in P.pkvs_last_error_message()
    assert P.pkvs_last_error_message() == P.last_error()
    assert err_code(lambda: P.pkvs_workspace_bytes(desc(head_dim=96), False)) == \
        P.PKVS_ERR_UNSUPPORTED
    assert err_code(lambda: P.pkvs_workspace_bytes(desc(), False, -1)) == P.PKVS_ERR_INVALID_ARG


def desc(kind=P.PKVS_PREFILL, **kw):
    base = dict(num_qo_heads=4, num_kv_heads=1, head_dim=128, page_size=16,
                dtype=torch.bfloat16, window_left=31, causal=True, batch_capacity=16,
                qo_capacity=8192, kv_capacity=8192)
    base.update(kw)
    return P.make_desc(kind, **base)


def err_code(fn):
    with pytest.raises(P.PkvsError) as ei:
        fn()
    return ei.value.code


@pytest.mark.parametrize("kw,code", [
    (dict(window_left=-2), P.PKVS_ERR_INVALID_ARG),
    (dict(num_qo_heads=6, num_kv_heads=4), P.PKVS_ERR_INVALID_ARG),
    (dict(head_dim=96), P.PKVS_ERR_UNSUPPORTED),
    (dict(page_size=12), P.PKVS_ERR_UNSUPPORTED),
    (dict(causal=False, window_left=7), P.PKVS_ERR_UNSUPPORTED),
    (dict(num_qo_heads=3, num_kv_heads=1), P.PKVS_ERR_UNSUPPORTED),
    (dict(num_qo_heads=3, num_kv_heads=1, dtype=torch.float16), P.PKVS_ERR_UNSUPPORTED),
    (dict(fixed_split_size=100), P.PKVS_ERR_INVALID_ARG),
    (dict(batch_capacity=0), P.PKVS_ERR_INVALID_ARG),
    (dict(prefill_variant=7), P.PKVS_ERR_INVALID_ARG),
    (dict(prefill_variant=2, head_dim=256), P.PKVS_ERR_UNSUPPORTED),
    (dict(prefill_variant=3, head_dim=256), P.PKVS_ERR_UNSUPPORTED),
    # one page of 1024 slots x 8192 kv heads x 256 dims is 2^31 elements
    (dict(num_qo_heads=8192, num_kv_heads=8192, head_dim=256, page_size=1024),
     P.PKVS_ERR_UNSUPPORTED),
])
def test_descriptor_rejections(kw, code):
    assert err_code(lambda: P.pkvs_plan_create(desc(**kw))) == code


def csr(qo_lens, kv_lens, page):
    npages = [(n + page - 1) // page for n in kv_lens]
    kvp = [0]
    for n in npages:
        kvp.append(kvp[-1] + n)
    qop = [0]
    for n in qo_lens:
        qop.append(qop[-1] + n)
    last = [0 if n == 0 else n - (m - 1) * page for n, m in zip(kv_lens, npages)]
    return qop, kvp, last


def visible(p, j, W, causal=True):
    return (not causal or j <= p) and (W < 0 or j >= p - W)


@pytest.mark.parametrize("W", [-1, 0, 4, 31, 511])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("cut", [False, True])
def test_prefill_items_cover_every_query_once(W, G, cut):
    """Every query in exactly one query tile whose key range holds all its
    visible keys and no wholly invisible key tile; with the key split allowed
    (cut) a tile may be several chunk items whose ranges partition it."""
    qo = [1, 0, 40, 300, 7, 129]
    kv = [1, 5, 40, 1000, 600, 129]
    h = P.pkvs_plan_create(desc(num_qo_heads=2 * G, num_kv_heads=2, window_left=W,
                                disable_split_kv=int(not cut)))
    qop, kvp, last = csr(qo, kv, 16)
    P.pkvs_prefill_plan(h, qop, kvp, last, len(kv), None, None)
    info = P.pkvs_plan_get_info(h)
    items = P.pkvs_plan_copy_items(h)
    assert info.query_tile in (128 // G, 256 // G)
    assert items.shape[0] == info.num_items
    # key tiles of the kernel the plan runs: 64 keys for variant 5, else 32
    kt = 64 if info.prefill_variant in (5, 6) else 32
    tiles = {}
    for it in items.tolist():
        b, hk, q0, qn, pos0, kv_len, pbase, kvb, split, kv_end, slot = it[:11]
        assert split == 2**31 - 1  # every key in the cache
        assert 1 <= qn <= info.query_tile and kv_len == kv[b] and pbase == kvp[b]
        assert pos0 == kv[b] - qo[b] + (q0 - qop[b])
        assert kvb % kt == 0 and (slot >= 0) <= cut
        tiles.setdefault((b, hk, q0, qn, pos0), []).append((kvb, kv_end))
    seen = {}
    for (b, hk, q0, qn, pos0), ranges in tiles.items():
        ranges.sort()
        for (_, e0), (b1, _) in zip(ranges, ranges[1:]):
            assert e0 == b1 and b1 % kt == 0
        kvb, kve = ranges[0][0], ranges[-1][1]
        assert kve == min(kv[b], pos0 + qn)
        for t in range(q0, q0 + qn):
            seen[(b, hk, t)] = seen.get((b, hk, t), 0) + 1
            p = pos0 + (t - q0)
            # every visible key of every query lies inside the tile's key range
            first_vis = max(0, p - W) if W >= 0 else 0
            assert kvb <= first_vis and p < kve
        # no key tile of the range is wholly invisible to the tile's queries
        for k0 in range(kvb, kve, kt):
            assert any(visible(pos0 + i, j, W) for i in range(qn)
                       for j in range(k0, min(k0 + kt, kve))), (b, hk, q0, k0)
    expect = {(b, hk, t) for b in range(len(kv)) for hk in range(2)
              for t in range(qop[b], qop[b + 1])}
    assert set(seen) == expect and set(seen.values()) == {1}
    if cut and W < 0:
        assert info.num_merges > 0  # request 3's long tiles are cut
    P.pkvs_plan_destroy(h)


def test_prefill_first_tile_matches_paged_trim():
    """The key range of a request's first query tile starts at the tile holding
    kv_start = seq - min(seq, W + seq - prefix) (sglang update_sliding_window,
    paged branch)."""
    W = 100
    qo, kv = [50, 10, 300], [1000, 10, 400]
    h = P.pkvs_plan_create(desc(window_left=W))
    qop, kvp, last = csr(qo, kv, 16)
    P.pkvs_prefill_plan(h, qop, kvp, last, 3, None, None)
    for it in P.pkvs_plan_copy_items(h).tolist():
        b, _, q0, _, _, _, _, kvb = it[:8]
        if q0 == qop[b]:
            seq, prefix = kv[b], kv[b] - qo[b]
            kv_start = seq - min(seq, W + seq - prefix)
            assert kvb == kv_start // 32 * 32


@pytest.mark.parametrize("W,split", [(-1, -1), (-1, 2048), (0, -1), (31, 64), (1023, 256),
                                     (4095, 2048), (-1, 32), (4095, 1024), (100, 64)])
def test_decode_chunks_partition_the_window(W, split):
    kv = [0, 1, 2, 31, 32, 33, 500, 4096, 5000, 17]
    h = P.pkvs_plan_create(desc(P.PKVS_DECODE, num_qo_heads=32, num_kv_heads=8, window_left=W,
                                fixed_split_size=split, batch_capacity=len(kv)))
    _, kvp, last = csr([1] * len(kv), kv, 16)
    P.pkvs_decode_plan(h, kvp, last, len(kv), None, None)
    info = P.pkvs_plan_get_info(h)
    items = P.pkvs_plan_copy_items(h).tolist()
    if split > 0:
        assert info.split_size == split
    by = {}
    for b_, hk, t0, t1, lo, pbase, slot, kv_len in items:
        assert kv_len == kv[b_] and pbase == kvp[b_]
        by.setdefault((b_, hk), []).append((t0, t1, lo, slot))
    slots = []
    for b, n in enumerate(kv):
        ws = max(0, n - 1 - W) if W >= 0 else 0
        # the window of a decode query: the last min(kv_len, W+1) keys
        assert n - ws == (min(n, W + 1) if W >= 0 else n)
        for hk in range(8):
            ch = sorted(by[(b, hk)])
            if n == 0:
                assert ch == [(0, 0, 0, -1)]
                continue
            assert ch[0][0] == ws // 32 * 32 and ch[-1][1] == n
            for (a0, a1, alo, _), (b0, _, _, _) in zip(ch, ch[1:]):
                assert a1 == b0  # contiguous, disjoint
            for t0, t1, lo, slot in ch:
                assert t0 % 32 == 0 and t0 < t1 and lo == max(ws, t0) and lo < t1
                if split > 0:
                    # only a last chunk grows, by a piece shorter than one 32-key block
                    assert t1 - t0 <= split or (t1 == n and t1 - t0 < split + 32)
            if split > 0 and len(ch) > 1:
                assert ch[-1][1] - ch[-1][0] >= 32
            if len(ch) == 1:
                assert ch[0][3] == -1
            else:
                slots.append(sorted(c[3] for c in ch))
    for s in slots:
        assert s == list(range(s[0], s[0] + len(s)))
    assert info.num_merges == len(slots)


def test_prefill_variant_choice_and_page_table_fallback():
    """Large head_dim-128 prefill plans pick the 64-key-step direct-to-LDS
    kernel (variant 5) at page sizes of 8 keys or more, the 256-row kernel
    (variant 2) below.  The direct-to-LDS variants hold an item's page ids in
    an LDS table (variants 4 and 6: 2048 entries, 5: 8192), so a plan whose
    capacities let one item span more pages runs the register-staged 256-row
    kernel (variant 2) from creation on; the variant never changes between
    plan() calls of one plan object (a captured run keeps launching the kernel
    it was captured with)."""
    big = dict(num_qo_heads=32, num_kv_heads=8, window_left=-1, qo_capacity=32768,
               kv_capacity=32768, batch_capacity=4)
    for v, table in ((0, 8192), (4, 2048), (5, 8192), (6, 2048)):
        # no window, keys of 16 per page: at most `table` pages per item -> kept
        cap = table * 16
        hv = P.pkvs_plan_create(desc(page_size=16, prefill_variant=v, **dict(big, kv_capacity=cap)))
        assert P.pkvs_plan_get_info(hv).prefill_variant == (v or 5)
        for qo, kv in (([4096], [4096]), ([64], [cap]), ([1] * 4, [1, 40, cap - 100, 7])):
            qop, kvp, last = csr(qo, kv, 16)
            P.pkvs_prefill_plan(hv, qop, kvp, last, len(kv), None, None)
            assert P.pkvs_plan_get_info(hv).prefill_variant == (v or 5)
        # one key more per request allows one page more -> variant 2 from creation
        hv = P.pkvs_plan_create(desc(page_size=16, prefill_variant=v,
                                     **dict(big, kv_capacity=cap + 1)))
        assert P.pkvs_plan_get_info(hv).prefill_variant == 2
        qop, kvp, last = csr([64], [4096], 16)
        P.pkvs_prefill_plan(hv, qop, kvp, last, 1, None, None)
        assert P.pkvs_plan_get_info(hv).prefill_variant == 2
    # page size 1 without a window: 8193 keys are 8193 pages -> variant 2
    h = P.pkvs_plan_create(desc(page_size=1, prefill_variant=5, **dict(big, kv_capacity=8193)))
    assert P.pkvs_plan_get_info(h).prefill_variant == 2
    # the planner's choice at page size 1 with the device full: variant 2
    h = P.pkvs_plan_create(desc(page_size=1, **dict(big, window_left=1023, kv_capacity=4096)))
    assert P.pkvs_plan_get_info(h).prefill_variant == 2
    # with a window the span is bounded by window_left: 1023 + 64 + 128 keys
    h1 = P.pkvs_plan_create(desc(page_size=1, prefill_variant=5,
                                 **dict(big, window_left=1023, kv_capacity=65536)))
    for qo, kv in (([8192], [8192]), ([100, 3000], [1000, 60000])):
        qop, kvp, last = csr(qo, kv, 1)
        P.pkvs_prefill_plan(h1, qop, kvp, last, len(kv), None, None)
        assert P.pkvs_plan_get_info(h1).prefill_variant == 5
    # largest window that still fits: W + 64 + 2*64 - 3 keys -> W/1 + 2 pages
    for W, want in ((8001, 5), (8002, 2)):
        hw = P.pkvs_plan_create(desc(page_size=1, prefill_variant=5,
                                     **dict(big, window_left=W, kv_capacity=65536)))
        assert P.pkvs_plan_get_info(hw).prefill_variant == want, W
        if want == 5:
            # the worst item of that window spans exactly the table or less
            qop, kvp, last = csr([4096], [65536], 1)
            P.pkvs_prefill_plan(hw, qop, kvp, last, 1, None, None)
            items = P.pkvs_plan_copy_items(hw).numpy()
            spans = []
            for it in items:
                kb, kv_len, pos0, qn = it[7], it[5], it[4], it[3]
                kv_end = min(kv_len, pos0 + qn)
                lastk = min(kb + -(-(kv_end - kb) // 64) * 64, kv_len) - 1
                spans.append(lastk - kb + 1)
            assert max(spans) <= 8192
    # head_dim 64 keeps the register-staged kernel; asking for 4 is refused
    assert P.pkvs_plan_get_info(P.pkvs_plan_create(desc(head_dim=64, **big))).prefill_variant == 2
    for v in (4, 5, 6):
        assert err_code(lambda: P.pkvs_plan_create(desc(head_dim=64, prefill_variant=v))) == \
            P.PKVS_ERR_UNSUPPORTED


def test_grid_does_not_depend_on_the_batch():
    h = P.pkvs_plan_create(desc(P.PKVS_DECODE, num_qo_heads=32, num_kv_heads=8, window_left=-1,
                                batch_capacity=64, kv_capacity=4096))
    grids = []
    for kv in ([5], [4096] * 64, [1, 2, 3]):
        _, kvp, last = csr([1] * len(kv), kv, 16)
        P.pkvs_decode_plan(h, kvp, last, len(kv), None, None)
        grids.append(P.pkvs_plan_get_info(h).grid_blocks)
    assert len(set(grids)) == 1


def test_decode_waves_choice_and_validation():
    """decode_waves: 1 or 4 as asked; 0 lets the planner take four waves per
    item only for a batch of at most one (request, kv head) pair per 32
    resident one-wave items (32 pairs on 256 CUs without an occupancy query)
    whose requests can present more than 2048 keys after the window trim;
    anything else is an error.  The plan reports the choice and sizes its
    workgroups by it."""
    base = dict(num_qo_heads=32, num_kv_heads=8, batch_capacity=4, kv_capacity=8192)
    for nw in (1, 4):
        h = P.pkvs_plan_create(desc(P.PKVS_DECODE, window_left=-1, decode_waves=nw, **base))
        info = P.pkvs_plan_get_info(h)
        assert info.decode_waves == nw and info.block_threads == 64 * nw
        P.pkvs_plan_destroy(h)
    auto = lambda **kw: P.pkvs_plan_get_info(
        P.pkvs_plan_create(desc(P.PKVS_DECODE, **dict(dict(base, window_left=-1), **kw)))).decode_waves
    assert auto() == 4
    assert auto(window_left=2047) == 1 and auto(window_left=2048) == 4
    assert auto(kv_capacity=2048) == 1
    assert auto(batch_capacity=5) == 1 and auto(batch_capacity=4096) == 1
    for bad in (2, 3, -1, 8):
        assert err_code(lambda: P.pkvs_plan_create(desc(P.PKVS_DECODE, decode_waves=bad, **base))) \
            == P.PKVS_ERR_INVALID_ARG
    # prefill plans report no decode waves
    assert P.pkvs_plan_get_info(P.pkvs_plan_create(desc())).decode_waves == 0


def test_capacity_is_enforced_not_underlaunched():
    """A larger batch than the plan was made for is rejected at plan time
    (AMD-Ecosystem/flashinfer PR 234, "Why each fix" 2)."""
    h = P.pkvs_plan_create(desc(P.PKVS_DECODE, num_qo_heads=32, num_kv_heads=8,
                                batch_capacity=4, kv_capacity=1024))
    _, kvp, last = csr([1] * 4, [10, 20, 30, 1024], 16)
    P.pkvs_decode_plan(h, kvp, last, 4, None, None)
    _, kvp, last = csr([1] * 5, [10] * 5, 16)
    assert err_code(lambda: P.pkvs_decode_plan(h, kvp, last, 5, None, None)) == P.PKVS_ERR_CAPACITY
    _, kvp, last = csr([1], [1025], 16)
    assert err_code(lambda: P.pkvs_decode_plan(h, kvp, last, 1, None, None)) == P.PKVS_ERR_CAPACITY
    hp = P.pkvs_plan_create(desc(qo_capacity=100))
    qop, kvp, last = csr([60, 50], [60, 50], 16)
    assert err_code(lambda: P.pkvs_prefill_plan(hp, qop, kvp, last, 2, None, None)) == \
        P.PKVS_ERR_CAPACITY


def test_layout_rejections():
    h = P.pkvs_plan_create(desc())
    qop, kvp, last = csr([10], [5], 16)
    assert err_code(lambda: P.pkvs_prefill_plan(h, qop, kvp, last, 1, None, None)) == \
        P.PKVS_ERR_INVALID_ARG
    qop, kvp, last = csr([5], [5], 16)
    last[0] = 17
    assert err_code(lambda: P.pkvs_prefill_plan(h, qop, kvp, last, 1, None, None)) == \
        P.PKVS_ERR_INVALID_ARG
    assert err_code(lambda: P.pkvs_prefill_plan(h, [0, 5], [0, 2, 1], [5, 5], 2, None, None)) == \
        P.PKVS_ERR_INVALID_ARG


def test_workspace_too_small_is_reported():
    h = P.pkvs_plan_create(desc())
    _, ib = P.pkvs_workspace_size(h)
    qop, kvp, last = csr([5], [5], 16)
    small = torch.empty(ib // 2, dtype=torch.uint8)
    # the size check happens before any device copy
    (qp, qt), (kp, kt), (lp, lt) = P._host_i32(qop), P._host_i32(kvp), P._host_i32(last)
    rc = P._lib.pkvs_prefill_plan(h, qp, kp, lp, 1, None, 0, ctypes.c_void_p(small.data_ptr()),
                                  small.numel(), None)
    assert rc == P.PKVS_ERR_WORKSPACE, P.last_error()


def test_noalloc_scratch_size_matches_the_header():
    m = re.search(r"#define PKVS_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m, "PKVS_NOALLOC_SCRATCH_BYTES not found in include/pkvs.h"
    assert int(m.group(1)) << int(m.group(2)) == P.NOALLOC_SCRATCH_BYTES


def test_noalloc_decode_checks_come_before_any_device_work():
    """pkvs_decode_noalloc refuses a missing or non-decode plan, an fp32 plan
    and a plan whose workspaces exceed the library's scratch array before it
    touches a device; nothing falls back to allocating."""
    lib = P._lib
    (kp, _k), (lp, _l) = P._host_i32([0, 1]), P._host_i32([1])

    def call(h):
        return lib.pkvs_decode_noalloc(h, kp, lp, 1, None, None, None, 1, None, None, None, 1.0,
                                       -1, 1.0, 1.0, None)

    assert call(None) == P.PKVS_ERR_INVALID_ARG
    plans = []
    try:
        plans.append(P.pkvs_plan_create(desc(window_left=-1)))
        assert call(plans[-1]) == P.PKVS_ERR_INVALID_ARG  # a prefill plan
        plans.append(P.pkvs_plan_create(desc(P.PKVS_DECODE, dtype=torch.float32, window_left=-1)))
        assert call(plans[-1]) == P.PKVS_ERR_INVALID_ARG
        shape = dict(num_qo_heads=64, num_kv_heads=8, batch_capacity=256, qo_capacity=256,
                     kv_capacity=32768, fixed_split_size=2048)
        big = desc(P.PKVS_DECODE, window_left=-1, **shape)
        fb, ib = P.pkvs_workspace_bytes(big, True)
        assert (ib + 255) // 256 * 256 + fb > P.NOALLOC_SCRATCH_BYTES
        plans.append(P.pkvs_plan_create(big))
        assert call(plans[-1]) == P.PKVS_ERR_WORKSPACE
        assert "scratch array" in P.last_error()
        # the same shape with a 4096-key window fits; without a GPU the call
        # stops at the device check, with one it stops at the null tensors
        fits = desc(P.PKVS_DECODE, window_left=4095, **shape)
        fb, ib = P.pkvs_workspace_bytes(fits, True)
        assert (ib + 255) // 256 * 256 + fb <= P.NOALLOC_SCRATCH_BYTES
        plans.append(P.pkvs_plan_create(fits))
        assert call(plans[-1]) in (P.PKVS_ERR_HIP, P.PKVS_ERR_INVALID_ARG)
    finally:
        for h in plans:
            P.pkvs_plan_destroy(h)


def test_run_rejects_a_window_other_than_the_planned_one():
    """run(window_left != plan) fails before touching any data (sglang PR
    'Pass window_left at plan time...', section What)."""
    h = P.pkvs_plan_create(desc(window_left=31))
    qop, kvp, last = csr([5], [5], 16)
    P.pkvs_prefill_plan(h, qop, kvp, last, 1, None, None)
    lib = P._lib
    rc = lib.pkvs_prefill_run(h, None, None, None, 1, None, None, None, 1.0, 30, 1, 1.0, 1.0,
                              None)
    assert rc == P.PKVS_ERR_PLAN_MISMATCH
    rc = lib.pkvs_prefill_run(h, None, None, None, 1, None, None, None, 1.0, 31, 0, 1.0, 1.0,
                              None)
    assert rc == P.PKVS_ERR_PLAN_MISMATCH
    rc = lib.pkvs_prefill_run(h, None, None, None, 1, None, None, None, 1.0, 31, 1, 1.0, 1.0,
                              None)
    assert rc == P.PKVS_ERR_NOT_PLANNED  # a dry plan cannot run
    hd = P.pkvs_plan_create(desc(P.PKVS_DECODE, num_qo_heads=4, window_left=0))
    rc = lib.pkvs_decode_run(hd, None, None, None, 1, None, None, None, 1.0, -1, 1.0, 1.0, None)
    assert rc == P.PKVS_ERR_PLAN_MISMATCH


def test_misaligned_tensors_and_workspaces_are_rejected():
    """q, o, the caches, a cascade's new-token K/V and both workspaces must be
    16-byte aligned; the checks run before any device work (the pointers are
    never dereferenced here)."""
    lib = P._lib
    A, M = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 8)  # aligned, misaligned
    h = P.pkvs_plan_create(desc(window_left=31))
    qop, kvp, last = csr([5], [5], 16)
    P.pkvs_prefill_plan(h, qop, kvp, last, 1, None, None)
    for i in range(4):
        t = [A, A, A, A]
        t[i] = M
        rc = lib.pkvs_prefill_run(h, t[0], t[1], t[2], 1, None, t[3], None, 1.0, 31, 1, 1.0,
                                  1.0, None)
        assert rc == P.PKVS_ERR_INVALID_ARG and "aligned" in P.last_error(), i
    hd = P.pkvs_plan_create(desc(P.PKVS_DECODE, num_qo_heads=4, window_left=0))
    rc = lib.pkvs_decode_run(hd, M, A, A, 1, None, A, None, 1.0, 0, 1.0, 1.0, None)
    assert rc == P.PKVS_ERR_INVALID_ARG
    hc = P.pkvs_plan_create(desc(P.PKVS_CASCADE, window_left=31))
    rc = lib.pkvs_cascade_run(hc, A, M, A, A, A, 1, None, A, None, 1.0, 31, 1.0, 1.0, None)
    assert rc == P.PKVS_ERR_INVALID_ARG
    # a plan into misaligned workspaces (sizes large enough) fails before any copy
    fb, ib = P.pkvs_workspace_size(h)
    big = torch.empty(ib + 64, dtype=torch.uint8)
    (qp, _a), (kp, _b), (lp, _c) = P._host_i32(qop), P._host_i32(kvp), P._host_i32(last)
    fbig = torch.empty(fb + 64, dtype=torch.uint8)
    rc = lib.pkvs_prefill_plan(h, qp, kp, lp, 1, ctypes.c_void_p(fbig.data_ptr()), fb,
                               ctypes.c_void_p(big.data_ptr() + 4), ib, None)
    assert rc == P.PKVS_ERR_INVALID_ARG and "aligned" in P.last_error()
    for x in (h, hd, hc):
        P.pkvs_plan_destroy(x)


def test_workload_plans_fit_their_capacities():
    """The five workloads plan within the workspaces their capacities give."""
    for name in ("tiny_prefill", "prefix_prefill", "decode_sweep", "long_prefill",
                 "split_decode"):
        qo, kv = workload_lengths(name, torch.Generator().manual_seed(1), 12)
        decode = name.endswith("decode") or name == "decode_sweep"
        kind = P.PKVS_DECODE if decode else P.PKVS_PREFILL
        dims = dict(tiny_prefill=(2, 1, 64, 4, torch.float32),
                    prefix_prefill=(4, 1, 256, 16, torch.bfloat16),
                    decode_sweep=(32, 8, 128, 16, torch.bfloat16),
                    long_prefill=(32, 8, 128, 16, torch.bfloat16),
                    split_decode=(64, 8, 128, 16, torch.bfloat16))[name]
        h = P.pkvs_plan_create(desc(kind, num_qo_heads=dims[0], num_kv_heads=dims[1],
                                    head_dim=dims[2], page_size=dims[3], dtype=dims[4],
                                    window_left=4095, batch_capacity=len(kv),
                                    qo_capacity=sum(qo), kv_capacity=max(kv),
                                    fixed_split_size=2048 if name == "split_decode" else -1))
        qop, kvp, last = csr(qo, kv, dims[3])
        if decode:
            P.pkvs_decode_plan(h, kvp, last, len(kv), None, None)
        else:
            P.pkvs_prefill_plan(h, qop, kvp, last, len(kv), None, None)
        assert P.pkvs_plan_get_info(h).num_items > 0
        P.pkvs_plan_destroy(h)


# ----------------------------------------------------------------- cascade prefill


def test_cascade_passes_cover_every_query_once():
    """A two-pass cascade plan (a kernel variant without split key ranges: the
    4x64-row one) lists its extend pass (keys = the request's own query
    tokens, read through a row-index table) and then its prefix pass (queries
    placed after every cached key of the table), each covering every query
    once.  A request may have more new tokens than cached keys."""
    W = 40
    qo = [1, 70, 0, 33, 129, 300]
    tab = [0, 20, 9, 267, 2, 100]  # cached keys in each request's table
    h = P.pkvs_plan_create(desc(P.PKVS_CASCADE, num_qo_heads=8, num_kv_heads=2, window_left=W,
                                prefill_variant=3))
    assert P.pkvs_plan_get_info(h).float_ws_bytes > 0, "expected the two-pass plan"
    qop, kvp, last = csr(qo, tab, 16)
    P.pkvs_cascade_plan(h, qop, kvp, last, len(qo), None, None)
    info = P.pkvs_plan_get_info(h)
    items = P.pkvs_plan_copy_items(h).tolist()
    assert len(items) == info.num_items
    n_ext = sum(1 for it in items if it[6] >= 0 and it[5] == qo[it[0]] and it[4] < qo[it[0]])
    ext, pre = items[:n_ext], items[n_ext:]
    for part, name in ((ext, "extend"), (pre, "prefix")):
        seen = {}
        for b, hk, q0, qn, pos0, kv_len, pbase, kvb in (it[:8] for it in part):
            i0 = q0 - qop[b]
            if name == "extend":
                assert kv_len == qo[b] and pos0 == i0
            else:
                assert kv_len == tab[b] and pbase == kvp[b] and pos0 == tab[b] + i0
            assert kvb % 32 == 0 and kvb <= max(0, pos0 - W)
            for t in range(q0, q0 + qn):
                seen[(b, hk, t)] = seen.get((b, hk, t), 0) + 1
        expect = {(b, hk, t) for b in range(len(qo)) for hk in range(2)
                  for t in range(qop[b], qop[b + 1])}
        assert set(seen) == expect and set(seen.values()) == {1}, name
    # extend tables of consecutive requests do not overlap
    bases = sorted({(it[0], it[6]) for it in ext})
    for (b0, p0), (b1, p1) in zip(bases, bases[1:]):
        assert p1 - p0 >= (qo[b0] + 255) // 256
    P.pkvs_plan_destroy(h)


def test_cascade_one_pass_work_list():
    """With a kernel that reads split key ranges (variant 5, the default for
    head_dim 128, and the register-staged 1 and 2) a cascade runs in one pass:
    one prefill item list over each request's cached keys followed by its new
    tokens (kv_len = table + new, queries at the end, split = table length),
    no float workspace; the other kernels keep the two passes."""
    W = 40
    qo = [1, 70, 0, 33, 129, 300]
    tab = [0, 20, 9, 267, 2, 100]
    h = P.pkvs_plan_create(desc(P.PKVS_CASCADE, num_qo_heads=8, num_kv_heads=2, window_left=W,
                                prefill_variant=5, disable_split_kv=1))
    assert P.pkvs_plan_get_info(h).prefill_variant == 5
    assert P.pkvs_plan_get_info(h).cascade_passes == 1
    assert P.pkvs_workspace_size(h)[0] == 0  # no key split: no float workspace
    qop, kvp, last = csr(qo, tab, 16)
    P.pkvs_cascade_plan(h, qop, kvp, last, len(qo), None, None)
    items = P.pkvs_plan_copy_items(h).tolist()
    assert len(items) == P.pkvs_plan_get_info(h).num_items
    seen = {}
    for it in items:
        b, hk, q0, qn, pos0, kv_len, pbase, kvb, split = it[:9]
        assert kv_len == tab[b] + qo[b] and split == tab[b] and pbase == kvp[b]
        assert pos0 == tab[b] + (q0 - qop[b]) and kvb % 64 == 0 and kvb <= max(0, pos0 - W)
        for t in range(q0, q0 + qn):
            seen[(b, hk, t)] = seen.get((b, hk, t), 0) + 1
    expect = {(b, hk, t) for b in range(len(qo)) for hk in range(2)
              for t in range(qop[b], qop[b + 1])}
    assert set(seen) == expect and set(seen.values()) == {1}
    P.pkvs_plan_destroy(h)
    for variant, one_pass in ((1, True), (2, True), (3, False), (4, False), (6, False)):
        h2 = P.pkvs_plan_create(desc(P.PKVS_CASCADE, num_qo_heads=8, num_kv_heads=2,
                                     window_left=W, prefill_variant=variant))
        info = P.pkvs_plan_get_info(h2)
        assert info.cascade_passes == (1 if one_pass else 2), variant
        # one pass: the key split's partial slots (variants 1 and 2 cut key
        # ranges); two passes: no key split, the paged pass's (o, lse)
        assert info.key_chunks == (8 if one_pass else 1), variant
        assert P.pkvs_workspace_size(h2)[0] > 0, variant
        P.pkvs_plan_destroy(h2)


@pytest.mark.parametrize("kind", [P.PKVS_PREFILL, P.PKVS_CASCADE])
@pytest.mark.parametrize("variant", [1, 2, 5])
def test_key_split_rules(kind, variant):
    """The key split is fixed at plan creation for prefill variants 1, 2 and 5
    (one-pass cascades included), whatever the capacities, with partial slots
    sized from the grid: a batch is cut only with at most one query tile per
    two resident workgroups, into at most one grid of chunks of whole key
    tiles.  disable_split_kv turns it off; variants 3, 4 and 6, the two-pass
    cascade and decode plans never cut."""
    kw = dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, window_left=-1,
              batch_capacity=4, qo_capacity=16384, kv_capacity=16384, prefill_variant=variant)
    h = P.pkvs_plan_create(desc(kind, **kw))
    info = P.pkvs_plan_get_info(h)
    assert info.key_chunks == 8 and info.prefill_variant == variant
    grid, tq = info.grid_blocks, info.query_tile
    fb, _ = P.pkvs_workspace_size(h)
    # 16-bit o + fp32 lse per (slot, query head of the group)
    assert fb == tq * grid * 4 * (128 * 2 + 4)
    plan = P.pkvs_prefill_plan if kind == P.PKVS_PREFILL else P.pkvs_cascade_plan
    # few tiles with long key ranges: cut
    qo, kv = [100, 3], [3000, 1003]
    if kind == P.PKVS_CASCADE:
        kv = [k - q for q, k in zip(qo, kv)]  # cached keys only
    qop, kvp, last = csr(qo, kv, 16)
    plan(h, qop, kvp, last, 2, None, None)
    info = P.pkvs_plan_get_info(h)
    assert info.num_merges == 2 * 103  # every token of both requests, both kv heads
    assert info.num_items <= grid
    # as many tiles as resident workgroups: not cut
    qo, kv = [tq * grid // 2], [tq * grid // 2 + 4000]
    if kind == P.PKVS_CASCADE:
        kv = [4000]
    qop, kvp, last = csr(qo, kv, 16)
    plan(h, qop, kvp, last, 1, None, None)
    assert P.pkvs_plan_get_info(h).num_merges == 0
    P.pkvs_plan_destroy(h)
    h = P.pkvs_plan_create(desc(kind, **{**kw, "disable_split_kv": 1}))
    assert P.pkvs_plan_get_info(h).key_chunks == 1 and P.pkvs_workspace_size(h)[0] == 0
    P.pkvs_plan_destroy(h)


def test_key_split_only_on_its_variants():
    kw = dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, window_left=-1, batch_capacity=4,
              qo_capacity=256, kv_capacity=4096)
    for v in (3, 4, 6):
        h = P.pkvs_plan_create(desc(P.PKVS_PREFILL, prefill_variant=v, **kw))
        assert P.pkvs_plan_get_info(h).key_chunks == 1, v
        assert P.pkvs_workspace_size(h)[0] == 0, v
        P.pkvs_plan_destroy(h)
    h = P.pkvs_plan_create(desc(P.PKVS_CASCADE, prefill_variant=3, **kw))
    assert P.pkvs_plan_get_info(h).cascade_passes == 2
    assert P.pkvs_plan_get_info(h).key_chunks == 1
    P.pkvs_plan_destroy(h)
    kw.pop("qo_capacity")
    h = P.pkvs_plan_create(desc(P.PKVS_DECODE, **kw))
    assert P.pkvs_plan_get_info(h).key_chunks == 1
    P.pkvs_plan_destroy(h)


def test_cascade_workspace_and_errors():
    """The two-pass form (variant 3 reads no split key ranges): its float
    workspace holds the paged pass's (o, lse)."""
    kw = dict(num_qo_heads=8, num_kv_heads=2, window_left=31, qo_capacity=1000,
              kv_capacity=500, batch_capacity=4)
    h = P.pkvs_plan_create(desc(P.PKVS_CASCADE, prefill_variant=3, **kw))
    fb, ib = P.pkvs_workspace_size(h)
    rows = 1000 * 8
    assert fb >= rows * 128 * 2 + rows * 4  # the paged pass's (o, lse)
    hp = P.pkvs_plan_create(desc(P.PKVS_PREFILL, disable_split_kv=1, **kw))
    assert ib > P.pkvs_workspace_size(hp)[1]
    qop, kvp, last = csr([10, 600], [0, 5], 16)
    # the wrong entry point for each kind
    assert err_code(lambda: P.pkvs_prefill_plan(h, qop, kvp, last, 2, None, None)) == \
        P.PKVS_ERR_INVALID_ARG
    assert err_code(lambda: P.pkvs_cascade_plan(hp, qop, kvp, last, 2, None, None)) == \
        P.PKVS_ERR_INVALID_ARG
    P.pkvs_cascade_plan(h, qop, kvp, last, 2, None, None)  # 600 new tokens over 5 cached keys
    # capacities: total new tokens, cached keys per request, batch
    qop2, kvp2, last2 = csr([600, 401], [1, 1], 16)
    assert err_code(lambda: P.pkvs_cascade_plan(h, qop2, kvp2, last2, 2, None, None)) == \
        P.PKVS_ERR_CAPACITY
    qop2, kvp2, last2 = csr([1], [501], 16)
    assert err_code(lambda: P.pkvs_cascade_plan(h, qop2, kvp2, last2, 1, None, None)) == \
        P.PKVS_ERR_CAPACITY
    qop2, kvp2, last2 = csr([1] * 5, [1] * 5, 16)
    assert err_code(lambda: P.pkvs_cascade_plan(h, qop2, kvp2, last2, 5, None, None)) == \
        P.PKVS_ERR_CAPACITY
    # workspaces too small are reported before any device copy
    (qp, _a), (kp, _b), (lp, _c) = P._host_i32(qop), P._host_i32(kvp), P._host_i32(last)
    small = torch.empty(ib // 2, dtype=torch.uint8)
    rc = P._lib.pkvs_cascade_plan(h, qp, kp, lp, 2, None, 0, ctypes.c_void_p(small.data_ptr()),
                                  small.numel(), None)
    assert rc == P.PKVS_ERR_WORKSPACE, P.last_error()
    big = torch.empty(ib, dtype=torch.uint8)
    fsmall = torch.empty(fb // 2, dtype=torch.uint8)
    rc = P._lib.pkvs_cascade_plan(h, qp, kp, lp, 2, ctypes.c_void_p(fsmall.data_ptr()),
                                  fsmall.numel(), ctypes.c_void_p(big.data_ptr()), big.numel(),
                                  None)
    assert rc == P.PKVS_ERR_WORKSPACE, P.last_error()
    # run: window other than the planned one, a dry plan, the wrong kind
    lib = P._lib
    rc = lib.pkvs_cascade_run(h, None, None, None, None, None, 1, None, None, None, 1.0, 30,
                              1.0, 1.0, None)
    assert rc == P.PKVS_ERR_PLAN_MISMATCH
    rc = lib.pkvs_cascade_run(h, None, None, None, None, None, 1, None, None, None, 1.0, 31,
                              1.0, 1.0, None)
    assert rc == P.PKVS_ERR_NOT_PLANNED
    rc = lib.pkvs_cascade_run(hp, None, None, None, None, None, 1, None, None, None, 1.0, 31,
                              1.0, 1.0, None)
    assert rc == P.PKVS_ERR_INVALID_ARG
    # a window needs causal attention, as for prefill
    assert err_code(lambda: P.pkvs_plan_create(desc(P.PKVS_CASCADE, causal=False))) == \
        P.PKVS_ERR_UNSUPPORTED
    P.pkvs_plan_destroy(h)
    P.pkvs_plan_destroy(hp)


# ----------------------------------------------------------------- cache writes, page-table build


def test_append_and_build_reject_bad_arguments():
    """Argument checks run before any launch (so they hold without a GPU)."""
    lib = P._lib
    buf = torch.empty(64, dtype=torch.uint8)
    p = ctypes.c_void_p(buf.data_ptr())
    odd = ctypes.c_void_p(buf.data_ptr() + 2)
    # append: negative count, unsupported dtype, a row that is not 16 bytes, nulls, misalignment
    assert lib.pkvs_append_kv(p, p, p, -1, p, p, 4, 1, 64,
                              P.PKVS_BF16, 0, 1.0, 1.0, None, None) == \
        P.PKVS_ERR_INVALID_ARG
    assert lib.pkvs_append_kv(p, p, p, 1, p, p, 4, 1, 64,
                              7, 0, 1.0, 1.0, None, None) == P.PKVS_ERR_UNSUPPORTED
    assert lib.pkvs_append_kv(p, p, p, 1, p, p, 4, 1, 4, P.PKVS_BF16, 0, 1.0, 1.0, None, None) == \
        P.PKVS_ERR_UNSUPPORTED
    assert lib.pkvs_append_kv(None, p, p, 1, p, p, 4, 1, 64,
                              P.PKVS_BF16, 0, 1.0, 1.0, None, None) == \
        P.PKVS_ERR_INVALID_ARG
    assert lib.pkvs_append_kv(odd, p, p, 1, p, p, 4, 1, 64,
                              P.PKVS_BF16, 0, 1.0, 1.0, None, None) == \
        P.PKVS_ERR_INVALID_ARG
    assert lib.pkvs_append_kv(None, None, None, 0, None, None, 0, 1, 64, P.PKVS_BF16, 0, 1.0,
                              1.0, None, None) == P.PKVS_OK  # nothing to write
    # 8-bit cache: a kv_format outside the enum, scales that are not positive finite
    assert lib.pkvs_append_kv(p, p, p, 1, p, p, 4, 1, 64, P.PKVS_BF16, 3, 1.0, 1.0, None,
                              None) == P.PKVS_ERR_INVALID_ARG
    for ks, vs in ((0.0, 1.0), (1.0, float("nan")), (-1.0, 1.0)):
        assert lib.pkvs_append_kv(p, p, p, 1, p, p, 4, 1, 64, P.PKVS_BF16, 1, ks, vs, None,
                                  None) == P.PKVS_ERR_INVALID_ARG
    # build: negative sizes, missing outputs or inputs
    assert lib.pkvs_build_kv_indices(p, 2, 2, p, None, p, -1, p, p, 4, None, None) == \
        P.PKVS_ERR_INVALID_ARG
    assert lib.pkvs_build_kv_indices(p, 2, 2, p, None, p, 1, None, p, 4, None, None) == \
        P.PKVS_ERR_INVALID_ARG
    assert lib.pkvs_build_kv_indices(None, 2, 2, p, None, p, 1, p, p, 4, None, None) == \
        P.PKVS_ERR_INVALID_ARG
    assert lib.pkvs_build_kv_indices(p, 2, 2, p, None, p, 1, p, None, 4, None, None) == \
        P.PKVS_ERR_INVALID_ARG


@pytest.mark.parametrize("cap", [-1.0, float("nan"), float("inf")])
def test_soft_cap_must_be_zero_or_positive_finite(cap):
    assert err_code(lambda: P.pkvs_plan_create(desc(logits_soft_cap=cap))) == \
        P.PKVS_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(kv_dtype=torch.float8_e4m3fn, dtype=torch.float32), P.PKVS_ERR_UNSUPPORTED),
    (dict(kv_dtype=torch.float8_e5m2, prefill_variant=4), P.PKVS_ERR_UNSUPPORTED),
    (dict(kv_dtype=torch.float8_e4m3fn, prefill_variant=5), P.PKVS_ERR_UNSUPPORTED),
    (dict(kv_dtype=torch.float8_e5m2, prefill_variant=3), P.PKVS_ERR_UNSUPPORTED),
])
def test_fp8_kv_descriptor_rules(kw, code):
    assert err_code(lambda: P.pkvs_plan_create(desc(**kw))) == code


def test_fp8_kv_format_and_scales_are_checked():
    d = desc()
    d.kv_format = 7
    assert err_code(lambda: P.pkvs_plan_create(d)) == P.PKVS_ERR_INVALID_ARG
    # an 8-bit cache never takes the direct-to-LDS kernel, even where it would be chosen
    h = P.pkvs_plan_create(desc(kv_dtype=torch.float8_e4m3fn, head_dim=128, num_qo_heads=32,
                                num_kv_heads=8, qo_capacity=32768, kv_capacity=32768))
    assert P.pkvs_plan_get_info(h).prefill_variant in (1, 2)
    lib = P._lib
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0), (1.0, float("nan"))):
        rc = lib.pkvs_prefill_run(h, None, None, None, 1, None, None, None, 1.0, 31, 1, ks, vs,
                                  None)
        assert rc == P.PKVS_ERR_INVALID_ARG, (ks, vs)
        rc = lib.pkvs_decode_run(h, None, None, None, 1, None, None, None, 1.0, 31, ks, vs, None)
        assert rc == P.PKVS_ERR_INVALID_ARG, (ks, vs)
    P.pkvs_plan_destroy(h)
