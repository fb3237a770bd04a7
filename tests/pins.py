"""Checks that pin the CPU oracle to facts fixed outside it.

Each ``check_*`` takes an ``oracle.OracleLib`` (or None for the default build)
and raises AssertionError when the oracle disagrees with:

* closed forms (all-zero queries: LSE = ln(number of visible keys) and the
  output is the plain mean of the visible values),
* exact special cases (window_left = 0 returns the value at the query's own
  position; one-hot values expose the attention support),
* a library routine (torch scaled_dot_product_attention and logsumexp in
  float64; scipy softmax / logsumexp in the brute force),
* invariants (page size and page placement, grouped-query heads = repeated
  heads, window saturation, merge of a split = unsplit result),
* the trims the pages state for the sliding-window wrappers,
* hand-derived counts stored under ``tests/golden``.

They are small so the whole set also runs against deliberately broken copies
of the oracle (see ``test_oracle_mutants.py``).
"""
from __future__ import annotations

import dataclasses
import math
import os

import numpy as np
import torch

import oracle
from oracle import dense
from paged_kv_sliding_amd.synth import case_from_lengths  # noqa: F401 (also used directly)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def small_case(qo_lens, kv_lens, *, H_q=2, H_kv=1, D=16, P=4, W=4, seed=0,
               dtype=torch.float32, spare=2, causal=True, sm_scale=None, soft_cap=0.0):
    return case_from_lengths("pin", qo_lens, kv_lens, num_qo_heads=H_q, num_kv_heads=H_kv,
                             head_dim=D, page_size=P, dtype=dtype, window_left=W, seed=seed,
                             causal=causal, spare_pages=spare, sm_scale=sm_scale,
                             logits_soft_cap=soft_cap)


def run(case, impl, **kw):
    return oracle.case_attention(case, impl=impl, **kw)


def dense_kv(case, b):
    """Logical [kv_len, H_kv, D] keys and values of request b (host, float64)."""
    P = case.page_size
    pages = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]].long()
    n = case.kv_lens[b]
    K = case.k_cache[pages].reshape(-1, case.num_kv_heads, case.head_dim)[:n]
    V = case.v_cache[pages].reshape(-1, case.num_kv_heads, case.head_dim)[:n]
    assert len(pages) * P >= n
    return K.double().numpy(), V.double().numpy()


def visible_range(p, W):
    """First and last visible key of a causal query at position p."""
    return (max(0, p - W) if W >= 0 else 0), p


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return rows


def close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    with np.errstate(invalid="ignore"):
        ok = same_inf | (np.abs(a - b) <= tol * np.maximum(1.0, np.abs(b)))
    return bool(ok.all())


# --------------------------------------------------------------------------- closed forms


def check_zero_query_closed_form(impl=None):
    """q = 0: every visible logit is 0, so LSE = ln n and O = mean of visible V."""
    for W in (-1, 0, 1, 3, 4, 9, 40):
        for P in (1, 4):
            case = small_case([5, 3, 7], [5, 9, 20], W=W, P=P, H_q=4, H_kv=2, seed=11 + W)
            case.q.zero_()
            o, lse = run(case, impl)
            t = 0
            for b in range(case.batch_size):
                _, V = dense_kv(case, b)
                prefix = case.kv_lens[b] - case.qo_lens[b]
                for i in range(case.qo_lens[b]):
                    p = prefix + i
                    lo, hi = visible_range(p, W)
                    n = hi - lo + 1
                    for h in range(case.num_qo_heads):
                        hk = h // (case.num_qo_heads // case.num_kv_heads)
                        assert lse[t, h] == math.log(n), (W, P, b, i, lse[t, h], n)
                        assert close(o[t, h], V[lo:hi + 1, hk].mean(axis=0)), (W, P, b, i)
                    t += 1


def check_golden_decode_counts(impl=None):
    """Decode query at kv_len-1 sees W+1 keys (tests/golden/window_counts.txt)."""
    for kv_len, W, count in read_golden("window_counts.txt"):
        case = small_case([1], [kv_len], W=W, P=16, H_q=1, H_kv=1, D=4, seed=kv_len)
        case.q.zero_()
        _, lse = run(case, impl)
        assert lse[0, 0] == math.log(count), (kv_len, W, count, math.exp(lse[0, 0]))


def check_golden_extend_counts(impl=None):
    """No-prefix extend 6/8/12 with window 4 (tests/golden/extend_window4_counts.txt)."""
    table = read_golden("extend_window4_counts.txt")
    for E in (6, 8, 12):
        case = small_case([E], [E], W=4, P=4, H_q=2, H_kv=1, D=8, seed=E)
        case.q.zero_()
        _, lse = run(case, impl)
        for e, pos, count in table:
            if e == E:
                assert lse[pos, 0] == math.log(count), (E, pos, count)
                assert lse[pos, 1] == math.log(count), (E, pos, count)


# --------------------------------------------------------------------------- exact cases


def check_one_hot_support(impl=None):
    """V_j = e_j: row O[i] holds the attention weights, nonzero exactly on V(p)."""
    D = 32
    for W in (-1, 0, 2, 5):
        case = small_case([6, 10], [9, 30], W=W, P=4, H_q=2, H_kv=1, D=D, seed=3 + W)
        for b in range(case.batch_size):
            n = case.kv_lens[b]
            assert n <= D
            for j in range(n):
                pg = int(case.kv_indices[int(case.kv_indptr[b]) + j // case.page_size])
                case.v_cache[pg, j % case.page_size].zero_()
                case.v_cache[pg, j % case.page_size, :, j] = 1.0
        o, _ = run(case, impl)
        t = 0
        for b in range(case.batch_size):
            prefix = case.kv_lens[b] - case.qo_lens[b]
            for i in range(case.qo_lens[b]):
                lo, hi = visible_range(prefix + i, W)
                for h in range(2):
                    row = o[t, h]
                    support = set(np.nonzero(row)[0].tolist())
                    assert support == set(range(lo, hi + 1)), (W, b, i, h, support)
                    assert abs(row.sum() - 1.0) < 1e-12
                t += 1


def check_window_zero_is_own_value(impl=None):
    """W = 0: O = V at the query position bit for bit; LSE = its own logit."""
    case = small_case([4, 6], [10, 6], W=0, P=4, H_q=4, H_kv=2, D=16, seed=21,
                      dtype=torch.bfloat16)
    o, lse = run(case, impl)
    q = case.q.double().numpy()
    t = 0
    for b in range(case.batch_size):
        K, V = dense_kv(case, b)
        prefix = case.kv_lens[b] - case.qo_lens[b]
        for i in range(case.qo_lens[b]):
            p = prefix + i
            for h in range(4):
                hk = h // 2
                assert np.array_equal(o[t, h], V[p, hk]), (b, i, h)
                ref = case.sm_scale * float(np.dot(q[t, h], K[p, hk]))
                assert close(lse[t, h], ref), (b, i, h, lse[t, h], ref)
            t += 1


# --------------------------------------------------------------------------- library routines


def _sdpa_reference(case, W):
    """torch SDPA (float64, CPU) with an explicit bottom-right window mask."""
    G = case.num_qo_heads // case.num_kv_heads
    q = case.q.double()
    outs, lses = [], []
    for b in range(case.batch_size):
        K, V = dense_kv(case, b)
        K = torch.from_numpy(K).repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        V = torch.from_numpy(V).repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        qb = q[case.qo_indptr[b]:case.qo_indptr[b + 1]].transpose(0, 1).contiguous()
        nq, nk = qb.shape[1], K.shape[1]
        pos = torch.arange(nk - nq, nk)[:, None]
        key = torch.arange(nk)[None, :]
        mask = key <= pos
        if W >= 0:
            mask &= key >= pos - W
        o = torch.nn.functional.scaled_dot_product_attention(
            qb[None], K[None], V[None], attn_mask=mask[None, None], scale=case.sm_scale)[0]
        logits = case.sm_scale * torch.matmul(qb, K.transpose(1, 2).contiguous())
        lse = torch.logsumexp(logits.masked_fill(~mask[None], float("-inf")), dim=-1)
        outs.append(o.transpose(0, 1))
        lses.append(lse.transpose(0, 1))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def check_matches_sdpa(impl=None):
    """W = -1 (plain causal) and W >= 0 against torch SDPA in float64."""
    for W in (-1, 0, 3, 17):
        case = small_case([7, 1, 12], [7, 20, 40], W=W, P=4, H_q=4, H_kv=2, D=16, seed=40 + W)
        o, lse = run(case, impl)
        ro, rl = _sdpa_reference(case, W)
        assert close(o, ro, 1e-11), W
        assert close(lse, rl, 1e-11), W


def check_brute_force_dense(impl=None):
    """Every W in -1..kv_len on kv_len <= 16 against the dense SciPy version."""
    for P in (1, 2, 4, 16):
        for W in range(-1, 17):
            case = small_case([3, 5, 1, 16], [7, 5, 1, 16], W=W, P=P, H_q=3, H_kv=1, D=8,
                              seed=100 + 17 * P + W)
            o, lse = run(case, impl)
            ro, rl = dense.attention(case)
            assert close(o, ro), (P, W)
            assert close(lse, rl), (P, W)


# --------------------------------------------------------------------------- invariants


def check_saturation_is_no_window(impl=None):
    """W >= kv_len - 1 gives exactly the W = -1 result."""
    case = small_case([5, 9], [12, 9], W=-1, P=4, H_q=2, H_kv=1, D=16, seed=5)
    o_ref, l_ref = run(case, impl, window_left=-1)
    for W in (11, 12, 50):
        o, l = run(case, impl, window_left=W)
        assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref), W
    o, l = run(case, impl, window_left=10)
    assert not np.array_equal(l, l_ref)


def check_gqa_is_repeated_heads(impl=None):
    """Grouped heads equal MHA over KV heads repeated G times, bit for bit."""
    case = small_case([4, 6], [9, 13], W=5, P=4, H_q=6, H_kv=2, D=16, seed=8)
    o, l = run(case, impl)
    G = 3
    o2, l2 = oracle.paged_attention(
        case.q, case.k_cache.repeat_interleave(G, dim=2), case.v_cache.repeat_interleave(G, dim=2),
        case.qo_indptr, case.kv_indptr, case.kv_indices, case.kv_last_page_len,
        num_qo_heads=6, num_kv_heads=6, head_dim=16, page_size=4, causal=True, window_left=5,
        sm_scale=case.sm_scale, impl=impl)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def repage(case, P, seed):
    """Same logical keys/values stored with page size P in a new random placement."""
    Ks, Vs = [], []
    for b in range(case.batch_size):
        K, V = dense_kv(case, b)
        Ks.append(torch.from_numpy(K).to(case.dtype))
        Vs.append(torch.from_numpy(V).to(case.dtype))
    npages = [(n + P - 1) // P for n in case.kv_lens]
    total = sum(npages)
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(total + 3, generator=g)[:total]
    kc = torch.full((total + 3, P, case.num_kv_heads, case.head_dim), float("nan"),
                    dtype=case.dtype)
    vc = kc.clone()
    pi = 0
    for b in range(case.batch_size):
        for j in range(case.kv_lens[b]):
            pg = int(perm[pi + j // P])
            kc[pg, j % P] = Ks[b][j]
            vc[pg, j % P] = Vs[b][j]
        pi += npages[b]
    kvp = torch.zeros(case.batch_size + 1, dtype=torch.int32)
    kvp[1:] = torch.tensor(npages).cumsum(0)
    last = torch.tensor([0 if n == 0 else n - (m - 1) * P for n, m in zip(case.kv_lens, npages)],
                        dtype=torch.int32)
    return kc, vc, kvp, perm.to(torch.int32), last


def check_paging_invariance(impl=None):
    """Page size and page placement do not change a single bit of the result."""
    case = small_case([5, 3, 9], [11, 3, 17], W=6, P=4, H_q=2, H_kv=1, D=16, seed=9,
                      dtype=torch.bfloat16)
    o, l = run(case, impl)
    for P, seed in ((1, 1), (2, 2), (16, 3), (4, 4)):
        kc, vc, kvp, kvi, last = repage(case, P, seed)
        o2, l2 = oracle.paged_attention(
            case.q, kc, vc, case.qo_indptr, kvp, kvi, last, num_qo_heads=2, num_kv_heads=1,
            head_dim=16, page_size=P, causal=True, window_left=6, sm_scale=case.sm_scale,
            impl=impl)
        assert np.array_equal(o, o2) and np.array_equal(l, l2), P


def check_empty_sets(impl=None):
    """An empty request, or a key range with nothing visible: O = 0, LSE = -inf."""
    case = small_case([0, 2, 0, 1], [0, 5, 3, 0], W=1, P=4, H_q=2, H_kv=1, D=8, seed=13)
    o, l = run(case, impl)
    assert o.shape[0] == 3 and np.isfinite(l[:2]).all()
    assert (o[2] == 0).all() and np.isneginf(l[2]).all()  # queries of a keyless request
    o, l = run(case, impl, key_lo=0, key_hi=2)  # queries at p=3,4 with W=1 see keys >= 2
    assert (o == 0).all() and np.isneginf(l).all()


# --------------------------------------------------------------------------- trims on the pages


def check_decode_trim(impl=None):
    """Decode: the window equals the last min(kv_len, W+1) keys, unwindowed
    (sglang FlashInferIndicesUpdaterDecode.update_sliding_window)."""
    for W in (0, 3, 31):
        case = small_case([1] * 4, [1, 7, 33, 64], W=W, P=4, H_q=4, H_kv=1, D=16, seed=50 + W)
        o, l = run(case, impl)
        for b, n in enumerate(case.kv_lens):
            start = n - min(n, W + 1)
            o2, l2 = run(case, impl, window_left=-1, rows=[b], key_lo=start)
            assert np.array_equal(o[b], o2[0]) and l[b].tolist() == l2[0].tolist(), (W, b)


def check_prefill_trim(impl=None):
    """Paged extend: keys before seq - min(seq, W + seq - prefix) are invisible to
    every query, and the first extend query sees all keys from there on
    (sglang FlashInferIndicesUpdaterPrefill.update_sliding_window, paged branch)."""
    W = 5
    case = small_case([4, 3], [12, 3], W=W, P=4, H_q=2, H_kv=1, D=16, seed=61)
    o, l = run(case, impl)
    for b in range(case.batch_size):
        seq, ext = case.kv_lens[b], case.qo_lens[b]
        prefix = seq - ext
        paged_len = min(seq, W + seq - prefix)
        start = seq - paged_len
        rows = list(range(int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])))
        o2, l2 = run(case, impl, rows=rows, key_lo=start)
        assert np.array_equal(o[rows], o2) and np.array_equal(l[rows], l2)
        if start > 0:
            o3, l3 = run(case, impl, rows=rows[:1], key_lo=start + 1)
            assert l3[0].tolist() != l[rows[0]].tolist()


# --------------------------------------------------------------------------- merge


def check_merge_split_equals_unsplit(impl=None):
    """Merging the partials of two (and of many) key ranges gives the unsplit result."""
    for W in (-1, 0, 7, 20):
        case = small_case([1, 1, 6], [40, 25, 30], W=W, P=4, H_q=4, H_kv=2, D=16, seed=70 + W)
        o, l = run(case, impl)
        rng = np.random.default_rng(W + 5)
        cuts = sorted(set(rng.integers(1, 40, size=4).tolist()))
        edges = [0] + cuts + [10 ** 9]
        parts = [run(case, impl, key_lo=a, key_hi=b) for a, b in zip(edges[:-1], edges[1:])]
        v, s = oracle.merge_many(parts, impl=impl)
        assert close(v, o, 1e-12) and close(s, l, 1e-12), W


def check_merge_algebra(impl=None):
    """-inf partial is an identity; merge is commutative; associative to 1e-12."""
    rng = np.random.default_rng(0)
    n, H, D = 5, 3, 8
    va, vb, vc = (rng.standard_normal((n, H, D)) for _ in range(3))
    sa, sb, sc = (rng.standard_normal((n, H)) * 4 for _ in range(3))
    ninf = np.full((n, H), -np.inf)
    v, s = oracle.merge_state(va, sa, np.zeros_like(va), ninf, impl=impl)
    assert np.array_equal(v, va) and np.array_equal(s, sa)
    v, s = oracle.merge_state(np.zeros_like(va), ninf, np.zeros_like(va), ninf, impl=impl)
    assert (v == 0).all() and np.isneginf(s).all()
    v1, s1 = oracle.merge_state(va, sa, vb, sb, impl=impl)
    v2, s2 = oracle.merge_state(vb, sb, va, sa, impl=impl)
    assert np.array_equal(v1, v2) and np.array_equal(s1, s2)
    l1 = oracle.merge_state(*oracle.merge_state(va, sa, vb, sb, impl=impl), vc, sc, impl=impl)
    l2 = oracle.merge_state(va, sa, *oracle.merge_state(vb, sb, vc, sc, impl=impl), impl=impl)
    assert close(l1[0], l2[0]) and close(l1[1], l2[1])
    # a closed form: equal LSEs average the values and add ln 2
    v, s = oracle.merge_state(va, sa, vb, sa, impl=impl)
    assert close(v, (va + vb) / 2) and close(s, sa + math.log(2.0))


# --------------------------------------------------------------------------- input widening


def check_widening_every_8_bit_pattern(impl=None):
    """Every OCP e4m3 ("fn") and e5m2 byte widens to the float64 torch's
    float8 types give (NaN to NaN, e5m2 infinities to infinities)."""
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for dt in (torch.float8_e4m3fn, torch.float8_e5m2):
        got = oracle.widen(bits.view(dt), impl=impl)
        want = bits.view(dt).to(torch.float64).numpy()
        assert np.array_equal(got, want, equal_nan=True), dt


def check_kv_scales(impl=None):
    """An 8-bit cache with scales reads as k_scale * k, v_scale * v: with
    power-of-two scales the oracle equals the oracle on an fp32 cache holding
    those products (exact), and for any scale k_scale moves into sm_scale
    and v_scale multiplies the output."""
    for dt in (torch.float8_e4m3fn, torch.float8_e5m2):
        case = case_from_lengths("pin8", [3, 5], [9, 5], num_qo_heads=4, num_kv_heads=2,
                                 head_dim=16, page_size=4, dtype=torch.float32, window_left=4,
                                 seed=12, spare_pages=2, kv_dtype=dt, k_scale=0.125,
                                 v_scale=4.0)
        o, lse = run(case, impl)
        wide = dataclasses.replace(case, k_cache=case.k_cache.float() * 0.125,
                                   v_cache=case.v_cache.float() * 4.0, k_scale=1.0, v_scale=1.0)
        o2, l2 = run(wide, impl)
        assert np.array_equal(o, o2, equal_nan=True) and np.array_equal(lse, l2), dt
        odd = dataclasses.replace(case, k_scale=0.37, v_scale=1.9)
        o3, l3 = run(odd, impl)
        ref = dataclasses.replace(case, k_scale=1.0, v_scale=1.0, sm_scale=case.sm_scale * 0.37)
        o4, l4 = run(ref, impl)
        assert close(l3, l4) and close(o3, 1.9 * o4), dt


def check_quantize_every_16_bit_pattern(impl=None):
    """An 8-bit cache write divides by the scale in the input dtype and
    rounds to the 8-bit type: for every bf16 and half bit pattern and three
    scales the code equals torch's (x / scale).to(float8) (a NaN input gives a
    NaN code; its sign is the platform's)."""
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    for src in (torch.bfloat16, torch.float16):
        x = bits.view(src)
        nan = torch.isnan(x).numpy()
        for dt in (torch.float8_e4m3fn, torch.float8_e5m2):
            for sc in (1.0, 0.0625, 0.37):
                want = (x / torch.tensor(sc, dtype=torch.float32)).to(dt).view(torch.uint8).numpy()
                got = oracle.quantize(x, sc, dt, impl=impl)
                assert np.array_equal(got[~nan], want[~nan]), (src, dt, sc)
                assert (got[nan] & 0x7F == 0x7F).all(), (src, dt, sc)


def check_widening_every_16_bit_pattern(impl=None):
    """Every bf16 and every IEEE half bit pattern widens to the float64 that
    torch's / numpy's own conversions give (NaN patterns to NaN); fp32 values
    pass through unchanged."""
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    for dt in (torch.bfloat16, torch.float16):
        got = oracle.widen(bits.view(dt), impl=impl)
        want = bits.view(dt).to(torch.float64).numpy()
        if dt == torch.float16:
            want_np = bits.numpy().view(np.float16).astype(np.float64)
            assert np.array_equal(want, want_np, equal_nan=True)
        assert np.array_equal(got, want, equal_nan=True), dt
    x = torch.randn(1000, dtype=torch.float32) * 1e3
    assert np.array_equal(oracle.widen(x, impl=impl), x.double().numpy())


# --------------------------------------------------------------------------- logits soft cap


def check_soft_cap_brute_force(impl=None):
    """With a cap c each scaled logit x becomes c * tanh(x / c): the oracle
    equals the dense NumPy version (numpy's tanh) on tiny inputs."""
    for cap in (0.7, 3.0, 30.0):
        for W in (-1, 0, 3):
            case = small_case([3, 6], [8, 6], W=W, P=2, H_q=4, H_kv=2, seed=int(cap * 10) + W,
                              sm_scale=0.9, soft_cap=cap)
            o, lse = run(case, impl)
            ro, rl = dense.attention(case)
            assert close(o, ro) and close(lse, rl), (cap, W)


def check_soft_cap_saturation(impl=None):
    """Keys all equal to u and queries = 1000 u: every logit is huge, the cap
    saturates at c, so LSE = c + ln n and O is the plain mean of the visible
    values."""
    cap = 5.0
    case = small_case([4], [9], W=3, P=4, H_q=1, H_kv=1, D=8, seed=3, soft_cap=cap)
    u = torch.linspace(0.5, 1.5, 8)
    case.k_cache[:] = u
    case.q[:] = 1000.0 * u
    o, lse = run(case, impl)
    _, V = dense_kv(case, 0)
    for i in range(4):
        lo, hi = visible_range(5 + i, 3)
        assert close(lse[i, 0], cap + math.log(hi - lo + 1)), (i, lse[i, 0])
        assert close(o[i, 0], V[lo:hi + 1, 0].mean(axis=0)), i


def check_soft_cap_large_is_no_cap(impl=None):
    """c * tanh(x / c) -> x as c grows: a cap of 1e6 changes nothing beyond
    1e-9."""
    case = small_case([5], [12], W=6, P=4, H_q=2, H_kv=1, seed=9, soft_cap=1e6)
    o, lse = run(case, impl)
    case.logits_soft_cap = 0.0
    o0, l0 = run(case, impl)
    assert close(o, o0, tol=1e-9) and close(lse, l0, tol=1e-9)
    assert not np.array_equal(lse, l0)  # the cap is applied at all


# --------------------------------------------------------------------------- cache writes, page tables


def check_append_round_trip(impl=None):
    """Writing every key / value of a paged batch into an empty pool at slot
    page * P + (position mod P) rebuilds the cache at those slots, and the
    attention over the rebuilt pool equals the attention over the original."""
    for P in (1, 4):
        case = small_case([3, 5, 1], [7, 5, 13], P=P, H_q=4, H_kv=2, D=8, seed=20 + P)
        kvp = case.kv_indptr.tolist()
        loc, ks, vs = [], [], []
        for b in range(case.batch_size):
            K, V = dense_kv(case, b)
            pages = case.kv_indices[kvp[b]:kvp[b + 1]].tolist()
            for j in range(case.kv_lens[b]):
                loc.append(pages[j // P] * P + j % P)
            ks.append(torch.from_numpy(K).float())
            vs.append(torch.from_numpy(V).float())
        order = np.random.default_rng(P).permutation(len(loc))  # any write order
        k_new = torch.cat(ks)[order]
        v_new = torch.cat(vs)[order]
        loc = torch.tensor(loc)[order]
        empty_k = torch.full_like(case.k_cache, float("nan"))
        empty_v = torch.full_like(case.v_cache, float("nan"))
        kc, vc, skipped = oracle.append_kv(k_new, v_new, loc, empty_k, empty_v, impl=impl)
        assert skipped == 0
        flat = lambda t: t.reshape(-1, case.num_kv_heads, case.head_dim)
        assert torch.equal(flat(kc)[loc], flat(case.k_cache)[loc])
        assert torch.equal(flat(vc)[loc], flat(case.v_cache)[loc])
        rebuilt = dataclasses.replace(case, k_cache=kc, v_cache=vc)
        o1, l1 = run(case, impl)
        o2, l2 = run(rebuilt, impl)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), P


def check_append_matches_scatter(impl=None):
    """Row i lands in slot loc[i] (numpy indexed assignment); rows whose slot
    lies outside the pool are skipped and counted; other slots keep their
    bytes (bf16 rows, compared bit for bit)."""
    rng = np.random.default_rng(5)
    cache_k = torch.from_numpy(rng.standard_normal((6, 4, 2, 8))).to(torch.bfloat16)
    cache_v = torch.from_numpy(rng.standard_normal((6, 4, 2, 8))).to(torch.bfloat16)
    k_new = torch.from_numpy(rng.standard_normal((7, 2, 8))).to(torch.bfloat16)
    v_new = torch.from_numpy(rng.standard_normal((7, 2, 8))).to(torch.bfloat16)
    loc = np.array([23, 0, -1, 5, 24, 17, 9])
    kc, vc, skipped = oracle.append_kv(k_new, v_new, torch.from_numpy(loc), cache_k, cache_v,
                                       impl=impl)
    assert skipped == 2
    for got, cache, new in ((kc, cache_k, k_new), (vc, cache_v, v_new)):
        want = cache.view(torch.int16).numpy().reshape(24, 2, 8).copy()
        ok = (loc >= 0) & (loc < 24)
        want[loc[ok]] = new.view(torch.int16).numpy()[ok]
        assert np.array_equal(got.view(torch.int16).numpy().reshape(24, 2, 8), want)


def check_append_into_8_bit_cache(impl=None):
    """Rows written into an 8-bit cache land at their slots as torch's
    (row / scale).to(float8) (bf16 rows, e4m3 and e5m2, K and V with their
    own scales); other slots keep their bytes; out-of-pool slots are counted."""
    g = torch.Generator().manual_seed(8)
    for dt in (torch.float8_e4m3fn, torch.float8_e5m2):
        cache_k = (torch.randn(5, 4, 2, 8, generator=g) * 3).to(dt)
        cache_v = (torch.randn(5, 4, 2, 8, generator=g) * 3).to(dt)
        k_new = (torch.randn(6, 2, 8, generator=g) * 40).to(torch.bfloat16)
        v_new = (torch.randn(6, 2, 8, generator=g) * 40).to(torch.bfloat16)
        loc = torch.tensor([19, 0, -1, 7, 20, 3])
        kc, vc, skipped = oracle.append_kv_quant(k_new, v_new, loc, cache_k, cache_v, 0.25, 0.4,
                                                 impl=impl)
        assert skipped == 2
        for got, cache, new, sc in ((kc, cache_k, k_new, 0.25), (vc, cache_v, v_new, 0.4)):
            want = cache.view(torch.uint8).reshape(20, 2, 8).clone()
            ok = (loc >= 0) & (loc < 20)
            q = (new / torch.tensor(sc, dtype=torch.float32)).to(dt).view(torch.uint8)
            want[loc[ok]] = q[ok]
            assert torch.equal(got.view(torch.uint8).reshape(20, 2, 8), want), dt


def check_build_indices_golden(impl=None):
    """The hand-derived example of tests/golden/kv_indices_build.txt."""
    rows = {}
    with open(os.path.join(GOLDEN, "kv_indices_build.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                rows.setdefault(key, []).append([int(v) for v in vals])
    m = np.array([[100 * r + c for c in range(6)] for r in range(4)], dtype=np.int32)
    spec = np.array(rows["map"])
    indptr, idx, err = oracle.build_kv_indices(m, spec[:, 0], spec[:, 2], start=spec[:, 1],
                                               impl=impl)
    assert err == 0
    assert indptr.tolist() == rows["indptr"][0]
    assert idx.tolist() == rows["indices"][0]


def check_build_indices_reproduce_page_tables(impl=None):
    """A map whose rows hold each request's pages (rows in shuffled order, junk
    after the last page) gives back the batch's CSR page table; with a start it
    gives the slice from that page on (numpy slicing)."""
    case = small_case([1, 1, 1, 1], [9, 1, 30, 17], P=4, seed=31, spare=5)
    kvp = case.kv_indptr.tolist()
    pages = [case.kv_indices[kvp[b]:kvp[b + 1]].tolist() for b in range(4)]
    cols = max(len(p) for p in pages) + 3
    row_of = [2, 0, 3, 1]
    m = np.full((4, cols), 999, dtype=np.int32)
    for b, p in enumerate(pages):
        m[row_of[b], :len(p)] = p
    lens = [len(p) for p in pages]
    indptr, idx, err = oracle.build_kv_indices(m, row_of, lens, impl=impl)
    assert err == 0 and indptr.tolist() == kvp
    assert idx.tolist() == case.kv_indices.tolist()
    start = [1, 0, 5, 2]
    lens2 = [lens[b] - start[b] for b in range(4)]
    indptr, idx, err = oracle.build_kv_indices(m, row_of, lens2, start=start, impl=impl)
    want = np.concatenate([m[row_of[b], start[b]:start[b] + lens2[b]] for b in range(4)])
    assert err == 0 and np.array_equal(idx, want)
    assert np.array_equal(np.diff(indptr), lens2)


def check_build_indices_errors(impl=None):
    """Entries outside the map come out as -1, a negative length counts as 0,
    entries past the capacity are not written; each is counted."""
    m = np.arange(12, dtype=np.int32).reshape(3, 4)
    indptr, idx, err = oracle.build_kv_indices(m, [0, 5, 2, 1], [2, 1, -3, 3],
                                               start=[3, 0, 0, -1], capacity=5, impl=impl)
    assert indptr.tolist() == [0, 2, 3, 3, 6]
    # request 0: col 3 ok, col 4 outside; request 1: row 5 outside;
    # request 2: negative length; request 3: col -1 outside, col 0 ok, dst 5 past capacity
    assert idx.tolist() == [3, -1, -1, -1, 4]
    assert err == 1 + 1 + 1 + 1 + 1


ALL_CHECKS = [
    check_zero_query_closed_form,
    check_golden_decode_counts,
    check_golden_extend_counts,
    check_one_hot_support,
    check_window_zero_is_own_value,
    check_matches_sdpa,
    check_brute_force_dense,
    check_saturation_is_no_window,
    check_gqa_is_repeated_heads,
    check_paging_invariance,
    check_empty_sets,
    check_decode_trim,
    check_widening_every_16_bit_pattern,
    check_widening_every_8_bit_pattern,
    check_quantize_every_16_bit_pattern,
    check_kv_scales,
    check_soft_cap_brute_force,
    check_soft_cap_saturation,
    check_soft_cap_large_is_no_cap,
    check_append_round_trip,
    check_append_matches_scatter,
    check_append_into_8_bit_cache,
    check_build_indices_golden,
    check_build_indices_reproduce_page_tables,
    check_build_indices_errors,
    check_prefill_trim,
    check_merge_split_equals_unsplit,
    check_merge_algebra,
]
