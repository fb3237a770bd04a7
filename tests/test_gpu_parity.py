"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Tolerances: max |O - O_ref| <= 2e-2 and max |LSE - LSE_ref| <= 1e-3, compared
in fp32; masking is checked bit-exactly (window_left = 0 returns V at the
query's own position; one-hot values expose the attention support)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (assert_all_written, compare, gpu_run, kv_dtype_of, log, make_attention,
                         oracle_for, poisoned_outputs, sub_case)
from paged_kv_sliding_amd import pkvs as P
from paged_kv_sliding_amd.synth import build_case, cascade_inputs, case_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda"


def small(qo, kv, *, H_q=4, H_kv=1, D=128, P_=16, W=31, seed=0, dtype=torch.bfloat16,
          decode=False, split=-1, spare=3, cap=0.0, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    return case_from_lengths("small", qo, kv, num_qo_heads=H_q, num_kv_heads=H_kv, head_dim=D,
                             page_size=P_, dtype=dtype, window_left=W, seed=seed,
                             spare_pages=spare, device=DEV, is_decode=decode,
                             fixed_split_size=split, logits_soft_cap=cap, kv_dtype=kv_dtype,
                             k_scale=k_scale, v_scale=v_scale)


# ----------------------------------------------------------------- the five workloads


@pytest.mark.parametrize("E", [6, 8, 12])
def test_tiny_prefill_fp32(E):
    case = build_case("tiny_prefill", device=DEV, extend_len=E)
    log(f"tiny_prefill E={E} W={case.window_left}")
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"tiny E={E}")
    # positions past the window really lose keys: LSE differs from no window
    if E > 5:
        _, rl_full = oracle_for(case, window_left=-1)
        assert np.abs(rl[5:] - rl_full[5:]).max() > 1e-3


def test_tiny_prefill_fp32_batched():
    cases = [build_case("tiny_prefill", device="cpu", extend_len=E) for E in (6, 8, 12)]
    qo = [c.qo_lens[0] for c in cases]
    case = case_from_lengths("tiny3", qo, qo, num_qo_heads=2, num_kv_heads=1, head_dim=64,
                             page_size=4, dtype=torch.float32, window_left=4, seed=7,
                             spare_pages=6, device=DEV)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="tiny batch of 3")


def test_prefix_prefill_full():
    """The 8-request batch with cached prefixes: its 56 query tiles leave most
    CUs idle, so the planner cuts their key ranges (key split) and merges the
    chunk partials; every row written, against the oracle."""
    case = build_case("prefix_prefill", device=DEV)
    log(f"prefix_prefill qo={case.qo_lens} kv={case.kv_lens}")
    att = make_attention(case)
    o, lse = gpu_run(case, att=att)
    info = att.info()
    log(f"  key chunks {info.key_chunks}, items {info.num_items}, merges {info.num_merges}")
    assert info.num_merges > 0
    assert_all_written(case, o, lse, "prefix_prefill")
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="prefix_prefill")


@pytest.mark.parametrize("W", [-1, 0, 31, 127, 1023])
def test_decode_sweep_full(W):
    case = build_case("decode_sweep", device=DEV, window_left=W)
    log(f"decode_sweep W={W}")
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"decode_sweep W={W}")


def test_decode_sweep_saturation_equals_no_window():
    case = build_case("decode_sweep", device=DEV, window_left=-1)
    o1, l1 = gpu_run(case, window_left=-1)
    o2, l2 = gpu_run(case, window_left=max(case.kv_lens) - 1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


LONG_ROWS = [0, 1, 2, 7, 8, 31, 32, 33, 127, 128, 129, 4094, 4095, 4096, 4097, 4127, 4128, 8191,
             8192, 12345, 16384, 20000, 24575, 30001, 32735, 32736, 32766, 32767]


def test_long_prefill_every_item():
    """The full 32k-token prefill in the benchmark's launch configuration (the
    64-key-step kernel, work items claimed at run time), into NaN-filled
    outputs: every output row must be written, and the oracle checks one
    token of every 64-token query tile (each tile is one work item per kv head;
    all 32 heads of the token are compared, so every item owns a checked row),
    plus the window edges."""
    case = build_case("long_prefill", device=DEV)
    log("long_prefill run")
    att = make_attention(case)
    o, lse = gpu_run(case, att=att)
    info = att.info()
    assert info.prefill_variant == 5  # the 64-key-step kernel the bench times
    tile = info.query_tile
    assert tile == 64 and info.num_items == (32768 // tile) * case.num_kv_heads
    assert info.num_items > info.grid_blocks  # workgroups take several items each
    assert_all_written(case, o, lse, tag="long_prefill")
    rng = np.random.default_rng(4)
    rows = set(LONG_ROWS)
    rows |= {t0 + int(rng.integers(0, tile)) for t0 in range(0, 32768, tile)}
    rows = sorted(rows)
    log(f"long_prefill oracle on {len(rows)} rows ({oracle.default_threads()} threads)")
    ro, rl = oracle_for(case, rows=rows)
    compare(o, lse, ro, rl, rows=rows, tag="long_prefill, a row of every item")


@pytest.mark.parametrize("W", [4095, -1])
def test_split_decode_every_request(W):
    """The full 256-request split-KV decode (2048-key chunks merged) in the
    benchmark's launch configuration, into NaN-filled outputs, against the
    oracle on every request and head."""
    case = build_case("split_decode", device=DEV, window_left=W)
    log(f"split_decode W={W} run")
    att = make_attention(case)
    o, lse = gpu_run(case, att=att)
    info = att.info()
    assert info.split_size == 2048 and info.num_merges > 0
    assert info.num_items > info.grid_blocks  # waves take several items each
    assert_all_written(case, o, lse, tag=f"split_decode W={W}")
    log(f"split_decode W={W} oracle on all {case.batch_size} requests "
        f"({oracle.default_threads()} threads)")
    host = dataclasses.replace(case, q=case.q.cpu(), k_cache=case.k_cache.cpu(),
                               v_cache=case.v_cache.cpu())
    ro, rl = oracle_for(host)
    del host
    compare(o, lse, ro, rl, tag=f"split_decode W={W}, every request")


# ----------------------------------------------------------------- edge cases and tails


@pytest.mark.parametrize("P_", [1, 4, 16, 64])
@pytest.mark.parametrize("W", [-1, 0, 1, 31, 33, 200])
def test_prefill_small_ragged(P_, W):
    qo = [1, 70, 0, 33, 129, 5]
    kv = [1, 70, 9, 300, 129, 700]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=P_, W=W, seed=P_ * 100 + W)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"prefill P={P_} W={W}")


# every bf16 prefill kernel variant on the ragged batch: 1 = 4x32 rows, 2 = 8x32
# rows (register staging), 3 = 4x64 rows, 4 = 8x32 rows with direct-to-LDS
# row loads, 5 = 4 with 64-key steps and 16-byte loads into a swizzled layout
# (page sizes 1, 2 and 4 take their per-row page paths (variant 4: below 4),
# the others their same-page paths; the last tile of each item the
# clamped-row path)
@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("P_", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("W", [-1, 0, 33, 200])
def test_prefill_variants_ragged(variant, P_, W):
    qo = [1, 70, 0, 33, 129, 5, 300]
    kv = [1, 70, 9, 300, 129, 700, 301]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=P_, W=W, seed=variant * 1000 + P_ * 10 + W)
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    assert att.info().prefill_variant == variant
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"prefill variant={variant} P={P_} W={W}")


@pytest.mark.parametrize("variant", [4, 5, 6])
def test_prefill_dma_variant_prefix_non_causal_and_fallback(variant):
    # non-causal, no window: every item loads all keys of its request
    case = small([20, 7, 64], [50, 7, 400], H_q=8, H_kv=2, D=128, W=-1, seed=21)
    case.causal = False
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    assert att.info().prefill_variant == variant
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"dma variant {variant} non-causal")
    # page size 1 and 2100 keys (variant 5: 8300): an item spans more pages
    # than the LDS page table holds, so the plan runs the register-staged
    # 256-row kernel
    case = small([40], [8300 if variant == 5 else 2100], H_q=8, H_kv=2, D=128, P_=1, W=-1,
                 seed=22)
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    assert att.info().prefill_variant == 2
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="dma fallback")


@pytest.mark.parametrize("D,G", [(64, 1), (64, 8), (128, 2), (128, 16), (256, 4), (256, 1)])
def test_prefill_head_shapes(D, G):
    qo, kv = [40, 130, 3], [300, 130, 64]
    case = small(qo, kv, H_q=2 * G, H_kv=2, D=D, P_=16, W=63, seed=D + G)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"prefill D={D} G={G}")


def test_prefill_fp32_ragged():
    case = small([5, 17, 1], [40, 17, 3], H_q=4, H_kv=2, D=128, P_=4, W=6, seed=3,
                 dtype=torch.float32)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="prefill fp32")


def test_prefill_non_causal_no_window():
    case = small([20, 7], [50, 7], H_q=4, H_kv=1, D=128, W=-1, seed=9)
    case.causal = False
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="prefill non-causal")


@pytest.mark.parametrize("P_", [1, 4, 16])
@pytest.mark.parametrize("W", [-1, 0, 5, 31, 32, 100])
@pytest.mark.parametrize("split", [-1, 32, 96])
def test_decode_small_ragged(P_, W, split):
    kv = [1, 2, 31, 32, 33, 64, 65, 200, 1000, 0]
    case = small([1] * len(kv), kv, H_q=32, H_kv=8, D=128, P_=P_, W=W, seed=P_ + W + split,
                 decode=True, split=split)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"decode P={P_} W={W} split={split}")
    assert (o[-1] == 0).all() and torch.isneginf(lse[-1]).all()  # keyless request


@pytest.mark.parametrize("decode", [False, True])
def test_empty_batch_then_a_real_one(decode):
    """A plan of zero requests launches kernels that find no work and write
    nothing (the NaN-filled outputs stay NaN); the same plan object then runs
    a real batch correctly."""
    qo = [1, 1, 1] if decode else [30, 1, 64]
    kv = [40, 700, 5] if decode else [30, 200, 64]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=63, seed=41, decode=decode,
                 split=64 if decode else -1)
    att = make_attention(case)
    z = torch.zeros(1, dtype=torch.int32)
    att.plan(qo_indptr=None if decode else z, kv_indptr=z,
             kv_last_page_len=torch.zeros(0, dtype=torch.int32))
    assert att.info().num_items == 0
    o, lse = poisoned_outputs(case.q)
    att.run(case.q, case.k_cache, case.v_cache, case.kv_indices, sm_scale=case.sm_scale,
            window_left=63, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all(), "an empty batch wrote outputs"
    o, lse = gpu_run(case, att=att)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"after an empty batch, decode={decode}")


@pytest.mark.parametrize("D,G", [(64, 4), (128, 1), (128, 8), (128, 16), (256, 2)])
def test_decode_head_shapes(D, G):
    kv = [7, 300, 1500, 64]
    case = small([1] * 4, kv, H_q=2 * G, H_kv=2, D=D, P_=16, W=511, seed=D * G, decode=True)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"decode D={D} G={G}")


def test_decode_fp32():
    kv = [7, 300, 0, 64]
    case = small([1] * 4, kv, H_q=8, H_kv=2, D=64, P_=4, W=20, seed=11, decode=True,
                 dtype=torch.float32)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="decode fp32")


@pytest.mark.parametrize("split,disable", [(32, False), (64, False), (256, False), (-1, False),
                                           (-1, True), (2048, False)])
def test_decode_split_invariance(split, disable):
    kv = [3000, 5000, 17, 4096, 2049]
    case = small([1] * 5, kv, H_q=64, H_kv=8, D=128, W=-1, seed=21, decode=True)
    o, lse = gpu_run(case, fixed_split_size=split, disable_split_kv=disable)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"split={split} disable={disable}")


@pytest.mark.parametrize("nw", [1, 4])
@pytest.mark.parametrize("W,split,P_", [(-1, -1, 16), (-1, 64, 4), (100, -1, 1), (0, -1, 16),
                                        (2047, 96, 8), (-1, 2048, 16), (4095, -1, 2)])
def test_decode_waves_per_item(nw, W, split, P_):
    """One or four waves per work item (the four split the item's key blocks
    into contiguous runs and combine in LDS): ragged lengths around block and
    run boundaries, windows, chunked and whole requests, a keyless request."""
    kv = [1, 2, 31, 33, 64, 97, 128, 129, 200, 1000, 3000, 5000, 0]
    case = small([1] * len(kv), kv, H_q=32, H_kv=8, D=128, P_=P_, W=W, seed=7 * nw + W + P_,
                 decode=True, split=split)
    att = make_attention(case, decode_waves=nw)
    o, lse = gpu_run(case, att=att)
    info = att.info()
    assert info.decode_waves == nw and info.block_threads == 64 * nw
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"decode nw={nw} W={W} split={split} P={P_}")
    assert (o[-1] == 0).all() and torch.isneginf(lse[-1]).all()


@pytest.mark.parametrize("D,G,dtype,kv_dtype,cap", [
    (64, 4, torch.bfloat16, None, 0.0), (128, 16, torch.bfloat16, None, 0.0),
    (256, 2, torch.bfloat16, None, 0.0), (128, 8, torch.float16, None, 0.0),
    (128, 4, torch.bfloat16, torch.float8_e4m3fn, 0.0), (128, 4, torch.float16, torch.float8_e5m2, 0.0),
    (128, 4, torch.bfloat16, None, 30.0)])
def test_decode_four_waves_shapes_and_types(D, G, dtype, kv_dtype, cap):
    kv = [7, 300, 1500, 64, 4100, 0]
    case = small([1] * len(kv), kv, H_q=2 * G, H_kv=2, D=D, P_=16, W=-1, seed=D + G, decode=True,
                 dtype=dtype, kv_dtype=kv_dtype, cap=cap)
    att = make_attention(case, decode_waves=4)
    o, lse = gpu_run(case, att=att)
    assert att.info().decode_waves == 4
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"decode nw=4 D={D} G={G} {dtype} kv={kv_dtype} cap={cap}")


def test_decode_waves_automatic_choice():
    """A batch of a few long requests takes four waves per item; short requests
    (or a window of at most 2048 keys) and larger batches one."""
    long_kv = [5000, 3000, 100, 4500]
    case = small([1] * 4, long_kv, H_q=32, H_kv=8, D=128, P_=16, W=-1, seed=5, decode=True)
    att = make_attention(case)
    o, lse = gpu_run(case, att=att)
    assert att.info().decode_waves == 4
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="decode auto nw")
    assert make_attention(case, window_left=2047).info().decode_waves == 1
    assert make_attention(case, kv_capacity=2048).info().decode_waves == 1
    assert make_attention(case, batch_capacity=4096).info().decode_waves == 1


# ----------------------------------------------------------------- exact masking


@pytest.mark.parametrize("decode", [False, True])
def test_window_zero_returns_own_value_bit_exact(decode):
    if decode:
        kv = [1, 17, 300, 4096]
        case = small([1] * 4, kv, H_q=32, H_kv=8, D=128, W=0, seed=31, decode=True)
    else:
        kv = [40, 300, 77]
        case = small([40, 100, 7], kv, H_q=8, H_kv=2, D=128, W=0, seed=32)
    o, lse = gpu_run(case)
    G = case.num_qo_heads // case.num_kv_heads
    # expected: the value row of the query's own position, per KV head
    expect = torch.empty_like(o)
    kvp = case.kv_indptr.cpu()
    for b in range(case.batch_size):
        prefix = case.kv_lens[b] - case.qo_lens[b]
        for i in range(case.qo_lens[b]):
            p = prefix + i
            pg = int(case.kv_indices[int(kvp[b]) + p // case.page_size])
            vrow = case.v_cache[pg, p % case.page_size]  # [H_kv, D]
            expect[int(case.qo_indptr[b]) + i] = vrow.repeat_interleave(G, dim=0)
    assert torch.equal(o, expect)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"W=0 decode={decode}")


@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("W", [-1, 0, 3, 40])
def test_one_hot_values_expose_exact_support(decode, W):
    """V_j = e_j (D >= kv_len): the output row is the attention weight vector;
    its nonzero set must be exactly the visible keys."""
    D = 128
    if decode:
        kv = [1, 50, 128, 97]
        case = small([1] * 4, kv, H_q=8, H_kv=2, D=D, P_=4, W=W, seed=40 + W, decode=True,
                     split=32)
    else:
        kv = [128, 60, 100]
        case = small([70, 60, 1], kv, H_q=8, H_kv=2, D=D, P_=4, W=W, seed=50 + W)
    kvp = case.kv_indptr.cpu()
    for b in range(case.batch_size):
        for j in range(case.kv_lens[b]):
            pg = int(case.kv_indices[int(kvp[b]) + j // case.page_size])
            case.v_cache[pg, j % case.page_size] = 0
            case.v_cache[pg, j % case.page_size, :, j] = 1
    o, lse = gpu_run(case)
    o = o.float().cpu()
    for b in range(case.batch_size):
        prefix = case.kv_lens[b] - case.qo_lens[b]
        for i in range(case.qo_lens[b]):
            p = prefix + i
            lo = max(0, p - W) if W >= 0 else 0
            want = torch.zeros(D, dtype=torch.bool)
            want[lo:p + 1] = True
            got = o[int(case.qo_indptr[b]) + i] != 0
            assert (got == want.unsqueeze(0)).all(), (b, i, p, lo)


# ----------------------------------------------------------------- plan lifecycle


def _sub_layout(case, picks):
    """Layout of the requests `picks` of `case`, over the same cache pages:
    (q rows, kv_indices, qo_indptr, kv_indptr, kv_last_page_len)."""
    qop, kvp = case.qo_indptr.cpu(), case.kv_indptr.cpu()
    idx = case.kv_indices.cpu()
    rows, pages, qo_ind, kv_ind, last = [], [], [0], [0], []
    for b in picks:
        rows += list(range(int(qop[b]), int(qop[b + 1])))
        pages.append(idx[int(kvp[b]):int(kvp[b + 1])])
        qo_ind.append(qo_ind[-1] + int(qop[b + 1] - qop[b]))
        kv_ind.append(kv_ind[-1] + int(kvp[b + 1] - kvp[b]))
        last.append(int(case.kv_last_page_len[b]))
    i32 = dict(dtype=torch.int32)
    return (rows, torch.cat(pages).to(**i32), torch.tensor(qo_ind, **i32),
            torch.tensor(kv_ind, **i32), torch.tensor(last, **i32))


@pytest.mark.parametrize("decode,nw,split,variant", [
    (False, 0, -1, 0), (True, 1, 64, 0), (True, 4, 64, 0), (True, 1, -1, 0), (False, 0, -2, 1),
    (False, 0, -2, 5)])
def test_graph_replay_follows_replans(decode, nw, split, variant):
    """run() captured once in a HIP graph stays valid for every later plan() of
    the same capacities (AMD-Ecosystem/flashinfer PR 234, "Why each fix" 2: the
    grid and the launch set come from the capacities, the work from the
    workspace).  Each replay, with eager work and synchronisations between
    replays, must equal an eager run() of the batch planned last, bit for bit.
    split = -2: a prefill whose full batch is key-split (chunk partials and a
    merge launch) and whose one-request batch is not, on prefill variant
    `variant`."""
    if not decode and split == -2:
        qo, kv = [40, 1, 130, 7, 64], [1300, 1, 130, 2500, 64]
        case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=-1, seed=63)
    elif decode:
        # split = -1: the planner's choice; the first planned batch (request 2
        # alone, 77 keys) splits nothing, the later ones split their long
        # requests, so the graph must hold the merge launch an eager run of
        # the first batch skips
        qo, kv = [1] * 6, [300, 1, 77, 2000, 64, 900]
        case = small(qo, kv, H_q=16, H_kv=2, D=128, P_=16, W=-1 if split < 0 else 255, seed=61,
                     decode=True, split=split)
    else:
        qo, kv = [40, 1, 130, 7, 64], [300, 1, 130, 500, 64]
        case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=100, seed=62)
    att = make_attention(case, decode_waves=nw, prefill_variant=variant)
    if decode:
        assert att.info().decode_waves == nw
    elif variant:
        assert att.info().prefill_variant == variant
    B, n_q = case.batch_size, case.q.shape[0]
    q_buf = case.q.clone()
    idx_buf = case.kv_indices.clone()
    o_buf = torch.zeros_like(case.q)
    l_buf = torch.zeros(n_q, case.num_qo_heads, dtype=torch.float32, device=DEV)

    def plan(layout):
        _, _, qo_ind, kv_ind, last = layout
        if decode:
            att.plan(kv_indptr=kv_ind, kv_last_page_len=last)
        else:
            att.plan(qo_indptr=qo_ind, kv_indptr=kv_ind, kv_last_page_len=last)

    def load(layout):
        rows, pages, *_ = layout
        q_buf.zero_()
        q_buf[:len(rows)] = case.q[torch.tensor(rows, device=DEV)]
        idx_buf.zero_()
        idx_buf[:len(pages)] = pages.to(DEV)

    def run():
        att.run(q_buf, case.k_cache, case.v_cache, idx_buf, sm_scale=case.sm_scale,
                window_left=case.window_left, out=o_buf, lse=l_buf)

    req_sets = [list(range(B)), [2], [0, 3, 4], list(range(B))]
    if decode and split < 0:
        req_sets = [[2]] + req_sets
    layouts = [_sub_layout(case, r) for r in req_sets]
    load(layouts[0])
    plan(layouts[0])
    if decode and split < 0:
        assert att.info().num_merges == 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for k, layout in enumerate(layouts):
        load(layout)
        plan(layout)
        n = len(layout[0])
        o_buf.fill_(7.0)
        run()
        torch.cuda.synchronize()
        want_o, want_l = o_buf[:n].clone(), l_buf[:n].clone()
        for rep in range(3):
            o_buf.fill_(-3.0)
            l_buf.fill_(-3.0)
            junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
            g.replay()
            torch.cuda.synchronize()
            assert torch.isfinite(junk).all()
            assert torch.equal(o_buf[:n], want_o), (k, rep)
            assert torch.equal(l_buf[:n], want_l), (k, rep)
        if decode and split < 0 and len(layout[0]) == B:
            assert att.info().num_merges > 0
        if not decode and split == -2:
            assert (att.info().num_merges > 0) == (len(req_sets[k]) > 1), k
        if len(layout[0]) == B:
            ro, rl = oracle_for(case)
            compare(want_o, want_l, ro, rl,
                    tag=f"graph decode={decode} nw={nw} split={split} variant={variant}")


@pytest.mark.parametrize("decode,variant", [(False, 5), (False, 6), (True, 0)])
def test_run_time_claiming_repeats_and_replays(decode, variant):
    """Batches with more work items than the launch has workgroups, so items
    are handed out at run time and each launch must leave its claim counters
    at 0: three eager runs in a row into NaN-filled outputs, each checked
    row by row against the oracle, then one captured run replayed after
    re-plans that alternate between batches with and without run-time
    claiming, every replay equal to an eager run of the batch planned last."""
    rng = np.random.default_rng(5 + decode)
    if decode:
        B = 300
        kv = [int(x) for x in rng.integers(1, 200, size=B)]
        case = small([1] * B, kv, H_q=32, H_kv=8, D=128, P_=16, W=31, seed=71, decode=True,
                     spare=5)
        att = make_attention(case, disable_split_kv=True)
        few = list(range(0, B, 8))
    else:
        qo = [1200, 900, 1100, 1000]
        case = small(qo, [q + 50 for q in qo], H_q=32, H_kv=8, D=128, P_=16, W=127, seed=72)
        att = make_attention(case, prefill_variant=variant)
        assert att.info().prefill_variant == variant
        few = [1]
    ro, rl = oracle_for(case)
    for rep in range(3):
        o, lse = gpu_run(case, att=att)
        info = att.info()
        assert info.num_items > info.grid_blocks, (info.num_items, info.grid_blocks)
        assert_all_written(case, o, lse, tag=f"claiming run {rep}")
        compare(o, lse, ro, rl, tag=f"claiming run {rep}, decode={decode}")
    # one captured run, replayed after re-plans with and without claiming
    B, n_q = case.batch_size, case.q.shape[0]
    q_buf, idx_buf = case.q.clone(), case.kv_indices.clone()
    o_buf = torch.zeros_like(case.q)
    l_buf = torch.zeros(n_q, case.num_qo_heads, dtype=torch.float32, device=DEV)

    def plan(layout):
        _, pages, qo_ind, kv_ind, last = layout
        q_buf.zero_()
        q_buf[:len(layout[0])] = case.q[torch.tensor(layout[0], device=DEV)]
        idx_buf.zero_()
        idx_buf[:len(pages)] = pages.to(DEV)
        if decode:
            att.plan(kv_indptr=kv_ind, kv_last_page_len=last)
        else:
            att.plan(qo_indptr=qo_ind, kv_indptr=kv_ind, kv_last_page_len=last)

    def run():
        att.run(q_buf, case.k_cache, case.v_cache, idx_buf, sm_scale=case.sm_scale,
                window_left=case.window_left, out=o_buf, lse=l_buf)

    everything = _sub_layout(case, list(range(B)))
    plan(everything)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for k, picks in enumerate([list(range(B)), few, list(range(B)), few]):
        layout = _sub_layout(case, picks)
        plan(layout)
        claims = att.info().num_items > att.info().grid_blocks
        assert claims == (len(picks) == B), (k, att.info().num_items)
        n = len(layout[0])
        run()
        torch.cuda.synchronize()
        want_o, want_l = o_buf[:n].clone(), l_buf[:n].clone()
        for rep in range(2):
            o_buf.fill_(float("nan"))
            l_buf.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(o_buf[:n], want_o), (k, rep)
            assert torch.equal(l_buf[:n], want_l), (k, rep)
        if len(picks) == B:
            compare(want_o, want_l, ro, rl, tag=f"claiming replay {k}, decode={decode}")


def _layout_case(case, picks):
    """The requests `picks` of `case` as a case of their own over the same cache
    pages (for the oracle)."""
    rows, pages, qo_ind, kv_ind, last = _sub_layout(case, picks)
    return dataclasses.replace(
        case, qo_lens=[case.qo_lens[b] for b in picks], kv_lens=[case.kv_lens[b] for b in picks],
        q=case.q[torch.tensor(rows, device=case.q.device)], qo_indptr=qo_ind, kv_indptr=kv_ind,
        kv_indices=pages, kv_last_page_len=last)


@pytest.mark.parametrize("W,kv_cap,want", [(-1, 8300, 2), (1023, 8192, 5), (-1, 8000, 5)])
def test_graph_replay_variant_fixed_by_capacity(W, kv_cap, want):
    """The prefill kernel is chosen when the plan is created, from its
    capacities: a run() captured while a short batch is planned replays the
    same kernel after a re-plan whose items span thousands of keys (page size 1,
    so every key is a page; the 64-key kernel holds 8192 page ids per item).
    Every replay matches the oracle of the batch planned last."""
    case = small([64, 3, 40], [kv_cap, 700, 1000], H_q=8, H_kv=2, D=128, P_=1, W=W,
                 seed=64 + W)
    att = make_attention(case, prefill_variant=5)
    assert att.info().prefill_variant == want
    n_q = case.q.shape[0]
    q_buf = torch.zeros_like(case.q)
    idx_buf = torch.zeros_like(case.kv_indices)
    o_buf = torch.zeros_like(case.q)
    l_buf = torch.zeros(n_q, case.num_qo_heads, dtype=torch.float32, device=DEV)

    def load_and_plan(picks):
        rows, pages, qo_ind, kv_ind, last = _sub_layout(case, picks)
        q_buf.zero_()
        q_buf[:len(rows)] = case.q[torch.tensor(rows, device=DEV)]
        idx_buf.zero_()
        idx_buf[:len(pages)] = pages.to(DEV)
        att.plan(qo_indptr=qo_ind, kv_indptr=kv_ind, kv_last_page_len=last)
        return len(rows)

    def run():
        att.run(q_buf, case.k_cache, case.v_cache, idx_buf, sm_scale=case.sm_scale,
                window_left=W, out=o_buf, lse=l_buf)

    load_and_plan([1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for picks in ([0, 1, 2], [1], [2, 0]):
        n = load_and_plan(picks)
        assert att.info().prefill_variant == want
        ro, rl = oracle_for(_layout_case(case, picks))
        for rep in range(2):
            o_buf.fill_(float("nan"))
            l_buf.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            compare(o_buf[:n], l_buf[:n], ro, rl, tag=f"replay W={W} picks={picks} rep={rep}")


def test_replan_in_place_then_capacity_error():
    big = small([1] * 6, [500, 2000, 33, 4096, 1, 700], H_q=32, H_kv=8, D=128, W=127, seed=61,
                decode=True)
    att = make_attention(big, batch_capacity=6, kv_capacity=4096)
    o, lse = gpu_run(big, att=att)
    ro, rl = oracle_for(big)
    compare(o, lse, ro, rl, tag="plan A")
    smaller = small([1] * 3, [4096, 5, 900], H_q=32, H_kv=8, D=128, W=127, seed=62, decode=True)
    o, lse = gpu_run(smaller, att=att)
    ro, rl = oracle_for(smaller)
    compare(o, lse, ro, rl, tag="re-plan B (smaller)")
    larger = small([1] * 7, [10] * 7, H_q=32, H_kv=8, D=128, W=127, seed=63, decode=True)
    with pytest.raises(P.PkvsError) as ei:
        att.plan(kv_indptr=larger.kv_indptr.cpu(), kv_last_page_len=larger.kv_last_page_len.cpu())
    assert ei.value.code == P.PKVS_ERR_CAPACITY


def test_run_without_lse():
    case = small([30], [90], H_q=4, H_kv=1, D=128, W=10, seed=71)
    o = gpu_run(case, return_lse=False)
    ro, _ = oracle_for(case)
    compare(o, None, ro, None, tag="no lse")


def test_run_rejects_mismatched_window_on_gpu():
    case = small([30], [90], H_q=4, H_kv=1, D=128, W=10, seed=72)
    att = make_attention(case)
    att.plan(qo_indptr=case.qo_indptr.cpu(), kv_indptr=case.kv_indptr.cpu(),
             kv_last_page_len=case.kv_last_page_len.cpu())
    with pytest.raises(P.PkvsError) as ei:
        att.run(case.q, case.k_cache, case.v_cache, case.kv_indices, sm_scale=case.sm_scale,
                window_left=11)
    assert ei.value.code == P.PKVS_ERR_PLAN_MISMATCH


# ----------------------------------------------------------------- merge_state


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("H,D,n", [(64, 128, 37), (128, 64, 37), (128, 256, 37), (8, 96, 37),
                                   (64, 128, 3001), (32, 64, 4099)])
def test_merge_state_against_oracle(dtype, H, D, n):
    """merge_state against the oracle (16 bytes per lane where a (token, head)
    row is a power of two of 16-byte chunks, one wave per row otherwise), into
    NaN-filled outputs; a partial whose LSE is -inf contributes nothing even
    when its values are NaN; in place equals out of place."""
    g = torch.Generator(device=DEV).manual_seed(H * D + n)
    va = torch.randn(n, H, D, generator=g, device=DEV).to(dtype)
    vb = torch.randn(n, H, D, generator=g, device=DEV).to(dtype)
    sa = torch.randn(n, H, generator=g, device=DEV) * 5
    sb = torch.randn(n, H, generator=g, device=DEV) * 5
    sa[0, :3] = float("-inf")
    sb[0, 1:4] = float("-inf")
    va[0, :3] = float("nan")
    vb[0, 1:4] = float("nan")
    v = torch.full_like(va, float("nan"))
    s = torch.full_like(sa, float("nan"))
    P.pkvs_merge_state(va, sa, vb, sb, v_out=v, s_out=s)
    torch.cuda.synchronize()
    va = va.clone()
    vb = vb.clone()
    va[0, :3] = 0
    vb[0, 1:4] = 0
    rv, rs = oracle.merge_state(va.double().cpu().numpy(), sa.double().cpu().numpy(),
                                vb.double().cpu().numpy(), sb.double().cpu().numpy())
    compare(v, s, rv, rs, tag=f"merge {dtype} H={H} D={D}")
    assert (v[0, 1:3] == 0).all() and torch.isneginf(s[0, 1:3]).all()
    # in place (v_out aliases v_a)
    va2, sa2 = va.clone(), sa.clone()
    P.pkvs_merge_state(va2, sa2, vb, sb, v_out=va2, s_out=sa2)
    torch.cuda.synchronize()
    assert torch.equal(va2, v) and torch.equal(sa2, s)
    # v not 16-byte aligned: the one-wave-per-row kernel, same arithmetic
    off = 16 // va.element_size() - 1 if va.element_size() < 16 else 0
    if off:
        def shifted(t):
            buf = torch.empty(t.numel() + off, dtype=t.dtype, device=DEV)
            view = buf[off:].view(t.shape)
            view.copy_(t)
            return view
        va3, vb3 = shifted(va), shifted(vb)
        v3 = shifted(torch.full_like(v, float("nan")))
        s3 = torch.full_like(s, float("nan"))
        P.pkvs_merge_state(va3, sa, vb3, sb, v_out=v3, s_out=s3)
        torch.cuda.synchronize()
        assert torch.equal(v3, v) and torch.equal(s3, s)


def test_merge_state_of_prefill_split_equals_unsplit():
    """Attention over keys [0, c) merged with attention over keys [c, kv_len)
    gives the one-pass result (decode split at a chunk boundary, in the GPU)."""
    case = small([1] * 3, [1000, 64, 3000], H_q=32, H_kv=8, D=128, W=-1, seed=81, decode=True)
    o1, l1 = gpu_run(case, fixed_split_size=256)
    o2, l2 = gpu_run(case, disable_split_kv=True)
    assert (o1.float() - o2.float()).abs().max() <= 2e-2
    assert (l1 - l2).abs().max() <= 1e-3


# ----------------------------------------------------------------- cascade prefill
# sglang flashinfer_backend.py, FlashInferAttnBackend.forward_extend (the
# branch with cached prefixes): a ragged pass over the new tokens' own keys, a
# paged pass over the cached prefix, merged.  The result must equal the one
# paged prefill over prefix + new keys (the oracle on the combined layout).


# ----------------------------------------------------------------- key-split prefill

# small batches whose query tiles reach far back: the plan cuts their key ranges
SPLIT_QO = [3, 70, 129, 1, 40]
SPLIT_KV = [1500, 900, 2129, 1, 600]


@pytest.mark.parametrize("variant,D,G", [(1, 64, 4), (1, 128, 8), (1, 256, 4), (2, 64, 2),
                                         (2, 128, 4), (5, 128, 4), (5, 128, 1)])
@pytest.mark.parametrize("W,P_", [(-1, 16), (0, 4), (100, 1), (511, 16), (1023, 2)])
def test_key_split_prefill(variant, D, G, W, P_):
    """The key split on the register-staged kernels: chunks of whole key
    tiles, each writing per-token partials, merged per token; every row
    written (NaN-filled outputs), against the oracle, and the same batch with
    the split disabled runs one item per tile."""
    case = small(SPLIT_QO, SPLIT_KV, H_q=2 * G, H_kv=2, D=D, P_=P_, W=W,
                 seed=11 * variant + D + W + P_)
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    info = att.info()
    assert info.prefill_variant == variant and info.key_chunks > 1
    if W < 0 or W >= 511:
        assert info.num_merges > 0
    tag = f"key split v={variant} D={D} G={G} W={W} P={P_} merges={info.num_merges}"
    assert_all_written(case, o, lse, tag)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=tag)
    whole = make_attention(case, prefill_variant=variant, disable_split_kv=True)
    assert whole.info().key_chunks == 1 and whole.info().float_ws_bytes == 0
    o1, l1 = gpu_run(case, att=whole)
    assert whole.info().num_merges == 0
    compare(o1, l1, ro, rl, tag=tag + " (no split)")


@pytest.mark.parametrize("dtype,kv_dtype,cap", [
    (torch.float16, None, 0.0), (torch.bfloat16, None, 30.0),
    (torch.bfloat16, torch.float8_e4m3fn, 0.0), (torch.float16, torch.float8_e5m2, 0.0)])
def test_key_split_prefill_types(dtype, kv_dtype, cap):
    """The key split with fp16 queries, a logits soft cap and 8-bit caches
    (the chunks' partials carry v_scale; the merge rounds once to the dtype)."""
    case = small(SPLIT_QO, SPLIT_KV, H_q=8, H_kv=2, D=128, P_=16, W=-1, seed=19, dtype=dtype,
                 kv_dtype=kv_dtype, cap=cap, k_scale=0.5 if kv_dtype else 1.0,
                 v_scale=0.25 if kv_dtype else 1.0)
    att = make_attention(case)
    o, lse = gpu_run(case, att=att)
    assert att.info().num_merges > 0
    tag = f"key split {dtype} kv={kv_dtype} cap={cap}"
    assert_all_written(case, o, lse, tag)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=tag)


@pytest.mark.parametrize("W", [2047, -1])
@pytest.mark.parametrize("variant", [0, 1, 5])
def test_key_split_chunked_prefill(W, variant):
    """A 512-token chunk of a long prompt over its 4096 cached keys (32/8
    heads, head_dim 128; the 128-row kernel, the 64-key one, and the
    planner's choice for these capacities, the 64-key one): 128 or 64 query
    tiles for 256 workgroups, so every tile's keys are cut into chunks; every
    row written, against the oracle."""
    case = small([512], [4608], H_q=32, H_kv=8, D=128, P_=16, W=W, seed=29 + variant)
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    info = att.info()
    assert info.prefill_variant == (variant or 5) and info.num_merges == 512 * 8
    tag = f"key split chunked prefill W={W} items={info.num_items}"
    assert_all_written(case, o, lse, tag)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=tag)


def test_key_split_prefill_non_causal_and_without_lse():
    """Non-causal without a window (every key of the request), and run()
    without an LSE output: the merge writes o only."""
    case = dataclasses.replace(small(SPLIT_QO, SPLIT_KV, H_q=4, H_kv=1, D=128, W=-1, seed=23),
                               causal=False)
    att = make_attention(case)
    o, lse = gpu_run(case, att=att)
    assert att.info().num_merges > 0
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="key split non-causal")
    o2 = gpu_run(case, att=att, return_lse=False)
    o2 = o2[0] if isinstance(o2, tuple) else o2
    assert torch.equal(o2, o)


def make_cascade(case, window_left=None, prefill_variant=0, qo_capacity=None,
                 kv_capacity=None, batch_capacity=None):
    W = case.window_left if window_left is None else window_left
    prefix = [k - q for q, k in zip(case.qo_lens, case.kv_lens)]
    return P.CascadeAttention(
        num_qo_heads=case.num_qo_heads, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
        page_size=case.page_size, dtype=case.dtype, window_left=W, causal=case.causal,
        batch_capacity=batch_capacity or max(case.batch_size, 1),
        qo_capacity=qo_capacity or max(int(case.qo_indptr[-1]), 1),
        kv_capacity=kv_capacity or max(max(prefix, default=1), 1),
        prefill_variant=prefill_variant, logits_soft_cap=case.logits_soft_cap,
        kv_dtype=kv_dtype_of(case))


def cascade_run(case, trim=False, att=None, return_lse=True, **kw):
    W = case.window_left
    cin = cascade_inputs(case, trim_to=W if trim else None)
    if att is None:
        att = make_cascade(case, **kw)
    att.plan(qo_indptr=case.qo_indptr.cpu(), kv_indptr=cin.kv_indptr,
             kv_last_page_len=cin.kv_last_page_len)
    k_ext, v_ext = cin.k_extend, cin.v_extend
    if kv_dtype_of(case) is not None:
        # the new tokens' K/V arrive in the query dtype (the cache values times
        # their scales: power-of-two scales keep them exact)
        k_ext = (k_ext.float() * case.k_scale).to(case.dtype)
        v_ext = (v_ext.float() * case.v_scale).to(case.dtype)
    o, lse = poisoned_outputs(case.q)
    res = att.run(case.q, k_ext, v_ext, cin.k_cache, cin.v_cache, cin.kv_indices,
                  sm_scale=case.sm_scale, window_left=W, return_lse=return_lse,
                  k_scale=case.k_scale, v_scale=case.v_scale, out=o,
                  lse=lse if return_lse else None)
    torch.cuda.synchronize()
    return res, att


@pytest.mark.parametrize("P_", [1, 16])
@pytest.mark.parametrize("W", [-1, 0, 5, 100, 511])
@pytest.mark.parametrize("trim", [False, True])
@pytest.mark.parametrize("variant", [0, 1, 5])
def test_cascade_equals_one_paged_prefill(P_, W, trim, variant):
    """Cascade prefill against the one paged prefill over prefix + new keys;
    variants 1 and 5 run the cascade in one pass (cached keys from the pages,
    new keys from the contiguous K/V, split per request), 0 is the planner's
    choice for the capacities (variant 5 where an item can span 512 keys)."""
    qo = [1, 70, 0, 33, 129, 5, 300, 40]
    kv = [1, 90, 9, 300, 129, 700, 301, 1000]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=P_, W=W, seed=P_ * 31 + W + 7 * trim)
    (o, lse), att = cascade_run(case, trim=trim, prefill_variant=variant)
    if variant:
        assert att.info().prefill_variant == variant
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"cascade P={P_} W={W} trim={trim} "
                                f"variant={att.info().prefill_variant}")


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6])
def test_cascade_prefill_variants(variant):
    qo = [64, 1, 257, 33, 600]
    kv = [64, 800, 300, 1000, 700]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=200, seed=900 + variant)
    (o, lse), att = cascade_run(case, prefill_variant=variant)
    assert att.info().prefill_variant == variant
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"cascade variant={variant}")


@pytest.mark.parametrize("D,G", [(64, 8), (128, 1), (256, 4)])
def test_cascade_head_shapes(D, G):
    case = small([40, 130, 7], [90, 130, 500], H_q=2 * G, H_kv=2, D=D, P_=16, W=63,
                 seed=D + G)
    (o, lse), _ = cascade_run(case, trim=True)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"cascade D={D} G={G}")


def test_cascade_fp32_and_no_window_non_causal():
    case = small([6, 8, 12], [10, 8, 20], H_q=2, H_kv=1, D=64, P_=4, W=4, seed=5,
                 dtype=torch.float32)
    (o, lse), _ = cascade_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="cascade fp32")
    # non-causal (no window): the one-pass plans (variants 1 and 5) keep the
    # cascade's causality, the two-pass one (variant 3) its passes'
    for variant in (0, 1, 3, 5):
        case = small([20, 7, 64], [50, 7, 400], H_q=8, H_kv=2, D=128, W=-1, seed=23)
        case.causal = False
        (o, lse), att = cascade_run(case, prefill_variant=variant)
        ro, rl = oracle_for(case)
        compare(o, lse, ro, rl, tag=f"cascade non-causal, variant {att.info().prefill_variant}")


def test_cascade_prefix_prefill_workload():
    """The batched prefill with cached prefixes (8 requests, prefix up to 1024,
    up to 512 new tokens, window 511, head_dim 256) run as a cascade with the
    prefix table trimmed to the window."""
    case = build_case("prefix_prefill", device=DEV)
    (o, lse), _ = cascade_run(case, trim=True)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="cascade prefix_prefill")


@pytest.mark.parametrize("variant", [0, 5])
def test_cascade_without_lse_and_without_cached_keys(variant):
    case = small([30, 9], [90, 40], H_q=4, H_kv=1, D=128, W=10, seed=73)
    (o), _ = cascade_run(case, return_lse=False, prefill_variant=variant)
    ro, _ = oracle_for(case)
    compare(o, None, ro, None, tag="cascade no lse")
    # no request has cached keys: the paged pass sees empty tables (one pass:
    # every key comes from the contiguous K/V, the cache is never read)
    case = small([30, 9], [30, 9], H_q=4, H_kv=1, D=128, W=10, seed=74)
    (o, lse), _ = cascade_run(case, prefill_variant=variant)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="cascade without cached keys")


@pytest.mark.parametrize("P_", [1, 16])
def test_cascade_one_pass_split_mid_group(P_):
    """One-pass cascade where the boundary between cached and new keys falls
    inside a wave's 8-key staging group and inside a page (tables of 13, 4101
    -- 1501 with single-key pages, whose plan must not span more than 2048
    pages -- 1 and 30 cached keys), long new-token runs, window and no
    window."""
    qo = [200, 77, 1, 130]
    tab = [13, 4101 if P_ > 1 else 1501, 1, 30]
    kv = [t + q for t, q in zip(tab, qo)]
    for W in (-1, 300):
        case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=P_, W=W, seed=77 + W + P_)
        (o, lse), att = cascade_run(case, prefill_variant=5)
        assert att.info().prefill_variant == 5
        ro, rl = oracle_for(case)
        compare(o, lse, ro, rl, tag=f"one-pass cascade P={P_} W={W}")


@pytest.mark.parametrize("dtype,cap", [(torch.float16, 0.0), (torch.bfloat16, 30.0),
                                       (torch.float16, 20.0)])
def test_cascade_one_pass_fp16_and_soft_cap(dtype, cap):
    """The one-pass cascade (variant 5) in IEEE half and with a logits soft
    cap, against the oracle on the combined layout."""
    qo = [70, 1, 129, 300]
    kv = [90, 300, 129, 1000]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=100, seed=int(cap) + 3, dtype=dtype,
                 cap=cap)
    (o, lse), att = cascade_run(case, prefill_variant=5)
    info = att.info()
    assert info.prefill_variant == 5 and info.cascade_passes == 1, "expected the one-pass plan"
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"one-pass cascade {dtype} cap={cap}")


@pytest.mark.parametrize("variant", [0, 5])
def test_cascade_graph_replay_follows_replans(variant):
    """The cascade's launches captured once replay correctly after re-plans of
    the same capacities (the kernels read their work from the workspace), bit
    for bit against eager runs; variant 5 is the one-pass cascade."""
    qo, kv = [40, 1, 130, 7, 64], [300, 1, 200, 500, 64]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=100, seed=64)
    cin = cascade_inputs(case)
    att = make_cascade(case, prefill_variant=variant)
    qop = case.qo_indptr.cpu().tolist()
    q_buf = case.q.clone()
    ke_buf, ve_buf = cin.k_extend.clone(), cin.v_extend.clone()
    idx_buf = cin.kv_indices.clone()
    o_buf = torch.zeros_like(case.q)
    l_buf = torch.zeros(case.q.shape[0], case.num_qo_heads, dtype=torch.float32, device=DEV)
    kvp = cin.kv_indptr.tolist()

    def plan_and_load(picks):
        rows, pages, qo_ind, kv_ind, last = [], [], [0], [0], []
        for b in picks:
            rows += list(range(qop[b], qop[b + 1]))
            pages.append(cin.kv_indices[kvp[b]:kvp[b + 1]])
            qo_ind.append(qo_ind[-1] + qop[b + 1] - qop[b])
            kv_ind.append(kv_ind[-1] + kvp[b + 1] - kvp[b])
            last.append(int(cin.kv_last_page_len[b]))
        r = torch.tensor(rows, device=DEV)
        for buf, src in ((q_buf, case.q), (ke_buf, cin.k_extend), (ve_buf, cin.v_extend)):
            buf.zero_()
            buf[:len(rows)] = src[r]
        idx_buf.zero_()
        pg = torch.cat(pages)
        idx_buf[:len(pg)] = pg
        att.plan(qo_indptr=qo_ind, kv_indptr=kv_ind, kv_last_page_len=last)
        return len(rows)

    def run():
        att.run(q_buf, ke_buf, ve_buf, cin.k_cache, cin.v_cache, idx_buf,
                sm_scale=case.sm_scale, window_left=case.window_left, out=o_buf, lse=l_buf)

    B = case.batch_size
    picks = [list(range(B)), [2], [0, 3, 4], list(range(B))]
    plan_and_load(picks[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for k, pk in enumerate(picks):
        n = plan_and_load(pk)
        o_buf.fill_(7.0)
        run()
        torch.cuda.synchronize()
        want_o, want_l = o_buf[:n].clone(), l_buf[:n].clone()
        for rep in range(3):
            o_buf.fill_(-3.0)
            l_buf.fill_(-3.0)
            junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
            g.replay()
            torch.cuda.synchronize()
            assert torch.isfinite(junk).all()
            assert torch.equal(o_buf[:n], want_o), (k, rep)
            assert torch.equal(l_buf[:n], want_l), (k, rep)
        if k == 0:
            ro, rl = oracle_for(case)
            compare(want_o, want_l, ro, rl, tag="cascade graph")



# ----------------------------------------------------------------- cache writes, page-table build
# sglang flashinfer_backend.py: set_kv_buffer before the paged attention reads
# the new keys; call_begin_forward builds kv_indptr / kv_indices on the device.
# Integer and byte work: bit-exact against the oracle.


@pytest.mark.parametrize("dtype,H,D", [(torch.bfloat16, 8, 128), (torch.bfloat16, 1, 256),
                                       (torch.float32, 2, 64), (torch.bfloat16, 3, 64),
                                       (torch.float16, 8, 128)])
def test_append_kv_bit_exact(dtype, H, D):
    g = torch.Generator().manual_seed(H * D)
    pages, Psz = 40, 16
    slots = pages * Psz
    k_cache = torch.randn(pages, Psz, H, D, generator=g).to(dtype)
    v_cache = torch.randn(pages, Psz, H, D, generator=g).to(dtype)
    n = 300
    loc = torch.randperm(slots, generator=g)[:n].to(torch.int64)
    loc[7], loc[100], loc[299] = -1, slots, -5  # outside the pool: skipped and counted
    k_new = torch.randn(n, H, D, generator=g).to(dtype)
    v_new = torch.randn(n, H, D, generator=g).to(dtype)
    rk, rv, skipped = oracle.append_kv(k_new, v_new, loc, k_cache, v_cache)
    kc, vc = k_cache.to(DEV), v_cache.to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    log(f"append dtype={dtype} H={H} D={D} n={n}")
    P.pkvs_append_kv(k_new.to(DEV), v_new.to(DEV), loc.to(DEV), kc, vc, status=status)
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu().view(torch.uint8), rk.view(torch.uint8))
    assert torch.equal(vc.cpu().view(torch.uint8), rv.view(torch.uint8))
    assert int(status) == skipped == 3


@pytest.mark.parametrize("batch", [0, 1, 37, 3000])
@pytest.mark.parametrize("with_start", [False, True])
def test_build_kv_indices_bit_exact(batch, with_start):
    g = torch.Generator().manual_seed(batch + 7 * with_start)
    rows, cols = 64, 300
    page_map = torch.randint(0, 1 << 20, (rows, cols), generator=g, dtype=torch.int32)
    slot = torch.randint(0, rows, (batch,), generator=g, dtype=torch.int32)
    length = torch.randint(0, 40 if batch < 1000 else 6, (batch,), generator=g,
                           dtype=torch.int32)
    start = torch.randint(0, cols - 40, (batch,), generator=g, dtype=torch.int32)
    if batch >= 37:
        length[3] = -2          # negative: counts as 0
        slot[5] = rows          # row outside the map: -1 entries
        start[9] = cols - 2     # runs off the row end: -1 past it
    if not with_start:
        start = None
    total = int(length.clamp(min=0).sum())
    capacity = max(total - 3, 0) if batch >= 37 else total  # the last entries do not fit
    indptr, idx, err = oracle.build_kv_indices(page_map, slot, length, start=start,
                                               capacity=capacity)
    out_idx = torch.full((max(capacity, 1),), 0x7FFFFFFF, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    log(f"build batch={batch} start={with_start} capacity={capacity}")
    kp, ki = P.pkvs_build_kv_indices(page_map.to(DEV), slot.to(DEV), length.to(DEV),
                                     start=None if start is None else start.to(DEV),
                                     kv_indices=out_idx, capacity=capacity, status=status)
    torch.cuda.synchronize()
    assert kp.cpu().tolist() == indptr.tolist()
    assert ki.cpu()[:capacity].tolist() == idx.tolist()
    assert int(status) == err


@pytest.mark.parametrize("W", [-1, 127])
def test_decode_step_appends_and_builds_its_page_table(W):
    """One decode step the way a serving loop runs it: write each request's new
    key/value into its slot, build the page table on the device from the
    request-to-page map (from the first page of the window when W >= 0), plan
    with the host lengths, decode; equal to the oracle on the full batch."""
    kv = [1, 300, 77, 2000, 16, 129]
    case = small([1] * len(kv), kv, H_q=16, H_kv=2, D=128, P_=16, W=W, seed=91,
                 decode=True)
    Psz, B = case.page_size, case.batch_size
    kvp = case.kv_indptr.cpu().tolist()
    pages = [case.kv_indices.cpu()[kvp[b]:kvp[b + 1]] for b in range(B)]
    # the new tokens' rows, taken out of the cache and poisoned there
    loc, k_new, v_new = [], [], []
    flat_k = case.k_cache.view(-1, case.num_kv_heads, case.head_dim)
    flat_v = case.v_cache.view(-1, case.num_kv_heads, case.head_dim)
    for b in range(B):
        j = kv[b] - 1
        s = int(pages[b][j // Psz]) * Psz + j % Psz
        loc.append(s)
        k_new.append(flat_k[s].clone())
        v_new.append(flat_v[s].clone())
    kc, vc = case.k_cache.clone(), case.v_cache.clone()
    kc.view(-1, case.num_kv_heads, case.head_dim)[torch.tensor(loc, device=DEV)] = float("nan")
    vc.view(-1, case.num_kv_heads, case.head_dim)[torch.tensor(loc, device=DEV)] = float("nan")
    P.pkvs_append_kv(torch.stack(k_new), torch.stack(v_new), torch.tensor(loc, device=DEV), kc, vc)
    # request b's pages live in map row (b * 5) % 8, the window trims whole pages
    rows = [(b * 5) % 8 for b in range(B)]
    page_map = torch.full((8, 200), -7, dtype=torch.int32)
    for b in range(B):
        page_map[rows[b], :len(pages[b])] = pages[b]
    first = [0 if W < 0 else max(0, kv[b] - 1 - W) // Psz for b in range(B)]
    npg = [len(pages[b]) - first[b] for b in range(B)]
    kp, ki = P.pkvs_build_kv_indices(
        page_map.to(DEV), torch.tensor(rows, dtype=torch.int32, device=DEV),
        torch.tensor(npg, dtype=torch.int32, device=DEV),
        start=torch.tensor(first, dtype=torch.int32, device=DEV), capacity=sum(npg))
    table_len = [kv[b] - first[b] * Psz for b in range(B)]
    last = [t - (n - 1) * Psz for t, n in zip(table_len, npg)]
    att = make_attention(case)
    host_indptr = [0]
    for n in npg:
        host_indptr.append(host_indptr[-1] + n)
    att.plan(kv_indptr=host_indptr, kv_last_page_len=last)
    o, lse = poisoned_outputs(case.q)
    att.run(case.q, kc, vc, ki, sm_scale=case.sm_scale, window_left=W, out=o, lse=lse)
    torch.cuda.synchronize()
    assert kp.cpu().tolist() == host_indptr
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"decode step with append + device page table W={W}")


# ----------------------------------------------------------------- logits soft cap
# sglang flashinfer_backend.py forward_extend / forward_decode pass
# logits_soft_cap to the wrappers; every logit x becomes c * tanh(x / c).
# sm_scale 0.3 on N(0,1) data puts many logits near and past the cap.


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("cap", [2.0, 30.0])
@pytest.mark.parametrize("W", [-1, 33])
def test_soft_cap_prefill_variants(variant, cap, W):
    qo = [1, 70, 33, 129, 300]
    kv = [1, 70, 300, 129, 301]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=W, seed=int(cap) * 10 + variant, cap=cap)
    case.sm_scale = 0.3
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"soft cap {cap} variant={variant} W={W}")
    if cap == 2.0:  # the cap matters: without it the LSE differs
        _, rl0 = oracle.paged_attention(
            case.q, case.k_cache, case.v_cache, case.qo_indptr, case.kv_indptr, case.kv_indices,
            case.kv_last_page_len, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
            causal=True, window_left=W, sm_scale=0.3)
        assert np.abs(rl0 - rl).max() > 0.1


@pytest.mark.parametrize("D,G", [(64, 4), (128, 8), (256, 2)])
@pytest.mark.parametrize("split", [-1, 64])
def test_soft_cap_decode(D, G, split):
    kv = [1, 300, 77, 2000, 64, 900]
    case = small([1] * len(kv), kv, H_q=2 * G, H_kv=2, D=D, P_=16, W=127, seed=D + G + split,
                 decode=True, split=split, cap=5.0)
    case.sm_scale = 0.3
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"soft cap decode D={D} G={G} split={split}")


def test_soft_cap_fp32_and_cascade():
    case = small([6, 8, 12], [6, 10, 12], H_q=2, H_kv=1, D=64, P_=4, W=4, seed=3,
                 dtype=torch.float32, cap=1.5)
    case.sm_scale = 0.3
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="soft cap fp32 prefill")
    dec = small([1] * 3, [9, 40, 100], H_q=2, H_kv=1, D=64, P_=4, W=20, seed=4,
                dtype=torch.float32, decode=True, cap=1.5)
    dec.sm_scale = 0.3
    o, lse = gpu_run(dec)
    ro, rl = oracle_for(dec)
    compare(o, lse, ro, rl, tag="soft cap fp32 decode")
    cas = small([40, 130, 7], [90, 130, 500], H_q=8, H_kv=2, D=128, P_=16, W=63, seed=5, cap=4.0)
    cas.sm_scale = 0.3
    (o, lse), _ = cascade_run(cas, trim=True)
    ro, rl = oracle_for(cas)
    compare(o, lse, ro, rl, tag="soft cap cascade")


# ----------------------------------------------------------------- fp16 inputs
# The dtype sweep of AMD-Ecosystem/flashinfer PR 234 ("Tests added") runs fp16
# and bf16; the 16-bit kernels read IEEE half on the fp16 matrix instructions.


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("W", [-1, 0, 33])
def test_fp16_prefill_variants(variant, W):
    qo = [1, 70, 0, 33, 129, 5, 300]
    kv = [1, 70, 9, 300, 129, 700, 301]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=4, W=W, seed=700 + variant * 10 + W,
                 dtype=torch.float16)
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    assert o.dtype == torch.float16 and att.info().prefill_variant == variant
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"fp16 prefill variant={variant} W={W}")


@pytest.mark.parametrize("D,G", [(64, 8), (128, 4), (256, 1)])
def test_fp16_prefill_head_shapes(D, G):
    case = small([40, 130, 7], [90, 130, 500], H_q=2 * G, H_kv=2, D=D, P_=16, W=63,
                 seed=D * G, dtype=torch.float16)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"fp16 prefill D={D} G={G}")


@pytest.mark.parametrize("D,G", [(64, 4), (128, 8), (256, 2)])
@pytest.mark.parametrize("W,split", [(-1, 64), (127, -1), (0, -1)])
def test_fp16_decode(D, G, W, split):
    kv = [1, 300, 77, 2000, 64, 900]
    case = small([1] * len(kv), kv, H_q=2 * G, H_kv=2, D=D, P_=16, W=W, seed=D + G + W,
                 decode=True, split=split, dtype=torch.float16)
    o, lse = gpu_run(case)
    assert o.dtype == torch.float16
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"fp16 decode D={D} G={G} W={W} split={split}")


def test_fp16_cascade_and_soft_cap():
    case = small([40, 130, 7], [90, 130, 500], H_q=8, H_kv=2, D=128, P_=16, W=63, seed=77,
                 dtype=torch.float16)
    (o, lse), _ = cascade_run(case, trim=True)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="fp16 cascade")
    capped = small([70, 33], [70, 300], H_q=8, H_kv=2, D=128, P_=16, W=-1, seed=78,
                   dtype=torch.float16, cap=3.0)
    capped.sm_scale = 0.3
    o, lse = gpu_run(capped)
    ro, rl = oracle_for(capped)
    compare(o, lse, ro, rl, tag="fp16 soft cap")


# ----------------------------------------------------------------- 8-bit KV caches
# sglang flashinfer_backend.py passes k_scale / v_scale with the cache; an
# 8-bit (OCP e4m3 / e5m2) cache holds K / k_scale and V / v_scale.  The oracle
# widens every byte exactly; the kernels widen on the way to the matrix cores.

FP8 = [torch.float8_e4m3fn, torch.float8_e5m2]


@pytest.mark.parametrize("kv_dtype", FP8)
@pytest.mark.parametrize("variant", [0, 1, 2])
@pytest.mark.parametrize("W", [-1, 33])
def test_fp8_kv_prefill(kv_dtype, variant, W):
    qo = [1, 70, 0, 33, 129, 5, 300]
    kv = [1, 70, 9, 300, 129, 700, 301]
    case = small(qo, kv, H_q=8, H_kv=2, D=128, P_=16, W=W, seed=800 + variant * 10 + W,
                 kv_dtype=kv_dtype, k_scale=0.05, v_scale=0.07)
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    assert att.info().prefill_variant in (1, 2)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"fp8 {kv_dtype} prefill variant={variant} W={W}")


@pytest.mark.parametrize("kv_dtype", FP8)
@pytest.mark.parametrize("D,G", [(64, 4), (128, 8), (256, 2)])
@pytest.mark.parametrize("W,split", [(-1, 64), (127, -1)])
def test_fp8_kv_decode(kv_dtype, D, G, W, split):
    kv = [1, 300, 77, 2000, 64, 900]
    case = small([1] * len(kv), kv, H_q=2 * G, H_kv=2, D=D, P_=16, W=W, seed=D + G + W,
                 decode=True, split=split, kv_dtype=kv_dtype, k_scale=0.05, v_scale=0.07)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"fp8 {kv_dtype} decode D={D} G={G} W={W} split={split}")


@pytest.mark.parametrize("kv_dtype", FP8)
def test_fp8_kv_head_shapes_fp16_cascade(kv_dtype):
    for D, G in ((64, 8), (256, 1)):
        case = small([40, 130, 7], [90, 130, 500], H_q=2 * G, H_kv=2, D=D, P_=16, W=63,
                     seed=D * G, kv_dtype=kv_dtype, k_scale=0.05, v_scale=0.07)
        o, lse = gpu_run(case)
        ro, rl = oracle_for(case)
        compare(o, lse, ro, rl, tag=f"fp8 prefill D={D} G={G}")
    case = small([70, 33], [70, 300], H_q=8, H_kv=2, D=128, P_=16, W=-1, seed=81,
                 dtype=torch.float16, kv_dtype=kv_dtype, k_scale=0.05, v_scale=0.07)
    o, lse = gpu_run(case)
    assert o.dtype == torch.float16
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="fp8 K/V with fp16 queries")
    cas = small([40, 130, 7], [90, 130, 500], H_q=8, H_kv=2, D=128, P_=16, W=63, seed=82,
                kv_dtype=kv_dtype, k_scale=0.0625, v_scale=0.125)
    (o, lse), _ = cascade_run(cas, trim=True)
    ro, rl = oracle_for(cas)
    compare(o, lse, ro, rl, tag="fp8 cascade")


def test_kv_scales_on_a_16_bit_cache():
    """The scales apply to every cache type: a bf16 cache read as 0.5 K, 1.5 V."""
    case = small([30, 9], [90, 40], H_q=8, H_kv=2, D=128, W=10, seed=83, k_scale=0.5,
                 v_scale=1.5)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag="scales on bf16")


@pytest.mark.parametrize("kv_dtype", FP8)
@pytest.mark.parametrize("src", [torch.bfloat16, torch.float16, torch.float32])
def test_append_into_8_bit_cache_bit_exact(kv_dtype, src):
    """Every new element x lands as the 8-bit code of x / scale (fp32 quotient
    rounded to the input type, then to nearest even; overflow, infinities and
    NaN by the format's rules), bit for bit against the oracle: for 16-bit
    inputs every bit pattern of the type, for fp32 a spread with the edge
    values."""
    H, D = 8, 128
    if src == torch.float32:
        g = torch.Generator().manual_seed(3)
        x = torch.randn(65536, generator=g) * torch.logspace(-12, 6, 65536, base=2.0)
        x[:12] = torch.tensor([0.0, -0.0, 464.0, 464.01, 448.0, 61440.0, 57344.0, 1e-40,
                               float("inf"), float("-inf"), float("nan"), -2.0 ** -17])
    else:
        x = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16).view(src)
    rows = x.numel() // (H * D)
    k_new = x.reshape(rows, H, D).contiguous()
    v_new = k_new.flip(0).contiguous()
    pages, Psz = 16, 8
    g = torch.Generator().manual_seed(7)
    k_cache = torch.randint(0, 256, (pages, Psz, H, D), generator=g,
                            dtype=torch.uint8).view(kv_dtype)
    v_cache = torch.randint(0, 256, (pages, Psz, H, D), generator=g,
                            dtype=torch.uint8).view(kv_dtype)
    loc = torch.randperm(pages * Psz, generator=g)[:rows].to(torch.int64)
    loc[1] = -1  # skipped and counted
    rk, rv, skipped = oracle.append_kv_quant(k_new, v_new, loc, k_cache, v_cache, 0.37, 0.0625)
    kc, vc = k_cache.to(DEV), v_cache.to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    log(f"8-bit append {src} -> {kv_dtype}: {rows} rows")
    P.pkvs_append_kv(k_new.to(DEV), v_new.to(DEV), loc.to(DEV), kc, vc, status=status,
                     k_scale=0.37, v_scale=0.0625)
    torch.cuda.synchronize()
    assert int(status) == skipped == 1
    nan_mask = 0x7F if kv_dtype == torch.float8_e4m3fn else 0x7C
    for got, want in ((kc.cpu().view(torch.uint8), rk.view(torch.uint8)),
                      (vc.cpu().view(torch.uint8), rv.view(torch.uint8))):
        g8, w8 = got.reshape(-1).numpy(), want.reshape(-1).numpy()
        # NaN codes may differ in sign; every other code is exact
        wnan = ((w8 & 0x7F) > nan_mask) | ((w8 & 0x7F) == 0x7F)
        gnan = ((g8 & 0x7F) > nan_mask) | ((g8 & 0x7F) == 0x7F)
        assert np.array_equal(gnan, wnan)
        diff = np.nonzero((g8 != w8) & ~wnan)[0]
        assert diff.size == 0, [(int(i), hex(g8[i]), hex(w8[i])) for i in diff[:8]]


@pytest.mark.parametrize("kv_dtype", FP8)
def test_decode_over_an_8_bit_cache_written_by_append(kv_dtype):
    """A decode batch whose 8-bit cache was filled by pkvs_append_kv from bf16
    keys and values equals the oracle over that cache."""
    kv = [1, 300, 77, 900]
    src = small([1] * len(kv), kv, H_q=16, H_kv=2, D=128, P_=16, W=127, seed=95, decode=True)
    Psz = src.page_size
    kvp = src.kv_indptr.cpu().tolist()
    loc = []
    for b in range(len(kv)):
        pages = src.kv_indices.cpu()[kvp[b]:kvp[b + 1]]
        loc += [int(pages[j // Psz]) * Psz + j % Psz for j in range(kv[b])]
    loc_t = torch.tensor(loc, device=DEV)
    flat = lambda t: t.view(-1, src.num_kv_heads, src.head_dim)
    k_rows, v_rows = flat(src.k_cache)[loc_t].contiguous(), flat(src.v_cache)[loc_t].contiguous()
    k8 = torch.zeros(src.k_cache.shape, dtype=torch.uint8, device=DEV).view(kv_dtype)
    v8 = torch.zeros_like(k8)
    P.pkvs_append_kv(k_rows, v_rows, loc_t, k8, v8, k_scale=0.05, v_scale=0.07)
    case = dataclasses.replace(src, k_cache=k8, v_cache=v8, k_scale=0.05, v_scale=0.07)
    o, lse = gpu_run(case)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=f"decode over an appended {kv_dtype} cache")
