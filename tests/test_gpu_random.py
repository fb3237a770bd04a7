"""Seeded random GPU parity cases: prefill, decode and cascade batches whose
shape (batch, lengths, window, page size, head dim and group, dtype, logits
soft cap, kernel variant, split size, waves per item) is drawn from a fixed
seed, each run into NaN-filled outputs and compared with the oracle at the
parity tolerances; and chunks of long prompts (few query tiles over many
cached keys, the shape the key split cuts), checked on sampled rows of every
query tile.  The draws cover combinations the hand-written cases do not list
one by one."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_all_written, compare, gpu_run, make_attention, oracle_for
from paged_kv_sliding_amd.synth import case_from_lengths
from test_gpu_parity import cascade_run

pytestmark = pytest.mark.gpu
DEV = "cuda"


def draw_shape(rng):
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8]))
    H_kv = int(rng.choice([1, 2]))
    dtype = torch.float16 if rng.random() < 0.3 else torch.bfloat16
    cap = float(rng.choice([0.0, 0.0, 0.0, 30.0]))
    W = int(rng.choice([-1, 0, 1, 17, 64, 255, 1000]))
    P_ = int(rng.choice([1, 4, 16]))
    return D, G, H_kv, dtype, cap, W, P_


def make_case(name, qo, kv, D, G, H_kv, dtype, cap, W, P_, seed, decode=False, split=-1):
    return case_from_lengths(name, qo, kv, num_qo_heads=G * H_kv, num_kv_heads=H_kv, head_dim=D,
                             page_size=P_, dtype=dtype, window_left=W, seed=seed, spare_pages=3,
                             device=DEV, is_decode=decode, fixed_split_size=split,
                             logits_soft_cap=cap)


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(seed):
    rng = np.random.default_rng(1000 + seed)
    D, G, H_kv, dtype, cap, W, P_ = draw_shape(rng)
    B = int(rng.integers(1, 6))
    qo = [int(x) for x in rng.integers(0, 200, size=B)]
    kv = [q + int(p) for q, p in zip(qo, rng.integers(0, 400, size=B))]
    # variants 3-6 need head_dim 128 (3: <= 128) and 16-bit K/V
    variants = [0, 1] + ([2] if D <= 128 else []) + ([3] if D <= 128 else []) + \
        ([4, 5, 6] if D == 128 else [])
    variant = int(rng.choice(variants))
    case = make_case("rp", qo, kv, D, G, H_kv, dtype, cap, W, P_, seed)
    o, lse = gpu_run(case, prefill_variant=variant)
    tag = f"prefill seed={seed} D={D} G={G} Hkv={H_kv} {dtype} cap={cap} W={W} P={P_} v={variant}"
    assert_all_written(case, o, lse, tag)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=tag)


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(seed):
    rng = np.random.default_rng(2000 + seed)
    D, G, H_kv, dtype, cap, W, P_ = draw_shape(rng)
    B = int(rng.integers(1, 40))
    kv = [int(x) for x in rng.integers(0, 3000, size=B)]
    split = int(rng.choice([-1, 32, 256, 2048]))
    nw = int(rng.choice([0, 1, 4]))
    case = make_case("rd", [1] * B, kv, D, G, H_kv, dtype, cap, W, P_, seed, decode=True,
                     split=split)
    o, lse = gpu_run(case, decode_waves=nw)
    tag = f"decode seed={seed} D={D} G={G} Hkv={H_kv} {dtype} cap={cap} W={W} P={P_} split={split} nw={nw}"
    assert_all_written(case, o, lse, tag)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=tag)


@pytest.mark.parametrize("seed", range(12))
def test_random_cascade(seed):
    rng = np.random.default_rng(3000 + seed)
    D, G, H_kv, dtype, cap, W, P_ = draw_shape(rng)
    B = int(rng.integers(1, 5))
    qo = [int(x) for x in rng.integers(0, 200, size=B)]
    kv = [q + int(p) for q, p in zip(qo, rng.integers(0, 400, size=B))]
    variants = [0, 1] + ([2, 3] if D <= 128 else []) + ([5] if D == 128 else [])
    variant = int(rng.choice(variants))
    trim = bool(rng.random() < 0.5)
    case = make_case("rc", qo, kv, D, G, H_kv, dtype, cap, W, P_, seed)
    (o, lse), att = cascade_run(case, trim=trim, prefill_variant=variant)
    tag = (f"cascade seed={seed} D={D} G={G} Hkv={H_kv} {dtype} cap={cap} W={W} P={P_} "
           f"v={att.info().prefill_variant} trim={trim}")
    assert_all_written(case, o, lse, tag)
    ro, rl = oracle_for(case)
    compare(o, lse, ro, rl, tag=tag)


@pytest.mark.parametrize("seed", range(10))
def test_random_chunked_prefill(seed):
    rng = np.random.default_rng(4000 + seed)
    B = int(rng.integers(1, 4))
    qo = [int(x) for x in rng.integers(1, 700, size=B)]
    kv = [q + int(p) for q, p in zip(qo, rng.integers(500, 6000, size=B))]
    W = int(rng.choice([-1, 511, 2047, 4095]))
    G = int(rng.choice([1, 4, 8]))
    P_ = int(rng.choice([1, 16]))
    dtype = torch.float16 if rng.random() < 0.3 else torch.bfloat16
    variant = int(rng.choice([0, 1, 2, 5]))
    case = make_case("rk", qo, kv, 128, G, 2, dtype, 0.0, W, P_, seed)
    att = make_attention(case, prefill_variant=variant)
    o, lse = gpu_run(case, att=att)
    info = att.info()
    tag = (f"chunked seed={seed} qo={qo} kv={kv} W={W} G={G} P={P_} {dtype} "
           f"v={info.prefill_variant} items={info.num_items} merges={info.num_merges}")
    assert_all_written(case, o, lse, tag)
    # a row of every query tile (and each request's first and last token)
    rows = set()
    for b in range(B):
        q0, q1 = int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])
        rows |= {q0, q1 - 1}
        rows |= {t + int(rng.integers(0, min(info.query_tile, q1 - t)))
                 for t in range(q0, q1, info.query_tile)}
    rows = sorted(rows)
    ro, rl = oracle_for(case, rows=rows)
    compare(o, lse, ro, rl, rows=rows, tag=tag)
