"""The allocation-free decode (pkvs_decode_noalloc: plan and run in the
library's fixed device scratch array) against the decode entry points with
caller workspaces (pkvs_decode_plan + pkvs_decode_run) and the oracle.

Each case makes two calls in a row on one plan, the second with a smaller
batch, so the second runs over what the first left in the array.  The two
paths plan the same work list for the same kernels, so their outputs must be
equal bit for bit; both are also checked against the oracle within the parity
tolerances (|O| 2e-2, |LSE| 1e-3)."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_all_written, compare, log, make_attention, oracle_for, \
    poisoned_outputs
from paged_kv_sliding_amd import pkvs as P
from paged_kv_sliding_amd.synth import case_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda"


def decode_case(name, kv_lens, *, H_q, H_kv, W, dtype, split, seed):
    return case_from_lengths(name, [1] * len(kv_lens), kv_lens, num_qo_heads=H_q,
                             num_kv_heads=H_kv, head_dim=128, page_size=16, dtype=dtype,
                             window_left=W, seed=seed, spare_pages=5, device=DEV,
                             is_decode=True, fixed_split_size=split)


# (H_q, H_kv, W, dtype, split, decode_waves, first batch, second batch)
CASES = [
    # GQA 4 with the decode sweep's shape, 256-key chunks and their merge
    (32, 8, 1023, torch.bfloat16, 256, 1, (64, 1, 4096), (17, 1, 1500)),
    # four waves per item, the planner's own split, no window
    (8, 1, -1, torch.bfloat16, -1, 4, (3, 3000, 16384), (2, 1, 9000)),
    # fp16 with 512-key chunks of a 2048-key window
    (16, 2, 2047, torch.float16, 512, 1, (40, 1, 5000), (9, 1, 700)),
]


@pytest.mark.parametrize("H_q,H_kv,W,dtype,split,nw,first,second", CASES)
def test_noalloc_decode_equals_the_workspace_path(H_q, H_kv, W, dtype, split, nw, first,
                                                  second):
    rng = np.random.default_rng(11)
    batches = []
    for i, (B, lo, hi) in enumerate((first, second)):
        kv = [int(x) for x in rng.integers(lo, hi + 1, size=B)]
        kv[0] = hi  # the longest request of the batch
        batches.append(decode_case(f"noalloc{i}", kv, H_q=H_q, H_kv=H_kv, W=W, dtype=dtype,
                                   split=split, seed=20 + i))
    big = batches[0]
    ref = make_attention(big, batch_capacity=first[0], kv_capacity=first[2], decode_waves=nw)
    handle = P.pkvs_plan_create(ref.desc)
    try:
        fb, ib = P.pkvs_workspace_size(handle)
        assert (ib + 255) // 256 * 256 + fb <= P.NOALLOC_SCRATCH_BYTES
        for call, case in enumerate(batches):
            tag = f"call {call}: batch {case.batch_size}, W={W}, split={split}, waves={nw}"
            log(tag)
            # the workspace path
            ref.plan(qo_indptr=case.qo_indptr.cpu(), kv_indptr=case.kv_indptr.cpu(),
                     kv_last_page_len=case.kv_last_page_len.cpu())
            o_ref, lse_ref = poisoned_outputs(case.q)
            ref.run(case.q, case.k_cache, case.v_cache, case.kv_indices,
                    sm_scale=case.sm_scale, window_left=W, out=o_ref, lse=lse_ref)
            # the allocation-free path, into its own NaN-filled outputs
            o, lse = poisoned_outputs(case.q)
            P.pkvs_decode_noalloc(handle, case.kv_indptr.cpu(), case.kv_last_page_len.cpu(),
                                  case.batch_size, case.q, case.k_cache, case.v_cache,
                                  case.kv_indices, o, lse, case.sm_scale, W)
            torch.cuda.synchronize()
            info = P.pkvs_plan_get_info(handle)
            assert info.decode_waves == nw
            if call == 0 and split > 0:
                assert info.num_merges > 0, "the first batch must split some request"
            assert_all_written(case, o, lse, tag)
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), \
                f"{tag}: O differs from the workspace path"
            assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), \
                f"{tag}: LSE differs from the workspace path"
            ro, rl = oracle_for(case)
            compare(o, lse, ro, rl, tag=tag)
    finally:
        P.pkvs_plan_destroy(handle)
        ref.close()


def test_noalloc_rejects_a_plan_larger_than_the_array():
    """A plan whose capacities need more than the array is refused before any
    device work, with the workspace error."""
    ref = P.make_desc(P.PKVS_DECODE, num_qo_heads=64, num_kv_heads=8, head_dim=128, page_size=16,
                      dtype=torch.bfloat16, window_left=-1, batch_capacity=256,
                      qo_capacity=256, kv_capacity=32768, fixed_split_size=2048)
    handle = P.pkvs_plan_create(ref)
    try:
        case = decode_case("noalloc_big", [40, 70], H_q=64, H_kv=8, W=-1,
                           dtype=torch.bfloat16, split=2048, seed=3)
        o, lse = poisoned_outputs(case.q)
        with pytest.raises(P.PkvsError) as ei:
            P.pkvs_decode_noalloc(handle, case.kv_indptr.cpu(), case.kv_last_page_len.cpu(),
                                  case.batch_size, case.q, case.k_cache, case.v_cache,
                                  case.kv_indices, o, lse, case.sm_scale, -1)
        assert ei.value.code == P.PKVS_ERR_WORKSPACE
        torch.cuda.synchronize()
        assert torch.isnan(o.float()).all(), "a refused call must not write its outputs"
    finally:
        P.pkvs_plan_destroy(handle)
