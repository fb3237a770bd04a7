"""The CPU oracle against facts fixed outside it (closed forms, library
routines, invariants, brute force, hand-derived golden counts)."""
import pytest

from pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(check):
    check(None)


def test_oracle_threads_do_not_change_results():
    """Rows spread over several threads give the single-thread result bit for
    bit (each row is computed by one thread with the same arithmetic)."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_sliding_amd.synth import case_from_lengths

    case = case_from_lengths("threads", [5, 40, 1, 17], [9, 300, 1, 17], num_qo_heads=4,
                             num_kv_heads=2, head_dim=32, page_size=4, dtype=torch.bfloat16,
                             window_left=13, seed=3, spare_pages=3)
    o1, l1 = oracle.case_attention(case, threads=1)
    for nt in (2, 7, 200):
        o2, l2 = oracle.case_attention(case, threads=nt)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), nt
    rows = [60, 0, 44, 3, 62]
    o3, l3 = oracle.case_attention(case, rows=rows, threads=3)
    assert np.array_equal(o3, o1[rows]) and np.array_equal(l3, l1[rows])
