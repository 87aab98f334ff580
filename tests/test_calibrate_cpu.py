"""Host logic of the retention calibration (no GPU): the retained-count rule
matches the oracle's count rule for every ratio of a fine grid."""
import oracle
from sparse_attention_kv_amd import calibrate


def test_retained_count_matches_oracle_rule():
    for N in (1, 7, 100, 384, 1000, 4096, 32768):
        for n_prev in sorted({N, max(1, N // 2), max(1, N // 7)}):
            for i in range(1, 101):
                rho = i / 100
                assert calibrate.retained_count(rho, N, n_prev) == \
                    oracle.active_count(rho, N, n_prev), (rho, N, n_prev)
