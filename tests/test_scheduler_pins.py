"""Pins of the prefix-scheduler oracle against things other than itself.

Brute force over every choice of per-request prefix lengths, the unimodal
case in which early stopping reaches the global optimum, a staircase cost
table on which only the search without early stopping crosses the cliff,
the decode-round worked example, tie order and confidence clamping.
"""
import itertools
import json
import os

import numpy as np

from oracle import prefix_scheduler as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(conf, sps):
    """Largest throughput over every vector of prefix lengths, summed directly in float64."""
    conf = np.asarray(conf, dtype=np.float32)
    R, g = conf.shape
    a = S.survival(conf).astype(np.float64)
    best, best_L = -1.0, None
    for L in itertools.product(range(g + 1), repeat=R):
        tau = R + sum(a[r, :L[r]].sum() for r in range(R))
        th = tau * float(np.float32(sps[R + sum(L)]))
        if th > best * (1 + 1e-12):
            best, best_L = th, L
    return best, best_L


def direct_theta(conf, sps, verify_len):
    a = S.survival(conf).astype(np.float64)
    R = len(verify_len)
    tau = R + sum(a[r, :verify_len[r]].sum() for r in range(R))
    return tau * float(np.float32(sps[R + int(np.sum(verify_len))]))


def test_survival_is_running_product_with_clamping():
    conf = np.array([[0.5, 0.5, 2.0, -1.0], [np.nan, 0.9, 0.9, 0.9], [1.0, 1.0, 0.25, 1.0]],
                    np.float32)
    a = S.survival(conf)
    assert a[0].tolist() == [0.5, 0.25, 0.25, 0.0]
    assert a[1].tolist() == [0.0, 0.0, 0.0, 0.0]
    assert a[2].tolist() == [1.0, 1.0, 0.25, 0.25]


def test_global_search_equals_brute_force_on_any_table():
    """Top-K by survival is the best K-subset under the prefix rule, so the search over K
    reaches the maximum over all prefix-length vectors for an arbitrary cost table."""
    rng = np.random.default_rng(3)
    for trial in range(60):
        R, g = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        conf = rng.uniform(0.05, 1.0, (R, g)).astype(np.float32)
        sps = rng.uniform(0.2, 1.0, R * (g + 1) + 1).astype(np.float32)
        vl, offs, K = S.schedule_prefix(conf, sps, S.ASYNC_TOP_K)
        best, _ = brute_force(conf, sps)
        got = direct_theta(conf, sps, vl)
        assert abs(got - best) <= 1e-9 * best, (trial, got, best)
        assert int(vl.sum()) == K and offs[-1] == R + K
        assert np.array_equal(np.diff(offs), vl + 1)


def test_early_stop_is_optimal_when_theta_is_unimodal():
    """With SPS(B) = 1 / (t0 + t1 B) the throughput is concave over linear along the
    sorted order, hence unimodal, and early stopping finds the global maximum."""
    rng = np.random.default_rng(4)
    for trial in range(60):
        R, g = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        conf = rng.uniform(0.05, 1.0, (R, g)).astype(np.float32)
        t0, t1 = rng.uniform(0.5, 2.0), rng.uniform(0.01, 1.0)
        B = np.arange(R * (g + 1) + 1)
        sps = (1.0 / (t0 + t1 * B)).astype(np.float32)
        vl, _, _ = S.schedule_prefix(conf, sps, S.SYNC_EARLY_STOP)
        best, _ = brute_force(conf, sps)
        got = direct_theta(conf, sps, vl)
        assert abs(got - best) <= 1e-9 * best, (trial, got, best)


def test_staircase_cliff_early_stop_versus_global_search():
    """A cost step after the first row and a flat stretch behind it: admitting the second
    candidate lowers throughput, so early stopping halts, while the global search goes on
    to the better plateau (the pages' reason for the asynchronous variant)."""
    conf = np.array([[0.9, 0.9, 0.9, 0.9, 0.9, 0.9]], np.float32)
    sps = np.array([1.0, 1.0, 1.0, 0.6, 0.6, 0.6, 0.6, 0.6], np.float32)
    vl_s, _, K_s = S.schedule_prefix(conf, sps, S.SYNC_EARLY_STOP)
    vl_a, _, K_a = S.schedule_prefix(conf, sps, S.ASYNC_TOP_K)
    assert K_s == 1 and vl_s.tolist() == [1]
    assert K_a == 6 and vl_a.tolist() == [6]
    assert direct_theta(conf, sps, vl_a) > direct_theta(conf, sps, vl_s)


def test_async_uses_stale_confidences_for_k_and_current_ones_for_the_set():
    conf = np.array([[0.2, 0.2], [0.95, 0.9]], np.float32)
    stale = np.array([[0.99, 0.99], [0.99, 0.99]], np.float32)
    sps = np.ones(7, np.float32)   # flat table: every candidate raises throughput
    vl, _, K = S.schedule_prefix(conf, sps, S.ASYNC_TOP_K, conf_stale=stale)
    assert K == 4 and vl.tolist() == [2, 2]
    sps = np.array([1, 1, 1, 1, 1, 0.1, 0.1], np.float32)   # 2 drafts (B = 4) before the cliff
    vl, _, K = S.schedule_prefix(conf, sps, S.ASYNC_TOP_K, conf_stale=stale)
    assert K == 2 and vl.tolist() == [0, 2]    # the two current best: request 1's prefix


def test_ties_go_to_lower_request_then_position():
    conf = np.ones((3, 4), np.float32)
    sps = np.array([1.0] * 10 + [0.01] * 6, np.float32)   # 6 drafts (B = 9) before the drop
    vl, offs, K = S.schedule_prefix(conf, sps, S.ASYNC_TOP_K)
    assert K == 6 and vl.tolist() == [4, 2, 0] and offs.tolist() == [0, 5, 8, 9]
    vl, _, _ = S.schedule_prefix(conf, sps, S.SYNC_EARLY_STOP)
    assert vl.tolist() == [4, 2, 0]


def test_decode_round_worked_example():
    gold = json.load(open(os.path.join(GOLDEN, "dspark_scheduler_round.json")))
    conf = np.array(gold["conf"], np.float32)
    sps = np.array(gold["sps"], np.float32)
    for mode in (S.SYNC_EARLY_STOP, S.ASYNC_TOP_K):
        vl, offs, K = S.schedule_prefix(conf, sps, mode)
        assert vl.tolist() == gold["expected"]["verify_len"]
        assert offs.tolist() == gold["expected"]["row_offsets"]
        assert K == gold["expected"]["admitted"]


def test_zero_confidence_never_helps_and_full_confidence_fills_a_flat_table():
    conf = np.zeros((4, 3), np.float32)
    sps = np.linspace(1.0, 0.5, 17).astype(np.float32)
    vl, _, K = S.schedule_prefix(conf, sps, S.SYNC_EARLY_STOP)
    assert K == 0 and vl.tolist() == [0, 0, 0, 0]
    conf = np.ones((4, 3), np.float32)
    vl, _, K = S.schedule_prefix(conf, np.ones(17, np.float32), S.SYNC_EARLY_STOP)
    assert K == 12 and vl.tolist() == [3, 3, 3, 3]
