"""CPU oracle for the hardware-aware prefix scheduler (test infrastructure, not product).

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this module. The HIP library never
calls it and shares no code with it.

What it computes (DSpark summary, "Architecture", "Confidence-Scheduled
Verification" -> "Hardware-Aware Prefix Scheduler", and "Engineering" ->
"the scheduler in practice"):

* each request r of the R active ones carries per-position conditional
  confidences c[r][k] (the chance that position k passes given that the
  earlier ones did); its survival is the running product
  a[r][j] = c[r][0] * ... * c[r][j], which never grows with j;
* verifying K draft candidates in total costs a batch of B = R + K target
  rows (each request always verifies its bonus row); SPS(B) is the engine's
  steps per second at that batch, a table profiled once;
* the objective is throughput, Theta = tau * SPS(B), with tau the expected
  number of tokens one step emits: one per request plus the survival of
  every admitted candidate;
* all candidates are sorted by survival (largest first) and admitted in that
  order; because survival falls along a block, every prefix of the sorted
  list keeps each request's admitted positions a prefix of its block;
* synchronous variant: admit one candidate at a time and stop at the first
  candidate whose admission lowers Theta;
* asynchronous variant: the number of candidates K is chosen from
  confidences two steps old, by a search over every K with no early stop
  (a dynamic top-K); the current step then admits its own K most confident
  candidates.

Readings where the pages leave the step open (both sides share them, since
floating point here decides integers):

* confidences are clamped into [0, 1] (NaN counts as 0) and the running
  product is taken left to right in float32;
* sort order: larger survival first, ties broken by request, then position;
* tau is accumulated in fixed point: each admitted survival contributes
  floor(a * 2^40) units of 2^-40 tokens, and Theta_K is the float64 product
  of (R * 2^40 + sum of the first K units), converted to float64 with
  round-to-nearest-even, and the float64 value of SPS(R + K). This makes the
  sum independent of summation order;
* synchronous: K is the first K with Theta_{K+1} < Theta_K (equal values
  keep admitting), else every candidate;
* asynchronous: K is the smallest K attaining the largest Theta over
  K = 0 .. R * gamma computed from the stale confidences.

Outputs are those of confidence truncation: verify_len[r] = admitted
candidates of request r, and row_offsets = exclusive scan of verify_len + 1.
"""
from __future__ import annotations

import numpy as np

FIX_BITS = 40
SYNC_EARLY_STOP = 0
ASYNC_TOP_K = 1


def survival(conf: np.ndarray) -> np.ndarray:
    """Running float32 product of the clamped confidences along each block."""
    conf = np.asarray(conf, dtype=np.float32)
    R, g = conf.shape
    a = np.zeros((R, g), dtype=np.float32)
    for r in range(R):
        run = np.float32(1.0)
        for j in range(g):
            c = conf[r, j]
            c = c if c > 0 else np.float32(0.0)           # NaN and negatives -> 0
            c = c if c < 1 else np.float32(1.0)
            run = np.float32(run * c)
            a[r, j] = run
    return a


def sorted_candidates(a: np.ndarray):
    """(r, j) of every candidate, larger survival first, ties by request then position."""
    R, g = a.shape
    cand = [(-float(a[r, j]), r, j) for r in range(R) for j in range(g)]
    cand.sort()
    return [(r, j) for _, r, j in cand]


def fixed_units(x: np.float32) -> int:
    return int(np.floor(np.float64(x) * float(1 << FIX_BITS)))


def theta_curve(a: np.ndarray, sps: np.ndarray):
    """Theta_K for K = 0 .. R*gamma along the sorted candidate order, and that order."""
    R, g = a.shape
    order = sorted_candidates(a)
    units = R << FIX_BITS
    theta = [float(units) * float(np.float32(sps[R]))]
    for K, (r, j) in enumerate(order, start=1):
        units += fixed_units(a[r, j])
        theta.append(float(units) * float(np.float32(sps[R + K])))
    return np.array(theta), order


def choose_k(theta: np.ndarray, mode: int) -> int:
    N = len(theta) - 1
    if mode == SYNC_EARLY_STOP:
        for K in range(N):
            if theta[K + 1] < theta[K]:
                return K
        return N
    best = 0
    for K in range(1, N + 1):
        if theta[K] > theta[best]:
            best = K
    return best


def schedule_prefix(conf: np.ndarray, sps: np.ndarray, mode: int = SYNC_EARLY_STOP,
                    conf_stale: np.ndarray | None = None):
    """verify_len[R], row_offsets[R + 1] and the admitted candidate count K."""
    conf = np.asarray(conf, dtype=np.float32)
    R, g = conf.shape
    sps = np.asarray(sps, dtype=np.float32)
    assert sps.shape[0] >= R * (g + 1) + 1
    a = survival(conf)
    if mode == ASYNC_TOP_K and conf_stale is not None:
        theta, _ = theta_curve(survival(conf_stale), sps)
        _, order = theta_curve(a, sps)
    else:
        theta, order = theta_curve(a, sps)
    K = choose_k(theta, mode)
    verify_len = np.zeros(R, dtype=np.int32)
    for r, j in order[:K]:
        verify_len[r] += 1
    row_offsets = np.zeros(R + 1, dtype=np.int32)
    for r in range(R):
        row_offsets[r + 1] = row_offsets[r] + verify_len[r] + 1
    return verify_len, row_offsets, K
