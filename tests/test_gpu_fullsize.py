"""GPU parity at the full vocabulary sizes, on the acceptance paths that the seeded
workloads rarely reach there.

With planting 4 along the drafted token's LM-head row and V ~ 1.3e5-1.5e5, a kept
draft survives rejection sampling only about a quarter of the time, so the named
rejection workloads mostly stop at the first position and almost never draw a bonus
token. These cases change only the inputs, never the path:

* stress planting (+12 along the drafted row, long planted prefixes): long accepted
  prefixes, late acceptance decisions, bonus draws from p;
* u_accept = 0 everywhere: every kept draft survives (p(x) > 0), so every request
  draws its bonus token from p at row L_r with u_resample[r][L_r] (DSpark summary,
  "Architecture": the round emits a bonus token when all drafts survive);
* u_accept = 0 before the last kept position and 0.999 there: the request reaches
  its last kept draft and, unless p(x)/q(x) > 0.999, draws the correction from the
  residual norm(max(0, p - q)) at that late row (DSpark summary, "Problem
  definition": the first rejected position is replaced by a draw from the residual).

Every request is compared with the oracle as in the named-workload tests.
"""
import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as sd
from synth import make_step, workload

from _parity import (Report, attach_inputs, check_logits_rows, compare, lm_head, run_gpu,
                     run_oracle, upload_step)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    yield


def run_case(w, steps, edit=None, label=""):
    """Every request of `steps` against the oracle; `edit(step_inputs)` rewrites the
    uniforms in place before both sides see them."""
    W, W64, W_dev = lm_head(w)
    vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold)
    rep = Report()
    residual_late = 0
    for st in steps:
        say(w.name, label, f"B={w.B} g={w.gamma} d={w.d} V={w.V} T={w.T} plant={w.plant} "
            f"step={st}")
        s = make_step(w, W, st)
        if edit is not None:
            edit(s)
        g = run_gpu(w, W_dev, upload_step(s), vr, fetch_all_logits=True)
        assert g.flags == 0, f"device flags {g.flags}"
        o = attach_inputs(run_oracle(w, W64, s), s)
        compare(w, g, o, range(w.B), rep)
        check_logits_rows(w, g.logits, o.z, rep)
        assert np.array_equal(g.counters, o.accept.counters)
        residual_late += int(np.sum(o.diag.residual & (o.accept.accept_len >= 8)))
        del g, o
    say("report", label, rep, f"residual draws at position >= 8: {residual_late}")
    return rep, residual_late


STRESS = [
    # Long planted prefixes (geometric(0.05), mean 19 before the cap) planted at +12.
    ("rejection-b1", 6),
    ("concurrency-b128", 1),
]


@pytest.mark.parametrize("case", STRESS, ids=[c[0] for c in STRESS])
def test_stress_planting_full_vocab(case):
    key, steps = case
    w = workload(key, plant=12.0, geo_p=(0.05,), name=f"{key}-stress")
    rep, _ = run_case(w, range(steps), label="stress")
    assert rep.accepted >= 4 * rep.requests, rep
    assert rep.full_accepts >= 1, rep
    assert rep.bonus_draws >= 1, rep


def _all_survive(s):
    s.u_accept[:] = 0.0


BONUS = [("rejection-b1", 2), ("ragged-b32", 1), ("concurrency-b128", 1)]


@pytest.mark.parametrize("case", BONUS, ids=[c[0] for c in BONUS])
def test_bonus_draw_full_vocab(case):
    key, steps = case
    w = workload(key)
    rep, _ = run_case(w, range(steps), edit=_all_survive, label="u_accept=0")
    # Every request accepted all of its kept drafts and drew from p at row L_r.
    assert rep.bonus_draws == rep.requests, rep
    assert rep.accepted == rep.rows - rep.requests, rep


def _reject_last(s, threshold):
    """Survive every kept position before the last; at the last one accept only if
    p(x)/q(x) > 0.999. Kept lengths come from the same truncation on both sides."""
    from oracle import sd_oracle as O
    B, g = s.u_accept.shape
    if s.conf is not None:
        L, _ = O.truncate_by_confidence(s.conf, threshold)
    else:
        L = np.full(B, g, np.int32)
    s.u_accept[:] = 0.0
    for r in range(B):
        if L[r] >= 1:
            s.u_accept[r, L[r] - 1] = np.float32(0.999)


LATE = [("rejection-b1", 2), ("ragged-b32", 1), ("concurrency-b128", 1)]


@pytest.mark.parametrize("case", LATE, ids=[c[0] for c in LATE])
def test_late_residual_draw_full_vocab(case):
    key, steps = case
    w = workload(key)
    rep, late = run_case(w, range(steps), edit=lambda s: _reject_last(s, w.threshold),
                         label="reject-last")
    # Most requests reach their last kept draft and draw from the residual there.
    assert rep.draws - rep.bonus_draws >= rep.requests // 2, rep
    assert late >= 1
