"""GPU parity of the W12 LM-head stream: the verify path run on the W12 encoding of
the LM head must give the oracle's results computed on the bf16 LM head itself
(lossless format; logits differ from the bf16 kernel only in fp32 summation order)."""
import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as sd
from oracle import sd_oracle as O
from synth import make_step, make_weights, workload

from _parity import (Report, attach_inputs, check_logits_rows, compare, run_gpu, run_oracle,
                     upload_step)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    yield


def w12_case(w, steps, fused=True, W=None, tokens=None):
    W = make_weights(w) if W is None else W
    W64 = O.lm_head_f64(W)
    head = sd.W12Weights.from_bf16(W)
    say(w.name, f"W12 cap={head.cap} b2={head.b2} fused={fused}")
    vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold, fused=fused)
    rep = Report()
    for st in steps:
        say(w.name, f"B={w.B} g={w.gamma} d={w.d} V={w.V} T={w.T} step={st}")
        s = make_step(w, W, st)
        if tokens is not None:
            s.draft_tokens = tokens(s.draft_tokens.shape)
        g = run_gpu(w, head, upload_step(s), vr, fetch_all_logits=w.T > 0)
        o = attach_inputs(run_oracle(w, W64, s), s)
        assert g.flags == 0, f"device flags {g.flags}"
        compare(w, g, o, range(w.B), rep)
        if g.logits is not None:
            check_logits_rows(w, g.logits, o.z, rep)
        assert np.array_equal(g.counters, o.accept.counters)
    say("report", rep)
    return rep


SMALL = [
    ("w12-skinny16-greedy", 1, 4, 256, 1000, 0.0, False),
    ("w12-skinny32-rej", 1, 20, 384, 2000, 1.0, False),
    ("w12-skinny64-trunc", 3, 16, 512, 3001, 0.8, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
def test_w12_small_shapes(case, fused):
    name, B, g, d, V, T, trunc = case
    w = workload("ragged-b32", B=B, gamma=g, d=d, V=V, T=T, truncate=trunc, geo_p=(0.2,),
                 name=name)
    w12_case(w, range(3), fused)


def test_w12_many_corrections_and_crowded_slab():
    """Tiny weights scattered over every region (dozens of corrections per region) and
    every drafted token inside the first slab (the merge's own W12 dot)."""
    w = workload("ragged-b32", B=2, gamma=16, d=512, V=4000, T=1.0, truncate=False,
                 geo_p=(0.2,), name="w12-corrections")
    W = make_weights(w).copy()
    rng = np.random.default_rng(11)
    flat = W.reshape(-1)
    idx = rng.choice(flat.size, 8000, replace=False)
    flat[idx[:6000]] = (rng.integers(1, 40, 6000) << 8 | rng.integers(0, 256, 6000)).astype(np.uint16)
    flat[idx[6000:]] = 0x8000
    head = sd.W12Weights.from_bf16(W)
    assert head.cap >= 16
    for fused in (True, False):
        w12_case(w, range(2), fused, W=W)
        w12_case(w, range(2), fused, W=W,
                 tokens=lambda shape: rng.integers(0, 64, shape).astype(np.int32))


def test_w12_greedy_block9():
    w = workload("greedy-block9")
    w12_case(w, range(30), fused=True)
    w12_case(w, range(5), fused=False)


def test_w12_rejection_b1():
    w = workload("rejection-b1")
    w12_case(w, range(3), fused=True)
