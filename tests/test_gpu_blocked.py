"""GPU parity of the slab-blocked bf16 LM head: the copy sd_lm_head_block writes has the
documented layout, and the verify path reading it gives the oracle's results on the
[V][d] LM head and the same accepted lengths, tokens and argmax as the [V][d] path."""
import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as sd
from oracle import sd_oracle as O
from synth import make_step, make_weights, workload

from _parity import (Report, attach_inputs, bf16_dev, check_logits_rows, compare, run_gpu,
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


def expected_blocks(W: np.ndarray) -> np.ndarray:
    """The layout by its definition: [d/128][ceil(V/64)][64][128] (block (st, s) holds rows
    64 s .. 64 s + 63 at columns 128 st .. 128 st + 127), row r's chunk j of a block at
    chunk position j ^ (r & 15), rows past V zero."""
    V, d = W.shape
    ns, nst = (V + 63) // 64, d // 128
    pad = np.zeros((ns * 64, d), np.uint16)
    pad[:V] = W
    out = np.zeros((nst, ns, 64, 16, 8), np.uint16)
    for st in range(nst):
        for s in range(ns):
            for r in range(64):
                row = pad[64 * s + r, 128 * st:128 * (st + 1)].reshape(16, 8)
                for j in range(16):
                    out[st, s, r, j ^ (r & 15), :] = row[j]
    return out.reshape(-1)


@pytest.mark.parametrize("V,d", [(1000, 256), (64, 128), (3001, 512)])
def test_block_layout_bytes(V, d):
    w = workload("ragged-b32", B=1, gamma=4, d=d, V=V, T=0.0, truncate=False, name="layout")
    W = make_weights(w)
    say("layout", f"V={V} d={d}")
    head = sd.BlockedWeights(bf16_dev(W))
    torch.cuda.synchronize()
    assert head.nbytes == ((V + 63) // 64) * (d // 128) * 16384
    got = head.buf.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, expected_blocks(W))


def blocked_case(w, steps, fused=True, tokens=None):
    W = make_weights(w)
    W64 = O.lm_head_f64(W)
    W_dev = bf16_dev(W)
    head = sd.BlockedWeights(W_dev)
    vr_b = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold, fused=fused)
    vr_r = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold, fused=fused)
    rep = Report()
    rng = np.random.default_rng(5)
    for st in steps:
        say(w.name, f"blocked B={w.B} g={w.gamma} d={w.d} V={w.V} T={w.T} step={st} fused={fused}")
        s = make_step(w, W, st)
        if tokens is not None:
            s.draft_tokens = tokens(rng, s.draft_tokens.shape)
        ds = upload_step(s)
        g = run_gpu(w, head, ds, vr_b, fetch_all_logits=w.T > 0)
        g_r = run_gpu(w, W_dev, ds, vr_r)
        o = attach_inputs(run_oracle(w, W64, s), s)
        assert g.flags == 0, f"device flags {g.flags}"
        compare(w, g, o, range(w.B), rep)
        if g.logits is not None:
            check_logits_rows(w, g.logits, o.z, rep)
        assert np.array_equal(g.counters, o.accept.counters)
        # Same weights: the same decisions as the [V][d] path.
        assert np.array_equal(g.accept_len, g_r.accept_len)
        assert np.array_equal(g.next_token, g_r.next_token)
        assert np.array_equal(g.stats["argmax"], g_r.stats["argmax"])
        # The drafted-token logit: fp64 sums of exact products, stage order aside.
        assert np.allclose(g.stats["z_draft"], g_r.stats["z_draft"], rtol=1e-12, atol=1e-12)
    say("report", rep)


SMALL = [
    ("blk-skinny16-greedy", 1, 4, 256, 1000, 0.0, False),
    ("blk-skinny32-rej", 1, 20, 384, 2000, 1.0, False),
    ("blk-skinny64-trunc", 3, 16, 512, 3001, 0.8, True),
    ("blk-one-slab", 2, 5, 128, 64, 1.0, False),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
def test_blocked_small_shapes(case, fused):
    name, B, g, d, V, T, trunc = case
    w = workload("ragged-b32", B=B, gamma=g, d=d, V=V, T=T, truncate=trunc, geo_p=(0.2,),
                 name=name)
    blocked_case(w, range(3), fused)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
def test_blocked_crowded_slab(fused):
    """Every drafted token in the first 64 ids: beyond the four drafted logits the
    contraction forms per slab, the merge dots the blocked LM-head row itself."""
    w = workload("ragged-b32", B=3, gamma=16, d=512, V=3001, T=1.0, truncate=False,
                 geo_p=(0.2,), name="blk-crowded")
    blocked_case(w, range(2), fused,
                 tokens=lambda rng, shape: rng.integers(0, 64, shape).astype(np.int32))


def test_blocked_greedy_block9():
    blocked_case(workload("greedy-block9"), range(20))


def test_blocked_rejection_b1():
    blocked_case(workload("rejection-b1"), range(3))


def test_blocked_outside_the_streaming_regime_is_refused():
    w = workload("ragged-b32", B=8, gamma=16, d=256, V=1000, T=0.0, truncate=False, name="refuse")
    W_dev = bf16_dev(make_weights(w))
    head = sd.BlockedWeights(W_dev)
    hidden = torch.zeros((8, 17, 256), dtype=torch.bfloat16, device="cuda")   # 136 rows > 64
    with pytest.raises(sd.SdError):
        sd.sd_verify_logits(hidden, head)
