"""The toy multi-step decode loop on the GPU: greedy speculative decoding through the
whole path (draft -> keep a prefix -> verify -> accept -> commit) must emit exactly the
target's own greedy chain, whatever prefix the threshold or the scheduler keeps
(LFM2.5-DSpark blog, "Quality parity"), eagerly and when the steps replay from a
captured HIP graph."""
import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as sd
from draft_block_verification_amd.decode_loop import ToyDecodeLoop
from oracle import sd_oracle as O
from synth import bf16_round, make_weights, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    yield


V, D = 4096, 256


def toy(seed=0):
    """LM head, bigram embedding with a planted successor, the target's greedy next-token
    table (fp64 oracle) with its top-1/top-2 gaps, and a drafter table that is right 75%."""
    rng = np.random.default_rng(seed)
    W = make_weights(workload("ragged-b32", V=V, d=D, name="toy-decode"))
    W64 = O.lm_head_f64(W)
    succ = rng.permutation(V)
    unit = W64[succ] / np.linalg.norm(W64[succ], axis=1, keepdims=True)
    E = bf16_round((0.3 * rng.standard_normal((V, D)) / np.sqrt(D) + 4.0 * unit).astype(np.float32))
    z = O.bf16_decode(E) @ W64.T
    nxt = np.argmax(z, axis=1)
    srt = np.sort(z, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    right = rng.random(V) < 0.75
    dnext = np.where(right, nxt, rng.integers(0, V, V))
    dconf = np.where(right, 0.92, rng.uniform(0.2, 0.6, V)).astype(np.float32)
    return W, E, nxt, gap, dnext, dconf


def to_dev(W, E, dnext, dconf):
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)
    return bf(W), bf(E), torch.from_numpy(dnext).cuda(), torch.from_numpy(dconf).cuda()


def check_chain(outs, start, nxt, gap):
    """Each output must be start, nxt[start], nxt[nxt[start]], ... (no near-ties on the way)."""
    for r, toks in enumerate(outs):
        t = int(start[r])
        assert toks[0] == t
        for i in range(1, len(toks)):
            assert gap[t] > 1e-3, "near-tie on the chain"
            t = int(nxt[t])
            assert toks[i] == t, f"request {r}: token {i} is {toks[i]}, target chain has {t}"


def run_loop(loop, start, steps):
    loop.reset(start)
    for i in range(steps):
        loop.step(i % 3)
    torch.cuda.synchronize()
    return loop.tokens()


@pytest.mark.parametrize("mode", ["threshold", "early-stop", "top-k"])
def test_decode_loop_emits_target_greedy_chain(mode):
    W, E, nxt, gap, dnext, dconf = toy()
    Wd, Ed, dn, dc = to_dev(W, E, dnext, dconf)
    B, g, steps = 8, 6, 30
    sched = {"threshold": None, "early-stop": sd.SCHED_EARLY_STOP, "top-k": sd.SCHED_TOP_K}[mode]
    sps = None
    if sched is not None:
        rows = np.arange(B * (g + 1) + 1)
        sps = torch.from_numpy((1.0 / (1.0 + 0.02 * np.ceil(rows / 16.0))).astype(np.float32)).cuda()
    say("decode-loop", mode, f"B={B} g={g} steps={steps} V={V} d={D}")
    loop = ToyDecodeLoop(Wd, Ed, dn, dc, B, g, steps, scheduler=sched, sps=sps)
    start = torch.from_numpy(np.random.default_rng(1).integers(0, V, B)).cuda()
    outs = run_loop(loop, start, steps)
    check_chain(outs, start.cpu().numpy(), nxt, gap)
    drafted, accepted = loop.vr.counters.cpu().numpy().tolist()
    emitted = sum(len(o) - 1 for o in outs)
    assert emitted == accepted + steps * B                        # a_r + 1 tokens per step
    assert 0 < accepted <= drafted <= steps * B * g
    say("tokens", emitted, "accepted", accepted, "drafted", drafted)


def test_decode_loop_graph_replays_match_eager():
    """Three steps captured in one HIP graph, replayed with host work in between; every
    replay's outputs equal the eager run's and the target chain."""
    W, E, nxt, gap, dnext, dconf = toy(seed=3)
    Wd, Ed, dn, dc = to_dev(W, E, dnext, dconf)
    B, g, reps = 6, 5, 5
    start = torch.from_numpy(np.random.default_rng(2).integers(0, V, B)).cuda()
    eager = ToyDecodeLoop(Wd, Ed, dn, dc, B, g, 3 * reps)
    want = run_loop(eager, start, 3 * reps)
    check_chain(want, start.cpu().numpy(), nxt, gap)
    loop = ToyDecodeLoop(Wd, Ed, dn, dc, B, g, 3 * reps)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):                                    # warm-up outside capture
        loop.reset(start)
        for i in range(3):
            loop.step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for i in range(3):
            loop.step(i)
    for attempt in range(2):
        with torch.cuda.stream(s):
            loop.reset(start)
        torch.cuda.synchronize()
        for rep in range(reps):
            graph.replay()
            torch.cuda.synchronize()
            got = loop.tokens()                                   # host work between replays
            n = 3 * (rep + 1)
            ref = ToyDecodeLoop(Wd, Ed, dn, dc, B, g, 3 * reps)
            assert got == run_loop(ref, start, n), f"replay {rep} of attempt {attempt}"
        assert got == want
    say("graph", f"{2 * reps} replays of 3 steps match")
