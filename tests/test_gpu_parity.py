"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case draws seeded inputs, runs truncate -> verify -> accept on the GPU
and the same round in the oracle, and compares per request (see _parity for
the bars and the exemptions). Full-size workloads that the oracle cannot
finish in seconds are checked on sampled requests, whose rows the oracle
computes exactly.
"""
import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as sd
from oracle import sd_oracle as O
from synth import make_step, make_weights, workload

from _parity import (Report, attach_inputs, bf16_dev, check_logits_rows, compare, lm_head,
                     run_gpu, run_oracle, upload_step)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    yield


def full_case(w, steps, seed=0, check_all_logits=True, named=False):
    """Oracle over whole batches: every request and every logit compared. On the named
    workloads (named=True) no exemption may be used: every accepted length, token and
    argmax equals the oracle's."""
    W = make_weights(w, seed)
    W64 = O.lm_head_f64(W)
    W_dev = bf16_dev(W)
    vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold)
    rep = Report()
    for st in steps:
        say(w.name, f"B={w.B} g={w.gamma} d={w.d} V={w.V} T={w.T} step={st} seed={seed}")
        s = make_step(w, W, st, seed)
        g = run_gpu(w, W_dev, upload_step(s), vr, fetch_all_logits=check_all_logits and w.T > 0)
        o = attach_inputs(run_oracle(w, W64, s), s)
        assert g.flags == 0, f"device flags {g.flags}"
        compare(w, g, o, range(w.B), rep)
        if g.logits is not None:
            check_logits_rows(w, g.logits, o.z, rep)
        assert np.array_equal(g.counters, o.accept.counters)
    say("report", rep)
    if named:
        assert rep.exempt == 0, rep
    return rep


# ---------------------------------------------------------------- small shapes

SHAPES = [
    # (name, B, gamma, d, V, T, truncate): skinny 16/32/64-row tiles (direct-to-LDS
    # when d % 128 == 0, register-staged otherwise), LDS-tiled path, a K tail
    # (d % 32 != 0), vocabulary tails (V % 64 != 0, V % 8 != 0).
    ("skinny16-greedy", 1, 4, 256, 1000, 0.0, False),
    ("skinny32-dma-rej", 1, 20, 384, 2000, 1.0, False),
    ("skinny64-dma-trunc", 3, 16, 512, 3001, 0.8, True),
    ("skinny16-rej", 2, 5, 40, 1001, 1.0, False),
    ("skinny32-rej", 1, 16, 264, 3000, 0.7, False),
    ("skinny64-trunc", 3, 16, 128, 777, 1.3, True),
    ("tiled-greedy", 9, 9, 512, 2050, 0.0, False),
    ("tiled-d96-trunc", 20, 8, 96, 3000, 0.9, True),
    ("tiled-d32-one-stage", 8, 16, 32, 777, 1.0, False),
    ("tiled-trunc-rej", 40, 16, 200, 5000, 1.0, True),
    ("gamma64", 2, 64, 64, 300, 1.0, False),
    ("many-requests", 300, 3, 64, 129, 0.0, True),
    # Degenerate sizes: one vocabulary id, the smallest hidden size, one drafted token.
    ("edge-d8-V1-rej", 1, 1, 8, 1, 1.0, False),
    ("edge-gamma1-V5-greedy", 2, 1, 16, 5, 0.0, False),
    ("edge-d8-V64-trunc", 4, 3, 8, 64, 0.7, True),
    # More vocabulary tiles than the chip holds at once (a second, partial round).
    ("tiled-two-rounds-rej", 5, 16, 64, 70000, 1.0, True),
    ("tiled-two-rounds-greedy", 4, 20, 128, 69999, 0.0, False),
    # Row counts around the 256-row tile: the verified rows' 16-row tiles are dealt over
    # the row tiles (255 rows: one tile, last 16-row tile partial; 513: three tiles of
    # 11/11/11 16-row tiles; 775: four tiles of 13/12/12/12).
    ("tiled-rows-255", 15, 16, 128, 3000, 1.0, False),
    ("tiled-rows-513", 27, 18, 64, 2000, 0.0, False),
    ("tiled-rows-775", 25, 30, 64, 1500, 0.9, False),
    # More partial columns per row (547 vocabulary tiles of 128) than the rejection
    # decision holds in registers (512): its second loop over the partials.
    ("tiled-d96-547-tiles-rej", 5, 16, 96, 70000, 1.0, True),
    # Vocabularies of 256 and 269 chunks of 4096: the largest one-launch draw, and the
    # first one that falls back to two launches.
    ("vocab-256-chunks-rej", 1, 2, 8, 1048000, 1.0, False),
    ("vocab-269-chunks-rej", 1, 2, 8, 1100000, 0.8, False),
    # 64 requests x 35 chunks: more draw workgroups than the chip holds, so the one-launch
    # draw takes two chunks per workgroup.
    ("draw-2-chunks-per-group-rej", 64, 1, 64, 140000, 1.0, False),
]


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_small_shapes(case):
    name, B, g, d, V, T, trunc = case
    w = workload("ragged-b32", B=B, gamma=g, d=d, V=V, T=T, truncate=trunc,
                 geo_p=(0.2,), name=name)
    full_case(w, steps=range(3))


def test_stress_long_prefixes():
    """Planting 12 along the drafted row: long accepted prefixes exercise late positions."""
    w = workload("rejection-b1", V=20000, d=512, plant=12.0, name="stress-rej")
    rep = full_case(w, steps=range(6))
    assert rep.accepted >= 6 * 4
    w = workload("greedy-block9", V=20000, d=512, plant=12.0, geo_p=(0.05,), name="stress-greedy")
    rep = full_case(w, steps=range(20))
    assert rep.accepted >= 20 * 5


def test_truncation_edge_thresholds():
    """Threshold above every confidence (only bonus rows) and at zero (all kept)."""
    for thr in (1.5, 0.0):
        w = workload("ragged-b32", V=4096, d=256, threshold=thr, name=f"thr{thr}")
        full_case(w, steps=range(2))


@pytest.mark.parametrize("case", [("rows-past-grid-y-rej", 4200, 16, 64, 300, 1.0, True),
                                  ("rows-past-grid-y-greedy", 4200, 16, 64, 300, 0.0, False)],
                         ids=["rej-trunc", "greedy"])
def test_rows_beyond_one_grid_dimension(case):
    """4200 requests x 17 rows (71400 > 65535): the kernels whose grid y is capped at
    65535 stride over the remaining rows."""
    name, B, g, d, V, T, trunc = case
    w = workload("ragged-b32", B=B, gamma=g, d=d, V=V, T=T, truncate=trunc,
                 geo_p=(0.2,), name=name)
    rep = full_case(w, steps=range(1))
    assert rep.requests == B


# ----------------------------------------------------------- named workloads

def test_workload_tiny_greedy_all_steps():
    w = workload("tiny-greedy")
    rep = full_case(w, steps=range(w.steps), named=True)
    assert rep.requests == 1000


def test_workload_greedy_block9():
    w = workload("greedy-block9")
    rep = full_case(w, steps=range(w.steps), named=True)
    assert rep.requests == w.steps


def test_workload_rejection_b1():
    w = workload("rejection-b1")
    full_case(w, steps=range(10), named=True)


def test_workload_ragged_b32():
    w = workload("ragged-b32")
    full_case(w, steps=range(4), named=True)


def test_workload_concurrency_b128():
    """Full size (W 1.85 GB): every request of two steps, every logit row, the row
    statistics and the batch counters against the oracle."""
    w = workload("concurrency-b128")
    W, W64, W_dev = lm_head(w)
    vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold)
    rep = Report()
    for st in range(2):
        say(w.name, f"B={w.B} g={w.gamma} d={w.d} V={w.V} T={w.T} step={st} whole batch")
        s = make_step(w, W, st)
        g = run_gpu(w, W_dev, upload_step(s), vr, fetch_all_logits=True)
        assert g.flags == 0, f"device flags {g.flags}"
        o = attach_inputs(run_oracle(w, W64, s), s)
        compare(w, g, o, range(w.B), rep)
        check_logits_rows(w, g.logits, o.z, rep)
        assert np.array_equal(g.counters, o.accept.counters)
        del g, o
    say("report", rep)
    assert rep.requests == 2 * w.B
    assert rep.exempt == 0, rep


# --------------------------------------------------------------- properties

def test_determinism_bytes():
    w = workload("ragged-b32", V=30000, d=1024, name="determinism")
    W = make_weights(w)
    W_dev = bf16_dev(W)
    ds = upload_step(make_step(w, W, 0))
    outs = []
    for _ in range(2):
        vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold)
        vr.run(ds.hidden, W_dev, ds.draft_tokens, ds.conf, ds.draft_logits, ds.u_accept,
               ds.u_resample)
        torch.cuda.synchronize()
        M = int(vr.row_offsets[-1].item())
        outs.append([t.clone() for t in (vr.stats[:M], vr.logits[:M], vr.accept_len,
                                         vr.next_token, vr.row_offsets)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("case", [
    ("greedy-block9", {}),
    ("fused-trunc-skinny", dict(B=3, gamma=16, d=256, V=3001, truncate=True)),
    ("fused-tiled", dict(B=20, gamma=8, d=128, V=5000, truncate=True)),
    ("fused-gamma64", dict(B=2, gamma=64, d=64, V=700)),
    ("fused-many", dict(B=300, gamma=3, d=64, V=129, truncate=True)),
    # Streaming contractions of at most 16 requests of at most 12 rows, whose grid leaves
    # a compute unit per request, decide inside the contraction's launch (workgroups
    # appended to its grid merge published partials); greedy-block9 (512 workgroups) and
    # the last three take the separate launch.
    ("tail-tiny", dict(B=1, gamma=4, d=256, V=1024)),
    ("tail-32-trunc", dict(B=2, gamma=9, d=384, V=2048, truncate=True)),
    ("tail-blocked", dict(B=2, gamma=7, d=256, V=1500, blocked=True)),
    ("tail-33-slabs", dict(B=1, gamma=9, d=256, V=2049)),
    ("tail-16-requests", dict(B=16, gamma=3, d=256, V=5000, truncate=True)),
    ("tail-12-rows-188-slabs", dict(B=4, gamma=11, d=128, V=12000)),
    ("tail-13-rows-separate", dict(B=4, gamma=12, d=128, V=7000)),
    ("tail-17-requests-separate", dict(B=17, gamma=2, d=128, V=7000)),
    ("tail-512-grid-separate", dict(B=4, gamma=11, d=128, V=70000)),
], ids=lambda c: c[0])
def test_fused_greedy_matches_separate_calls(case):
    """sd_verify_greedy writes the same bytes as sd_verify_logits + sd_accept_greedy."""
    name, over = case
    over = dict(over)
    blocked = over.pop("blocked", False)
    base = "greedy-block9" if name == "greedy-block9" else "ragged-b32"
    over = dict(over, T=0.0, name=name) if name != "greedy-block9" else dict(name=name)
    w = workload(base, **over)
    W = make_weights(w)
    W_dev = bf16_dev(W)
    if blocked:
        W_dev = sd.BlockedWeights(W_dev)
    for step in range(2):
        ds = upload_step(make_step(w, W, step))
        outs = []
        for fused in (True, False):
            vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, 0.0, w.truncate, w.threshold, fused=fused)
            vr.counters.zero_()
            vr.run(ds.hidden, W_dev, ds.draft_tokens, ds.conf)
            torch.cuda.synchronize()
            M = int(vr.row_offsets[-1].item()) if w.truncate else w.B * (w.gamma + 1)
            outs.append([t.clone() for t in (vr.stats[:M], vr.accept_len, vr.next_token,
                                             vr.counters)])
            assert sd.device_flags(vr.ws_verify) == 0
        for a, b in zip(*outs):
            assert torch.equal(a, b)


def test_in_launch_decision_across_shapes_on_one_workspace():
    """One verify workspace serves greedy calls of changing shapes (grids of 16 to 512
    workgroups, 4 to 64 rows, truncated and not, deciding in the launch or not), with
    sd_verify_logits calls on it in between. The in-launch decision relies on the
    workspace's publication area being empty whenever a launch starts on it, so every
    call must equal the two-call path."""
    shapes = [dict(B=1, gamma=9, d=256, V=14000), dict(B=3, gamma=5, d=128, V=3001, truncate=True),
              dict(B=16, gamma=3, d=256, V=1000), dict(B=1, gamma=11, d=128, V=16000, truncate=True),
              dict(B=1, gamma=4, d=256, V=1024), dict(B=1, gamma=9, d=256, V=32768)]
    ws = sd.new_workspace(max(sd.verify_workspace_bytes(sh["B"], sh["gamma"], sh["d"], sh["V"])
                              for sh in shapes), "cuda")
    heads = {}
    for i, k in enumerate([0, 1, 2, 0, 3, 5, 1, 4, 0, 2, 5, 3, 3, 4, 0]):
        w = workload("ragged-b32", T=0.0, name=f"seq{k}", **shapes[k])
        if k not in heads:
            W = make_weights(w)
            heads[k] = (W, bf16_dev(W))
        W, W_dev = heads[k]
        say("sequence", i, shapes[k])
        ds = upload_step(make_step(w, W, i))
        vlen = offs = None
        if w.truncate:
            vlen, offs = sd.sd_truncate_by_confidence(ds.conf, w.threshold)
        M = int(offs[-1].item()) if w.truncate else w.B * (w.gamma + 1)
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        st_f, acc_f, nxt_f = sd.sd_verify_greedy(ds.hidden, W_dev, ds.draft_tokens, vlen, offs,
                                                 counters=cnt, workspace=ws)
        _, st_s = sd.sd_verify_logits(ds.hidden, W_dev, ds.draft_tokens, vlen, offs, 0.0)
        cnt_s = torch.zeros(2, dtype=torch.int64, device="cuda")
        acc_s, nxt_s = sd.sd_accept_greedy(st_s, ds.draft_tokens, vlen, offs, counters=cnt_s)
        if i % 3 == 2:
            # A plain verify on the shared workspace: row partials, not the publication area.
            sd.sd_verify_logits(ds.hidden, W_dev, ds.draft_tokens, vlen, offs, 0.0, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(st_f[:M], st_s[:M])
        assert torch.equal(acc_f, acc_s) and torch.equal(nxt_f, nxt_s)
        assert torch.equal(cnt, cnt_s)
    assert sd.device_flags(ws) == 0


REJ_FUSED = [
    # Streaming contraction with idle workgroup slots (the drafter rows are normalised in
    # its launch), without them (65536 ids: 1024 slabs, the grid fills every slot, so a
    # separate drafter launch runs), the register-staged streaming kernel (d % 128 != 0:
    # the drafted-token logits come from the drafter launch too), the tiled kernel,
    # gamma = 64 (three passes of row slots), many small requests, and the blocked head.
    ("rej-skinny-appended", dict(B=1, gamma=16, d=512, V=20000, truncate=False)),
    ("rej-skinny-full-grid", dict(B=1, gamma=9, d=256, V=65536, truncate=False)),
    ("rej-stream-d200", dict(B=2, gamma=12, d=200, V=5001, truncate=True)),
    ("rej-tiled", dict(B=20, gamma=16, d=256, V=7000, truncate=True)),
    ("rej-gamma64", dict(B=2, gamma=64, d=64, V=4099, truncate=False)),
    ("rej-many", dict(B=300, gamma=3, d=64, V=129, truncate=True)),
    ("rej-blocked", dict(B=3, gamma=16, d=256, V=9000, truncate=True, blocked=True)),
    # The W12 stream (decoded in the streaming contraction), with appended drafter
    # workgroups and on a full grid.
    ("rej-w12", dict(B=3, gamma=16, d=256, V=9000, truncate=True, w12=True)),
    ("rej-w12-full-grid", dict(B=1, gamma=9, d=256, V=65536, truncate=False, w12=True)),
    # A one-launch draw with two chunks per workgroup (64 requests x 35 chunks).
    ("rej-draw-2-chunks-per-group", dict(B=64, gamma=1, d=64, V=140000, truncate=False)),
]


@pytest.mark.parametrize("case", REJ_FUSED, ids=lambda c: c[0])
def test_fused_rejection_matches_separate_calls(case):
    """sd_verify_rejection against sd_verify_logits + sd_accept_rejection_ex: logits,
    argmax, top-1/top-2, drafted-token logits, accepted lengths, tokens, counters,
    acceptance rates and flags equal; the log-normalisers (summed in another order) to
    fp64 rounding."""
    name, over = case
    over = dict(over)
    blocked = over.pop("blocked", False)
    w12 = over.pop("w12", False)
    w = workload("ragged-b32", T=0.9, geo_p=(0.2,), name=name, **over)
    W = make_weights(w)
    W_dev = bf16_dev(W)
    if blocked:
        W_dev = sd.BlockedWeights(W_dev)
    if w12:
        W_dev = sd.W12Weights.from_bf16(W)
    for step in range(2):
        say(name, f"B={w.B} g={w.gamma} d={w.d} V={w.V} T={w.T} step={step}")
        ds = upload_step(make_step(w, W, step))
        outs = []
        # The fused call without rates (small grids draw in one launch), with rates (two
        # draw launches), then the separate calls with rates.
        for fused, rate in ((True, False), (True, True), (False, True)):
            vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold,
                                fused=fused, accept_rate=rate)
            vr.counters.zero_()
            vr.run(ds.hidden, W_dev, ds.draft_tokens, ds.conf, ds.draft_logits, ds.u_accept,
                   ds.u_resample)
            torch.cuda.synchronize()
            M = int(vr.row_offsets[-1].item()) if w.truncate else w.B * (w.gamma + 1)
            st = sd.stats_to_numpy(vr.stats)[:M]
            lse_q = (vr.ws_accept[256:256 + 8 * w.B * w.gamma].cpu().numpy().view(np.float64)
                     .reshape(w.B, w.gamma))
            outs.append(dict(st=st, logits=vr.logits[:M].clone(), acc=vr.accept_len.clone(),
                             nxt=vr.next_token.clone(), cnt=vr.counters.clone(),
                             rate=None if vr.accept_rate is None else vr.accept_rate.clone(),
                             lse_q=lse_q,
                             vlen=None if vr.verify_len is None else vr.verify_len.clone(),
                             flags=sd.device_flags(vr.ws_verify) | sd.device_flags(vr.ws_accept)))
        s = outs[2]
        for f in outs[:2]:
            assert f["flags"] == 0 and s["flags"] == 0
            assert torch.equal(f["logits"], s["logits"])
            for k in ("argmax", "top1", "top2", "pos", "z_draft"):
                assert np.array_equal(f["st"][k], s["st"][k]), k
            assert np.allclose(f["st"]["lse"], s["st"]["lse"], rtol=1e-13, atol=1e-13)
            L = (f["vlen"].cpu().numpy() if f["vlen"] is not None
                 else np.full(w.B, w.gamma))
            kept = np.arange(w.gamma)[None, :] < L[:, None]
            assert np.allclose(f["lse_q"][kept], s["lse_q"][kept], rtol=1e-13, atol=1e-13)
            for k in ("acc", "nxt", "cnt"):
                assert torch.equal(f[k], s[k]), k
        assert torch.allclose(outs[1]["rate"], s["rate"], rtol=0, atol=1e-12)


def test_rejection_lossless_on_gpu():
    """Bigram target and drafter over V = 8: emitted first tokens follow the target."""
    from scipy import special, stats as sstats
    rng = np.random.default_rng(77)
    V, g, B = 8, 3, 40000
    Zt = rng.standard_normal((V, V)).astype(np.float32)
    Zd = rng.standard_normal((V, V)).astype(np.float32)
    from synth import bf16_round, bf16_to_f32
    Zt = bf16_to_f32(bf16_round(Zt)).astype(np.float64)
    Zd = bf16_to_f32(bf16_round(Zd)).astype(np.float64)
    qt = special.softmax(Zd, axis=1)
    x = np.zeros((B, g), np.int32)
    prev = np.zeros(B, np.int64)
    for j in range(g):
        cdf = np.cumsum(qt[prev], axis=1)
        x[:, j] = np.minimum((rng.random((B, 1)) > cdf).sum(1), V - 1)
        prev = x[:, j]
    prevs = np.concatenate([np.zeros((B, 1), np.int64), x], axis=1)
    hidden = bf16_round(Zt[prevs].astype(np.float32))
    dl = bf16_round(Zd[prevs[:, :g]].astype(np.float32))
    W = bf16_round(np.eye(V, dtype=np.float32))
    say("lossless-gpu", f"B={B} V={V}")
    vr = sd.VerifyRound(B, g, V, V, 1.0, False)
    vr.run(bf16_dev(hidden), bf16_dev(W), torch.from_numpy(x).cuda(), None, bf16_dev(dl),
           torch.from_numpy(rng.random((B, g)).astype(np.float32)).cuda(),
           torch.from_numpy(rng.random((B, g + 1)).astype(np.float32)).cuda())
    torch.cuda.synchronize()
    a = vr.accept_len.cpu().numpy()
    n = vr.next_token.cpu().numpy()
    first = np.where(a > 0, x[:, 0], n)
    pt = special.softmax(Zt, axis=1)
    cnt = np.bincount(first, minlength=V)
    assert sstats.chisquare(cnt, pt[0] / pt[0].sum() * B).pvalue > 1e-3
    rate = np.mean(a >= 1)
    want = 1 - 0.5 * np.abs(pt[0] - qt[0]).sum()
    assert abs(rate - want) < 4 * np.sqrt(want * (1 - want) / B)


CROWDED = [
    # (name, B, gamma, d, V, T): every drafted token in the first 64 vocabulary ids, so
    # one LM-head slab holds up to 51 drafted rows (the skinny contraction forms the
    # first four logits itself and leaves the rest to the merge).
    ("crowded-greedy", 1, 16, 256, 3000, 0.0),
    ("crowded-rej", 3, 16, 512, 3001, 1.0),
    ("crowded-trunc", 2, 20, 384, 2000, 0.8),
]


@pytest.mark.parametrize("case", CROWDED, ids=[c[0] for c in CROWDED])
def test_drafted_tokens_crowding_one_slab(case):
    name, B, g, d, V, T = case
    w = workload("ragged-b32", B=B, gamma=g, d=d, V=V, T=T, truncate=name.endswith("trunc"),
                 geo_p=(0.2,), name=name)
    W = make_weights(w)
    W64 = O.lm_head_f64(W)
    W_dev = bf16_dev(W)
    rng = np.random.default_rng(7)
    rep = Report()
    for fused in (True, False):
        vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold, fused=fused)
        for st in range(2):
            say(name, f"B={B} g={g} d={d} V={V} T={T} step={st} fused={fused}")
            s = make_step(w, W, st)
            s.draft_tokens = rng.integers(0, 64, s.draft_tokens.shape).astype(np.int32)
            g_res = run_gpu(w, W_dev, upload_step(s), vr, fetch_all_logits=w.T > 0)
            o = attach_inputs(run_oracle(w, W64, s), s)
            assert g_res.flags == 0
            compare(w, g_res, o, range(w.B), rep)
            assert np.array_equal(g_res.counters, o.accept.counters)
    say("report", rep)


RATE_CASES = [
    # (name, B, gamma, d, V, T, truncate, steps): chunk tails (V % 4096 != 0, V % 4 != 0),
    # ragged rows, gamma = 64, and the full-size single-request rejection shape.
    ("rate-small", 2, 5, 64, 1001, 1.0, False, 2),
    ("rate-ragged", 12, 16, 128, 9000, 0.8, True, 2),
    ("rate-gamma64", 2, 64, 64, 4099, 1.3, False, 1),
    ("rate-rejection-b1", None, None, None, None, None, None, 2),
    # B + B * gamma = 71400 draw-kernel rows: grid y (capped at 65535) strides over them.
    ("rate-rows-past-grid-y", 4200, 16, 64, 300, 1.0, True, 1),
]


@pytest.mark.parametrize("case", RATE_CASES, ids=[c[0] for c in RATE_CASES])
def test_acceptance_rate_matches_oracle(case):
    """sd_accept_rejection_ex: 1 - TV(p_j, q_j) per verified position, abs 1e-4 against
    the oracle; -1 past L_r; acceptance outputs byte-identical to sd_accept_rejection."""
    name, B, g, d, V, T, trunc, steps = case
    if B is None:
        w = workload("rejection-b1")
    else:
        w = workload("ragged-b32", B=B, gamma=g, d=d, V=V, T=T, truncate=trunc,
                     geo_p=(0.2,), name=name)
    W = make_weights(w)
    W64 = O.lm_head_f64(W)
    W_dev = bf16_dev(W)
    vr_ex = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold,
                           accept_rate=True)
    vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold)
    worst = 0.0
    for st in range(steps):
        say(name, f"B={w.B} g={w.gamma} d={w.d} V={w.V} T={w.T} step={st}")
        s = make_step(w, W, st)
        ds = upload_step(s)
        g_ex = run_gpu(w, W_dev, ds, vr_ex)
        g_pl = run_gpu(w, W_dev, ds, vr)
        assert g_ex.flags == 0
        assert np.array_equal(g_ex.accept_len, g_pl.accept_len)
        assert np.array_equal(g_ex.next_token, g_pl.next_token)
        assert np.array_equal(g_ex.counters, g_pl.counters)
        rate_g = vr_ex.accept_rate.cpu().numpy()
        o = run_oracle(w, W64, s)
        rate_o = O.acceptance_rate(o.z, s.draft_logits, o.verify_len, o.row_offsets, w.T,
                                   o.stats.lse)
        live = rate_o >= 0
        assert np.array_equal(rate_g < 0, ~live)
        assert np.all(rate_g[~live] == -1.0)
        err = float(np.max(np.abs(rate_g[live] - rate_o[live]))) if live.any() else 0.0
        worst = max(worst, err)
        assert err < 1e-4, f"acceptance rate error {err}"
    say("report", f"max |rate err| {worst:.3g}")


def test_out_of_range_lengths_are_clamped_and_flagged():
    w = workload("ragged-b32", B=4, V=2048, d=128, truncate=False, T=0.0, name="clamp")
    W = make_weights(w)
    s = make_step(w, W, 0)
    bad = np.array([99, -3, 5, 16], np.int32)
    L = np.clip(bad, 0, w.gamma)
    offs = np.concatenate([[0], np.cumsum(L + 1)]).astype(np.int32)
    ds = upload_step(s)
    say("clamp", bad.tolist())
    vlen_d = torch.from_numpy(bad).cuda()
    offs_d = torch.from_numpy(offs).cuda()
    ws = sd.new_workspace(sd.verify_workspace_bytes(w.B, w.gamma, w.d, w.V), "cuda")
    _, st = sd.sd_verify_logits(ds.hidden, bf16_dev(W), ds.draft_tokens, vlen_d, offs_d, 0.0,
                                workspace=ws)
    acc, nxt = sd.sd_accept_greedy(st, ds.draft_tokens, vlen_d, offs_d)
    torch.cuda.synchronize()
    assert sd.device_flags(ws) & sd.FLAG_VERIFY_LEN
    z = O.verify_logits(s.hidden, W, L)
    o = O.accept_greedy(np.argmax(z, axis=1), s.draft_tokens, L, offs)
    assert np.array_equal(acc.cpu().numpy(), o.accept_len)
    assert np.array_equal(nxt.cpu().numpy(), o.next_token)
