"""The allocation-free greedy verify (sd_verify_greedy_noalloc) against the
workspace-taking sd_verify_greedy, through the C ABI.

Two calls in a row share the library's per-GPU scratch; the second, smaller one must
not see anything the first left there. Every output byte (row statistics, accepted
lengths, tokens, counters) equals the workspace call's, and the flag word is clear.
"""
import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as sd
from synth import make_step, make_weights, workload

from _parity import bf16_dev, upload_step

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def run_both(w, step, truncate):
    W = make_weights(w)
    W_dev = bf16_dev(W)
    s = make_step(w, W, step)
    ds = upload_step(s)
    dev = ds.hidden.device
    vlen = offs = None
    if truncate:
        vlen, offs = sd.sd_truncate_by_confidence(ds.conf, w.threshold)
    M = w.B * (w.gamma + 1)
    ref_counters = torch.zeros(2, dtype=torch.int64, device=dev)
    ref = sd.sd_verify_greedy(ds.hidden, W_dev, ds.draft_tokens, vlen, offs, counters=ref_counters)
    got_stats = sd.new_stats(w.B, w.gamma, dev)
    got_acc = torch.full((w.B,), -7, dtype=torch.int32, device=dev)
    got_nxt = torch.full((w.B,), -7, dtype=torch.int32, device=dev)
    got_counters = torch.zeros(2, dtype=torch.int64, device=dev)
    flags = torch.full((1,), -1, dtype=torch.int32, device=dev)
    sd.sd_verify_greedy_noalloc(ds.hidden, W_dev, ds.draft_tokens, vlen, offs, got_stats, got_acc,
                                got_nxt, got_counters, flags)
    torch.cuda.synchronize()
    rows = int(offs[-1].item()) if truncate else M
    assert torch.equal(got_stats[:rows], ref[0][:rows])
    assert torch.equal(got_acc, ref[1])
    assert torch.equal(got_nxt, ref[2])
    assert torch.equal(got_counters, ref_counters)
    assert int(flags.item()) == 0
    return got_acc.cpu().numpy()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    yield


def test_noalloc_matches_workspace_call_twice_shrinking():
    # Calls in a row, each smaller than the one before: a tiled-regime problem (24
    # truncated requests), the greedy block of 9 at full size for 4 requests, a small
    # truncating one, then two tiny ones whose contractions also decide (workgroups
    # appended to their 16- and 8-workgroup grids merge partials published in the
    # scratch's publication area, which each call must leave empty for the next).
    # Partials and drafted-token logits of earlier calls remain in the scratch and must
    # not leak into later ones.
    tiled = workload("ragged-b32", B=24, gamma=16, d=256, V=20000, T=0.0, name="noalloc-tiled")
    big = workload("greedy-block9", B=4, name="noalloc-big")
    small = workload("ragged-b32", B=3, gamma=16, d=512, V=3001, T=0.0, name="noalloc-small")
    tiny = workload("ragged-b32", B=2, gamma=4, d=256, V=1024, T=0.0, name="noalloc-tiny")
    tinier = workload("ragged-b32", B=1, gamma=4, d=256, V=512, T=0.0, name="noalloc-tinier")
    ws = (tiled, big, small, tiny, tinier)
    sizes = [sd.verify_workspace_bytes(w.B, w.gamma, w.d, w.V) for w in ws]
    assert all(a > b for a, b in zip(sizes, sizes[1:])) and sizes[0] <= sd.NOALLOC_SCRATCH_BYTES
    for w, trunc in ((tiled, True), (big, False), (small, True), (tiny, True), (tinier, False)):
        say(w.name, f"B={w.B} g={w.gamma} d={w.d} V={w.V} truncate={trunc}")
        acc = run_both(w, 0, trunc)
        say("accept_len", acc.tolist())


def test_noalloc_flags_report_bad_lengths():
    # Out-of-range kept lengths are clamped and flagged in this call's flag word only.
    w = workload("ragged-b32", B=4, gamma=16, d=128, V=2048, T=0.0, name="noalloc-flags")
    W = make_weights(w)
    s = make_step(w, W, 0)
    ds = upload_step(s)
    dev = ds.hidden.device
    bad = torch.tensor([99, -3, 5, 16], dtype=torch.int32, device=dev)
    L = bad.clamp(0, w.gamma)
    offs = torch.cat([torch.zeros(1, dtype=torch.int32, device=dev),
                      torch.cumsum(L + 1, 0).to(torch.int32)])
    stats = sd.new_stats(w.B, w.gamma, dev)
    acc = torch.empty(w.B, dtype=torch.int32, device=dev)
    nxt = torch.empty(w.B, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    say("noalloc-flags", bad.tolist())
    sd.sd_verify_greedy_noalloc(ds.hidden, bf16_dev(W), ds.draft_tokens, bad, offs, stats, acc,
                                nxt, None, flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & sd.FLAG_VERIFY_LEN
    # The next call starts from a clear header.
    good = L
    sd.sd_verify_greedy_noalloc(ds.hidden, bf16_dev(W), ds.draft_tokens, good, offs, stats, acc,
                                nxt, None, flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
