"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to a fact fixed by the pages or by the
mathematics: exact integer arithmetic, closed forms, brute force, the
DSpark decode-round worked example, the greedy-equals-target property, the
1 - TV acceptance-rate identity and losslessness of rejection sampling.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

from oracle import sd_oracle as O
from synth import bf16_round, bf16_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------- bf16 decoding

def test_bf16_decode_known_patterns():
    # bf16 = sign | 8-bit exponent (bias 127) | 7-bit fraction.
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x7F7F, 0x8000, 0x3F81], dtype=np.uint16)
    want = [1.0, -2.0, 3.140625, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0, 1 + 2 ** -7]
    got = O.bf16_decode(bits)
    assert list(got) == want
    assert np.signbit(got[5])


def test_bf16_round_is_nearest_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even (1.0).
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert list(O.bf16_decode(bf16_round(x))) == [1.0, 1 + 2 * 2 ** -7, 1 + 2 ** -7]


# ------------------------------------------------------------------ logits

def _int_bf16(rng, shape, lo=-16, hi=17):
    """Small integers are exact in bf16, so fp64 dot products of them are exact."""
    return bf16_round(rng.integers(lo, hi, size=shape).astype(np.float32))


def test_logits_exact_integer_arithmetic_and_row_packing():
    rng = np.random.default_rng(7)
    B, g, d, V = 3, 4, 12, 9
    hidden = _int_bf16(rng, (B, g + 1, d))
    W = _int_bf16(rng, (V, d))
    verify_len = np.array([4, 0, 2], dtype=np.int32)
    z = O.verify_logits(hidden, W, verify_len)
    hi = bf16_to_f32(hidden).astype(np.int64)
    wi = bf16_to_f32(W).astype(np.int64)
    want = []
    for r in range(B):
        for j in range(int(verify_len[r]) + 1):
            want.append([sum(int(hi[r, j, k]) * int(wi[v, k]) for k in range(d)) for v in range(V)])
    assert z.shape == (int(np.sum(verify_len + 1)), V)
    assert np.array_equal(z, np.array(want, dtype=np.float64))


def test_logits_single_row_matches_packed():
    rng = np.random.default_rng(3)
    hidden = bf16_round(rng.standard_normal((2, 3, 16)).astype(np.float32))
    W = bf16_round(rng.standard_normal((10, 16)).astype(np.float32))
    z = O.verify_logits(hidden, W, np.array([2, 2], dtype=np.int32))
    assert np.allclose(O.logits_at(hidden, W, 1, 1), z[4], rtol=0, atol=1e-12)


# --------------------------------------------------------------- row stats

def test_argmax_ties_lowest_and_top2():
    z = np.array([[3.0, 5.0, 5.0, 1.0], [2.0, 2.0, 2.0, 2.0], [-1.0, 7.0, 0.5, 6.0]])
    st = O.row_stats(z, 0.0)
    assert list(st.argmax) == [1, 0, 1]
    assert list(st.top1) == [5.0, 2.0, 7.0]
    assert list(st.top2) == [5.0, 2.0, 6.0]


def test_lse_closed_forms():
    V, c, T = 1000, 0.37, 0.8
    st = O.row_stats(np.full((1, V), c), T)
    assert abs(st.lse[0] - (c / T + np.log(V))) < 1e-12
    a, b = 2.0, -1.5
    st = O.row_stats(np.array([[a, b]]), 1.0)
    assert abs(st.lse[0] - np.log(np.exp(a) + np.exp(b))) < 1e-12
    # Large logits: the max is taken out, so no overflow.
    st = O.row_stats(np.array([[1000.0, 1000.0]]), 1.0)
    assert abs(st.lse[0] - (1000.0 + np.log(2.0))) < 1e-9
    z = np.random.default_rng(1).standard_normal((4, 300)) * 3
    st = O.row_stats(z, 1.3)
    assert np.allclose(st.lse, special.logsumexp(z / 1.3, axis=1), atol=1e-12)
    p = np.exp(z / 1.3 - st.lse[:, None])
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)


# --------------------------------------------------------------- truncation

def test_decode_round_worked_example():
    gold = json.load(open(os.path.join(GOLDEN, "dspark_decode_round.json")))
    V = len(gold["vocab"])
    conf = np.array(gold["conf"], dtype=np.float32)
    x = np.array(gold["draft_tokens"], dtype=np.int32)
    g = x.shape[1]
    W = bf16_round(np.eye(V, dtype=np.float32))
    hidden = np.zeros((1, g + 1, V), dtype=np.float32)
    for j, t in enumerate(gold["target_argmax_rows"]):
        hidden[0, j, t] = 3.0
        hidden[0, j, (t + 1) % V] = 1.0
    res = O.verify_step(bf16_round(hidden), W, x, 0.0, conf=conf, threshold=gold["threshold"])
    exp = gold["expected"]
    assert list(res.verify_len) == exp["verify_len"]
    assert list(res.row_offsets) == exp["row_offsets"]
    assert list(res.accept.accept_len) == exp["accept_len"]
    assert list(res.accept.next_token) == exp["next_token"]
    a = int(res.accept.accept_len[0])
    emitted = [gold["vocab"][t] for t in list(x[0, :a]) + [int(res.accept.next_token[0])]]
    assert emitted == exp["emitted"]
    assert list(res.accept.counters) == [3, 2]


def test_truncation_invariants():
    rng = np.random.default_rng(11)
    B, g = 200, 16
    c1 = rng.uniform(0.6, 1.0, (B, 1))
    conf = np.cumprod(np.concatenate([c1, rng.uniform(0.7, 1.0, (B, g - 1))], 1), 1).astype(np.float32)
    prev = None
    for thr in [0.0, 0.1, 0.2, 0.3, 0.5, 0.7, 0.95, 1.01]:
        L, off = O.truncate_by_confidence(conf, thr)
        assert np.all((L >= 0) & (L <= g))
        assert off[0] == 0 and np.all(np.diff(off) == L + 1)
        if prev is not None:
            assert np.all(L <= prev)           # non-increasing in the threshold
        prev = L
        # Every kept position clears the threshold, the first cut one does not.
        for r in range(B):
            assert np.all(conf[r, :L[r]] >= np.float32(thr))
            if L[r] < g:
                assert conf[r, L[r]] < np.float32(thr)
    assert np.all(O.truncate_by_confidence(conf, 0.0)[0] == g)
    assert np.all(O.truncate_by_confidence(conf, 0.3)[0] >= 1)   # c1 >= 0.6
    # A confidence equal to the threshold is kept; a non-monotone tail is still cut.
    L, _ = O.truncate_by_confidence(np.array([[0.5, 0.3, 0.2, 0.9]], np.float32), 0.3)
    assert list(L) == [2]


# ------------------------------------------------------------------ greedy

def _bigram(rng, V, scale=2.0):
    return bf16_to_f32(bf16_round((rng.standard_normal((V, V)) * scale).astype(np.float32)))


def test_greedy_speculation_equals_target_greedy_decoding():
    """LFM2.5-DSpark blog, "Quality parity": greedy speculative output is the target's."""
    rng = np.random.default_rng(5)
    V, g, n_out = 16, 4, 200
    Z = _bigram(rng, V)                        # target next-token logits given previous token
    Zd = Z + rng.standard_normal((V, V)) * 1.5  # a drafter that is often right, sometimes not
    W = bf16_round(np.eye(V, dtype=np.float32))
    # Plain autoregressive greedy decoding of the target.
    ar = [0]
    while len(ar) < n_out + 1:
        ar.append(int(np.argmax(Z[ar[-1]])))
    # Speculative greedy decoding through the oracle.
    out = [0]
    accepted_total = 0
    while len(out) < n_out + 1:
        prev = out[-1]
        x = []
        for _ in range(g):
            prev = int(np.argmax(Zd[prev]))
            x.append(prev)
        prevs = [out[-1]] + x                  # row j is conditioned on the token before x_j
        hidden = bf16_round(np.stack([Z[p] for p in prevs]).astype(np.float32))[None]
        res = O.verify_step(hidden, W, np.array([x], np.int32), 0.0)
        a = int(res.accept.accept_len[0])
        accepted_total += a
        out += x[:a] + [int(res.accept.next_token[0])]
    assert out[:n_out + 1] == ar[:n_out + 1]
    assert accepted_total > 0


def test_greedy_first_mismatch_bruteforce():
    """Accepted length is the first mismatch index, over all 27 drafts for V=3, gamma=3."""
    t = np.array([2, 0, 1, 1])                 # target argmax per row (row 3 is the bonus row)
    for code in range(27):
        x = [(code // 9) % 3, (code // 3) % 3, code % 3]
        res = O.accept_greedy(t, np.array([x], np.int32), np.array([3], np.int32),
                              np.array([0, 4], np.int32))
        a = int(res.accept_len[0])
        assert x[:a] == list(t[:a]) and (a == 3 or x[a] != t[a])
        assert int(res.next_token[0]) == t[a]


# --------------------------------------------------------------- rejection

def test_inverse_cdf_hand_cases():
    w = np.array([0.0, 0.2, 0.0, 0.3, 0.5])
    assert O.inverse_cdf(w, 0.0)[0] == 1
    assert O.inverse_cdf(w, 0.1)[0] == 1
    assert O.inverse_cdf(w, 0.2)[0] == 3       # C_1 = 0.2 is not > 0.2
    assert O.inverse_cdf(w, 0.49)[0] == 3
    assert O.inverse_cdf(w, 0.5)[0] == 4
    assert O.inverse_cdf(w, 0.999)[0] == 4
    assert O.inverse_cdf(w * 7.0, 0.3)[0] == 3  # scale-free
    assert O.inverse_cdf(np.array([0.0, 0.4, 0.6, 0.0]), 1.0)[0] == 2   # fallback


def _softmax_rows(logits):
    return special.softmax(np.asarray(logits, dtype=np.float64), axis=-1)


def _chi2_p(counts, probs):
    """Goodness-of-fit p-value of counts against probabilities (renormalised in fp64)."""
    probs = np.asarray(probs, dtype=np.float64)
    return stats.chisquare(counts, probs / probs.sum() * counts.sum()).pvalue


def _tiny_rejection_case(rng, V, g, B, T=1.0, target=None, drafter=None):
    """Bigram target/drafter; drafts are sampled from the drafter's own distribution."""
    Zt = target if target is not None else _bigram(rng, V, 1.0)
    Zd = drafter if drafter is not None else _bigram(rng, V, 1.0)
    qt = _softmax_rows(Zd / T)
    x = np.zeros((B, g), np.int32)
    prev = np.zeros(B, np.int64)
    for j in range(g):
        cdf = np.cumsum(qt[prev], axis=1)
        x[:, j] = np.minimum((rng.random((B, 1)) > cdf).sum(1), V - 1)
        prev = x[:, j]
    prevs = np.concatenate([np.zeros((B, 1), np.int64), x], axis=1)
    hidden = bf16_round(Zt[prevs].astype(np.float32))
    dl = bf16_round(Zd[prevs[:, :g]].astype(np.float32))
    ua = rng.random((B, g)).astype(np.float32)
    ur = rng.random((B, g + 1)).astype(np.float32)
    return Zt, Zd, x, hidden, dl, ua, ur


def test_acceptance_rate_is_one_minus_tv():
    """DSpark summary, "Confidence head" / "Training": per-step acceptance = 1 - TV(p, q)."""
    rng = np.random.default_rng(21)
    V, T = 6, 1.0
    zt = bf16_to_f32(bf16_round(rng.standard_normal(V).astype(np.float32)))
    zd = bf16_to_f32(bf16_round(rng.standard_normal(V).astype(np.float32)))
    p, q = _softmax_rows(zt / T), _softmax_rows(zd / T)
    W = bf16_round(np.eye(V, dtype=np.float32))
    N = 2000
    acc_rate = 0.0
    for x in range(V):
        u = ((np.arange(N) + 0.5) / N).astype(np.float32)[:, None]
        hidden = np.broadcast_to(bf16_round(np.stack([zt, zt]).astype(np.float32)), (N, 2, V))
        dl = np.broadcast_to(bf16_round(zd.astype(np.float32))[None, None], (N, 1, V))
        res = O.verify_step(np.ascontiguousarray(hidden), W, np.full((N, 1), x, np.int32), T,
                            draft_logit_bits=np.ascontiguousarray(dl), u_accept=u,
                            u_resample=np.zeros((N, 2), np.float32))
        acc_rate += q[x] * res.accept.accept_len.mean()
    assert abs(acc_rate - (1 - 0.5 * np.abs(p - q).sum())) < 2.0 / N


def test_acceptance_rate_function_matches_integrated_acceptance():
    """acceptance_rate against the rejection rule itself, integrated exactly over u and x.

    For x ~ q the rule keeps x with probability min(1, p(x)/q(x)); summing q(x) times
    that over every x is the acceptance rate. The ratios come from accept_rejection's
    diagnostics, a separate route through the oracle.
    """
    rng = np.random.default_rng(31)
    V, g, T = 7, 3, 0.8
    zt = bf16_to_f32(bf16_round(rng.standard_normal((g + 1, V)).astype(np.float32)))
    dl = bf16_round(rng.standard_normal((1, g, V)).astype(np.float32) * 1.5)
    z = zt.astype(np.float64)
    vlen, offs = np.array([g], np.int32), np.array([0, g + 1], np.int32)
    rate = O.acceptance_rate(z, dl, vlen, offs, T)
    assert rate.shape == (1, g)
    q = _softmax_rows(bf16_to_f32(dl[0]).astype(np.float64) / T)
    integ = np.zeros(g)
    for x in range(V):
        res, diag = O.accept_rejection(z, dl, np.full((1, g), x, np.int32), vlen, offs,
                                       np.zeros((1, g), np.float32),
                                       np.zeros((1, g + 1), np.float32), T)
        integ += q[:, x] * np.minimum(1.0, diag.ratio[0, :g])
    assert np.allclose(rate[0], integ, rtol=0, atol=1e-12)


def test_acceptance_rate_closed_forms_and_ragged_rows():
    """V = 2: rate = 1 - |p(0) - q(0)|; p = q gives 1, disjoint supports give 0, and
    positions past L_r hold -1. Rows are packed with per-request offsets, so a shifted
    row or request index changes a value."""
    T = 1.0
    vlen = np.array([3, 0, 2], np.int32)
    offs = np.concatenate([[0], np.cumsum(vlen + 1)]).astype(np.int32)
    g = 3
    rng = np.random.default_rng(5)
    a = rng.uniform(0.05, 0.95, offs[-1])
    z = np.stack([np.log(a), np.log1p(-a)], axis=1)
    ld = rng.standard_normal((3, g, 2)).astype(np.float32)
    dl = bf16_round(ld)
    # Request 2 position 0: the drafter equals the target row (bf16-exact logits).
    dl[2, 0] = bf16_round(np.array([0.5, -0.25], np.float32))
    z[offs[2]] = [0.5, -0.25]
    # Request 2 position 1: disjoint supports.
    dl[2, 1] = bf16_round(np.array([-300.0, 0.0], np.float32))
    z[offs[2] + 1] = [0.0, -900.0]
    rate = O.acceptance_rate(z, dl, vlen, offs, T)
    for r in range(3):
        for j in range(g):
            if j >= vlen[r]:
                assert rate[r, j] == -1.0
                continue
            zr = z[offs[r] + j]
            p0 = 1.0 / (1.0 + np.exp(zr[1] - zr[0]))
            lq = bf16_to_f32(dl[r, j]).astype(np.float64)
            q0 = 1.0 / (1.0 + np.exp(lq[1] - lq[0]))
            assert abs(rate[r, j] - (1.0 - abs(p0 - q0))) < 1e-12
    assert abs(rate[2, 0] - 1.0) < 1e-15
    assert abs(rate[2, 1]) < 1e-100


def test_rejection_is_lossless_chi2():
    """DSpark summary, "Problem definition": rejection sampling keeps the target distribution.

    The first two emitted tokens of each round must be distributed as the
    target's own autoregressive samples p(v0 | anchor) p(v1 | v0).
    """
    rng = np.random.default_rng(2024)
    V, g, B = 4, 3, 60000
    Zt, Zd, x, hidden, dl, ua, ur = _tiny_rejection_case(rng, V, g, B)
    W = bf16_round(np.eye(V, dtype=np.float32))
    res = O.verify_step(hidden, W, x, 1.0, draft_logit_bits=dl, u_accept=ua, u_resample=ur)
    a = res.accept.accept_len
    nxt = res.accept.next_token
    emitted = [list(x[r, :a[r]]) + [int(nxt[r])] for r in range(B)]
    pt = _softmax_rows(Zt)
    # First token.
    first = np.bincount([e[0] for e in emitted], minlength=V)
    assert _chi2_p(first, pt[0]) > 1e-3
    # First two tokens, over the rounds that emitted at least two.
    two = [e[:2] for e in emitted if len(e) >= 2]
    # Emitting a second token requires x_0 accepted; condition on the first token v0 instead:
    # P(v1 | v0, at least two emitted) must be p(v1 | v0).
    for v0 in range(V):
        cnt = np.bincount([e[1] for e in two if e[0] == v0], minlength=V)
        if cnt.sum() > 500:
            assert _chi2_p(cnt, pt[v0]) > 1e-3
    # Acceptance at position 0 follows 1 - TV(p_0, q_0).
    q0 = _softmax_rows(Zd)[0]
    rate = np.mean(a >= 1)
    want = 1 - 0.5 * np.abs(pt[0] - q0).sum()
    assert abs(rate - want) < 4 * np.sqrt(want * (1 - want) / B)


def test_rejection_multi_round_three_tokens_chi2():
    """DSpark summary, "Problem definition": speculative sampling, round after round,
    emits the target's own autoregressive distribution. Bigram target and drafter over
    V = 3; rounds of gamma = 2 drafts (x ~ q) continue from the last emitted token until
    three tokens are out; their 27-cell distribution must match
    p(v0 | anchor) p(v1 | v0) p(v2 | v1) (chi-square, alpha = 1e-3)."""
    rng = np.random.default_rng(77)
    V, g, N = 3, 2, 40000
    Zt = _bigram(rng, V, 1.2)
    Zd = _bigram(rng, V, 1.2)
    pt, qt = _softmax_rows(Zt), _softmax_rows(Zd)
    W = bf16_round(np.eye(V, dtype=np.float32))
    out = [[0] for _ in range(N)]                 # token 0 is the anchor
    todo = np.arange(N)
    while todo.size:
        last = np.array([out[i][-1] for i in todo])
        B = todo.size
        x = np.zeros((B, g), np.int32)
        prev = last.copy()
        for j in range(g):
            cdf = np.cumsum(qt[prev], axis=1)
            x[:, j] = np.minimum((rng.random((B, 1)) > cdf).sum(1), V - 1)
            prev = x[:, j]
        prevs = np.concatenate([last[:, None], x], axis=1)
        hidden = bf16_round(Zt[prevs].astype(np.float32))
        dl = bf16_round(Zd[prevs[:, :g]].astype(np.float32))
        ua = rng.random((B, g)).astype(np.float32)
        ur = rng.random((B, g + 1)).astype(np.float32)
        res = O.verify_step(hidden, W, x, 1.0, draft_logit_bits=dl, u_accept=ua, u_resample=ur)
        for k, i in enumerate(todo):
            a = int(res.accept.accept_len[k])
            out[i] += [int(t) for t in x[k, :a]] + [int(res.accept.next_token[k])]
        todo = np.array([i for i in todo if len(out[i]) < 4], dtype=np.int64)
    cells = np.zeros(V ** 3)
    for o in out:
        cells[o[1] * 9 + o[2] * 3 + o[3]] += 1
    want = np.array([pt[0, a] * pt[a, b] * pt[b, c]
                     for a in range(V) for b in range(V) for c in range(V)])
    assert abs(want.sum() - 1.0) < 1e-12
    assert _chi2_p(cells, want) > 1e-3


def test_rejection_equal_distributions_accept_everything():
    rng = np.random.default_rng(8)
    V, g, B = 5, 3, 3000
    Z = _bigram(rng, V, 1.0)
    _, _, x, hidden, dl, ua, ur = _tiny_rejection_case(rng, V, g, B, target=Z, drafter=Z)
    W = bf16_round(np.eye(V, dtype=np.float32))
    res = O.verify_step(hidden, W, x, 1.0, draft_logit_bits=dl, u_accept=ua, u_resample=ur)
    assert np.all(res.accept.accept_len == g)
    # The bonus token is a sample of p(. | x_{g-1}).
    pt = _softmax_rows(Z)
    for last in range(V):
        sel = x[:, -1] == last
        if sel.sum() > 300:
            cnt = np.bincount(res.accept.next_token[sel], minlength=V)
            assert _chi2_p(cnt, pt[last]) > 1e-3


def test_rejection_of_impossible_draft_resamples_from_target():
    """q puts its mass on x where p(x) is 0: always rejected, the correction ~ p."""
    rng = np.random.default_rng(9)
    V, B = 6, 20000
    zt = np.array([0.5, -1.0, 2.0, 0.0, 1.0, -200.0])       # p(5) == 0 in fp64
    zd = np.array([-50.0, -50.0, -50.0, -50.0, -50.0, 8.0])  # q concentrated on 5
    hidden = np.broadcast_to(bf16_round(np.stack([zt, zt]).astype(np.float32)), (B, 2, V))
    dl = np.broadcast_to(bf16_round(zd.astype(np.float32))[None, None], (B, 1, V))
    W = bf16_round(np.eye(V, dtype=np.float32))
    res = O.verify_step(np.ascontiguousarray(hidden), W, np.full((B, 1), 5, np.int32), 1.0,
                        draft_logit_bits=np.ascontiguousarray(dl),
                        u_accept=rng.random((B, 1)).astype(np.float32),
                        u_resample=rng.random((B, 2)).astype(np.float32))
    assert np.all(res.accept.accept_len == 0)
    p = _softmax_rows(O.bf16_decode(bf16_round(zt.astype(np.float32))))
    cnt = np.bincount(res.accept.next_token, minlength=V)
    assert cnt[5] == 0
    assert _chi2_p(cnt[:5], p[:5]) > 1e-3


def test_low_temperature_rejection_matches_greedy():
    """As T -> 0 both softmaxes become one-hot and rejection reduces to greedy matching."""
    rng = np.random.default_rng(31)
    V, g, B = 12, 5, 400
    W = bf16_round(np.eye(V, dtype=np.float32))
    hidden = bf16_round((rng.standard_normal((B, g + 1, V)) * 4).astype(np.float32))
    zt = O.bf16_decode(hidden)
    tgt = np.argmax(zt, axis=2)
    # Drafts agree with the target argmax for a random prefix, then disagree.
    x = tgt[:, :g].copy()
    cut = rng.integers(0, g + 1, B)
    for r in range(B):
        if cut[r] < g:
            x[r, cut[r]] = (x[r, cut[r]] + 1 + rng.integers(0, V - 1)) % V
    x = x.astype(np.int32)
    dlog = np.full((B, g, V), -4.0, np.float32)
    dlog[np.arange(B)[:, None], np.arange(g)[None], x] = 4.0
    # Skip near-ties of the target, which a vanishing temperature cannot separate.
    srt = np.sort(zt, axis=2)
    ok = np.all(srt[:, :, -1] - srt[:, :, -2] > 0.05, axis=1)
    T = 1e-3
    res_r = O.verify_step(hidden, W, x, T, draft_logit_bits=bf16_round(dlog),
                          u_accept=rng.random((B, g)).astype(np.float32) * 0.999,
                          u_resample=rng.random((B, g + 1)).astype(np.float32))
    res_g = O.verify_step(hidden, W, x, 0.0)
    assert ok.sum() > 100
    assert np.array_equal(res_r.accept.accept_len[ok], res_g.accept.accept_len[ok])
    assert np.array_equal(res_r.accept.next_token[ok], res_g.accept.next_token[ok])
    assert np.array_equal(res_g.accept.accept_len, np.minimum(cut, g))


def test_rejection_hand_case_uniform_indexing():
    """Hand-derived round: which uniform drives the correction and the bonus draw.

    Row 1: p = (.5, .3, .2), q = (.1, .1, .8), draft 2 -> ratio .25, rejected by u = .999.
    Residual (.4, .2, 0) / .6 has CDF (2/3, 1, 1): u_resample[1] = .95 gives token 1
    (u_resample[0] = .05 or u_resample[2] = .5 would give token 0).
    With all drafts accepted the bonus row p_2 = (.2, .2, .6) is sampled with
    u_resample[2] = .3 -> token 1 (u_resample[0] -> 0, u_resample[1] -> 2).
    """
    lg = lambda p: bf16_round(np.log(np.array(p, np.float64)).astype(np.float32))
    W = bf16_round(np.eye(3, dtype=np.float32))
    hidden = np.stack([lg([.4, .4, .2]), lg([.5, .3, .2]), lg([.2, .2, .6])])[None]
    dl = np.stack([lg([.3, .3, .4]), lg([.1, .1, .8])])[None]
    x = np.array([[0, 2]], np.int32)
    ur = np.array([[0.05, 0.95, 0.3]], np.float32)
    rej = O.verify_step(hidden, W, x, 1.0, draft_logit_bits=dl,
                        u_accept=np.array([[0.0, 0.999]], np.float32), u_resample=ur)
    assert int(rej.accept.accept_len[0]) == 1 and int(rej.accept.next_token[0]) == 1
    assert bool(rej.diag.residual[0])
    ur2 = np.array([[0.05, 0.95, 0.3]], np.float32)
    allacc = O.verify_step(hidden, W, np.array([[0, 1]], np.int32), 1.0, draft_logit_bits=dl,
                           u_accept=np.array([[0.0, 0.0]], np.float32), u_resample=ur2)
    assert int(allacc.accept.accept_len[0]) == 2 and int(allacc.accept.next_token[0]) == 1
    assert not bool(allacc.diag.residual[0])
    assert list(allacc.accept.counters) == [2, 2]


def _bisect_first_change(f, lo, hi, iters=56):
    """f is monotone on [lo, hi] with f(lo) != f(hi): the boundary point (to ~1e-17)."""
    flo = f(lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid) == flo:
            lo = mid
        else:
            hi = mid
    return hi


@pytest.mark.parametrize("V,g,L,T,seed", [(3, 3, 3, 1.0, 5), (4, 2, 2, 0.7, 6), (3, 3, 2, 1.3, 7)])
def test_rejection_output_distribution_closed_form(V, g, L, T, seed):
    """Exact output distribution of the oracle's rejection step against the closed form.

    DSpark summary, "Problem definition" (rejection sampling keeps the target's output
    distribution exactly). Drafts x ~ q are enumerated exhaustively; the oracle's
    dependence on each uniform is integrated piecewise, every acceptance threshold and
    every inverse-CDF breakpoint located by bisection on the oracle's own outputs. The
    result must equal
      P(a = k, emitted s_0..s_k) = prod_{i<k} min(p_i(s_i), q_i(s_i))
                                   * (max(0, p_k(s_k) - q_k(s_k)) if k < L else p_L(s_L))
    to 1e-12, with p, q from scipy's softmax of the decoded logits.
    """
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, 1.2, (L + 1, V))                       # target logits, rows 0..L
    dl = bf16_round(rng.normal(0.0, 1.2, (1, g, V)).astype(np.float32))
    p = special.softmax(z / T, axis=1)
    q = special.softmax(bf16_to_f32(dl[0]).astype(np.float64) / T, axis=1)
    vlen = np.array([L], np.int32)
    offs = np.array([0, L + 1], np.int32)

    def run(x, ua, ur):
        tok = np.zeros((1, g), np.int32)
        tok[0, :L] = x
        res, _ = O.accept_rejection(z, dl, tok, vlen, offs, np.asarray(ua, np.float64)[None],
                                    np.asarray(ur, np.float64)[None], T)
        return int(res.accept_len[0]), int(res.next_token[0])

    top = 1.0 - 2.0 ** -53
    got = {}
    for code in range(V ** L):
        x = [(code // V ** i) % V for i in range(L)]
        px = float(np.prod([q[i, x[i]] for i in range(L)]))
        # Acceptance threshold of each position: with every earlier uniform 0 (always
        # kept), position j is kept for u < t_j and rejected for u >= t_j.
        t = []
        for j in range(L):
            def kept(u, j=j):
                ua = np.zeros(g)
                ua[j] = u
                return run(x, ua, np.full(g + 1, 0.5))[0] > j
            t.append(1.0 if kept(top) else _bisect_first_change(kept, 0.0, top))
            assert kept(0.0)
        for k in range(L + 1):
            ua = np.zeros(g)
            if k < L:
                if t[k] >= 1.0:
                    continue                                    # position k is never rejected
                ua[k] = 0.5 * (t[k] + 1.0)
            weight = px * float(np.prod(t[:k])) * ((1.0 - t[k]) if k < L else 1.0)

            def emitted(u, ua=ua, k=k):
                ur = np.full(g + 1, 0.5)
                ur[k] = u
                a, v = run(x, ua, ur)
                assert a == k
                return v
            u0 = 0.0
            while True:                                         # the draw is non-decreasing in u
                v = emitted(u0)
                b = top if emitted(top) == v else _bisect_first_change(emitted, u0, top)
                if b == top:
                    b = 1.0
                key = (k, tuple(x[:k]) + (v,))
                got[key] = got.get(key, 0.0) + weight * (b - u0)
                if b >= 1.0:
                    break
                u0 = b
    want = {}
    for k in range(L + 1):
        for code in range(V ** (k + 1)):
            s = [(code // V ** i) % V for i in range(k + 1)]
            pr = float(np.prod([min(p[i, s[i]], q[i, s[i]]) for i in range(k)]))
            pr *= max(0.0, p[k, s[k]] - q[k, s[k]]) if k < L else p[L, s[L]]
            if pr > 0.0:
                want[(k, tuple(s))] = pr
    assert abs(sum(got.values()) - 1.0) < 1e-12
    for key in set(got) | set(want):
        assert abs(got.get(key, 0.0) - want.get(key, 0.0)) < 1e-12, key
