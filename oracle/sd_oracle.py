"""CPU oracle for draft-block verification (test infrastructure, not product).

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this module. The HIP library never
calls it and shares no code with it.

It computes, plainly and slowly in float64, what one verify round of
speculative decoding produces:

* confidence truncation of each request's draft block
  (DSpark summary, "Architecture": the decode-round example in which the
  scheduler keeps the prefix E F G and cuts the low-confidence H; the
  confidence head gives per-position survival probabilities in (0, 1));
* target logits at every kept draft position plus the bonus position, from
  the LM-head contraction z = h . W^T (DSpark summary, "Production
  deployment": the LM head maps the d-vector to V logits; LFM2.5-DSpark
  blog, "How DSpark works": the target checks the whole block in one pass);
* greedy acceptance: a draft token survives iff it equals the target's
  argmax, and the first mismatch is replaced by the target's own token
  (LFM2.5-DSpark blog, "Quality parity" and the usage notes: greedy output
  equals the target's own greedy output);
* rejection-sampling acceptance of the longest prefix consistent with the
  target distribution (DSpark summary, "Problem definition"), with
  acceptance probability min(1, p/q) and, on the first rejection, a
  correction token drawn from norm(max(0, p - q)); when every draft
  survives, a bonus token is drawn from the target row after the block.
  The per-step acceptance probability of this rule is 1 - TV(p, q)
  (DSpark summary, "Confidence-Scheduled Verification" and "Training").

Where the pages leave a step open, the readings are:

* truncation keeps the leading positions whose confidence is >= threshold;
  kept drafts L_r = (1-based index of the first position below threshold)
  - 1, or gamma if none; rows 0..L_r (L_r + 1 of them, the last one being
  the bonus row) are verified;
* argmax ties go to the lowest vocabulary id;
* the draft distribution uses the same temperature: q = softmax(l / T);
* a draft survives iff u < min(1, p(x) / q(x)) with u in [0, 1);
* the correction/bonus token is the inverse CDF in ascending vocabulary id:
  the smallest v with C_v > u * S, where C is the running sum of the
  weights and S their total; the uniform used is u_resample[r][a_r], the
  one indexed by the row being sampled; if rounding leaves no such v the
  last v with positive weight is taken; if the residual has no positive
  weight at all (p == q at that row) the token is drawn from p instead.

Parity pins: every function here is checked in tests/test_oracle_pins.py
against closed forms, exact integer arithmetic, brute force, the pages'
worked example and distributional identities.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


# ---------------------------------------------------------------- decoding

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (the 16 bits are the top half of a float32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# -------------------------------------------------------------- truncation

def truncate_by_confidence(conf: np.ndarray, threshold: float):
    """Per-request kept draft count and packed row offsets.

    DSpark summary, "Architecture" (decode-round example and confidence
    head): each position carries the probability that it survives
    verification; the scheduler keeps the confident prefix and cuts the
    rest. L_r counts the leading positions with conf >= threshold; request r
    then owns rows row_offsets[r] .. row_offsets[r] + L_r (draft rows plus
    one bonus row), packed with no padding between requests (DSpark
    summary, "Production deployment": variable-length queries are
    flattened).
    """
    conf = np.asarray(conf, dtype=np.float32)
    B, g = conf.shape
    verify_len = np.zeros(B, dtype=np.int32)
    for r in range(B):
        L = 0
        while L < g and float(conf[r, L]) >= float(np.float32(threshold)):
            L += 1
        verify_len[r] = L
    row_offsets = np.zeros(B + 1, dtype=np.int32)
    for r in range(B):
        row_offsets[r + 1] = row_offsets[r] + verify_len[r] + 1
    return verify_len, row_offsets


def full_lengths(B: int, gamma: int):
    """Untruncated block: every request verifies all gamma drafts plus the bonus row."""
    verify_len = np.full(B, gamma, dtype=np.int32)
    row_offsets = (np.arange(B + 1, dtype=np.int64) * (gamma + 1)).astype(np.int32)
    return verify_len, row_offsets


# ------------------------------------------------------------------ logits

def verified_rows(hidden_bits: np.ndarray, verify_len: np.ndarray) -> np.ndarray:
    """Packed hidden states of the verified rows, float64 [M][d].

    Request r contributes its rows j = 0..L_r of hidden[r] in order.
    """
    h = bf16_decode(hidden_bits)
    rows = [h[r, : int(verify_len[r]) + 1] for r in range(h.shape[0])]
    return np.concatenate(rows, axis=0)


def lm_head_f64(W_bits: np.ndarray) -> np.ndarray:
    """The LM-head weight as float64 (bf16 bits are decoded; float64 input is returned as is)."""
    W = np.asarray(W_bits)
    return W if W.dtype == np.float64 else bf16_decode(W)


def verify_logits(hidden_bits: np.ndarray, W_bits: np.ndarray,
                  verify_len: np.ndarray) -> np.ndarray:
    """Target logits z[m][v] = sum_k h[m][k] * W[v][k] at every verified row (float64)."""
    H = verified_rows(hidden_bits, verify_len)
    return H @ lm_head_f64(W_bits).T


def logits_at(hidden_bits: np.ndarray, W_bits: np.ndarray, r: int, j: int) -> np.ndarray:
    """One target row z[v] for request r, block position j (float64); for sampled checks."""
    h = bf16_decode(hidden_bits[r, j])
    return lm_head_f64(W_bits) @ h


# --------------------------------------------------------------- row stats

@dataclasses.dataclass
class RowStats:
    argmax: np.ndarray   # int64 [M], lowest id on ties
    top1: np.ndarray     # float64 [M]
    top2: np.ndarray     # float64 [M], largest value over v != argmax
    lse: np.ndarray      # float64 [M], log sum_v exp(z_v / T) (T > 0), else zeros


def log_softmax_norm(x: np.ndarray) -> np.ndarray:
    """log sum_v exp(x_v) along the last axis, with the maximum taken out first."""
    m = np.max(x, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))[..., 0]


def row_stats(z: np.ndarray, T: float) -> RowStats:
    z = np.asarray(z, dtype=np.float64)
    am = np.argmax(z, axis=1)
    top1 = z[np.arange(z.shape[0]), am]
    rest = z.copy()
    rest[np.arange(z.shape[0]), am] = -np.inf
    top2 = np.max(rest, axis=1) if z.shape[1] > 1 else np.full(z.shape[0], -np.inf)
    lse = log_softmax_norm(z / T) if T > 0 else np.zeros(z.shape[0])
    return RowStats(am, top1, top2, lse)


# ------------------------------------------------------------------ greedy

@dataclasses.dataclass
class AcceptResult:
    accept_len: np.ndarray   # int32 [B]
    next_token: np.ndarray   # int32 [B]
    counters: np.ndarray     # int64 [2]: drafts verified, drafts accepted


def accept_greedy(argmax: np.ndarray, draft_tokens: np.ndarray,
                  verify_len: np.ndarray, row_offsets: np.ndarray) -> AcceptResult:
    """Greedy verification.

    LFM2.5-DSpark blog, "Quality parity": a draft token is kept only if it
    matches the target, and on the first mismatch the target's own token
    takes its place. a_r is the first kept position j with argmax != x_j (or
    L_r if all match); the emitted token is the target argmax at row a_r,
    which is the bonus token when every draft matched.
    """
    B = draft_tokens.shape[0]
    acc = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    for r in range(B):
        base, L = int(row_offsets[r]), int(verify_len[r])
        a = 0
        while a < L and int(argmax[base + a]) == int(draft_tokens[r, a]):
            a += 1
        acc[r] = a
        nxt[r] = int(argmax[base + a])
    counters = np.array([int(np.sum(verify_len)), int(np.sum(acc))], dtype=np.int64)
    return AcceptResult(acc, nxt, counters)


# --------------------------------------------------------------- rejection

def inverse_cdf(weights: np.ndarray, u: float):
    """Smallest v with C_v > u * S (C = running sum in ascending id, S = total).

    Returns (v, S, boundary distance min_v |u*S - C_v| / S). If rounding
    leaves no such v, the last v with positive weight.
    """
    C = np.cumsum(weights)
    S = float(C[-1])
    t = float(u) * S
    hit = np.nonzero(C > t)[0]
    if hit.size:
        v = int(hit[0])
    else:
        v = int(np.nonzero(weights > 0)[0][-1])
    dist = float(np.min(np.abs(C - t)) / S) if S > 0 else 0.0
    return v, S, dist


@dataclasses.dataclass
class RejectionDiag:
    ratio: np.ndarray        # float64 [B][gamma]: p(x)/q(x) at kept rows, nan elsewhere
    p_x: np.ndarray          # float64 [B][gamma]
    q_x: np.ndarray          # float64 [B][gamma]
    lse_q: np.ndarray        # float64 [B][gamma]
    cdf_dist: np.ndarray     # float64 [B]: boundary distance of the final draw
    residual: np.ndarray     # bool [B]: correction drawn from the residual (else bonus / p)
    mass: np.ndarray         # float64 [B]: S of the final draw
    cdf_conc: np.ndarray     # float64 [B]: sqrt(sum_v (w_v / S)^2) of the final draw's weights
    draw_row: np.ndarray     # int64 [B]: packed row the final draw was taken from


def accept_rejection(z: np.ndarray, draft_logit_bits: np.ndarray, draft_tokens: np.ndarray,
                     verify_len: np.ndarray, row_offsets: np.ndarray, u_accept: np.ndarray,
                     u_resample: np.ndarray, T: float, lse_p: Optional[np.ndarray] = None):
    """Rejection-sampling verification (lossless; DSpark summary, "Problem definition").

    z: float64 target logits of the verified rows [M][V] (packed by row_offsets).
    draft_logit_bits: bf16 bits of the drafter's logits [B][gamma][V].
    p_j = softmax(z_j / T), q_j = softmax(l_j / T). Position j < L_r survives iff
    u_accept[r][j] < min(1, p_j(x_j) / q_j(x_j)); a_r is the first failure (or L_r).
    If a_r < L_r the correction token is drawn from norm(max(0, p_a - q_a)), else the
    bonus token from p_{L_r}; both by inverse_cdf with u_resample[r][a_r].
    """
    assert T > 0
    B, g = draft_tokens.shape
    if lse_p is None:
        lse_p = log_softmax_norm(np.asarray(z) / T)
    acc = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    nan = np.full((B, g), np.nan)
    ratio, p_x, q_x, lse_q = nan.copy(), nan.copy(), nan.copy(), nan.copy()
    cdf_dist = np.zeros(B)
    residual = np.zeros(B, dtype=bool)
    mass = np.zeros(B)
    cdf_conc = np.zeros(B)
    draw_row = np.zeros(B, dtype=np.int64)
    for r in range(B):
        base, L = int(row_offsets[r]), int(verify_len[r])
        lq = bf16_decode(draft_logit_bits[r, :L]) / T          # [L][V]
        if L:
            lse_q[r, :L] = log_softmax_norm(lq)
        a = L
        for j in range(L):
            x = int(draft_tokens[r, j])
            p = np.exp(z[base + j, x] / T - lse_p[base + j])
            q = np.exp(lq[j, x] - lse_q[r, j])
            p_x[r, j], q_x[r, j] = p, q
            ratio[r, j] = p / q
            if a == L and not float(u_accept[r, j]) < min(1.0, p / q):
                a = j          # first rejection; later rows only fill the diagnostics
        acc[r] = a
        draw_row[r] = base + a
        p_row = np.exp(z[base + a] / T - lse_p[base + a])
        u = float(u_resample[r, a])
        weights = p_row
        if a < L:
            q_row = np.exp(lq[a] - lse_q[r, a])
            R = np.maximum(0.0, p_row - q_row)
            if np.any(R > 0):
                weights = R
                residual[r] = True
        nxt[r], mass[r], cdf_dist[r] = inverse_cdf(weights, u)
        # How concentrated the draw's weights are: the spread of a CDF value under
        # independent relative errors of the weights scales with this (diagnostic only).
        cdf_conc[r] = float(np.sqrt(np.sum((weights / mass[r]) ** 2))) if mass[r] > 0 else 0.0
    counters = np.array([int(np.sum(verify_len)), int(np.sum(acc))], dtype=np.int64)
    return AcceptResult(acc, nxt, counters), RejectionDiag(ratio, p_x, q_x, lse_q, cdf_dist,
                                                           residual, mass, cdf_conc, draw_row)


def acceptance_rate(z: np.ndarray, draft_logit_bits: np.ndarray, verify_len: np.ndarray,
                    row_offsets: np.ndarray, T: float, lse_p: Optional[np.ndarray] = None):
    """Analytic per-position acceptance rate c*_j = 1 - TV(q_j, p_j).

    DSpark summary, "Architecture" (confidence-scheduled verification): the confidence
    head is trained on the acceptance probability of each drafted position, which for
    the rejection rule is one minus the total-variation distance between the drafter's
    and the target's distributions at that position, 1 - (1/2) * sum_v |q(v) - p(v)|.
    Returns float64 [B][gamma]; positions at or past L_r hold -1 (not a probability).
    """
    assert T > 0
    B, g = draft_logit_bits.shape[:2]
    if lse_p is None:
        lse_p = log_softmax_norm(np.asarray(z) / T)
    out = np.full((B, g), -1.0)
    for r in range(B):
        base, L = int(row_offsets[r]), int(verify_len[r])
        for j in range(L):
            lq = bf16_decode(draft_logit_bits[r, j]) / T
            q = np.exp(lq - log_softmax_norm(lq[None, :])[0])
            p = np.exp(z[base + j] / T - lse_p[base + j])
            out[r, j] = 1.0 - 0.5 * float(np.sum(np.abs(q - p)))
    return out


# ------------------------------------------------------------ whole round

@dataclasses.dataclass
class StepResult:
    verify_len: np.ndarray
    row_offsets: np.ndarray
    z: np.ndarray
    stats: RowStats
    accept: AcceptResult
    diag: Optional[RejectionDiag]


def verify_step(hidden_bits, W_bits, draft_tokens, T, conf=None, threshold=0.3,
                draft_logit_bits=None, u_accept=None, u_resample=None) -> StepResult:
    """One verify round: truncate (if confidences are given), logits, stats, acceptance."""
    B, g = draft_tokens.shape
    if conf is not None:
        verify_len, row_offsets = truncate_by_confidence(conf, threshold)
    else:
        verify_len, row_offsets = full_lengths(B, g)
    z = verify_logits(hidden_bits, W_bits, verify_len)
    st = row_stats(z, T)
    if T > 0:
        res, diag = accept_rejection(z, draft_logit_bits, draft_tokens, verify_len, row_offsets,
                                     u_accept, u_resample, T, lse_p=st.lse)
    else:
        res, diag = accept_greedy(st.argmax, draft_tokens, verify_len, row_offsets), None
    return StepResult(verify_len, row_offsets, z, st, res, diag)
