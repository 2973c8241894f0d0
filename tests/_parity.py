"""Helpers shared by the GPU parity tests: run one verify round on the device
and on the CPU oracle from the same seeded inputs, then compare.

Bars (floating point in, integer decisions out):
  * logits: |gpu - oracle| <= max(2e-2, 1e-2 |oracle|);
  * probabilities p_j(x_j), q_j(x_j): abs 1e-4;
  * argmax, accepted lengths, emitted tokens: bit-exact, except
      - a greedy decision on a row whose oracle top-2 gap is below 1e-3,
      - a rejection decision with |u - min(1, p/q)| < 1e-6,
      - a correction/bonus draw whose u * S lies within draw_band() of a CDF
        boundary (see there: the spread that fp32 logits put on the CDF);
    exempt requests are counted by kind and reported.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

import draft_block_verification_amd as sd
from oracle import sd_oracle as O
from synth import StepInputs, Workload, make_weights

TIE_GAP = 1e-3
U_BAND = 1e-6
CDF_SIGMAS = 6.0


def draw_band(d: int, T: float, zmax: float, conc: float) -> float:
    """Half-width, as a fraction of S, of the band around a CDF boundary inside which a
    correction/bonus draw may differ between the kernel and the oracle.

    The kernel forms each weight from an fp32 logit. That logit is a sum of ceil(d/32)
    MFMA steps, each rounded to fp32, so its error against the exact fp64 logit has a
    standard deviation of at most sigma_z = 0.5 ulp(zmax) sqrt(ceil(d/32)), with zmax
    bounding the accumulator's magnitude; the hardware exp2 and the fp32 weight add
    about 2^-22 relative. With independent relative errors e_v of standard deviation
    sigma_e = sigma_z / T + 2^-22, a normalised CDF value C_v / S moves by a standard
    deviation of at most sigma_e sqrt(sum_v (w_v / S)^2) (conc). The band is CDF_SIGMAS
    of those. At V ~ 1.5e5 a flat band would cover most boundaries (their mean spacing
    is 1/V ~ 7e-6 of S); this one covers a few percent of draws.
    """
    e = np.floor(np.log2(max(abs(zmax), 2.0 ** -20)))
    sigma_z = 0.5 * 2.0 ** (e - 23) * np.sqrt(np.ceil(d / 32))
    sigma_e = sigma_z / T + 2.0 ** -22
    return CDF_SIGMAS * sigma_e * conc


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


_HEADS = {}


def lm_head(w: Workload, seed: int = 0):
    """(bf16 bits, float64, device bf16) of the workload's LM head, the last one kept.

    Full-size heads are large (config 5: 1.85 GB of bf16, 7.4 GB as float64), so only
    the most recent one stays cached across the tests that share it.
    """
    key = (w.wid, w.V, w.d, seed)
    if key not in _HEADS:
        _HEADS.clear()
        W = make_weights(w, seed)
        _HEADS[key] = (W, O.lm_head_f64(W), bf16_dev(W))
    return _HEADS[key]


def f32_dev(x, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def i32_dev(x, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


@dataclasses.dataclass
class DevStep:
    hidden: torch.Tensor
    draft_tokens: torch.Tensor
    conf: Optional[torch.Tensor]
    draft_logits: Optional[torch.Tensor]
    u_accept: torch.Tensor
    u_resample: torch.Tensor


def upload_step(s: StepInputs, device="cuda") -> DevStep:
    return DevStep(bf16_dev(s.hidden, device), i32_dev(s.draft_tokens, device),
                   None if s.conf is None else f32_dev(s.conf, device),
                   None if s.draft_logits is None else bf16_dev(s.draft_logits, device),
                   f32_dev(s.u_accept, device), f32_dev(s.u_resample, device))


@dataclasses.dataclass
class GpuResult:
    verify_len: np.ndarray
    row_offsets: np.ndarray
    stats: np.ndarray            # structured, ROW_STATS_DTYPE, first M rows
    logits: Optional[np.ndarray]  # [M][V] or None
    accept_len: np.ndarray
    next_token: np.ndarray
    counters: np.ndarray
    flags: int
    lse_q: Optional[np.ndarray]   # [B][gamma] drafter log-normalisers (rejection only)


def run_gpu(w: Workload, W_dev: torch.Tensor, ds: DevStep, vr: Optional[sd.VerifyRound] = None,
            fetch_logits_rows: Optional[Sequence[int]] = None, fetch_all_logits=False) -> GpuResult:
    if vr is None:
        vr = sd.VerifyRound(w.B, w.gamma, w.d, w.V, w.T, w.truncate, w.threshold)
    vr.counters.zero_()
    vr.run(ds.hidden, W_dev, ds.draft_tokens, ds.conf, ds.draft_logits, ds.u_accept,
           ds.u_resample)
    torch.cuda.synchronize()
    if w.truncate:
        vlen = vr.verify_len.cpu().numpy()
        offs = vr.row_offsets.cpu().numpy()
    else:
        vlen, offs = O.full_lengths(w.B, w.gamma)
    M = int(offs[-1])
    stats = sd.stats_to_numpy(vr.stats)[:M]
    logits = None
    if vr.logits is not None:
        if fetch_all_logits:
            logits = vr.logits[:M].cpu().numpy()
        elif fetch_logits_rows is not None:
            idx = torch.as_tensor(list(fetch_logits_rows), dtype=torch.long, device=vr.logits.device)
            logits = vr.logits.index_select(0, idx).cpu().numpy()
    flags = sd.device_flags(vr.ws_verify)
    lse_q = None
    if vr.ws_accept is not None:
        flags |= sd.device_flags(vr.ws_accept)
        # The accept workspace holds the drafter log-normalisers after its 256-byte header.
        lse_q = (vr.ws_accept[256:256 + 8 * w.B * w.gamma].cpu().numpy().view(np.float64)
                 .reshape(w.B, w.gamma))
    return GpuResult(vlen, offs, stats, logits, vr.accept_len.cpu().numpy(),
                     vr.next_token.cpu().numpy(), vr.counters.cpu().numpy(), flags, lse_q)


def slice_step(s: StepInputs, req: Sequence[int]) -> StepInputs:
    req = np.asarray(req)
    pick = lambda a: None if a is None else np.ascontiguousarray(a[req])
    return StepInputs(pick(s.draft_tokens), pick(s.planted), pick(s.hidden), pick(s.draft_logits),
                      pick(s.conf), pick(s.u_accept), pick(s.u_resample))


def run_oracle(w: Workload, W_bits: np.ndarray, s: StepInputs) -> O.StepResult:
    return O.verify_step(s.hidden, W_bits, s.draft_tokens, w.T,
                         conf=s.conf if w.truncate else None, threshold=w.threshold,
                         draft_logit_bits=s.draft_logits, u_accept=s.u_accept,
                         u_resample=s.u_resample)


@dataclasses.dataclass
class Report:
    requests: int = 0
    exempt: int = 0          # requests whose outputs differ inside an exemption
    exempt_tie: int = 0      # ... a greedy top-2 gap below TIE_GAP
    exempt_u: int = 0        # ... |u - min(1, p/q)| below U_BAND
    exempt_draw: int = 0     # ... a draw inside draw_band() of a CDF boundary
    fragile_draws: int = 0   # draws inside the band (whether or not they differed)
    draws: int = 0           # correction/bonus draws compared (T > 0)
    bonus_draws: int = 0     # of which drawn from p after every kept draft survived
    full_accepts: int = 0    # requests with a_r = L_r (L_r > 0)
    rows: int = 0
    max_logit_err: float = 0.0
    max_prob_err: float = 0.0
    max_lse_err: float = 0.0
    accepted: int = 0


def compare(w: Workload, g: GpuResult, o: O.StepResult, req: Sequence[int],
            rep: Optional[Report] = None, check_logits=True) -> Report:
    """Compare GPU results at requests `req` with an oracle run over exactly those requests."""
    rep = rep or Report()
    req = list(req)
    # Truncation is integer work: bit-exact.
    assert np.array_equal(g.verify_len[req], o.verify_len), "verify_len"
    if len(req) == w.B:
        assert np.array_equal(g.row_offsets, o.row_offsets), "row_offsets"
    for i, r in enumerate(req):
        L = int(o.verify_len[i])
        gb, ob = int(g.row_offsets[r]), int(o.row_offsets[i])
        grow = g.stats[gb:gb + L + 1]
        z = o.z[ob:ob + L + 1]
        st_top1, st_top2 = o.stats.top1[ob:ob + L + 1], o.stats.top2[ob:ob + L + 1]
        st_arg = o.stats.argmax[ob:ob + L + 1]
        rep.rows += L + 1
        assert np.all(grow["pos"] == np.arange(L + 1)), f"row positions of request {r}"
        tol = np.maximum(2e-2, 1e-2 * np.abs(st_top1))
        assert np.all(np.abs(grow["top1"] - st_top1) <= tol), f"top1 of request {r}"
        gap = st_top1 - st_top2
        tie = gap < TIE_GAP
        assert np.all((grow["argmax"] == st_arg) | tie), f"argmax of request {r}"
        # Exact drafted-token logits (fp64 dots of bf16 inputs on both sides).
        if L:
            zd_o = z[np.arange(L), np.asarray(o_draft(o, i, L))]
            assert np.allclose(grow["z_draft"][:L], zd_o, rtol=0, atol=1e-9), f"z_draft {r}"
        if w.T > 0:
            lse_err = np.max(np.abs(grow["lse"] - o.stats.lse[ob:ob + L + 1]))
            rep.max_lse_err = max(rep.max_lse_err, float(lse_err))
            assert lse_err < 1e-4, f"lse of request {r}: {lse_err}"
            if L:
                p_g = np.exp(grow["z_draft"][:L] / w.T - grow["lse"][:L])
                pe = float(np.max(np.abs(p_g - o.diag.p_x[i, :L])))
                rep.max_prob_err = max(rep.max_prob_err, pe)
                assert pe < 1e-4, f"p(x) of request {r}"
                lq_err = float(np.max(np.abs(g.lse_q[r, :L] - o.diag.lse_q[i, :L])))
                rep.max_lse_err = max(rep.max_lse_err, lq_err)
                assert lq_err < 1e-5, f"lse_q of request {r}: {lq_err}"
        # Acceptance decisions.
        a_o, a_g = int(o.accept.accept_len[i]), int(g.accept_len[r])
        n_o, n_g = int(o.accept.next_token[i]), int(g.next_token[r])
        rep.requests += 1
        rep.accepted += a_g
        if L and a_o == L:
            rep.full_accepts += 1
        if w.T > 0:
            decided = min(a_o, L - 1)
            ratio = o.diag.ratio[i, :decided + 1] if L else np.zeros(0)
            u = o_u(o, i, decided + 1) if L else np.zeros(0)
            fragile_acc = bool(np.any(np.abs(u - np.minimum(1.0, ratio)) < U_BAND))
            zmax = float(np.max(np.abs(o.z[int(o.diag.draw_row[i])])))
            band = draw_band(w.d, w.T, zmax, float(o.diag.cdf_conc[i]))
            fragile_draw = bool(o.diag.cdf_dist[i] < band)
            rep.draws += 1
            rep.bonus_draws += int(a_o == L)
            rep.fragile_draws += int(fragile_draw)
        else:
            fragile_acc = bool(np.any(tie[:min(a_o, L) + 1]))
            fragile_draw = bool(tie[min(a_o, L)])
        if a_g != a_o:
            assert fragile_acc, f"accept_len of request {r}: gpu {a_g} oracle {a_o}"
            rep.exempt += 1
            if w.T > 0:
                rep.exempt_u += 1
            else:
                rep.exempt_tie += 1
            continue
        if n_g != n_o:
            assert fragile_draw or fragile_acc, f"next_token of request {r}: gpu {n_g} oracle {n_o}"
            rep.exempt += 1
            if w.T > 0 and fragile_draw:
                rep.exempt_draw += 1
            elif w.T > 0:
                rep.exempt_u += 1
            else:
                rep.exempt_tie += 1
    return rep


# The oracle's step result does not keep its inputs; these read them from the
# attributes attached by attach_inputs().
def o_draft(o, i, L):
    return o._x[i, :L]


def o_u(o, i, n):
    return o._u[i, :n].astype(np.float64)


def attach_inputs(o: O.StepResult, s: StepInputs) -> O.StepResult:
    o._x = s.draft_tokens
    o._u = s.u_accept
    return o


def check_logits_rows(w: Workload, g_logits: np.ndarray, z_rows: np.ndarray, rep: Report) -> None:
    err = np.abs(g_logits.astype(np.float64) - z_rows)
    tol = np.maximum(2e-2, 1e-2 * np.abs(z_rows))
    assert np.all(err <= tol), f"logits: max err {err.max()}"
    rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
