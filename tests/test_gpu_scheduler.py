"""GPU parity of the hardware-aware prefix scheduler (sd_schedule_prefix) against the oracle.

The scheduler turns floating-point survivals into integer decisions; both sides take
them in the same arithmetic (fp32 running products, fixed-point sums, one fp64
multiply per throughput value), so verify_len and row_offsets must match bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as sd
from oracle import prefix_scheduler as S

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    yield


def tables(rng, R, g):
    B = np.arange(R * (g + 1) + 1, dtype=np.float64)
    t0, t1 = rng.uniform(0.5, 2.0), rng.uniform(1e-4, 0.05)
    yield "linear", (1.0 / (t0 + t1 * B)).astype(np.float32)
    yield "staircase", (1.0 / (t0 + 0.3 * np.ceil(B / 256.0) + 0.05 * np.ceil(B / 16.0))
                        ).astype(np.float32)
    yield "random", rng.uniform(0.1, 1.0, B.size).astype(np.float32)


def confidences(rng, R, g, kind):
    if kind == "uniform":
        return rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)
    if kind == "ones":
        return np.ones((R, g), np.float32)
    if kind == "steep":
        return rng.uniform(0.0, 0.5, (R, g)).astype(np.float32)
    c = rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)       # out-of-range entries
    m = rng.random((R, g))
    c[m < 0.05] = np.nan
    c[(m >= 0.05) & (m < 0.1)] = -0.5
    c[(m >= 0.1) & (m < 0.15)] = 1.75
    return c


SHAPES = [(1, 16), (32, 16), (128, 16), (300, 3), (2, 64), (1000, 7), (256, 64), (16384, 1)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"R{r}g{g}" for r, g in SHAPES])
def test_scheduler_matches_oracle(shape):
    R, g = shape
    rng = np.random.default_rng(R * 100 + g)
    kinds = ["uniform", "ones", "steep", "dirty"] if R * g <= 4096 else ["uniform", "dirty"]
    for kind in kinds:
        conf = confidences(rng, R, g, kind)
        stale = confidences(rng, R, g, "uniform")
        conf_d = torch.from_numpy(conf).cuda()
        stale_d = torch.from_numpy(stale).cuda()
        for tname, sps in tables(rng, R, g):
            sps_d = torch.from_numpy(sps).cuda()
            for mode, st in ((S.SYNC_EARLY_STOP, None), (S.ASYNC_TOP_K, None),
                             (S.ASYNC_TOP_K, stale)):
                say(f"R={R} g={g} conf={kind} sps={tname} mode={mode} stale={st is not None}")
                vl, ro = sd.sd_schedule_prefix(conf_d, sps_d, mode,
                                               stale_d if st is not None else None)
                torch.cuda.synchronize()
                vl_o, ro_o, K = S.schedule_prefix(conf, sps, mode, st)
                assert np.array_equal(vl.cpu().numpy(), vl_o)
                assert np.array_equal(ro.cpu().numpy(), ro_o)
                assert int(ro_o[-1]) == R + K


def test_scheduler_on_measured_table():
    """SPS(B) profiled from this library's verify call (32 requests, gamma 16, d 4096,
    V 151936, T 0.8), then the scheduler on synthetic survival-style confidences."""
    from synth import workload
    w = workload("ragged-b32")
    say("profile_sps", f"R={w.B} g={w.gamma} d={w.d} V={w.V}")
    W = torch.randn((w.V, w.d), dtype=torch.float32, device="cuda").div_(w.d ** 0.5)
    W = W.to(torch.bfloat16)
    sps = sd.profile_sps(w.B, w.gamma, W, w.T, repeats=5)
    torch.cuda.synchronize()
    s = sps.cpu().numpy()
    assert s.shape == (w.B * (w.gamma + 1) + 1,)
    assert np.all(np.isfinite(s)) and np.all(s > 0)
    assert s[-1] <= s[w.B] * 1.05          # more rows never run much faster
    say("sps", f"SPS(R)={s[w.B]:.1f}/s SPS(cap)={s[-1]:.1f}/s distinct={len(np.unique(s))}")
    del W
    rng = np.random.default_rng(5)
    for step in range(4):
        # Conditional confidences with the synthetic survival curves' law: the first
        # position U(0.6, 1), each later one a ratio U(0.7, 1).
        c = rng.uniform(0.6, 1.0, (w.B, w.gamma)).astype(np.float32)
        c[:, 1:] = rng.uniform(0.7, 1.0, (w.B, w.gamma - 1)).astype(np.float32)
        for mode in (S.SYNC_EARLY_STOP, S.ASYNC_TOP_K):
            vl, ro = sd.sd_schedule_prefix(torch.from_numpy(c).cuda(), sps, mode)
            torch.cuda.synchronize()
            vl_o, ro_o, K = S.schedule_prefix(c, s, mode)
            assert np.array_equal(vl.cpu().numpy(), vl_o)
            assert np.array_equal(ro.cpu().numpy(), ro_o)
            say(f"step {step} mode {mode}: admitted {K} of {w.B * w.gamma}")
