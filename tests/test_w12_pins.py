"""Pins of the W12 oracle (oracle/w12.py) against things other than itself.

Exact round trips over every one of the 65536 bf16 bit patterns and over
synthetic LM heads; bytes of a hand-encoded group; the edges of the exponent
window; the layout of the correction slots.
"""
import numpy as np

from oracle import w12 as X
from synth import make_weights, workload


def test_round_trip_every_bf16_pattern():
    """Zeros, subnormals, infinities, NaNs and every exponent come back bit for bit."""
    W = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    rng = np.random.default_rng(0)
    W = W[rng.permutation(512)]                      # mix the exponents across rows
    enc = X.encode(W)
    assert enc.b2 == 127 - 6                          # inf / NaN patterns have e2 = 127
    assert np.array_equal(X.decode(enc, 512, 128), W)
    assert enc.codes.shape == (512, 16, 12) and enc.codes.dtype == np.uint8


def test_round_trip_synthetic_lm_head_and_few_corrections():
    w = workload("tiny-greedy")
    W = make_weights(w)                               # N(0, 1/sqrt(d)) in bf16, V=1024, d=256
    enc = X.encode(W)
    assert np.array_equal(X.decode(enc, *W.shape), W)
    n_corr = int(np.count_nonzero(enc.corr))
    assert n_corr < 5e-3 * W.size                    # the window holds almost every weight
    assert enc.cap % 4 == 0 and enc.cap >= 4


def test_hand_encoded_group_and_correction():
    """One row of 128: the first group by hand, a tiny weight as a correction."""
    row = np.zeros(128, dtype=np.uint16)
    row[:8] = [0x3F80, 0xC000, 0x3F00, 0x0000, 0x8000, 0x4040, 0x3FC0, 0x3F40]
    #          1.0     -2.0    0.5     +0      -0      3.0     1.5     0.75
    row[9] = 0x3580                                   # 2^-20: e2 = 0x35, below the window
    enc = X.encode(row[None, :])
    assert enc.b2 == 0x40 - 6                         # -2.0 and 3.0 have e2 = 0x40
    # codes (sign << 3 | t): 1.0 -> 6, -2.0 -> 0xF, 0.5 -> 6, +0 -> 0, -0 -> 8,
    # 3.0 -> 7, 1.5 -> 6, 0.75 -> 6; low bytes verbatim
    assert enc.codes[0, 0].tolist() == [0x80, 0x00, 0x00, 0x00, 0x00, 0x40, 0xC0, 0x40,
                                        0xF6, 0x06, 0x78, 0x66]
    assert enc.codes[0, 1].tolist() == [0] * 12       # placeholder +0 for column 9
    assert enc.cap == 4
    assert enc.corr[0, 0].tolist() == [0x35800009, 0, 0, 0]
    assert np.array_equal(X.decode(enc, 1, 128), row[None, :])


def test_window_edges():
    """e2_max - 6 is the lowest pair in the window; e2_max - 7 needs a correction;
    zeros, subnormals and exponent 1 are coded (t = 0)."""
    row = np.full(128, 0x3F80, dtype=np.uint16)       # 1.0: e2 = 63
    row[1] = 57 << 8                                  # coded with t = 1
    row[2] = 56 << 8                                  # one below the window
    row[3] = 0x0001                                   # subnormal
    row[4] = 0x8000                                   # -0
    row[5] = 0x0080                                   # exponent 1
    enc = X.encode(row[None, :])
    assert enc.b2 == 57
    assert enc.codes[0, 0, 8] >> 4 == 1 and enc.codes[0, 0, 1] == 0x00
    assert [int(e) & 0x7F for e in enc.corr[0, 0] if e] == [2]
    assert np.array_equal(X.decode(enc, 1, 128), row[None, :])


def test_correction_regions_and_order():
    """Regions are 64 rows by 128 columns; slots sorted by (row, column); CAP rounds up."""
    V, d = 130, 256
    W = np.full((V, d), 0x3F80, dtype=np.uint16)
    tiny = 0x0400                                     # e2 = 4: far below the window
    spots = [(0, 5), (0, 3), (63, 127), (64, 0), (129, 200), (129, 130), (1, 3), (2, 0), (3, 1)]
    for v, k in spots:
        W[v, k] = tiny
    enc = X.encode(W)
    assert enc.corr.shape == (3, 2, 8)                # fullest region holds 6 -> CAP 8
    first = [int(e) for e in enc.corr[0, 0] if e]
    assert [((e >> 7) & 0x3F, e & 0x7F) for e in first] == [(0, 3), (0, 5), (1, 3), (2, 0), (3, 1), (63, 127)]
    assert [int(e) & 0xFFFF for e in enc.corr[2, 1] if e] == [2 | 1 << 7, 72 | 1 << 7]
    assert np.array_equal(X.decode(enc, V, d), W)


def test_device_layout_is_a_region_blocked_permutation():
    V, d = 70, 256
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (V, d // 8, 12)).astype(np.uint8)
    dev = X.device_layout(codes)
    assert dev.shape == (2, 2, 64, 16, 12)
    # Row v, group c lives in region (v // 64, c // 16) at (v % 64, c % 16).
    for v, c in [(0, 0), (5, 17), (63, 31), (64, 3), (69, 16)]:
        assert np.array_equal(dev[v // 64, c // 16, v % 64, c % 16], codes[v, c])
    assert not dev[1, :, 6:].any()                    # rows 70..127 are padding
