"""The library's host W12 encoder (sd_w12_encode) against the W12 oracle, byte for byte,
and host-side validation of the W12 entry points. No GPU work."""
import ctypes

import numpy as np

import draft_block_verification_amd as sd
from oracle import w12 as X
from synth import make_weights, workload

lib = ctypes.CDLL(sd.LIB_PATH)
FAKE = ctypes.c_void_p(0x10000)


def same_as_oracle(W):
    codes, corr, cap, b2, V = sd.w12_encode(W)
    enc = X.encode(W)
    assert (cap, b2, V) == (enc.cap, enc.b2, W.shape[0])
    assert np.array_equal(codes, X.device_layout(enc.codes))
    assert np.array_equal(corr, enc.corr)


def test_encoder_matches_oracle_on_every_bf16_pattern():
    W = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    same_as_oracle(W[np.random.default_rng(0).permutation(512)])


def test_encoder_matches_oracle_on_lm_heads():
    same_as_oracle(make_weights(workload("tiny-greedy")))
    rng = np.random.default_rng(3)
    W = make_weights(workload("ragged-b32", V=700, d=384, name="w12-host"))
    W = W.copy()
    # Scatter tiny and huge weights (corrections) and exact zeros (coded) over the rows.
    idx = rng.integers(0, W.size, 900)
    W.reshape(-1)[idx[:300]] = 0x0400          # tiny: below the window
    W.reshape(-1)[idx[300:600]] = 0x0000       # +0
    W.reshape(-1)[idx[600:]] = 0x8001          # negative subnormal
    same_as_oracle(W)


def test_encoder_sizing_and_short_capacity():
    W = np.full((70, 256), 0x3F80, dtype=np.uint16)
    W[3, 7] = W[5, 9] = W[69, 200] = 0x0100
    cap, b2 = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.sd_w12_encode(ctypes.c_void_p(W.ctypes.data), 70, 256, None, None,
                             ctypes.byref(cap), ctypes.byref(b2)) == 0
    assert cap.value == 4 and b2.value == 0x3F - 6
    codes = np.empty((2, 2, 64, 16, 12), np.uint8)
    corr = np.empty((2, 2, 8), np.uint32)
    small = ctypes.c_int32(0)                  # too few slots
    assert lib.sd_w12_encode(ctypes.c_void_p(W.ctypes.data), 70, 256,
                             ctypes.c_void_p(codes.ctypes.data), ctypes.c_void_p(corr.ctypes.data),
                             ctypes.byref(small), ctypes.byref(b2)) == 4
    assert small.value == 4
    wide = ctypes.c_int32(8)                   # more slots than needed: stride 8, zeros after
    assert lib.sd_w12_encode(ctypes.c_void_p(W.ctypes.data), 70, 256,
                             ctypes.c_void_p(codes.ctypes.data), ctypes.c_void_p(corr.ctypes.data),
                             ctypes.byref(wide), ctypes.byref(b2)) == 0
    assert wide.value == 8
    enc = X.encode(W)
    assert np.array_equal(corr[:, :, :4], enc.corr) and not corr[:, :, 4:].any()
    assert lib.sd_w12_encode(ctypes.c_void_p(W.ctypes.data), 70, 200, None, None,
                             ctypes.byref(cap), ctypes.byref(b2)) == 2   # d % 128 != 0


def test_w12_entry_point_validation():
    class D(ctypes.Structure):
        _fields_ = [("codes", ctypes.c_void_p), ("corr", ctypes.c_void_p), ("cap", ctypes.c_int32),
                    ("b2", ctypes.c_int32)]

    def call(desc, B=1, g=9, d=2048, V=32768, ws=1 << 30):
        return lib.sd_verify_logits_w12(FAKE, ctypes.byref(desc) if desc else None, FAKE, None, None,
                                        B, g, d, V, ctypes.c_float(0.0), None, FAKE, FAKE,
                                        ctypes.c_size_t(ws), None)

    good = D(0x10000, 0x20000, 16, 56)
    assert call(None) == 1
    assert call(D(None, 0x20000, 16, 56)) == 1
    assert call(D(0x10000, 0x20000, 16, 0)) == 1           # b2 out of range
    assert call(good, d=2112) == 2                         # d % 128 != 0
    assert call(good, B=7) == 2                            # 70 rows: not the streaming regime
    assert call(D(0x10000, 0x20000, 68, 56)) == 2          # more slots than the stage holds
    assert call(D(0x10000, 0x20000, 6, 56)) == 2           # not a multiple of 4
    assert call(D(0x10008, 0x20000, 16, 56)) == 3          # codes misaligned
    assert call(good, ws=64) == 4
