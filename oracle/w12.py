"""CPU oracle for the W12 LM-head weight stream (test infrastructure, not product).

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this module. The HIP library never
calls it and shares no code with it.

SpecPilot page, "Reasons": W12 is a lossless 12-bit weight format; BF16 is cut
into three 4-bit planes that the GEMM reassembles in registers, which the
authors credit with a 1.15-1.26x faster BF16 decode on dense 8-30B models.
The page gives no further detail, so the format below is this library's own
reading of it (parity unpinned against the pages' bytes; pinned to exact
round trips and hand-computed bytes instead):

* 12 bits per weight: sign (1), a 4-bit exponent code, the 7 mantissa bits.
  One exponent window per tensor, [b, b + 14] with b = max(1, E_max - 14),
  E_max the largest biased exponent of any finite normal weight (b = 1 if
  there is none). Code c in 1..15 means exponent b + c - 1; code 0 with a zero
  mantissa is a signed zero.
* Every weight the window cannot hold (a smaller or larger exponent, a
  subnormal, an infinity or NaN) is stored as a signed-zero code plus an exact
  correction: its bf16 bits, row and column. Corrections are kept per region
  of 64 LM-head rows by 128 columns (the unit the GEMM stages), in a fixed
  number CAP of slots per region (CAP = the fullest region's count rounded up
  to a multiple of 4, at least 4), sorted by (row, column), empty slots 0.
  A slot is the uint32 k_local | row_local << 7 | bits << 16.
* Bytes: each row is cut into groups of 8 consecutive columns, 12 bytes per
  group: bytes 0..7 hold the low 8 bits of the 8 codes, byte 8 + i holds the
  high 4 bits of code 2i (low nibble) and of code 2i + 1 (high nibble).

Decoding a weight = its correction bits if it has one, else the code read back.
"""
from __future__ import annotations

import dataclasses

import numpy as np

ROWS_PER_SLAB = 64
COLS_PER_STAGE = 128
GROUP = 8


@dataclasses.dataclass
class W12:
    base: int              # b: code c (1..15) means biased exponent b + c - 1
    codes: np.ndarray      # uint8 [V][d // 8][12]
    corr: np.ndarray       # uint32 [ceil(V / 64)][d // 128][cap]
    cap: int


def split_bf16(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return u >> 15, (u >> 7) & 0xFF, u & 0x7F


def window_base(W_bits: np.ndarray) -> int:
    _, E, _ = split_bf16(W_bits)
    normal = (E >= 1) & (E <= 254)
    if not normal.any():
        return 1
    return max(1, int(E[normal].max()) - 14)


def encode(W_bits: np.ndarray) -> W12:
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    V, d = W_bits.shape
    assert d % COLS_PER_STAGE == 0
    b = window_base(W_bits)
    s, E, m = split_bf16(W_bits)
    zero = (E == 0) & (m == 0)
    inside = (E >= b) & (E <= b + 14) & (E >= 1) & (E <= 254)
    code = np.where(inside, (s << 11) | ((E - b + 1) << 7) | m, s << 11).astype(np.uint32)
    needs = ~(zero | inside)
    # Bytes of each group of 8 codes.
    g = code.reshape(V, d // GROUP, GROUP)
    codes = np.zeros((V, d // GROUP, 12), dtype=np.uint8)
    codes[:, :, 0:8] = (g & 0xFF).astype(np.uint8)
    hi = (g >> 8) & 0xF
    codes[:, :, 8:12] = (hi[:, :, 0::2] | (hi[:, :, 1::2] << 4)).astype(np.uint8)
    # Corrections per (slab, stage) region, in (row, column) order.
    nslab, nst = (V + ROWS_PER_SLAB - 1) // ROWS_PER_SLAB, d // COLS_PER_STAGE
    lists = [[[] for _ in range(nst)] for _ in range(nslab)]
    for v, k in zip(*np.nonzero(needs)):
        lists[v // ROWS_PER_SLAB][k // COLS_PER_STAGE].append(
            int(k % COLS_PER_STAGE) | int(v % ROWS_PER_SLAB) << 7 | int(W_bits[v, k]) << 16)
    fullest = max((len(x) for row in lists for x in row), default=0)
    cap = max(4, (fullest + 3) // 4 * 4)
    corr = np.zeros((nslab, nst, cap), dtype=np.uint32)
    for i in range(nslab):
        for j in range(nst):
            ent = sorted(lists[i][j], key=lambda e: ((e >> 7) & 0x3F, e & 0x7F))
            corr[i, j, :len(ent)] = ent
    return W12(b, codes, corr, cap)


def decode(w: W12, V: int, d: int) -> np.ndarray:
    lo = w.codes[:, :, 0:8].astype(np.uint32)
    hb = w.codes[:, :, 8:12].astype(np.uint32)
    hi = np.empty_like(lo)
    hi[:, :, 0::2] = hb & 0xF
    hi[:, :, 1::2] = hb >> 4
    code = ((hi << 8) | lo).reshape(V, d)
    s, c, m = code >> 11, (code >> 7) & 0xF, code & 0x7F
    bits = np.where(c == 0, (s << 15) | m, (s << 15) | ((c + w.base - 1) << 7) | m)
    bits = bits.astype(np.uint16)
    nslab, nst, _ = w.corr.shape
    for i in range(nslab):
        for j in range(nst):
            for e in w.corr[i, j]:
                e = int(e)
                if e == 0:
                    continue
                v = i * ROWS_PER_SLAB + ((e >> 7) & 0x3F)
                k = j * COLS_PER_STAGE + (e & 0x7F)
                bits[v, k] = e >> 16
    return bits
