"""CPU oracle for the W12 LM-head weight stream (test infrastructure, not product).

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this module. The HIP library never
calls it and shares no code with it.

SpecPilot page, "Reasons": W12 is a lossless 12-bit weight format; BF16 is cut
into three 4-bit planes that the GEMM reassembles in registers, which the
authors credit with a 1.15-1.26x faster BF16 decode on dense 8-30B models.
The page gives no further detail, so the format below is this library's own
reading of it (the pages print no W12 bytes, so it is pinned to exact round
trips and hand-computed bytes instead):

* A bf16 weight is a high byte (sign, exponent bits 7..1) and a low byte
  (exponent bit 0, mantissa). The low byte is kept verbatim: two of the three
  4-bit planes. The third plane is a 4-bit code of the high byte: sign in bit 3
  and t in bits 0..2, where t = 0 stands for exponent bits 7..1 all zero (zeros,
  subnormals, exponent 1) and t = 1..7 for the pair value e2 = b2 + t - 1 of a
  window [b2, b2 + 6] chosen per tensor: b2 = max(1, largest e2 - 6) over every
  weight with e2 >= 1 (b2 = 1 if there is none).
* Every weight whose e2 is outside {0} and the window is stored as the code of a
  signed zero (t = 0, low byte 0) plus an exact correction: its bf16 bits, row
  and column. Corrections are kept per region of 64 LM-head rows by 128 columns
  (the unit the GEMM stages), in a fixed number CAP of slots per region (CAP =
  the fullest region's count rounded up to a multiple of 4, at least 4), sorted
  by (row, column), empty slots 0. A slot is the uint32
  k_local | row_local << 7 | bits << 16.
* Bytes: each row is cut into groups of 8 consecutive columns, 12 bytes per
  group: bytes 0..7 are the 8 low bytes, and byte 8 + i holds the code of
  column 2i (low nibble) and of column 2i + 1 (high nibble). `codes` below is
  indexed [row][group]; in device memory the groups are laid out by region,
  [V/64][d/128][64 rows][16 groups][12 bytes] with rows past V zero
  (device_layout), so each region the GEMM stages is one contiguous 12 KB block.

Decoding a weight = its correction bits if it has one, else
(sign << 15) | ((t ? b2 + t - 1 : 0) << 8) | low byte.
"""
from __future__ import annotations

import dataclasses

import numpy as np

ROWS_PER_SLAB = 64
COLS_PER_STAGE = 128
GROUP = 8


@dataclasses.dataclass
class W12:
    b2: int                # window start: t (1..7) means e2 = b2 + t - 1
    codes: np.ndarray      # uint8 [V][d // 8][12]
    corr: np.ndarray       # uint32 [ceil(V / 64)][d // 128][cap]
    cap: int


def window_start(W_bits: np.ndarray) -> int:
    e2 = (np.asarray(W_bits, dtype=np.uint16) >> 8) & 0x7F
    if not (e2 >= 1).any():
        return 1
    return max(1, int(e2[e2 >= 1].max()) - 6)


def encode(W_bits: np.ndarray) -> W12:
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    V, d = W_bits.shape
    assert d % COLS_PER_STAGE == 0
    b2 = window_start(W_bits)
    u = W_bits.astype(np.uint32)
    s, e2, lo = u >> 15, (u >> 8) & 0x7F, u & 0xFF
    inside = (e2 >= b2) & (e2 <= b2 + 6)
    held = (e2 == 0) | inside
    t = np.where(inside, e2 - b2 + 1, 0)
    nib = np.where(held, (s << 3) | t, s << 3).astype(np.uint32)
    low = np.where(held, lo, 0).astype(np.uint32)
    codes = np.zeros((V, d // GROUP, 12), dtype=np.uint8)
    codes[:, :, 0:8] = low.reshape(V, d // GROUP, GROUP).astype(np.uint8)
    n = nib.reshape(V, d // GROUP, GROUP)
    codes[:, :, 8:12] = (n[:, :, 0::2] | (n[:, :, 1::2] << 4)).astype(np.uint8)
    # Corrections per (slab, stage) region, in (row, column) order.
    nslab, nst = (V + ROWS_PER_SLAB - 1) // ROWS_PER_SLAB, d // COLS_PER_STAGE
    lists = [[[] for _ in range(nst)] for _ in range(nslab)]
    for v, k in zip(*np.nonzero(~held)):
        lists[v // ROWS_PER_SLAB][k // COLS_PER_STAGE].append(
            int(k % COLS_PER_STAGE) | int(v % ROWS_PER_SLAB) << 7 | int(W_bits[v, k]) << 16)
    fullest = max((len(x) for row in lists for x in row), default=0)
    cap = max(4, (fullest + 3) // 4 * 4)
    corr = np.zeros((nslab, nst, cap), dtype=np.uint32)
    for i in range(nslab):
        for j in range(nst):
            ent = sorted(lists[i][j], key=lambda e: ((e >> 7) & 0x3F, e & 0x7F))
            corr[i, j, :len(ent)] = ent
    return W12(b2, codes, corr, cap)


def decode(w: W12, V: int, d: int) -> np.ndarray:
    low = w.codes[:, :, 0:8].astype(np.uint32).reshape(V, d)
    nb = w.codes[:, :, 8:12].astype(np.uint32)
    nib = np.empty((V, d // GROUP, GROUP), dtype=np.uint32)
    nib[:, :, 0::2] = nb & 0xF
    nib[:, :, 1::2] = nb >> 4
    nib = nib.reshape(V, d)
    s, t = nib >> 3, nib & 7
    e2 = np.where(t == 0, 0, w.b2 + t - 1)
    bits = ((s << 15) | (e2 << 8) | low).astype(np.uint16)
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


def device_layout(codes: np.ndarray) -> np.ndarray:
    """codes [V][d/8][12] -> [ceil(V/64)][d/128][64][16][12], rows past V zero."""
    V, ng, _ = codes.shape
    nslab = (V + ROWS_PER_SLAB - 1) // ROWS_PER_SLAB
    pad = np.zeros((nslab * ROWS_PER_SLAB, ng, 12), dtype=np.uint8)
    pad[:V] = codes
    gps = COLS_PER_STAGE // GROUP
    return np.ascontiguousarray(
        pad.reshape(nslab, ROWS_PER_SLAB, ng // gps, gps, 12).transpose(0, 2, 1, 3, 4))
