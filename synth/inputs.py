"""Seeded synthetic workloads for draft-block verification.

Each workload mirrors one of the verify settings the pages describe:
block sizes of 9 (LFM2.5-DSpark blog, "Training & Architecture" and the
CPU/GPU speed-up section) and 16 (DSpark summary, "Problem definition",
parallel drafters with gamma = 16), batch 128 (DSpark summary, latency
overhead analysis), temperature 0 (LFM2.5 blog) and 1.0 (DSpark summary,
offline evaluation settings), and vocabulary / hidden sizes of the target
families the DSpark summary names (Qwen3, DeepSeek-V4 with V near 1e5).

No benchmark items are used: token ids, hidden states and draft logits are
random draws whose structure (planted accepted prefixes, code-like versus
chat-like prefix lengths, decreasing prefix-survival confidences) stands in
for real traffic.

Everything here is input synthesis. Values are drawn in float32/float64,
then rounded once to bf16 with round-to-nearest-even; both the CPU oracle
and the GPU path read the same bytes.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

# Rows of W drawn per independent generator; fixed so the bytes do not
# depend on how many threads draw them.
_W_CHUNK_ROWS = 2048


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and draw recipe of one synthetic verify workload."""
    wid: int                 # stable id, part of every seed
    name: str
    B: int                   # requests per step
    gamma: int               # drafted tokens per request
    d: int                   # hidden size
    V: int                   # vocabulary size
    T: float                 # sampling temperature (0 = greedy)
    geo_p: Sequence[float]   # planted-prefix geometric parameter per request half
    truncate: bool           # confidences drawn and truncation applied
    threshold: float = 0.3   # confidence threshold for truncation
    plant: float = 4.0       # planting magnitude along the unit draft-token row
    steps: int = 1           # distinct seeded steps the workload defines

    @property
    def rejection(self) -> bool:
        return self.T > 0.0

    @property
    def max_rows(self) -> int:
        return self.B * (self.gamma + 1)

    def geo_for_request(self, r: int) -> float:
        # The first half of the requests uses geo_p[0], the rest geo_p[-1].
        return float(self.geo_p[0] if r < self.B // 2 or len(self.geo_p) == 1
                     else self.geo_p[-1])


WORKLOADS = {
    "tiny-greedy": Workload(1, "tiny-greedy", 1, 4, 256, 1024, 0.0, (0.3,), False,
                            steps=1000),
    "greedy-block9": Workload(2, "greedy-block9", 1, 9, 2048, 32768, 0.0, (0.2,), False,
                              steps=1000),
    "rejection-b1": Workload(3, "rejection-b1", 1, 16, 4096, 151936, 1.0, (0.15,), False,
                             steps=16),
    "ragged-b32": Workload(4, "ragged-b32", 32, 16, 4096, 151936, 0.8, (0.15,), True,
                           steps=16),
    "concurrency-b128": Workload(5, "concurrency-b128", 128, 16, 7168, 129280, 1.0,
                                 (0.1, 0.5), True, steps=8),
}


def workload(key: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller V, stress planting)."""
    base = WORKLOADS[key]
    return dataclasses.replace(base, **overrides) if overrides else base


@dataclasses.dataclass
class StepInputs:
    """One verify step's inputs, as host arrays in the path's storage types."""
    draft_tokens: np.ndarray            # int32 [B][gamma]
    planted: np.ndarray                 # int32 [B] planted prefix length (diagnostic)
    hidden: np.ndarray                  # uint16 (bf16 bits) [B][gamma+1][d]
    draft_logits: Optional[np.ndarray]  # uint16 (bf16 bits) [B][gamma][V] or None
    conf: Optional[np.ndarray]          # float32 [B][gamma] or None
    u_accept: np.ndarray                # float32 [B][gamma] in [0, 1)
    u_resample: np.ndarray              # float32 [B][gamma+1] in [0, 1)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_weights(w: Workload, seed: int = 0) -> np.ndarray:
    """LM-head weight W[V][d] as bf16 bits, entries N(0, 1) / sqrt(d) before rounding."""
    out = np.empty((w.V, w.d), dtype=np.uint16)
    scale = np.float32(1.0 / np.sqrt(w.d))
    starts = list(range(0, w.V, _W_CHUNK_ROWS))

    def fill(ci: int) -> None:
        r0 = starts[ci]
        r1 = min(w.V, r0 + _W_CHUNK_ROWS)
        g = _rng(seed, w.wid, 0, ci)
        out[r0:r1] = bf16_round(g.standard_normal((r1 - r0, w.d), dtype=np.float32) * scale)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(starts))))
    return out


def make_step(w: Workload, W: np.ndarray, step: int, seed: int = 0) -> StepInputs:
    """Draw one step's inputs; draws follow a fixed order so every field is reproducible.

    Order: draft tokens, planted prefix lengths, hidden states (then planting),
    draft logits, confidences, acceptance uniforms, resample uniforms.
    """
    B, g, d, V = w.B, w.gamma, w.d, w.V
    rng = _rng(seed, w.wid, 1, step)
    x = rng.integers(0, V, size=(B, g), dtype=np.int64).astype(np.int32)
    # Trials to first success minus one, capped at gamma.
    k = np.array([min(int(rng.geometric(w.geo_for_request(r))) - 1, g) for r in range(B)],
                 dtype=np.int32)
    h = rng.standard_normal((B, g + 1, d), dtype=np.float32).astype(np.float64)
    for r in range(B):
        for j in range(int(k[r])):
            wr = bf16_to_f32(W[x[r, j]]).astype(np.float64)
            h[r, j] += w.plant * wr / np.sqrt(np.dot(wr, wr))
    hidden = bf16_round(h.astype(np.float32))

    draft_logits = None
    if w.rejection:
        draft_logits = np.empty((B, g, V), dtype=np.uint16)
        subs = [int(s) for s in rng.integers(0, 2**63 - 1, size=B, dtype=np.int64)]

        def fill(r: int) -> None:
            gr = _rng(subs[r])
            lq = gr.standard_normal((g, V), dtype=np.float32)
            lq[np.arange(g), x[r]] += np.float32(6.0)
            draft_logits[r] = bf16_round(lq)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(B)))

    conf = None
    if w.truncate:
        c1 = rng.uniform(0.6, 1.0, size=(B, 1))
        ratios = rng.uniform(0.7, 1.0, size=(B, g - 1))
        conf = np.cumprod(np.concatenate([c1, ratios], axis=1), axis=1).astype(np.float32)

    u_accept = rng.random((B, g), dtype=np.float32)
    u_resample = rng.random((B, g + 1), dtype=np.float32)
    return StepInputs(x, k, hidden, draft_logits, conf, u_accept, u_resample)
