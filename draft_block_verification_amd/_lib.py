"""ctypes binding of libsdverify.so: argument marshalling only.

Every step of the verify path runs in the library's HIP kernels; this module
checks tensor dtypes, devices and shapes, allocates outputs with torch when
the caller does not pass them, and forwards raw device pointers plus the
current HIP stream. There is no fallback: if the shared library is missing,
importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdverify.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)

_i32, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_SIGS = {
    "sd_abi_version": (_i32, []),
    "sd_status_string": (ctypes.c_char_p, [_i32]),
    "sd_verify_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "sd_accept_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "sd_workspace_init": (_i32, [_vp, _sz, _vp]),
    "sd_device_flags": (_i32, [_vp, _vp, ctypes.POINTER(ctypes.c_uint32), _i32]),
    "sd_truncate_by_confidence": (_i32, [_vp, _i32, _i32, _f32, _vp, _vp, _vp]),
    "sd_schedule_prefix": (_i32, [_vp, _vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp]),
    "sd_w12_encode": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "sd_verify_logits_w12": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                    _vp, _sz, _vp]),
    "sd_verify_contraction_w12": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                         _sz, _vp]),
    "sd_verify_greedy_w12": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                    _vp, _vp, _sz, _vp]),
    "sd_verify_logits": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                _vp, _sz, _vp]),
    "sd_lm_head_block_bytes": (_sz, [_i32, _i32]),
    "sd_lm_head_block": (_i32, [_vp, _i32, _i32, _vp, _sz, _vp]),
    "sd_verify_logits_blocked": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp,
                                        _vp, _vp, _sz, _vp]),
    "sd_verify_contraction_blocked": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp,
                                             _vp, _sz, _vp]),
    "sd_verify_greedy_blocked": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                        _vp, _vp, _vp, _sz, _vp]),
    "sd_verify_contraction": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _sz,
                                     _vp]),
    "sd_verify_greedy": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                _vp, _sz, _vp]),
    "sd_verify_greedy_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                        _vp, _vp, _vp, _vp]),
    "sd_accept_greedy": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "sd_accept_rejection": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _f32,
                                   _vp, _vp, _vp, _vp, _sz, _vp]),
    "sd_accept_rejection_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                      _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sd_verify_rejection": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                   _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz,
                                   _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)

# Layout of sd_row_stats (32 bytes).
ROW_STATS_DTYPE = np.dtype([("argmax", "<i4"), ("top1", "<f4"), ("top2", "<f4"), ("pos", "<i4"),
                            ("lse", "<f8"), ("z_draft", "<f8")])
assert ROW_STATS_DTYPE.itemsize == 32

FLAG_VERIFY_LEN, FLAG_ROW_OFFSETS, FLAG_NO_RESIDUAL, FLAG_WAIT = 1, 2, 4, 8
LM_HEAD_ROWS, LM_HEAD_BLOCKED, LM_HEAD_W12 = 0, 1, 2


class SdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_lib.sd_status_string(status).decode()} (status {status})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SdError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def abi_version() -> int:
    return int(_lib.sd_abi_version())


def verify_workspace_bytes(B: int, gamma: int, d: int, V: int) -> int:
    return int(_lib.sd_verify_workspace_bytes(B, gamma, d, V))


def accept_workspace_bytes(B: int, gamma: int, V: int) -> int:
    return int(_lib.sd_accept_workspace_bytes(B, gamma, V))


def new_workspace(nbytes: int, device, stream=None) -> torch.Tensor:
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    _check("sd_workspace_init", _lib.sd_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))
    return ws


def device_flags(workspace: torch.Tensor, clear: bool = True, stream=None) -> int:
    out = ctypes.c_uint32(0)
    _check("sd_device_flags", _lib.sd_device_flags(_ptr(workspace), _stream(stream),
                                                   ctypes.byref(out), int(clear)))
    return int(out.value)


def new_stats(B: int, gamma: int, device) -> torch.Tensor:
    """Device buffer for B * (gamma + 1) sd_row_stats records (viewed as int64 [rows][4])."""
    return torch.empty((B * (gamma + 1), 4), dtype=torch.int64, device=device)


def stats_to_numpy(stats: torch.Tensor) -> np.ndarray:
    """Host copy of a stats buffer as a structured array with the sd_row_stats fields."""
    return stats.detach().cpu().numpy().view(ROW_STATS_DTYPE).reshape(-1)


# ------------------------------------------------------------------ entry points

def sd_truncate_by_confidence(conf: torch.Tensor, threshold: float,
                              verify_len: Optional[torch.Tensor] = None,
                              row_offsets: Optional[torch.Tensor] = None, stream=None):
    _need(conf, "conf", torch.float32)
    B, g = conf.shape
    if verify_len is None:
        verify_len = torch.empty(B, dtype=torch.int32, device=conf.device)
    if row_offsets is None:
        row_offsets = torch.empty(B + 1, dtype=torch.int32, device=conf.device)
    _need(verify_len, "verify_len", torch.int32, (B,))
    _need(row_offsets, "row_offsets", torch.int32, (B + 1,))
    _check("sd_truncate_by_confidence",
           _lib.sd_truncate_by_confidence(_ptr(conf), B, g, float(threshold), _ptr(verify_len),
                                          _ptr(row_offsets), _stream(stream)))
    return verify_len, row_offsets


SCHED_EARLY_STOP, SCHED_TOP_K = 0, 1
SCHED_MAX_CANDIDATES = 16384


def sd_schedule_prefix(conf: torch.Tensor, sps: torch.Tensor, mode: int = SCHED_EARLY_STOP,
                       conf_stale: Optional[torch.Tensor] = None,
                       verify_len: Optional[torch.Tensor] = None,
                       row_offsets: Optional[torch.Tensor] = None, stream=None):
    """Hardware-aware prefix scheduler; same outputs as sd_truncate_by_confidence."""
    _need(conf, "conf", torch.float32)
    R, g = conf.shape
    _need(sps, "sps", torch.float32)
    if conf_stale is not None:
        _need(conf_stale, "conf_stale", torch.float32, (R, g))
    if verify_len is None:
        verify_len = torch.empty(R, dtype=torch.int32, device=conf.device)
    if row_offsets is None:
        row_offsets = torch.empty(R + 1, dtype=torch.int32, device=conf.device)
    _need(verify_len, "verify_len", torch.int32, (R,))
    _need(row_offsets, "row_offsets", torch.int32, (R + 1,))
    _check("sd_schedule_prefix",
           _lib.sd_schedule_prefix(_ptr(conf), _ptr(conf_stale), R, g, _ptr(sps), sps.numel(),
                                   int(mode), _ptr(verify_len), _ptr(row_offsets),
                                   _stream(stream)))
    return verify_len, row_offsets


def profile_sps(R: int, gamma: int, lm_head: torch.Tensor, temperature: float = 0.0,
                breakpoints: Optional[Sequence[int]] = None, repeats: int = 10,
                stream=None) -> torch.Tensor:
    """Steps-per-second table SPS(B), B = 0 .. R * (gamma + 1), of this library's own verify
    call (sd_verify_logits) for R requests with gamma drafts each.

    The verify cost is a staircase in the number of rows B (the contraction works on
    row tiles), so it is timed at the top of each stair -- every multiple of 256 rows
    and the full capacity, by default -- and every B takes the rate of the first timed
    point at or above it. Returns fp32 [R * (gamma + 1) + 1] on lm_head's device.
    """
    _need(lm_head, "lm_head", torch.bfloat16)
    V, d = lm_head.shape
    dev = lm_head.device
    cap = R * (gamma + 1)
    if breakpoints is None:
        breakpoints = sorted({min(cap, max(R, 256 * i)) for i in range(1, cap // 256 + 1)} | {cap})
    breakpoints = sorted({int(b) for b in breakpoints if R <= int(b) <= cap} | {cap})
    gen = torch.Generator(device="cpu").manual_seed(1234)
    hidden = (torch.randn((R, gamma + 1, d), generator=gen) / 4).to(torch.bfloat16).to(dev)
    drafts = torch.randint(0, V, (R, gamma), generator=gen, dtype=torch.int32).to(dev)
    stats = new_stats(R, gamma, dev)
    logits = (torch.empty((cap, V), dtype=torch.float32, device=dev) if temperature > 0
              else None)
    ws = new_workspace(verify_workspace_bytes(R, gamma, d, V), dev, stream)
    st = torch.cuda.Stream(device=dev) if stream is None else stream
    times = []
    for rows in breakpoints:
        extra = rows - R
        L = [min(gamma, max(0, extra - gamma * r)) for r in range(R)]
        offs = [0]
        for x in L:
            offs.append(offs[-1] + x + 1)
        vl = torch.tensor(L, dtype=torch.int32, device=dev)
        ro = torch.tensor(offs, dtype=torch.int32, device=dev)
        with torch.cuda.stream(st):
            for _ in range(2):
                sd_verify_logits(hidden, lm_head, drafts, vl, ro, temperature, logits, stats, ws,
                                 stream=st)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(repeats):
                sd_verify_logits(hidden, lm_head, drafts, vl, ro, temperature, logits, stats, ws,
                                 stream=st)
            e1.record(st)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / repeats)
    sps = torch.empty(cap + 1, dtype=torch.float32)
    i = 0
    for B in range(cap + 1):
        while breakpoints[i] < B:
            i += 1
        sps[B] = 1e3 / times[i]
    return sps.to(dev)


class _SdW12(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("corr", ctypes.c_void_p), ("cap", ctypes.c_int32),
                ("b2", ctypes.c_int32)]


def w12_encode(W_bits: np.ndarray):
    """Host W12 encoding of a bf16 LM head (uint16 bit patterns [V][d]) by the library's
    sd_w12_encode: returns (codes uint8 [V/64][d/128][64][16][12] (region-blocked),
    corr uint32 [V/64][d/128][cap], cap, b2, V)."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    V, d = W_bits.shape
    cap, b2 = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("sd_w12_encode", _lib.sd_w12_encode(W_bits.ctypes.data, V, d, None, None,
                                               ctypes.byref(cap), ctypes.byref(b2)))
    codes = np.empty(((V + 63) // 64, d // 128, 64, 16, 12), dtype=np.uint8)
    corr = np.empty(((V + 63) // 64, d // 128, cap.value), dtype=np.uint32)
    _check("sd_w12_encode", _lib.sd_w12_encode(W_bits.ctypes.data, V, d, codes.ctypes.data,
                                               corr.ctypes.data, ctypes.byref(cap),
                                               ctypes.byref(b2)))
    return codes, corr, int(cap.value), int(b2.value), V


class W12Weights:
    """A W12 LM head in device memory: 12-byte groups, correction slots, window start.
    Pass it as `lm_head` to sd_verify_logits / sd_verify_greedy / VerifyRound."""

    def __init__(self, codes: np.ndarray, corr: np.ndarray, cap: int, b2: int, V: int,
                 device="cuda"):
        self.V, self.d = int(V), codes.shape[1] * 128
        self.cap, self.b2 = int(cap), int(b2)
        self.codes = torch.from_numpy(np.ascontiguousarray(codes)).to(device)
        self.corr = torch.from_numpy(np.ascontiguousarray(corr).view(np.int32)).to(device)
        self.shape = (self.V, self.d)
        self.nbytes = self.codes.numel() + 4 * self.corr.numel()
        self._desc = _SdW12(self.codes.data_ptr(), self.corr.data_ptr(), self.cap, self.b2)

    @classmethod
    def from_bf16(cls, W_bits: np.ndarray, device="cuda") -> "W12Weights":
        return cls(*w12_encode(W_bits), device=device)

    def descriptor(self):
        return ctypes.byref(self._desc)


def sd_verify_logits_w12(hidden, lm_head: W12Weights, *args, **kwargs):
    return sd_verify_logits(hidden, lm_head, *args, **kwargs)


def sd_verify_contraction_w12(hidden, lm_head: W12Weights, *args, **kwargs):
    return sd_verify_contraction(hidden, lm_head, *args, **kwargs)


def sd_verify_greedy_w12(hidden, lm_head: W12Weights, *args, **kwargs):
    return sd_verify_greedy(hidden, lm_head, *args, **kwargs)


class BlockedWeights:
    """A bf16 LM head re-laid once into slab blocks (sd_lm_head_block) so the streaming
    contraction reads each stage as one contiguous 16 KB block. Same values as the
    [V][d] tensor; pass it as `lm_head` to sd_verify_logits / sd_verify_greedy /
    VerifyRound (the streaming regime: d % 128 == 0, B * (gamma + 1) <= 64)."""

    def __init__(self, lm_head: torch.Tensor, stream=None):
        _need(lm_head, "lm_head", torch.bfloat16)
        V, d = lm_head.shape
        nbytes = int(_lib.sd_lm_head_block_bytes(V, d))
        if nbytes == 0:
            raise ValueError(f"no blocked layout for a [{V}][{d}] LM head (d % 128 != 0)")
        self.V, self.d, self.shape, self.nbytes = int(V), int(d), (int(V), int(d)), nbytes
        self.buf = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=lm_head.device)
        _check("sd_lm_head_block", _lib.sd_lm_head_block(_ptr(lm_head), V, d, _ptr(self.buf),
                                                         nbytes, _stream(stream)))


def _lm_head(lm_head, d):
    """(pointer or descriptor, V, entry-point suffix) of a bf16 LM head tensor,
    W12Weights or BlockedWeights."""
    if isinstance(lm_head, (W12Weights, BlockedWeights)):
        if lm_head.d != d:
            raise ValueError("lm_head must be [V][d] with the hidden size of `hidden`")
        if isinstance(lm_head, W12Weights):
            return lm_head.descriptor(), lm_head.V, "_w12"
        return _ptr(lm_head.buf), lm_head.V, "_blocked"
    _need(lm_head, "lm_head", torch.bfloat16)
    if lm_head.shape[1] != d:
        raise ValueError("lm_head must be [V][d] with the hidden size of `hidden`")
    return _ptr(lm_head), lm_head.shape[0], ""


def sd_verify_logits(hidden: torch.Tensor, lm_head: torch.Tensor,
                     draft_tokens: Optional[torch.Tensor] = None,
                     verify_len: Optional[torch.Tensor] = None,
                     row_offsets: Optional[torch.Tensor] = None, temperature: float = 0.0,
                     logits: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (logits or None, stats). Pass logits=True to have one allocated.
    lm_head: bf16 [V][d] tensor, W12Weights (then sd_verify_logits_w12 runs) or
    BlockedWeights (sd_verify_logits_blocked)."""
    _need(hidden, "hidden", torch.bfloat16)
    B, g1, d = hidden.shape
    g = g1 - 1
    head, V, fmt = _lm_head(lm_head, d)
    dev = hidden.device
    if draft_tokens is not None:
        _need(draft_tokens, "draft_tokens", torch.int32, (B, g))
    if verify_len is not None:
        _need(verify_len, "verify_len", torch.int32, (B,))
    if row_offsets is not None:
        _need(row_offsets, "row_offsets", torch.int32, (B + 1,))
    if logits is True:
        logits = torch.empty((B * g1, V), dtype=torch.float32, device=dev)
    if logits is not None:
        _need(logits, "logits", torch.float32, (B * g1, V))
    if stats is None:
        stats = new_stats(B, g, dev)
    _need(stats, "stats", torch.int64, (B * g1, 4))
    if workspace is None:
        workspace = new_workspace(verify_workspace_bytes(B, g, d, V), dev, stream)
    name = "sd_verify_logits" + fmt
    _check(name, getattr(_lib, name)(_ptr(hidden), head, _ptr(draft_tokens), _ptr(verify_len),
                                     _ptr(row_offsets), B, g, d, V, float(temperature),
                                     _ptr(logits), _ptr(stats), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))
    return logits, stats


def sd_verify_contraction(hidden: torch.Tensor, lm_head: torch.Tensor,
                          verify_len: Optional[torch.Tensor] = None,
                          row_offsets: Optional[torch.Tensor] = None, temperature: float = 0.0,
                          logits: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """The contraction stage alone (logits and workspace partials, no row statistics).
    lm_head: bf16 [V][d] tensor, W12Weights (then sd_verify_contraction_w12 runs) or
    BlockedWeights (sd_verify_contraction_blocked)."""
    _need(hidden, "hidden", torch.bfloat16)
    B, g1, d = hidden.shape
    head, V, fmt = _lm_head(lm_head, d)
    if logits is not None:
        _need(logits, "logits", torch.float32, (B * g1, V))
    if workspace is None:
        workspace = new_workspace(verify_workspace_bytes(B, g1 - 1, d, V), hidden.device, stream)
    name = "sd_verify_contraction" + fmt
    _check(name, getattr(_lib, name)(_ptr(hidden), head, _ptr(verify_len), _ptr(row_offsets), B,
                                     g1 - 1, d, V, float(temperature), _ptr(logits),
                                     _ptr(workspace), workspace.numel(), _stream(stream)))
    return logits


def sd_verify_greedy(hidden: torch.Tensor, lm_head: torch.Tensor, draft_tokens: torch.Tensor,
                     verify_len: Optional[torch.Tensor] = None,
                     row_offsets: Optional[torch.Tensor] = None,
                     stats: Optional[torch.Tensor] = None,
                     accept_len: Optional[torch.Tensor] = None,
                     next_token: Optional[torch.Tensor] = None,
                     counters: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """Greedy verify in one call: returns (stats, accept_len, next_token).
    lm_head: bf16 [V][d] tensor, W12Weights (then sd_verify_greedy_w12 runs) or
    BlockedWeights (sd_verify_greedy_blocked)."""
    _need(hidden, "hidden", torch.bfloat16)
    B, g1, d = hidden.shape
    g = g1 - 1
    head, V, fmt = _lm_head(lm_head, d)
    dev = hidden.device
    _need(draft_tokens, "draft_tokens", torch.int32, (B, g))
    if verify_len is not None:
        _need(verify_len, "verify_len", torch.int32, (B,))
    if row_offsets is not None:
        _need(row_offsets, "row_offsets", torch.int32, (B + 1,))
    stats = new_stats(B, g, dev) if stats is None else stats
    _need(stats, "stats", torch.int64, (B * g1, 4))
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    next_token = torch.empty(B, dtype=torch.int32, device=dev) if next_token is None else next_token
    _need(accept_len, "accept_len", torch.int32, (B,))
    _need(next_token, "next_token", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    if workspace is None:
        workspace = new_workspace(verify_workspace_bytes(B, g, d, V), dev, stream)
    name = "sd_verify_greedy" + fmt
    _check(name, getattr(_lib, name)(_ptr(hidden), head, _ptr(draft_tokens), _ptr(verify_len),
                                     _ptr(row_offsets), B, g, d, V, _ptr(stats), _ptr(accept_len),
                                     _ptr(next_token), _ptr(counters), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))
    return stats, accept_len, next_token


NOALLOC_SCRATCH_BYTES = 16 << 20


def sd_verify_greedy_noalloc(hidden: torch.Tensor, lm_head: torch.Tensor,
                             draft_tokens: torch.Tensor, verify_len: Optional[torch.Tensor] = None,
                             row_offsets: Optional[torch.Tensor] = None,
                             stats: torch.Tensor = None, accept_len: torch.Tensor = None,
                             next_token: torch.Tensor = None,
                             counters: Optional[torch.Tensor] = None,
                             flags: Optional[torch.Tensor] = None, stream=None):
    """sd_verify_greedy with the library's own per-GPU scratch instead of a workspace.
    The caller passes every output (stats, accept_len, next_token; counters and the
    uint32 flag word optional), so the call allocates nothing; bf16 [V][d] LM head."""
    _need(hidden, "hidden", torch.bfloat16)
    B, g1, d = hidden.shape
    g = g1 - 1
    _need(lm_head, "lm_head", torch.bfloat16)
    V = lm_head.shape[0]
    _need(lm_head, "lm_head", torch.bfloat16, (V, d))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, g))
    if verify_len is not None:
        _need(verify_len, "verify_len", torch.int32, (B,))
    if row_offsets is not None:
        _need(row_offsets, "row_offsets", torch.int32, (B + 1,))
    if stats is None or accept_len is None or next_token is None:
        raise ValueError("sd_verify_greedy_noalloc: pass stats, accept_len and next_token")
    _need(stats, "stats", torch.int64, (B * g1, 4))
    _need(accept_len, "accept_len", torch.int32, (B,))
    _need(next_token, "next_token", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    if flags is not None:
        _need(flags, "flags", torch.int32, (1,))
    _check("sd_verify_greedy_noalloc",
           _lib.sd_verify_greedy_noalloc(_ptr(hidden), _ptr(lm_head), _ptr(draft_tokens),
                                         _ptr(verify_len), _ptr(row_offsets), B, g, d, V,
                                         _ptr(stats), _ptr(accept_len), _ptr(next_token),
                                         _ptr(counters), _ptr(flags), _stream(stream)))
    return stats, accept_len, next_token


def sd_accept_greedy(stats: torch.Tensor, draft_tokens: torch.Tensor,
                     verify_len: Optional[torch.Tensor] = None,
                     row_offsets: Optional[torch.Tensor] = None,
                     accept_len: Optional[torch.Tensor] = None,
                     next_token: Optional[torch.Tensor] = None,
                     counters: Optional[torch.Tensor] = None, stream=None):
    _need(draft_tokens, "draft_tokens", torch.int32)
    B, g = draft_tokens.shape
    dev = draft_tokens.device
    _need(stats, "stats", torch.int64, (B * (g + 1), 4))
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    next_token = torch.empty(B, dtype=torch.int32, device=dev) if next_token is None else next_token
    _need(accept_len, "accept_len", torch.int32, (B,))
    _need(next_token, "next_token", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    _check("sd_accept_greedy",
           _lib.sd_accept_greedy(_ptr(stats), _ptr(draft_tokens), _ptr(verify_len),
                                 _ptr(row_offsets), B, g, _ptr(accept_len), _ptr(next_token),
                                 _ptr(counters), _stream(stream)))
    return accept_len, next_token


def sd_accept_rejection(logits: torch.Tensor, stats: torch.Tensor, draft_logits: torch.Tensor,
                        draft_tokens: torch.Tensor, verify_len: Optional[torch.Tensor],
                        row_offsets: Optional[torch.Tensor], u_accept: torch.Tensor,
                        u_resample: torch.Tensor, temperature: float,
                        accept_len: Optional[torch.Tensor] = None,
                        next_token: Optional[torch.Tensor] = None,
                        counters: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    accept_len, next_token, _ = _accept_rejection(
        "sd_accept_rejection", logits, stats, draft_logits, draft_tokens, verify_len, row_offsets,
        u_accept, u_resample, temperature, accept_len, next_token, counters, None, workspace,
        stream)
    return accept_len, next_token


def sd_accept_rejection_ex(logits: torch.Tensor, stats: torch.Tensor, draft_logits: torch.Tensor,
                           draft_tokens: torch.Tensor, verify_len: Optional[torch.Tensor],
                           row_offsets: Optional[torch.Tensor], u_accept: torch.Tensor,
                           u_resample: torch.Tensor, temperature: float,
                           accept_len: Optional[torch.Tensor] = None,
                           next_token: Optional[torch.Tensor] = None,
                           counters: Optional[torch.Tensor] = None,
                           accept_rate: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """sd_accept_rejection plus accept_rate float64 [B][gamma] (allocated when None)."""
    B, g = draft_tokens.shape
    if accept_rate is None:
        accept_rate = torch.empty((B, g), dtype=torch.float64, device=draft_tokens.device)
    return _accept_rejection("sd_accept_rejection_ex", logits, stats, draft_logits, draft_tokens,
                             verify_len, row_offsets, u_accept, u_resample, temperature,
                             accept_len, next_token, counters, accept_rate, workspace, stream)


def _accept_rejection(name, logits, stats, draft_logits, draft_tokens, verify_len, row_offsets,
                      u_accept, u_resample, temperature, accept_len, next_token, counters,
                      accept_rate, workspace, stream):
    _need(draft_tokens, "draft_tokens", torch.int32)
    B, g = draft_tokens.shape
    dev = draft_tokens.device
    _need(draft_logits, "draft_logits", torch.bfloat16)
    V = draft_logits.shape[2]
    _need(draft_logits, "draft_logits", torch.bfloat16, (B, g, V))
    _need(logits, "logits", torch.float32, (B * (g + 1), V))
    _need(stats, "stats", torch.int64, (B * (g + 1), 4))
    _need(u_accept, "u_accept", torch.float32, (B, g))
    _need(u_resample, "u_resample", torch.float32, (B, g + 1))
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    next_token = torch.empty(B, dtype=torch.int32, device=dev) if next_token is None else next_token
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    if workspace is None:
        workspace = new_workspace(accept_workspace_bytes(B, g, V), dev, stream)
    args = [_ptr(logits), _ptr(stats), _ptr(draft_logits), _ptr(draft_tokens), _ptr(verify_len),
            _ptr(row_offsets), _ptr(u_accept), _ptr(u_resample), B, g, V, float(temperature),
            _ptr(accept_len), _ptr(next_token), _ptr(counters)]
    if name == "sd_accept_rejection_ex":
        _need(accept_rate, "accept_rate", torch.float64, (B, g))
        args.append(_ptr(accept_rate))
    args += [_ptr(workspace), workspace.numel(), _stream(stream)]
    _check(name, getattr(_lib, name)(*args))
    return accept_len, next_token, accept_rate


def sd_verify_rejection(hidden: torch.Tensor, lm_head, draft_tokens: torch.Tensor,
                        draft_logits: torch.Tensor, verify_len: Optional[torch.Tensor],
                        row_offsets: Optional[torch.Tensor], u_accept: torch.Tensor,
                        u_resample: torch.Tensor, temperature: float,
                        logits: Optional[torch.Tensor] = None,
                        stats: Optional[torch.Tensor] = None,
                        accept_len: Optional[torch.Tensor] = None,
                        next_token: Optional[torch.Tensor] = None,
                        counters: Optional[torch.Tensor] = None,
                        accept_rate: Optional[torch.Tensor] = None,
                        ws_verify: Optional[torch.Tensor] = None,
                        ws_accept: Optional[torch.Tensor] = None, stream=None):
    """Rejection verify in one call: returns (logits, stats, accept_len, next_token).
    lm_head: bf16 [V][d] tensor, BlockedWeights or W12Weights; accept_rate float64
    [B][gamma] or None (not computed)."""
    _need(hidden, "hidden", torch.bfloat16)
    B, g1, d = hidden.shape
    g = g1 - 1
    head, V, fmt = _lm_head(lm_head, d)
    layout = {"": LM_HEAD_ROWS, "_blocked": LM_HEAD_BLOCKED, "_w12": LM_HEAD_W12}[fmt]
    dev = hidden.device
    _need(draft_tokens, "draft_tokens", torch.int32, (B, g))
    _need(draft_logits, "draft_logits", torch.bfloat16, (B, g, V))
    if verify_len is not None:
        _need(verify_len, "verify_len", torch.int32, (B,))
    if row_offsets is not None:
        _need(row_offsets, "row_offsets", torch.int32, (B + 1,))
    _need(u_accept, "u_accept", torch.float32, (B, g))
    _need(u_resample, "u_resample", torch.float32, (B, g1))
    if logits is None:
        logits = torch.empty((B * g1, V), dtype=torch.float32, device=dev)
    _need(logits, "logits", torch.float32, (B * g1, V))
    if stats is None:
        stats = new_stats(B, g, dev)
    _need(stats, "stats", torch.int64, (B * g1, 4))
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    next_token = torch.empty(B, dtype=torch.int32, device=dev) if next_token is None else next_token
    _need(accept_len, "accept_len", torch.int32, (B,))
    _need(next_token, "next_token", torch.int32, (B,))
    if counters is not None:
        _need(counters, "counters", torch.int64, (2,))
    if accept_rate is not None:
        _need(accept_rate, "accept_rate", torch.float64, (B, g))
    if ws_verify is None:
        ws_verify = new_workspace(verify_workspace_bytes(B, g, d, V), dev, stream)
    if ws_accept is None:
        ws_accept = new_workspace(accept_workspace_bytes(B, g, V), dev, stream)
    _check("sd_verify_rejection", _lib.sd_verify_rejection(
        _ptr(hidden), head, layout, _ptr(draft_logits), _ptr(draft_tokens), _ptr(verify_len),
        _ptr(row_offsets), _ptr(u_accept), _ptr(u_resample), B, g, d, V, float(temperature),
        _ptr(logits), _ptr(stats), _ptr(accept_len), _ptr(next_token), _ptr(counters),
        _ptr(accept_rate), _ptr(ws_verify), ws_verify.numel(), _ptr(ws_accept),
        ws_accept.numel(), _stream(stream)))
    return logits, stats, accept_len, next_token


# --------------------------------------------------------------- a whole round

class VerifyRound:
    """Buffers for repeated verify rounds of one shape; each run() enqueues the whole path.

    truncate -> verify logits -> accept (greedy when temperature == 0, else rejection),
    all on one stream with no host synchronisation. The verify and accept steps run
    through sd_verify_greedy at temperature 0 and sd_verify_rejection otherwise (fewer
    launches, for every LM-head format); fused=False keeps the separate sd_verify_logits
    + sd_accept_* calls.
    """

    def __init__(self, B: int, gamma: int, d: int, V: int, temperature: float,
                 truncate: bool, threshold: float = 0.3, device="cuda", stream=None,
                 fused: bool = True, accept_rate: bool = False, scheduler: Optional[int] = None,
                 sps: Optional[torch.Tensor] = None):
        self.B, self.gamma, self.d, self.V = B, gamma, d, V
        # With a scheduler mode (SCHED_EARLY_STOP / SCHED_TOP_K) and an SPS table, the
        # prefix scheduler replaces the confidence threshold.
        self.scheduler, self.sps = scheduler, sps
        if scheduler is not None and (not truncate or sps is None):
            raise ValueError("a scheduler needs truncate=True and an SPS table")
        self.fused = fused
        self.T, self.truncate, self.threshold = float(temperature), truncate, float(threshold)
        dev = torch.device(device)
        rows = B * (gamma + 1)
        self.verify_len = torch.empty(B, dtype=torch.int32, device=dev) if truncate else None
        self.row_offsets = torch.empty(B + 1, dtype=torch.int32, device=dev) if truncate else None
        self.stats = new_stats(B, gamma, dev)
        self.logits = (torch.empty((rows, V), dtype=torch.float32, device=dev)
                       if self.T > 0 else None)
        self.accept_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.next_token = torch.empty(B, dtype=torch.int32, device=dev)
        self.counters = torch.zeros(2, dtype=torch.int64, device=dev)
        self.ws_verify = new_workspace(verify_workspace_bytes(B, gamma, d, V), dev, stream)
        self.ws_accept = (new_workspace(accept_workspace_bytes(B, gamma, V), dev, stream)
                          if self.T > 0 else None)
        # Analytic acceptance rate per verified draft position (rejection rounds only).
        self.accept_rate = (torch.empty((B, gamma), dtype=torch.float64, device=dev)
                            if accept_rate and self.T > 0 else None)

    def run(self, hidden, lm_head, draft_tokens, conf=None, draft_logits=None, u_accept=None,
            u_resample=None, stream=None, conf_stale=None):
        if self.truncate and self.scheduler is not None:
            sd_schedule_prefix(conf, self.sps, self.scheduler,
                               conf_stale if self.scheduler == SCHED_TOP_K else None,
                               self.verify_len, self.row_offsets, stream=stream)
        elif self.truncate:
            sd_truncate_by_confidence(conf, self.threshold, self.verify_len, self.row_offsets,
                                      stream=stream)
        if self.T == 0 and self.fused:
            sd_verify_greedy(hidden, lm_head, draft_tokens, self.verify_len, self.row_offsets,
                             self.stats, self.accept_len, self.next_token, self.counters,
                             self.ws_verify, stream=stream)
            return self.accept_len, self.next_token
        if self.T > 0 and self.fused:
            sd_verify_rejection(hidden, lm_head, draft_tokens, draft_logits, self.verify_len,
                                self.row_offsets, u_accept, u_resample, self.T, self.logits,
                                self.stats, self.accept_len, self.next_token, self.counters,
                                self.accept_rate, self.ws_verify, self.ws_accept, stream=stream)
            return self.accept_len, self.next_token
        sd_verify_logits(hidden, lm_head, draft_tokens, self.verify_len, self.row_offsets,
                         self.T, self.logits, self.stats, self.ws_verify, stream=stream)
        if self.T > 0 and self.accept_rate is not None:
            sd_accept_rejection_ex(self.logits, self.stats, draft_logits, draft_tokens,
                                   self.verify_len, self.row_offsets, u_accept, u_resample,
                                   self.T, self.accept_len, self.next_token, self.counters,
                                   self.accept_rate, self.ws_accept, stream=stream)
        elif self.T > 0:
            sd_accept_rejection(self.logits, self.stats, draft_logits, draft_tokens,
                                self.verify_len, self.row_offsets, u_accept, u_resample, self.T,
                                self.accept_len, self.next_token, self.counters, self.ws_accept,
                                stream=stream)
        else:
            sd_accept_greedy(self.stats, draft_tokens, self.verify_len, self.row_offsets,
                             self.accept_len, self.next_token, self.counters, stream=stream)
        return self.accept_len, self.next_token
