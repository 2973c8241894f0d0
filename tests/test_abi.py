"""The C ABI on the host: exported symbols, workspace sizing, argument validation.

Nothing here launches GPU work: every call below fails a host-side check
before the library touches the HIP runtime.
"""
import ctypes
import os
import re

import pytest

import draft_block_verification_amd as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sd_verify.h")

lib = ctypes.CDLL(sd.LIB_PATH)
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced on the host
MISALIGNED = ctypes.c_void_p(0x10002)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^SD_API\s+[\w\s\*]*?\b(sd_\w+)\s*\(", text, re.M)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(sd.EXPORTED) == names


def test_abi_version_and_status_strings():
    assert sd.abi_version() == 2
    lib.sd_status_string.restype = ctypes.c_char_p
    assert lib.sd_status_string(0) == b"ok"
    assert b"workspace" in lib.sd_status_string(4)
    assert b"scratch" in lib.sd_status_string(6)
    assert lib.sd_status_string(99) == b"unknown status"


def test_workspace_sizes():
    # Header; the publication area (two buffers of 2 * 64 * 512 + 64 words); one 16-byte
    # partial per (row, 64-wide vocabulary tile); fp64 drafted-token logits.
    up = lambda x: (x + 255) // 256 * 256
    pub = 2 * (2 * 64 * 512 + 64) * 8
    b = sd.verify_workspace_bytes(1, 9, 2048, 32768)
    assert b == 256 + pub + up(10 * 512 * 16) + up(10 * 8)
    assert sd.verify_workspace_bytes(32, 16, 4096, 151936) >= 32 * 17 * (151936 // 64) * 16
    assert sd.accept_workspace_bytes(128, 16, 129280) >= 256 + 128 * 16 * 8 + 128 * 16 * 32 * 16
    for bad in [(0, 9, 2048, 100), (1, 0, 2048, 100), (1, 65, 2048, 100), (1, 4, 12, 100),
                (1, 4, 2048, 0), (1, 4, 2048, 1 << 22)]:
        assert sd.verify_workspace_bytes(*bad) == 0, bad


def _verify(**kw):
    a = dict(hidden=FAKE, lm_head=FAKE, draft=None, vlen=None, offs=None, B=1, g=4, d=256,
             V=1024, T=0.0, logits=None, stats=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.sd_verify_logits(a["hidden"], a["lm_head"], a["draft"], a["vlen"], a["offs"],
                                ctypes.c_int32(a["B"]), ctypes.c_int32(a["g"]),
                                ctypes.c_int32(a["d"]), ctypes.c_int32(a["V"]),
                                ctypes.c_float(a["T"]), a["logits"], a["stats"], a["ws"],
                                ctypes.c_size_t(a["ws_bytes"]), a["stream"])


def test_verify_logits_host_validation():
    assert _verify(hidden=None) == 1
    assert _verify(stats=None) == 1
    assert _verify(vlen=FAKE) == 1                    # lengths without offsets
    assert _verify(T=-1.0) == 1
    assert _verify(T=float("nan")) == 1
    assert _verify(d=12) == 2
    assert _verify(g=65) == 2
    assert _verify(B=0) == 2
    assert _verify(V=0) == 2
    assert _verify(hidden=MISALIGNED) == 3
    assert _verify(logits=MISALIGNED) == 3
    assert _verify(ws=None) == 4
    assert _verify(ws_bytes=100) == 4
    assert _verify(ws=ctypes.c_void_p(0x10010)) == 3  # workspace must be 256-byte aligned


def test_truncate_and_accept_host_validation():
    f = lib.sd_truncate_by_confidence
    assert f(None, 1, 4, ctypes.c_float(0.3), FAKE, FAKE, None) == 1
    assert f(FAKE, 1, 4, ctypes.c_float(float("inf")), FAKE, FAKE, None) == 1
    assert f(FAKE, 0, 4, ctypes.c_float(0.3), FAKE, FAKE, None) == 2
    assert f(MISALIGNED, 1, 4, ctypes.c_float(0.3), FAKE, FAKE, None) == 3
    g = lib.sd_accept_greedy
    assert g(FAKE, None, None, None, 1, 4, FAKE, FAKE, None, None) == 1
    assert g(FAKE, FAKE, FAKE, None, 1, 4, FAKE, FAKE, None, None) == 1
    assert g(FAKE, FAKE, None, None, 1, 99, FAKE, FAKE, None, None) == 2
    assert g(MISALIGNED, FAKE, None, None, 1, 4, FAKE, FAKE, None, None) == 3
    r = lib.sd_accept_rejection
    args = [FAKE] * 8 + [1, 4, 1024, ctypes.c_float(1.0)] + [FAKE, FAKE, None, FAKE,
                                                             ctypes.c_size_t(1 << 20), None]
    bad_T = list(args)
    bad_T[11] = ctypes.c_float(0.0)
    assert r(*bad_T) == 1                             # rejection needs T > 0
    no_ws = list(args)
    no_ws[15] = None
    assert r(*no_ws) == 4
    small_ws = list(args)
    small_ws[16] = ctypes.c_size_t(64)
    assert r(*small_ws) == 4


def test_accept_rejection_ex_host_validation():
    r = lib.sd_accept_rejection_ex
    args = [FAKE] * 8 + [1, 4, 1024, ctypes.c_float(1.0)] + [FAKE, FAKE, None, FAKE, FAKE,
                                                             ctypes.c_size_t(1 << 20), None]
    bad_rate = list(args)
    bad_rate[15] = ctypes.c_void_p(0x10004)           # fp64 output must be 8-byte aligned
    assert r(*bad_rate) == 3
    bad_T = list(args)
    bad_T[11] = ctypes.c_float(0.0)
    assert r(*bad_T) == 1
    small_ws = list(args)
    small_ws[17] = ctypes.c_size_t(64)
    assert r(*small_ws) == 4


def test_lm_head_block_host_validation():
    assert lib.sd_lm_head_block_bytes(1000, 256) == 16 * 2 * 16384
    assert lib.sd_lm_head_block_bytes(64, 128) == 16384
    assert lib.sd_lm_head_block_bytes(65, 128) == 2 * 16384
    assert lib.sd_lm_head_block_bytes(100, 200) == 0          # d % 128 != 0
    assert lib.sd_lm_head_block_bytes(0, 256) == 0
    f = lib.sd_lm_head_block
    ok = [FAKE, 1000, 256, FAKE, ctypes.c_size_t(16 * 2 * 16384), None]
    bad = list(ok); bad[0] = None
    assert f(*bad) == 1
    bad = list(ok); bad[2] = 200
    assert f(*bad) == 2
    bad = list(ok); bad[3] = ctypes.c_void_p(0x10008)
    assert f(*bad) == 3
    bad = list(ok); bad[4] = ctypes.c_size_t(16 * 2 * 16384 - 1)
    assert f(*bad) == 4
    v = lib.sd_verify_logits_blocked
    args = [FAKE, FAKE, None, None, None, 8, 16, 256, 1000, ctypes.c_float(0.0), None, FAKE,
            FAKE, ctypes.c_size_t(1 << 24), None]
    assert v(*args) == 2                                       # 8 * 17 rows > 64
    args[5], args[7] = 2, 200
    assert v(*args) == 2                                       # d % 128 != 0


def test_schedule_prefix_host_validation():
    f = lib.sd_schedule_prefix

    def call(conf=FAKE, stale=None, R=4, g=16, sps=FAKE, n=4 * 17 + 1, mode=0, vl=FAKE,
             ro=FAKE):
        return f(conf, stale, ctypes.c_int32(R), ctypes.c_int32(g), sps, ctypes.c_int32(n),
                 ctypes.c_int32(mode), vl, ro, None)

    assert call(conf=None) == 1
    assert call(sps=None) == 1
    assert call(vl=None) == 1
    assert call(mode=2) == 1
    assert call(stale=FAKE, mode=0) == 1              # stale confidences only with top-K
    assert call(R=0) == 2
    assert call(g=65) == 2
    assert call(n=4 * 17) == 2                        # table must reach B = R * (gamma + 1)
    assert call(R=1025, g=16, n=1025 * 17 + 1) == 2  # more than 16384 candidates
    assert call(conf=MISALIGNED) == 3
    assert call(stale=MISALIGNED, mode=1) == 3


def _noalloc(**kw):
    a = dict(hidden=FAKE, lm_head=FAKE, draft=FAKE, vlen=None, offs=None, B=1, g=9, d=2048,
             V=32768, stats=FAKE, acc=FAKE, nxt=FAKE, counters=None, flags=None, stream=None)
    a.update(kw)
    f = lib.sd_verify_greedy_noalloc
    f.restype = ctypes.c_int32
    return f(a["hidden"], a["lm_head"], a["draft"], a["vlen"], a["offs"], ctypes.c_int32(a["B"]),
             ctypes.c_int32(a["g"]), ctypes.c_int32(a["d"]), ctypes.c_int32(a["V"]), a["stats"],
             a["acc"], a["nxt"], a["counters"], a["flags"], a["stream"])


def test_verify_greedy_noalloc_host_validation():
    """Every argument error, and a problem too large for the fixed scratch, is reported
    before the library looks up its scratch or launches anything."""
    assert _noalloc(hidden=None) == 1
    assert _noalloc(lm_head=None) == 1
    assert _noalloc(draft=None) == 1
    assert _noalloc(acc=None) == 1
    assert _noalloc(vlen=FAKE) == 1                   # lengths without offsets
    assert _noalloc(g=65) == 2
    assert _noalloc(d=12) == 2
    assert _noalloc(hidden=MISALIGNED) == 3
    assert _noalloc(flags=MISALIGNED) == 3
    # 16 MiB of scratch: the config-4 shape needs about 21 MB of row partials.
    assert sd.verify_workspace_bytes(32, 16, 4096, 151936) > sd.NOALLOC_SCRATCH_BYTES
    assert _noalloc(B=32, g=16, d=4096, V=151936) == 6
    assert sd.verify_workspace_bytes(1, 9, 2048, 32768) <= sd.NOALLOC_SCRATCH_BYTES


def _verify_rejection(**kw):
    a = dict(hidden=FAKE, lm_head=FAKE, layout=0, dlog=FAKE, draft=FAKE, vlen=None, offs=None,
             ua=FAKE, ur=FAKE, B=1, g=4, d=256, V=1024, T=1.0, logits=FAKE, stats=FAKE,
             acc=FAKE, nxt=FAKE, cnt=None, rate=None, wsv=FAKE, wsv_bytes=1 << 30, wsa=FAKE,
             wsa_bytes=1 << 30, stream=None)
    a.update(kw)
    i32 = ctypes.c_int32
    return lib.sd_verify_rejection(
        a["hidden"], a["lm_head"], i32(a["layout"]), a["dlog"], a["draft"], a["vlen"],
        a["offs"], a["ua"], a["ur"], i32(a["B"]), i32(a["g"]), i32(a["d"]), i32(a["V"]),
        ctypes.c_float(a["T"]), a["logits"], a["stats"], a["acc"], a["nxt"], a["cnt"],
        a["rate"], a["wsv"], ctypes.c_size_t(a["wsv_bytes"]), a["wsa"],
        ctypes.c_size_t(a["wsa_bytes"]), a["stream"])


def test_verify_rejection_host_validation():
    assert _verify_rejection(layout=3) == 1            # unknown LM-head layout
    assert _verify_rejection(lm_head=None) == 1
    assert _verify_rejection(logits=None) == 1         # the draws need the logits
    assert _verify_rejection(dlog=None) == 1
    assert _verify_rejection(ur=None) == 1
    assert _verify_rejection(T=0.0) == 1               # greedy has its own call
    assert _verify_rejection(vlen=FAKE) == 1           # lengths without offsets
    assert _verify_rejection(g=65) == 2
    assert _verify_rejection(layout=1, d=200) == 2     # blocked copy: d % 128 == 0 only
    assert _verify_rejection(layout=1, B=16) == 2      # blocked copy: streaming regime only
    assert _verify_rejection(dlog=MISALIGNED) == 3
    assert _verify_rejection(rate=ctypes.c_void_p(0x10004)) == 3
    assert _verify_rejection(wsv_bytes=100) == 4
    assert _verify_rejection(wsa=None) == 4
    assert _verify_rejection(wsa_bytes=100) == 4
    # A W12 head: a host descriptor, checked as for sd_verify_logits_w12.
    from draft_block_verification_amd._lib import _SdW12
    desc = lambda **f: ctypes.byref(_SdW12(**dict(dict(codes=0x10000, corr=0x10000, cap=12, b2=5), **f)))
    assert _verify_rejection(layout=2, lm_head=desc(codes=None)) == 1
    assert _verify_rejection(layout=2, lm_head=desc(b2=0)) == 1
    assert _verify_rejection(layout=2, lm_head=desc(), d=200) == 2   # streaming regime only
    assert _verify_rejection(layout=2, lm_head=desc(), B=16) == 2
    assert _verify_rejection(layout=2, lm_head=desc(cap=6)) == 2     # cap % 4 == 0
    assert _verify_rejection(layout=2, lm_head=desc(codes=0x10008)) == 3
    assert _verify_rejection(layout=2, lm_head=desc(), wsv_bytes=100) == 4


def test_import_fails_loudly_without_the_library(tmp_path):
    """No fallback: a copy of the package without libsdverify.so refuses to import."""
    import shutil
    import subprocess
    import sys
    shutil.copytree(os.path.join(ROOT, "draft_block_verification_amd"),
                    tmp_path / "draft_block_verification_amd",
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__", "csrc"))
    r = subprocess.run([sys.executable, "-c", "import draft_block_verification_amd"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "libsdverify.so is missing" in r.stderr
