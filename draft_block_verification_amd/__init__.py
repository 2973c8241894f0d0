"""Draft-block verification on AMD MI355X (gfx950).

Python face of libsdverify.so (C ABI declared in include/sd_verify.h). The
functions carry the C names and only marshal arguments; all computation runs
in the library's HIP kernels.
"""
from ._lib import (EXPORTED, FLAG_WAIT, FLAG_NO_RESIDUAL, FLAG_ROW_OFFSETS, FLAG_VERIFY_LEN, LIB_PATH,
                   LM_HEAD_BLOCKED, LM_HEAD_ROWS, LM_HEAD_W12, sd_verify_rejection,
                   ROW_STATS_DTYPE, SCHED_EARLY_STOP, SCHED_MAX_CANDIDATES, SCHED_TOP_K, SdError,
                   BlockedWeights, VerifyRound, W12Weights, abi_version, accept_workspace_bytes, device_flags, new_stats,
                   new_workspace, profile_sps, sd_accept_greedy, sd_accept_rejection,
                   sd_accept_rejection_ex, sd_schedule_prefix, sd_truncate_by_confidence,
                   sd_verify_contraction, sd_verify_contraction_w12, sd_verify_greedy,
                   sd_verify_greedy_noalloc, sd_verify_greedy_w12, NOALLOC_SCRATCH_BYTES,
                   sd_verify_logits, sd_verify_logits_w12, stats_to_numpy, verify_workspace_bytes,
                   w12_encode)

__all__ = ["EXPORTED", "FLAG_WAIT", "FLAG_NO_RESIDUAL", "FLAG_ROW_OFFSETS", "FLAG_VERIFY_LEN", "LIB_PATH",
           "LM_HEAD_BLOCKED", "LM_HEAD_ROWS", "LM_HEAD_W12", "sd_verify_rejection",
           "ROW_STATS_DTYPE", "SCHED_EARLY_STOP", "SCHED_MAX_CANDIDATES", "SCHED_TOP_K", "SdError",
           "BlockedWeights", "VerifyRound", "W12Weights", "abi_version", "accept_workspace_bytes", "device_flags", "new_stats",
           "new_workspace", "profile_sps", "sd_accept_greedy", "sd_accept_rejection",
           "sd_accept_rejection_ex",
           "sd_schedule_prefix", "sd_truncate_by_confidence",
           "sd_verify_contraction", "sd_verify_contraction_w12", "sd_verify_greedy",
           "sd_verify_greedy_noalloc", "sd_verify_greedy_w12", "NOALLOC_SCRATCH_BYTES",
           "sd_verify_logits",
           "sd_verify_logits_w12", "stats_to_numpy", "verify_workspace_bytes", "w12_encode"]
