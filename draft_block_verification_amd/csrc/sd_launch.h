// Host-side launchers and workspace layouts of the HIP library (defined in sd_gemm.hip,
// sd_accept.hip and sd_sched.hip; called by sd_api.hip). Each launcher enqueues its
// kernels on `stream` and returns the hipError_t of the launch.
#pragma once

#include "sd_internal.h"

namespace sdv {

// Bytes of verify workspace (header, then the row partials) for these sizes.
size_t verify_workspace_layout(int B, int gamma, int V, size_t *part_off, int *part_stride,
                               size_t *zx_off);

// LM-head verify.
hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream);
// Greedy verify in two launches: the contraction, then one kernel that merges each
// request's row statistics and decides acceptance (temperature 0, stats written too).
hipError_t launch_verify_greedy(const VerifyArgs &a, int32_t *accept_len, int32_t *next_token,
                                int64_t *counters, hipStream_t stream);
// The contraction kernel alone; *n_part receives the partial columns written per row and
// *zx_done whether it also wrote the drafted-token logits to a.zx.
hipError_t launch_contraction(const VerifyArgs &a, hipStream_t stream, int *n_part,
                              bool *zx_done);

// Stage-major blocked copy of a bf16 LM head (the layout VerifyArgs::w_blocked reads).
hipError_t launch_block_lm_head(const uint16_t *W, int V, int d, uint16_t *out,
                                hipStream_t stream);

hipError_t launch_truncate(const float *conf, int B, int gamma, float threshold,
                           int32_t *verify_len, int32_t *row_offsets, hipStream_t stream);

hipError_t launch_schedule(const float *conf, const float *conf_stale, int R, int gamma,
                           const float *sps, int mode, int32_t *verify_len, int32_t *row_offsets,
                           hipStream_t stream);

hipError_t launch_accept_greedy(const sd_row_stats *stats, const int32_t *draft_tokens,
                                const int32_t *verify_len, const RowMap &rm,
                                int32_t *accept_len, int32_t *next_token, int64_t *counters,
                                hipStream_t stream);

// Byte offsets inside the rejection-accept workspace.
struct AcceptLayout {
  int chunks;       // vocabulary chunks per row
  size_t lse_q;     // double [B][gamma] drafter log-normalisers (right after the header)
  size_t acc_a;     // int32 [B] accepted lengths
  size_t dpart;     // drafter chunk partials [B][gamma][chunks]
  size_t csum;      // double [B][chunks][2] draw-weight chunk sums
};
size_t accept_workspace_layout(int B, int gamma, int V, AcceptLayout *lay);

// Rejection acceptance. With normalized = true the drafter chunk partials are taken as
// already written to the workspace by launch_draft_normalizer for the same inputs.
hipError_t launch_accept_rejection(const float *logits, const sd_row_stats *stats,
                                   const uint16_t *draft_logits, const int32_t *draft_tokens,
                                   const int32_t *verify_len, const RowMap &rm,
                                   const float *u_accept, const float *u_resample, int V,
                                   float temperature, int32_t *accept_len, int32_t *next_token,
                                   int64_t *counters, double *accept_rate, void *workspace,
                                   bool normalized, hipStream_t stream);
// workgroups > 0: a fixed grid of that many workgroups walking the rows (bounded
// footprint beside another kernel); 0: one wave per (chunk, kept row) over a full grid.
hipError_t launch_draft_normalizer(const uint16_t *draft_logits, const int32_t *verify_len,
                                   int B, int gamma, int V, float temperature, void *workspace,
                                   int workgroups, hipStream_t stream);

}  // namespace sdv
