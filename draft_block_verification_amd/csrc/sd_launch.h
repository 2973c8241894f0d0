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
// *zx_done whether it also wrote the drafted-token logits to a.zx. With
// a.greedy_accept_len set, *greedy_done (when given) says whether the launch also wrote
// the greedy statistics and decisions (small streaming grids); otherwise the caller
// still has to.
// With a.dpart and a.draft_logits set, a streaming contraction may also write the drafter
// chunk partials of every kept draft row (workgroups appended to its grid); *draft_done
// (when given) says whether it did.
hipError_t launch_contraction(const VerifyArgs &a, hipStream_t stream, int *n_part,
                              bool *zx_done, bool *greedy_done = nullptr,
                              bool *draft_done = nullptr);
// Row statistics from the contraction's n_part partial columns (k_row_merge), with the
// drafted-token logits of a.zx when the contraction formed them (zx_done).
hipError_t launch_row_merge(const VerifyArgs &a, int n_part, bool zx_done, hipStream_t stream);
// Rejection verify's row merge and decision (k_merge_decide, gamma <= kDecideMaxGamma):
// statistics of every verified
// row, drafter log-normalisers, a_r and the counters, from the contraction's n_part
// partial columns, the drafter chunk partials and a.zx.
hipError_t launch_merge_decide(const VerifyArgs &a, const DecideArgs &o, int n_part,
                               hipStream_t stream);

// Workgroups of 256 threads of kernel fn that the current device holds at once.
int resident_workgroups(const void *fn);

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
  size_t rec;       // DrawRec [B] draw records
  size_t qx;        // float [B][gamma] drafter logits of the drafted tokens
  size_t dpart;     // drafter chunk partials [B][gamma][chunks]
  size_t csum;      // double [B][chunks][2] draw-weight chunk sums
};
size_t accept_workspace_layout(int B, int gamma, int V, AcceptLayout *lay);

// Rejection verify in one call: the contraction (v.logits and v.stats set), the drafter
// normaliser, k_merge_decide and the draws; v.draft_logits and v.draft_tokens are required.
hipError_t launch_verify_rejection(VerifyArgs v, const float *u_accept, const float *u_resample,
                                   int32_t *accept_len, int32_t *next_token, int64_t *counters,
                                   double *accept_rate, void *accept_workspace,
                                   hipStream_t stream);

// Rejection acceptance.
hipError_t launch_accept_rejection(const float *logits, const sd_row_stats *stats,
                                   const uint16_t *draft_logits, const int32_t *draft_tokens,
                                   const int32_t *verify_len, const RowMap &rm,
                                   const float *u_accept, const float *u_resample, int V,
                                   float temperature, int32_t *accept_len, int32_t *next_token,
                                   int64_t *counters, double *accept_rate, void *workspace,
                                   hipStream_t stream);
}  // namespace sdv
