/*
 * sd_verify.h -- C ABI of the draft-block verification library (libsdverify.so).
 *
 * One verify round of speculative decoding on an AMD MI355X (gfx950):
 *   1. sd_truncate_by_confidence  keep each request's confident draft prefix
 *      sd_schedule_prefix         or choose the prefixes that maximise throughput
 *   2. sd_verify_logits           LM-head logits at every kept position plus the
 *                                 bonus position, with per-row statistics
 *   3. sd_accept_greedy           greedy prefix acceptance + correction/bonus token
 *      sd_accept_rejection        rejection-sampling acceptance + residual/bonus draw
 *
 * Conventions shared by every call
 *   - All tensors are row-major, contiguous, caller-owned DEVICE memory unless
 *     stated otherwise. The library never allocates; scratch memory comes from a
 *     caller-provided workspace sized by the *_workspace_bytes functions.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work; outputs are valid once the stream has been synchronised.
 *   - Host-checkable errors (null pointers, bad sizes, misalignment, small
 *     workspace) are returned synchronously before any GPU work is enqueued.
 *     SD_EDEVICE reports a failed kernel launch. Nothing is printed.
 *   - Device-side anomalies (a verify length outside [0, gamma], row offsets
 *     that disagree with the lengths, a residual with no positive mass) are
 *     clamped or handled by a documented fallback and raise bits in a sticky
 *     flag word inside the workspace, read with sd_device_flags.
 *   - Identical inputs give identical output bytes (fixed-order reductions, no
 *     floating-point atomics).
 *   - Rows: request r verifies L_r kept drafts (0 <= L_r <= gamma) plus one bonus
 *     row, M = sum_r (L_r + 1) rows in total, packed with no padding. Row m of
 *     request r, block position j (0 <= j <= L_r) is m = row_offsets[r] + j and
 *     reads hidden[r][j][:]. Per-row outputs have capacity B * (gamma + 1) rows;
 *     only the first M are written.
 *
 * The operations follow these passages:
 *   DSpark summary (GeekNews), "Problem definition": the target checks a drafted
 *     block in one forward pass and rejection sampling accepts the longest
 *     prefix consistent with the target distribution, losslessly.
 *   DSpark summary, "Architecture" (decode-round example, confidence head,
 *     prefix scheduler): per-position survival confidences; the scheduler keeps
 *     the confident prefix and cuts the rest; on the first rejection the target
 *     emits a correction token.
 *   DSpark summary, "Production deployment": the LM head maps the d-dimensional
 *     hidden state to V logits; variable-length requests are flattened into
 *     independent elements instead of padded.
 *   LFM2.5-DSpark blog, "How DSpark works" and "Quality parity": verification
 *     shares one weight load across the block; in greedy decoding a draft is
 *     kept only if it matches the target and is otherwise replaced by the
 *     target's token, so the output equals the target's own greedy output.
 */
#ifndef SD_VERIFY_H
#define SD_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifndef SD_API
#define SD_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point (as int32_t). */
enum {
    SD_OK = 0,
    SD_EINVAL = 1,      /* null required pointer, bad temperature or threshold   */
    SD_ESHAPE = 2,      /* B < 1, gamma outside [1, 64], d % 8 != 0, V < 1, size overflow */
    SD_EALIGN = 3,      /* a bf16 / fp32 tensor not 16-byte aligned, stats not 8-byte aligned */
    SD_EWORKSPACE = 4,  /* workspace pointer null or smaller than required       */
    SD_EDEVICE = 5,     /* a HIP launch or copy failed                           */
    SD_ESCRATCH = 6     /* the problem needs more scratch than the allocation-free
                           entry point holds (SD_NOALLOC_SCRATCH_BYTES)            */
};

/* Sticky device flags (bit mask) accumulated in a workspace. */
enum {
    SD_FLAG_VERIFY_LEN = 1,   /* a verify_len entry was outside [0, gamma] and was clamped */
    SD_FLAG_ROW_OFFSETS = 2,  /* row_offsets disagreed with verify_len or overflowed the row capacity */
    SD_FLAG_NO_RESIDUAL = 4,  /* a residual max(0, p - q) had no positive mass; drew from p instead */
    SD_FLAG_WAIT = 8          /* a workgroup's bounded wait for results that other workgroups
                                 of the same launch publish ran out (sd_verify_rejection's
                                 one-launch draw, sd_verify_greedy's in-launch decision);
                                 the tokens of that call are not valid */
};

/* Per verified row statistics (32 bytes, 8-byte aligned). */
typedef struct sd_row_stats {
    int32_t argmax;   /* lowest vocabulary id attaining max_v z[v]                        */
    float top1;       /* z[argmax] (fp32 logit)                                          */
    float top2;       /* largest z[v] over v != argmax (equals top1 on an exact tie)      */
    int32_t pos;      /* block position j of this row (0..L_r; L_r is the bonus row)      */
    double lse;       /* log sum_v exp(z[v] / T) when T > 0, else 0                      */
    double z_draft;   /* logit of the drafted token x[r][j] for j < L_r, as an fp64 dot of
                         the bf16 inputs; 0 on the bonus row                              */
} sd_row_stats;

/* ABI version of this header (incremented on any signature or layout change). */
SD_API int32_t sd_abi_version(void);

/* Static text for a status code. */
SD_API const char *sd_status_string(int32_t status);

/* Workspace bytes sd_verify_logits needs for these sizes (0 on invalid sizes). */
SD_API size_t sd_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t d, int32_t V);

/* Workspace bytes sd_accept_rejection needs for these sizes (0 on invalid sizes). */
SD_API size_t sd_accept_workspace_bytes(int32_t B, int32_t gamma, int32_t V);

/* Prepare a freshly allocated workspace: clears its 256-byte header (flag word and
 * counters) and, in a workspace of at least 256 + 1049600 bytes (every verify workspace),
 * sets the 1049600-byte publication area that follows the header to all ones bytes (the
 * state sd_verify_greedy's in-launch decision expects; every later call leaves it so).
 * Must be called once per workspace before its first use; enqueued on `stream`. */
SD_API int32_t sd_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Synchronise `stream`, copy the sticky flag word of `workspace` to *flags (host) and,
 * if clear != 0, reset it to zero. */
SD_API int32_t sd_device_flags(void *workspace, void *stream, uint32_t *flags, int32_t clear);

/*
 * Confidence truncation (DSpark summary, "Architecture": the scheduler keeps
 * the confident prefix E F G and cuts the low-confidence H).
 *   conf        fp32 [B][gamma]  per-position prefix-survival confidences
 *   threshold   keep leading positions with conf >= threshold (finite, any value)
 *   verify_len  int32 [B]        out: L_r = number of leading positions kept
 *   row_offsets int32 [B + 1]    out: exclusive prefix sum of (L_r + 1); row_offsets[B] = M
 */
SD_API int32_t sd_truncate_by_confidence(const float *conf, int32_t B, int32_t gamma, float threshold,
                                  int32_t *verify_len, int32_t *row_offsets, void *stream);

/* Modes of sd_schedule_prefix. */
enum {
    SD_SCHED_EARLY_STOP = 0,  /* synchronous: admit by survival, stop when throughput drops */
    SD_SCHED_TOP_K = 1        /* asynchronous: K from (stale) confidences over every K, then top-K */
};

/* Largest R * gamma sd_schedule_prefix accepts (all candidates are sorted in one workgroup). */
#define SD_SCHED_MAX_CANDIDATES 16384

/*
 * Hardware-aware prefix scheduler (DSpark summary, "Architecture" ->
 * "Confidence-Scheduled Verification": survival-ordered admission that maximises
 * throughput tau * SPS(B) over a cost table profiled once, with early stopping;
 * "Engineering": the asynchronous form that sizes the batch from two-step-old
 * confidences by a search over every K and admits the current top-K). A drop-in
 * replacement for sd_truncate_by_confidence.
 *   conf        fp32 [R][gamma]  conditional confidences c[r][k] of the current step
 *   conf_stale  fp32 [R][gamma]  confidences of an earlier step (SD_SCHED_TOP_K only,
 *               may be NULL: then conf); must be NULL with SD_SCHED_EARLY_STOP
 *   sps         fp32 [n_sps]     steps per second at a batch of B target rows, for
 *               B = 0 .. n_sps - 1; n_sps >= R * (gamma + 1) + 1; finite and positive
 *   mode        SD_SCHED_EARLY_STOP or SD_SCHED_TOP_K
 *   verify_len  int32 [R]        out: admitted drafts of request r (a prefix of its block)
 *   row_offsets int32 [R + 1]    out: exclusive prefix sum of (verify_len + 1)
 * Survival a[r][j] = product of clamp(c[r][k], 0, 1) over k <= j (NaN counts as 0),
 * taken left to right in fp32. Candidates are ordered by larger survival, then lower
 * request, then lower position. With K admitted, the batch is B = R + K rows and
 * Theta_K = (R * 2^40 + sum over the first K candidates of floor(a * 2^40)) * SPS(B),
 * the integer converted to fp64 (round to nearest even) and one fp64 multiply.
 * SD_SCHED_EARLY_STOP: K = first K with Theta_{K+1} < Theta_K, else R * gamma.
 * SD_SCHED_TOP_K: K = smallest K attaining the largest Theta_K over K = 0 .. R * gamma
 * (computed from conf_stale when given); the admitted set is the first K candidates
 * in the order of conf.
 * Errors: SD_EINVAL for a null output or conf/sps, a bad mode or a stale array with
 * SD_SCHED_EARLY_STOP; SD_ESHAPE for R < 1, gamma outside [1, 64],
 * R * gamma > SD_SCHED_MAX_CANDIDATES or a short sps table; SD_EALIGN for arrays not
 * 4-byte aligned. One workgroup, no workspace.
 */
SD_API int32_t sd_schedule_prefix(const float *conf, const float *conf_stale, int32_t R,
                                  int32_t gamma, const float *sps, int32_t n_sps, int32_t mode,
                                  int32_t *verify_len, int32_t *row_offsets, void *stream);

/*
 * Target logits at every verified row and their statistics (LFM2.5-DSpark
 * blog, "How DSpark works"; DSpark summary, "Production deployment").
 *   hidden       bf16 [B][gamma + 1][d]  target hidden states before the LM head
 *   lm_head      bf16 [V][d]             LM-head weight, d-contiguous rows
 *   draft_tokens int32 [B][gamma] or NULL drafted tokens (for z_draft); NULL -> z_draft = 0
 *   verify_len   int32 [B] or NULL       kept drafts per request; NULL -> gamma for all
 *   row_offsets  int32 [B + 1] or NULL   packed row starts; NULL -> r * (gamma + 1).
 *                                        verify_len and row_offsets are both NULL or both set.
 *   temperature  >= 0; 0 computes argmax/top1/top2 only (lse = 0)
 *   logits       fp32 [B * (gamma + 1)][V] or NULL: out, z[m][v] for m < M
 *   stats        sd_row_stats [B * (gamma + 1)]: out, rows m < M
 *   workspace    device scratch of sd_verify_workspace_bytes(B, gamma, d, V) bytes
 * z[m][v] = sum_k hidden_row(m)[k] * lm_head[v][k], bf16 products accumulated in fp32.
 */
SD_API int32_t sd_verify_logits(const uint16_t *hidden, const uint16_t *lm_head,
                         const int32_t *draft_tokens, const int32_t *verify_len,
                         const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                         int32_t V, float temperature, float *logits, sd_row_stats *stats,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The LM-head contraction stage of sd_verify_logits on its own (same passages):
 * writes the fp32 logits (when logits != NULL) and leaves per-row partial
 * statistics in `workspace`; it does not produce sd_row_stats. It runs exactly the
 * contraction kernel sd_verify_logits runs first, so it serves to time that kernel
 * alone, and callers that only need the logits can use it. Arguments as for
 * sd_verify_logits.
 */
SD_API int32_t sd_verify_contraction(const uint16_t *hidden, const uint16_t *lm_head,
                                     const int32_t *verify_len, const int32_t *row_offsets,
                                     int32_t B, int32_t gamma, int32_t d, int32_t V,
                                     float temperature, float *logits, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * Greedy verify of a drafted block in one call (LFM2.5-DSpark blog, "How DSpark
 * works" and "Quality parity"): the LM-head contraction at temperature 0 followed
 * by one kernel that merges each request's row statistics and decides acceptance.
 * When the streaming contraction runs (B * (gamma + 1) <= 64, d % 128 == 0) for at most
 * 16 requests of at most 12 rows (gamma <= 11) on a grid that leaves a compute unit for
 * each request (up to about V = 16000 on MI355X), workgroups appended to its launch merge
 * and decide instead (no second launch): the contraction's workgroups publish their row
 * partials in the workspace's publication area, which the call leaves as it found it.
 * Outputs are the same bytes as sd_verify_logits (temperature 0, logits NULL)
 * followed by sd_accept_greedy, with one or two launches fewer.
 *   hidden, lm_head, draft_tokens, verify_len, row_offsets, B, gamma, d, V
 *                as for sd_verify_logits (draft_tokens required)
 *   stats        sd_row_stats [B * (gamma + 1)]  out, as for sd_verify_logits
 *   accept_len, next_token, counters  as for sd_accept_greedy
 *   workspace    the verify workspace (sd_verify_workspace_bytes)
 * Errors: as for sd_verify_logits and sd_accept_greedy.
 */
SD_API int32_t sd_verify_greedy(const uint16_t *hidden, const uint16_t *lm_head,
                                const int32_t *draft_tokens, const int32_t *verify_len,
                                const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                                int32_t V, sd_row_stats *stats, int32_t *accept_len,
                                int32_t *next_token, int64_t *counters, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * sd_verify_greedy for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc. The verify
 * workspace (header, per-tile row partials, drafted-token logits) lives in a file-scope
 * device array of the library, SD_NOALLOC_SCRATCH_BYTES bytes on every GPU the library
 * runs on, held until the process ends; its address is looked up once per device on
 * the first call made with that device current. The call itself allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).
 *   hidden, lm_head, draft_tokens, verify_len, row_offsets, B, gamma, d, V, stats,
 *   accept_len, next_token, counters   as for sd_verify_greedy (bf16 [V][d] LM head)
 *   flags   device uint32 [1] out, 4-byte aligned, or NULL: this call's sticky device
 *           flag word (SD_FLAG_*); the scratch's flag word is cleared at the start of
 *           every call, so flags cover this call only (the first call on a device also
 *           prepares the scratch as sd_workspace_init prepares a workspace)
 *   stream  hipStream_t of the device that is current at the call
 * Limit: sd_verify_workspace_bytes(B, gamma, d, V) <= SD_NOALLOC_SCRATCH_BYTES, else
 * SD_ESCRATCH before any GPU work (16 MiB holds, for example, 64 rows at V = 151936 or
 * 400 rows at V = 32768). Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (other streams, other host threads) race and must be serialised
 * by the caller. Outputs are the bytes sd_verify_greedy writes for the same inputs.
 * Errors: as for sd_verify_greedy (SD_EWORKSPACE does not occur), SD_ESCRATCH, and
 * SD_EDEVICE when the scratch address cannot be looked up.
 */
#define SD_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
SD_API int32_t sd_verify_greedy_noalloc(const uint16_t *hidden, const uint16_t *lm_head,
                                        const int32_t *draft_tokens, const int32_t *verify_len,
                                        const int32_t *row_offsets, int32_t B, int32_t gamma,
                                        int32_t d, int32_t V, sd_row_stats *stats,
                                        int32_t *accept_len, int32_t *next_token,
                                        int64_t *counters, uint32_t *flags, void *stream);

/*
 * W12 LM head (SpecPilot page, "Reasons": a lossless 12-bit weight format whose three
 * 4-bit planes the GEMM rebuilds in registers). This library's layout:
 *   - a bf16 weight's low byte (exponent bit 0, 7 mantissa bits) is kept verbatim;
 *   - its high byte (sign, exponent bits 7..1 = e2) becomes the 4-bit code
 *     sign << 3 | t: t = 0 for e2 = 0 (zeros, subnormals), t = e2 - b2 + 1 for e2 in
 *     the tensor's window [b2, b2 + 6], b2 = max(1, largest nonzero e2 - 6);
 *   - every other weight is coded as a signed zero and its exact bits go to a
 *     correction slot of its region of 64 LM-head rows by 128 columns: uint32
 *     k_local | row_local << 7 | bits << 16, sorted by (row_local, k_local), 0 = empty;
 *   - a group of 8 columns 8 g .. 8 g + 7 of one row is 12 bytes: the 8 low bytes, then
 *     byte 8 + i = code of column 8 g + 2 i | code of column 8 g + 2 i + 1 << 4; groups
 *     are stored region by region, [ceil(V / 64)][d / 128][64 rows][16 groups][12 bytes],
 *     rows past V zero (one region = one contiguous 12 KB block).
 * Decoding gives back every bf16 bit pattern exactly.
 */
typedef struct sd_w12 {
    const uint8_t *codes;    /* [ceil(V/64)][d/128][64][16][12], device, 16-byte aligned */
    const uint32_t *corr;    /* [ceil(V / 64)][d / 128][cap] correction slots, device     */
    int32_t cap;             /* slots per region: a multiple of 4 in [4, 64] for the GEMM */
    int32_t b2;              /* window start, 1..121                                     */
} sd_w12;

/*
 * Encode a bf16 LM head into W12 (host memory in and out; runs on the host).
 *   W      bf16 [V][d] (d a multiple of 128)
 *   codes  uint8 [ceil(V / 64)][d / 128][64][16][12] out (ignored by the sizing call)
 *   corr   uint32 [ceil(V / 64)][d / 128][*cap] out, or NULL for the sizing call
 *   cap    in: slots per region of corr; out: the slots needed (sizing call), or used
 *   b2     out: window start
 * A sizing call (corr NULL) sets *cap and *b2 only. SD_EWORKSPACE (with *cap set to
 * the need) when *cap is too small; SD_ESHAPE for V < 1 or d not a positive multiple
 * of 128.
 */
SD_API int32_t sd_w12_encode(const uint16_t *W, int32_t V, int32_t d, uint8_t *codes,
                             uint32_t *corr, int32_t *cap, int32_t *b2);

/*
 * sd_verify_logits, sd_verify_contraction and sd_verify_greedy with the LM head
 * given as W12 (lm_head:
 * host struct of device pointers). The contraction decodes the 12-bit groups in
 * registers and adds the corrected weights' products, so every result is that of
 * the bf16 LM head (logits up to fp32 summation order). Restricted to the streaming
 * regime: d % 128 == 0, B * (gamma + 1) <= 64 and cap <= 64, else SD_ESHAPE.
 * Other arguments, outputs and errors as for the bf16 calls.
 */
SD_API int32_t sd_verify_logits_w12(const uint16_t *hidden, const sd_w12 *lm_head,
                                    const int32_t *draft_tokens, const int32_t *verify_len,
                                    const int32_t *row_offsets, int32_t B, int32_t gamma,
                                    int32_t d, int32_t V, float temperature, float *logits,
                                    sd_row_stats *stats, void *workspace, size_t workspace_bytes,
                                    void *stream);
SD_API int32_t sd_verify_contraction_w12(const uint16_t *hidden, const sd_w12 *lm_head,
                                         const int32_t *verify_len, const int32_t *row_offsets,
                                         int32_t B, int32_t gamma, int32_t d, int32_t V,
                                         float temperature, float *logits, void *workspace,
                                         size_t workspace_bytes, void *stream);
SD_API int32_t sd_verify_greedy_w12(const uint16_t *hidden, const sd_w12 *lm_head,
                                    const int32_t *draft_tokens, const int32_t *verify_len,
                                    const int32_t *row_offsets, int32_t B, int32_t gamma,
                                    int32_t d, int32_t V, sd_row_stats *stats,
                                    int32_t *accept_len, int32_t *next_token, int64_t *counters,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Blocked bf16 LM head: the same weights re-laid once so that the streaming
 * contraction reads each of its stages (64 LM-head rows by 128 columns) as one
 * contiguous 16 KB block. Layout: [d/128][ceil(V/64)][64][128] bf16, stage-major: block
 * (st, s) holds LM-head rows 64 s .. 64 s + 63 at columns 128 st .. 128 st + 127, so the
 * blocks of one column range are adjacent. Within a block, row r's 16-byte chunk j
 * (columns 8j .. 8j + 7) sits at chunk position j ^ (r & 15); rows past V are zero. The values, and so every verify output, are those of the bf16
 * [V][d] LM head. The LM head is static, so the copy is made once, beside the original.
 *
 * sd_lm_head_block_bytes: bytes of the copy (0 unless V >= 1 and d is a positive
 * multiple of 128).
 * sd_lm_head_block: writes the copy on `stream`.
 *   lm_head  bf16 [V][d], 16-byte aligned; blocked: device buffer of
 *   sd_lm_head_block_bytes(V, d) bytes, 16-byte aligned, not overlapping lm_head.
 *   Errors: SD_EINVAL (null pointer), SD_ESHAPE (V < 1, d % 128 != 0), SD_EALIGN,
 *   SD_EWORKSPACE (blocked_bytes too small), SD_EDEVICE.
 * sd_verify_logits_blocked / sd_verify_contraction_blocked / sd_verify_greedy_blocked:
 * sd_verify_logits / sd_verify_contraction / sd_verify_greedy reading the blocked copy
 * (lm_head_blocked) instead of the [V][d] LM head; the streaming regime only, like W12:
 * d % 128 == 0 and B * (gamma + 1) <= 64, else SD_ESHAPE. All other arguments, outputs
 * and errors are those of the [V][d] calls.
 */
SD_API size_t sd_lm_head_block_bytes(int32_t V, int32_t d);
SD_API int32_t sd_lm_head_block(const uint16_t *lm_head, int32_t V, int32_t d, uint16_t *blocked,
                                size_t blocked_bytes, void *stream);
SD_API int32_t sd_verify_logits_blocked(const uint16_t *hidden, const uint16_t *lm_head_blocked,
                                        const int32_t *draft_tokens, const int32_t *verify_len,
                                        const int32_t *row_offsets, int32_t B, int32_t gamma,
                                        int32_t d, int32_t V, float temperature, float *logits,
                                        sd_row_stats *stats, void *workspace,
                                        size_t workspace_bytes, void *stream);
SD_API int32_t sd_verify_contraction_blocked(const uint16_t *hidden,
                                             const uint16_t *lm_head_blocked,
                                             const int32_t *verify_len,
                                             const int32_t *row_offsets, int32_t B, int32_t gamma,
                                             int32_t d, int32_t V, float temperature,
                                             float *logits, void *workspace,
                                             size_t workspace_bytes, void *stream);
SD_API int32_t sd_verify_greedy_blocked(const uint16_t *hidden, const uint16_t *lm_head_blocked,
                                        const int32_t *draft_tokens, const int32_t *verify_len,
                                        const int32_t *row_offsets, int32_t B, int32_t gamma,
                                        int32_t d, int32_t V, sd_row_stats *stats,
                                        int32_t *accept_len, int32_t *next_token,
                                        int64_t *counters, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * Greedy acceptance (LFM2.5-DSpark blog, "Quality parity"): a_r = first j < L_r
 * with stats[row_offsets[r] + j].argmax != draft_tokens[r][j], else L_r; the
 * emitted token is the target argmax of row a_r (a correction when a_r < L_r,
 * the bonus token otherwise).
 *   stats        from sd_verify_logits
 *   draft_tokens int32 [B][gamma]
 *   verify_len, row_offsets  as for sd_verify_logits (both NULL or both set)
 *   accept_len   int32 [B]  out: a_r
 *   next_token   int32 [B]  out
 *   counters     int64 [2] or NULL: counters[0] += sum_r L_r (drafts verified),
 *                counters[1] += sum_r a_r (drafts accepted)
 */
SD_API int32_t sd_accept_greedy(const sd_row_stats *stats, const int32_t *draft_tokens,
                         const int32_t *verify_len, const int32_t *row_offsets, int32_t B,
                         int32_t gamma, int32_t *accept_len, int32_t *next_token,
                         int64_t *counters, void *stream);

/*
 * Rejection-sampling acceptance (DSpark summary, "Problem definition":
 * lossless acceptance of the longest consistent prefix; "Architecture":
 * correction token on the first rejection). With p_j = softmax(z_j / T) and
 * q_j = softmax(draft_logits[r][j] / T):
 *   position j < L_r survives iff u_accept[r][j] < min(1, p_j(x_j) / q_j(x_j));
 *   a_r = first failing j, else L_r;
 *   if a_r < L_r the token is drawn from norm(max(0, p_a - q_a)), else from p_{L_r};
 *   draws are inverse-CDF in ascending vocabulary id: the smallest v whose running
 *   weight exceeds u_resample[r][a_r] times the total weight.
 *   logits       fp32 [B * (gamma + 1)][V] written by sd_verify_logits
 *   stats        from sd_verify_logits at the same temperature
 *   draft_logits bf16 [B][gamma][V]     drafter logits per block position
 *   draft_tokens int32 [B][gamma]
 *   u_accept     fp32 [B][gamma]        uniforms in [0, 1)
 *   u_resample   fp32 [B][gamma + 1]    uniforms in [0, 1), indexed by the row sampled
 *   temperature  > 0 (the same one given to sd_verify_logits)
 *   accept_len, next_token, counters   as for sd_accept_greedy
 *   workspace    device scratch of sd_accept_workspace_bytes(B, gamma, V) bytes
 */
SD_API int32_t sd_accept_rejection(const float *logits, const sd_row_stats *stats,
                            const uint16_t *draft_logits, const int32_t *draft_tokens,
                            const int32_t *verify_len, const int32_t *row_offsets,
                            const float *u_accept, const float *u_resample, int32_t B,
                            int32_t gamma, int32_t V, float temperature, int32_t *accept_len,
                            int32_t *next_token, int64_t *counters, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * sd_accept_rejection plus the analytic acceptance rate of every verified draft
 * position (DSpark summary, "Architecture": the confidence head learns, per drafted
 * position, the chance that rejection sampling keeps it, one minus the total-variation
 * distance between drafter and target distributions):
 *   accept_rate[r][j] = sum_v min(p_j(v), q_j(v)) = 1 - (1/2) sum_v |p_j(v) - q_j(v)|
 * for j < L_r, with p_j, q_j as above at the same temperature; -1 for j >= L_r and for
 * every position of a request whose rows leave the row capacity.
 *   accept_rate  fp64 [B][gamma], 8-byte aligned, or NULL (then identical to
 *                sd_accept_rejection)
 * All other arguments, outputs and errors are those of sd_accept_rejection; the
 * acceptance outputs are byte-identical to it. The extra work is one more pass over
 * the kept target and drafter rows (P * V * 6 bytes), with the same workspace.
 */
SD_API int32_t sd_accept_rejection_ex(const float *logits, const sd_row_stats *stats,
                            const uint16_t *draft_logits, const int32_t *draft_tokens,
                            const int32_t *verify_len, const int32_t *row_offsets,
                            const float *u_accept, const float *u_resample, int32_t B,
                            int32_t gamma, int32_t V, float temperature, int32_t *accept_len,
                            int32_t *next_token, int64_t *counters, double *accept_rate,
                            void *workspace, size_t workspace_bytes, void *stream);

/* LM-head layouts of sd_verify_rejection. */
enum {
    SD_LM_HEAD_ROWS = 0,     /* bf16 [V][d]                                              */
    SD_LM_HEAD_BLOCKED = 1,  /* the stage-major blocked copy written by sd_lm_head_block */
    SD_LM_HEAD_W12 = 2       /* lm_head points to an sd_w12 descriptor (host memory)     */
};

/*
 * Rejection verify of a drafted block in one call (DSpark summary, "Problem definition":
 * the target checks the block in one pass and rejection sampling keeps the longest
 * prefix consistent with its distribution; "Architecture": a correction token on the
 * first rejection, a bonus token when every draft survives): sd_verify_logits at
 * `temperature` followed by sd_accept_rejection_ex, in fewer launches. The row merge and
 * the acceptance test run in one kernel; in the streaming regime (d % 128 == 0,
 * B * (gamma + 1) <= 64) the contraction's launch also normalises the drafter rows when
 * the GPU has workgroup slots its grid leaves idle.
 *   hidden, draft_tokens, verify_len, row_offsets, B, gamma, d, V
 *                as for sd_verify_logits (draft_tokens required)
 *   lm_head      bf16 [V][d] (lm_head_layout SD_LM_HEAD_ROWS), its blocked copy
 *                (SD_LM_HEAD_BLOCKED), or a host sd_w12 descriptor of the W12 stream
 *                (SD_LM_HEAD_W12, checked as for sd_verify_logits_w12); the last two in
 *                the streaming regime only, else SD_ESHAPE
 *   draft_logits, u_accept, u_resample, temperature (> 0)
 *                as for sd_accept_rejection
 *   logits, stats  out, as for sd_verify_logits (both required)
 *   accept_len, next_token, counters, accept_rate (NULL: not computed)
 *                out, as for sd_accept_rejection_ex
 *   verify_workspace  sd_verify_workspace_bytes(B, gamma, d, V) bytes
 *   accept_workspace  sd_accept_workspace_bytes(B, gamma, V) bytes
 * The logits, argmax, top-1/top-2, drafted-token logits, accepted lengths, tokens,
 * counters and flags are those of the two separate calls; the per-row log-normalisers
 * (stats lse and the drafter's) are summed in another order and agree with them to
 * fp64 rounding.
 * Errors: those of sd_verify_logits and sd_accept_rejection_ex; SD_EINVAL for an unknown
 * lm_head_layout.
 */
SD_API int32_t sd_verify_rejection(const uint16_t *hidden, const void *lm_head,
                                   int32_t lm_head_layout, const uint16_t *draft_logits,
                                   const int32_t *draft_tokens, const int32_t *verify_len,
                                   const int32_t *row_offsets, const float *u_accept,
                                   const float *u_resample, int32_t B, int32_t gamma, int32_t d,
                                   int32_t V, float temperature, float *logits,
                                   sd_row_stats *stats, int32_t *accept_len,
                                   int32_t *next_token, int64_t *counters, double *accept_rate,
                                   void *verify_workspace, size_t verify_workspace_bytes,
                                   void *accept_workspace, size_t accept_workspace_bytes,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SD_VERIFY_H */
