// Internal declarations shared by the HIP translation units of libsdverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sd_verify.h"

namespace sdv {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workspace header: a 256-byte block at the start of every workspace.
struct WsHeader {
  uint32_t flags;      // sticky SD_FLAG_* bits
  // Publication area state of the in-launch greedy decision (verify workspaces):
  uint32_t pub_done;   // deciding workgroups finished in the running launch (returns to 0)
  uint32_t pub_epoch;  // launches that published; buffer pub_epoch & 1 is the next one's
  uint32_t pub_prev;   // words the last of them published into its buffer
  uint32_t pad[60];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

// Publication area of a verify workspace (right after its header): two buffers of
// kPubWords 64-bit words that a streaming contraction's workgroups publish their row
// partials and drafted-token logits into, with device-scope atomic stores, for the
// workgroups appended to the same launch that merge them and decide greedy acceptance.
// A word that holds kPubEmpty has not been published in the running launch. Launches
// alternate buffers; each one returns the other buffer's published words to kPubEmpty,
// so a buffer is empty whenever a launch starts on it. Holds 64 rows x 512 workgroups
// (two words per partial) and 64 drafted-token logits.
constexpr int kPubMaxGrid = 512;
constexpr int kPubWords = 2 * 64 * kPubMaxGrid + 64;
constexpr size_t kPubBytes = 2 * (size_t)kPubWords * 8;
constexpr unsigned long long kPubEmpty = ~0ull;

// Statistics of one verified row over one vocabulary tile.
struct TilePartial {
  float top1;   // max z over the tile
  float top2;   // max z over the tile excluding the argmax position
  int32_t arg;  // lowest vocabulary id attaining top1
  float sum;    // sum over the tile of exp((z - top1) / T); 0 when T == 0
};
static_assert(sizeof(TilePartial) == 16, "partials are 16 bytes");

// Drafter-row normaliser of one vocabulary chunk (kDraftChunk ids) of one kept draft row.
struct DraftPart {
  float m;       // max drafter logit of the chunk (raw, before / T)
  float pad;
  double s;      // sum over the chunk of exp((l - m) / T)
};
static_assert(sizeof(DraftPart) == 16, "drafter partials are 16 bytes");

// Vocabulary ids per chunk of the rejection kernels (drafter normaliser and draws).
constexpr int kDraftChunk = 4096;

// What the draw kernels read of request r's decision: the row they sample and its scale
// constants, written by the decision kernel so the draws need one load before the logits.
struct DrawRec {
  int32_t row;     // packed row of the draw (base + a_r), -1 for a request outside the row capacity
  int32_t acc;     // a_r
  int32_t qrow;    // drafter row r * gamma + a_r of a residual draw, -1 for the bonus draw from p
  int32_t pad;
  float cp, cq;    // T * log-normaliser of that target row and of that drafter row, in fp32
  int32_t pad2[2];
};
static_assert(sizeof(DrawRec) == 32, "draw records are 32 bytes");

// Bit pattern of a chunk-sum slot that the one-launch draw has not yet published.
constexpr unsigned long long kUnpublished = ~0ull;

// Largest W12 correction-slot count per (64-row, 128-column) region the contraction stages.
constexpr int kW12MaxCap = 64;

// Smallest vocabulary tile used by any GEMM variant; sizes the partials array.
constexpr int kMinVocabTile = 64;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Rows of the verify problem: request r owns rows row_offsets[r] .. + L_r.
struct RowMap {
  const int32_t *row_offsets;  // [B + 1] or null (then rows are r * (gamma + 1) + j)
  int32_t B;
  int32_t gamma;
};

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Number of verified rows, clamped to the row capacity B * (gamma + 1).
__device__ inline int rows_total(const RowMap &rm) {
  const int cap = rm.B * (rm.gamma + 1);
  if (!rm.row_offsets) return cap;
  int M = rm.row_offsets[rm.B];
  return M < 0 ? 0 : (M > cap ? cap : M);
}

// Request owning row m: the largest r with row_offsets[r] <= m.
__device__ inline int row_request(const RowMap &rm, int m) {
  if (!rm.row_offsets) return m / (rm.gamma + 1);
  int lo = 0, hi = rm.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rm.row_offsets[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Row index into hidden[B][gamma + 1] for packed row m, or -1 if the offsets are inconsistent.
__device__ inline int hidden_row(const RowMap &rm, int m, int *req, int *pos) {
  const int r = row_request(rm, m);
  const int j = rm.row_offsets ? m - rm.row_offsets[r] : m - r * (rm.gamma + 1);
  *req = r;
  *pos = j;
  if (j < 0 || j > rm.gamma) return -1;
  return r * (rm.gamma + 1) + j;
}

__device__ inline void raise_flag(WsHeader *ws, uint32_t bit) {
  if (ws) atomicOr(&ws->flags, bit);
}

// A kept-draft count clamped to [0, gamma] (flagged when out of range).
__device__ inline int clamp_len_value(int L, int gamma, WsHeader *ws) {
  if (L < 0 || L > gamma) {
    raise_flag(ws, SD_FLAG_VERIFY_LEN);
    L = L < 0 ? 0 : gamma;
  }
  return L;
}

// Kept drafts of request r, clamped to [0, gamma] (flagged when out of range).
__device__ inline int clamp_len(const int32_t *verify_len, int r, int gamma, WsHeader *ws) {
  if (!verify_len) return gamma;
  return clamp_len_value(verify_len[r], gamma, ws);
}

// fp64 sum of h[k] * w[k] over eight bf16 pairs (every product is exact in fp64).
__device__ inline double dot8_f64(const u32x4 &hv, const u32x4 &wv) {
  double part = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    part += (double)__uint_as_float(hv[e] << 16) * (double)__uint_as_float(wv[e] << 16);
    part += (double)__uint_as_float(hv[e] & 0xffff0000u) * (double)__uint_as_float(wv[e] & 0xffff0000u);
  }
  return part;
}

// 2^x by the hardware instruction. It returns no denormals: results below 2^-126 are 0,
// far below anything the sums and draws resolve (each draw or sum is relative to a row
// whose weights add up to 1).
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Weight exp((v - top) / T) = 2^((v - top) * sl), sl = log2(e) / T, of a partial whose
// maximum is v when a row's partials are merged under the row maximum top. Each partial's
// own sum is already an fp32 sum of the same hardware exponential, so forming its weight
// the same way keeps the merged sum at that precision (about 1e-7 relative); the terms
// are added in fp64.
__device__ inline double partial_weight(float v, float top, float sl) {
  return (double)exp2_hw((v - top) * sl);
}

// Order used for argmax: larger value first, then lower index.
__device__ inline bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Arguments of the LM-head verify kernels (sd_verify_logits).
struct VerifyArgs {
  const uint16_t *hidden;       // bf16 [B][gamma + 1][d]
  const uint16_t *W;            // bf16 [V][d], or the stage-major blocked copy (w_blocked)
  const int32_t *draft_tokens;  // [B][gamma] or null
  const int32_t *verify_len;    // [B] or null
  RowMap rm;
  int d, V;
  float temperature;            // 0: greedy statistics only
  float scale_log2;             // log2(e) / T, or 0
  double invT;                  // 1 / T, or 0
  float *logits;                // fp32 [cap][V] or null
  TilePartial *partials;        // [cap][part_stride]
  int part_stride;
  double *zx;                   // [cap] drafted-token logits left by the contraction (NaN:
                                // not computed there), or null when it leaves none
  // W12 LM head (W null): region-blocked 12-byte groups [V/64][d/128][64][16][12],
  // correction slots [V/64][d/128][cap], and the high bytes of codes t = 0..7 (sign
  // clear) in two words: lut0 = t 0..3, lut1 = t 4..7. Null codes: W is bf16.
  const uint8_t *w12_codes;
  const uint32_t *w12_corr;
  int w12_cap;
  uint32_t w12_lut0, w12_lut1;
  sd_row_stats *stats;          // [cap]
  WsHeader *ws;
  // Blocked bf16 LM head: W holds [d/128][ceil(V/64)][64][128] (stage-major), row r's
  // 16-byte chunk j of a block at position j ^ (r & 15), rows past V zero.
  bool w_blocked;
  // Greedy verify decided inside the streaming contraction's launch: with pub set (the
  // workspace's publication area), workgroups g_main .. g_main + B - 1 appended to the
  // grid merge request r = g - g_main's published partials and write its statistics and
  // these outputs (counters may be null).
  unsigned long long *pub;
  int32_t *greedy_accept_len;
  int32_t *greedy_next_token;
  int64_t *greedy_counters;
  // Rejection verify in one call: the streaming contraction's launch gains workgroups
  // g_main .. gridDim.x - 1 that write the drafter chunk partials dpart [B][gamma][dchunks]
  // of every kept draft row (draft_logits bf16 [B][gamma][V]). g_main is the contraction's
  // own grid, set by its launcher.
  // qx [B][gamma] receives, with dpart, the drafter logit of each kept row's drafted token.
  const uint16_t *draft_logits;
  DraftPart *dpart;
  float *qx;
  int dchunks;
  int g_main;
};

// Largest gamma whose rows k_merge_decide merges in one workgroup pass (32 row slots).
constexpr int kDecideMaxGamma = 31;

// Outputs of the rejection decision that k_merge_decide takes after merging the row
// statistics (with VerifyArgs for the rows and the drafter inputs).
struct DecideArgs {
  const float *u_accept;    // [B][gamma]
  double *lse_q;            // [B][gamma] out: drafter log-normaliser of each kept row
  DrawRec *rec;             // [B] out: the draw each request takes
  int32_t *accept_len;      // [B] out
  int32_t *next_token;      // [B] out (-1 for a request outside the row capacity)
  int64_t *counters;        // [2] or null
  // Chunk-sum slots [B][chunks][2] of the one-launch draw that follows, set here to
  // kUnpublished; null when the draw runs in two launches.
  unsigned long long *pub;
  int pub_chunks;
};

// LM-head formats of the streaming contraction.
constexpr int kLmBf16 = 0;      // bf16 [V][d]
constexpr int kLmW12 = 1;       // W12 groups plus correction slots
constexpr int kLmBlocked = 2;   // stage-major blocked bf16

// Prefix scheduler: one workgroup sorts all R * gamma candidates in LDS.
constexpr int kSchedMaxCandidates = 16384;

}  // namespace sdv
