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
  uint32_t ticket;     // arrival counter for last-workgroup epilogues (returns to 0)
  uint32_t pad[62];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

// Statistics of one verified row over one vocabulary tile.
struct TilePartial {
  float top1;   // max z over the tile
  float top2;   // max z over the tile excluding the argmax position
  int32_t arg;  // lowest vocabulary id attaining top1
  float sum;    // sum over the tile of exp((z - top1) / T); 0 when T == 0
};
static_assert(sizeof(TilePartial) == 16, "partials are 16 bytes");

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

// Kept drafts of request r, clamped to [0, gamma] (flagged when out of range).
__device__ inline int clamp_len(const int32_t *verify_len, int r, int gamma, WsHeader *ws) {
  if (!verify_len) return gamma;
  int L = verify_len[r];
  if (L < 0 || L > gamma) {
    raise_flag(ws, SD_FLAG_VERIFY_LEN);
    L = L < 0 ? 0 : gamma;
  }
  return L;
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
};

// LM-head formats of the streaming contraction.
constexpr int kLmBf16 = 0;      // bf16 [V][d]
constexpr int kLmW12 = 1;       // W12 groups plus correction slots
constexpr int kLmBlocked = 2;   // stage-major blocked bf16

// Prefix scheduler: one workgroup sorts all R * gamma candidates in LDS.
constexpr int kSchedMaxCandidates = 16384;

}  // namespace sdv
