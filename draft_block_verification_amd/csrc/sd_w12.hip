// W12 encoder (host): bf16 LM head -> 12-bit groups plus exact correction slots.
//
// SpecPilot page, "Reasons": W12 is a lossless 12-bit weight format whose three
// 4-bit planes are rebuilt in the GEMM's registers. Layout of this library:
//   * a weight's low byte (exponent bit 0, 7 mantissa bits) is kept verbatim;
//   * its high byte (sign, exponent bits 7..1 = e2) becomes a 4-bit code
//     sign << 3 | t, with t = 0 for e2 = 0 and t = e2 - b2 + 1 for e2 in the tensor's
//     window [b2, b2 + 6], b2 = max(1, largest nonzero e2 - 6);
//   * any other weight is coded as a signed zero and listed, with its bits, in the
//     correction slots of its (64-row, 128-column) region, sorted by (row, column);
//   * a group of 8 columns is 12 bytes: the 8 low bytes, then byte 8 + i = code of
//     column 2 i | code of column 2 i + 1 << 4; groups are stored region by region,
//     [V/64][d/128][64 rows][16 groups][12 bytes], rows past V zero, so one region is
//     one contiguous 12 KB block.
#include <string.h>

#include <algorithm>
#include <vector>

#include "sd_internal.h"

namespace {

constexpr int kSlabRows = 64;
constexpr int kStageCols = 128;

inline int pair_of(uint16_t w) { return (w >> 8) & 0x7F; }

}  // namespace

extern "C" {

int32_t sd_w12_encode(const uint16_t *W, int32_t V, int32_t d, uint8_t *codes, uint32_t *corr,
                      int32_t *cap, int32_t *b2) {
  if (!W || !cap || !b2) return SD_EINVAL;
  if (V < 1 || d < kStageCols || d % kStageCols != 0) return SD_ESHAPE;
  const size_t n = (size_t)V * d;
  int top = 0;
  for (size_t i = 0; i < n; ++i) {
    const int p = pair_of(W[i]);
    if (p > top) top = p;
  }
  const int lo = top >= 1 ? (top - 6 > 1 ? top - 6 : 1) : 1;
  auto held = [lo](uint16_t w) {
    const int p = pair_of(w);
    return p == 0 || (p >= lo && p <= lo + 6);
  };
  // Corrections per region, counted row by row.
  const int nslab = (V + kSlabRows - 1) / kSlabRows, nst = d / kStageCols;
  std::vector<int32_t> count((size_t)nslab * nst, 0);
  for (int v = 0; v < V; ++v)
    for (int k = 0; k < d; ++k)
      if (!held(W[(size_t)v * d + k])) ++count[(size_t)(v / kSlabRows) * nst + k / kStageCols];
  int fullest = 0;
  for (int32_t c : count) fullest = c > fullest ? c : fullest;
  const int need = fullest <= 4 ? 4 : (fullest + 3) / 4 * 4;
  *b2 = lo;
  if (!corr) {                       // sizing call
    *cap = need;
    return SD_OK;
  }
  if (!codes) return SD_EINVAL;
  if (*cap < need) {
    *cap = need;
    return SD_EWORKSPACE;
  }
  const int slots = *cap;
  memset(corr, 0, sizeof(uint32_t) * (size_t)nslab * nst * slots);
  memset(codes, 0, (size_t)nslab * kSlabRows * (d / 8) * 12);
  std::fill(count.begin(), count.end(), 0);
  for (int v = 0; v < V; ++v) {
    const uint16_t *row = W + (size_t)v * d;
    for (int g = 0; g < d / 8; ++g) {
      const int st = g / (kStageCols / 8);
      uint8_t *out = codes + ((((size_t)(v / kSlabRows) * nst + st) * kSlabRows + v % kSlabRows) *
                                  (kStageCols / 8) + g % (kStageCols / 8)) * 12;
      uint8_t nib[8];
      for (int j = 0; j < 8; ++j) {
        const int k = 8 * g + j;
        const uint16_t w = row[k];
        const int sign = w >> 15, p = pair_of(w);
        if (held(w)) {
          out[j] = (uint8_t)(w & 0xFF);
          nib[j] = (uint8_t)(sign << 3 | (p == 0 ? 0 : p - lo + 1));
        } else {
          out[j] = 0;
          nib[j] = (uint8_t)(sign << 3);
          const size_t r = (size_t)(v / kSlabRows) * nst + k / kStageCols;
          // Rows, then columns, arrive in increasing order: the slots stay sorted.
          corr[r * slots + count[r]++] =
              (uint32_t)(k % kStageCols) | (uint32_t)(v % kSlabRows) << 7 | (uint32_t)w << 16;
        }
      }
      for (int i = 0; i < 4; ++i) out[8 + i] = (uint8_t)(nib[2 * i] | nib[2 * i + 1] << 4);
    }
  }
  *cap = slots;
  return SD_OK;
}

}  // extern "C"
