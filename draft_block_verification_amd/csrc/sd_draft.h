// Drafter-row normaliser of one vocabulary chunk, shared by the standalone rejection
// kernel and the workgroups the streaming contraction runs beside its own.
//
// DSpark summary, "Problem definition": rejection sampling compares the target's p with
// the drafter's q = softmax(l / T), so every kept draft row needs log sum_v exp(l_v / T).
// One wave reduces one chunk of kDraftChunk ids to its max and its sum of
// exp((l - max) / T): fp32 weights from the hardware base-2 exponential, summed in fp64.
#pragma once

#include "sd_internal.h"

namespace sdv {

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Loads of chunk c of an aligned row (V % 8 == 0, so V >= 8 and v0 < V means v0 + 8 <= V):
// load h gives lane l ids c * kDraftChunk + 512 h + 8 l .. + 7. The address is clamped
// into the row, so every lane loads; past V the value is -inf.
__device__ inline void draft_chunk_load(const uint16_t *row, int V, int c, int lane,
                                        u32x4 (&w)[8]) {
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int v0 = c * kDraftChunk + 512 * h + 8 * lane;
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + min(v0, V - 8)));
    const u32x4 ninf{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};   // bf16 -inf
    w[h] = v0 < V ? x : ninf;
  }
}

// Ids at -inf add exp2(-inf) = 0; a chunk that is -inf throughout sums to 0.
__device__ inline DraftPart draft_part(float m, const float (&sh)[8]) {
  double S = 0.0;
  if (m != -INFINITY) {
#pragma unroll
    for (int h = 0; h < 8; ++h) S += (double)sh[h];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) S += __shfl_xor(S, off);
  }
  DraftPart p;
  p.m = m; p.pad = 0.f; p.s = S;
  return p;
}

__device__ inline DraftPart draft_chunk_stats(const u32x4 (&w)[8], float sl) {
  float m = -INFINITY;
#pragma unroll
  for (int h = 0; h < 8; ++h)
#pragma unroll
    for (int q = 0; q < 4; ++q) m = fmaxf(m, fmaxf(bf_lo(w[h][q]), bf_hi(w[h][q])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float sh[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    sh[h] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sh[h] += exp2_hw((bf_lo(w[h][q]) - m) * sl);
      sh[h] += exp2_hw((bf_hi(w[h][q]) - m) * sl);
    }
  }
  return draft_part(m, sh);
}

// Rows that are not 16-byte aligned (V % 8 != 0): one id at a time, two passes.
__device__ inline DraftPart draft_chunk_unaligned(const uint16_t *row, int V, int c, int lane,
                                                  float sl) {
  float m = -INFINITY;
#pragma unroll 1
  for (int h = 0; h < 8; ++h)
#pragma unroll 1
    for (int e = 0; e < 8; ++e) {
      const int v = c * kDraftChunk + 512 * h + 8 * lane + e;
      if (v < V) m = fmaxf(m, bf16_to_f32(row[v]));
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float sh[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    sh[h] = 0.f;
#pragma unroll 1
    for (int e = 0; e < 8; ++e) {
      const int v = c * kDraftChunk + 512 * h + 8 * lane + e;
      if (v < V) sh[h] += exp2_hw((bf16_to_f32(row[v]) - m) * sl);
    }
  }
  return draft_part(m, sh);
}

// The partial of chunk c of one drafter row, by one whole wave (every lane returns it).
__device__ inline DraftPart draft_chunk_partial(const uint16_t *row, int V, int c, int lane,
                                                float sl) {
  if ((V & 7) == 0) {
    u32x4 w[8];
    draft_chunk_load(row, V, c, lane, w);
    return draft_chunk_stats(w, sl);
  }
  return draft_chunk_unaligned(row, V, c, lane, sl);
}

// Request r's draw record after the decision a_r = acc over L kept drafts (row base + acc;
// base < 0 marks a request outside the row capacity). lse_p and lse_q are the target and
// drafter log-normalisers of that row; the scale constants are T * lse rounded to fp32.
__device__ inline DrawRec draw_record(int base, int acc, int L, int qrow, double lse_p,
                                      double lse_q, double invT) {
  DrawRec d{};
  d.row = base < 0 ? -1 : base + acc;
  d.acc = acc;
  d.qrow = acc < L ? qrow : -1;
  d.cp = (float)(lse_p / invT);
  d.cq = acc < L ? (float)(lse_q / invT) : 0.f;
  return d;
}

}  // namespace sdv
