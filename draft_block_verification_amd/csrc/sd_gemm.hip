// LM-head verify contraction with fused row statistics (gfx950).
//
// z[m][v] = sum_k h[m][k] * W[v][k] for the M packed verified rows (LFM2.5-DSpark
// blog, "How DSpark works": the target checks the whole drafted block in one pass
// and shares one weight load across it; DSpark summary, "Production deployment":
// the LM head maps the d-vector to V logits, and variable-length requests are
// flattened rather than padded).
//
// Both operands are K-contiguous bf16 (hidden rows [M][d], LM head [V][d]); products
// run on the 16x16x32 bf16 MFMA with fp32 accumulation. Regimes by row capacity:
//   * streaming (M <= 64): a persistent grid walks the vocabulary in 64-row slabs and
//     reads W from HBM exactly once. k_gemm_skinny (d % 128 == 0) moves each stage
//     straight into LDS with global_load_lds and keeps NS-1 stages in flight;
//     k_gemm_stream (any d % 8 == 0) stages through registers. One partial per
//     (row, workgroup).
//   * tiled (M > 64): BM x BN output tiles, k_gemm_dma (direct-to-LDS, 8 waves, for
//     d % 64 == 0) or k_gemm_tile (register-staged, any d); one partial per (row,
//     vocabulary tile).
// k_row_merge then combines each row's partials (one workgroup per row).
// Row statistics: max, second max, lowest argmax and sum of exp((z - max) / T); the
// drafted token's logit is recomputed exactly as an fp64 dot of the bf16 inputs.
#include <math.h>

#include "sd_draft.h"
#include "sd_launch.h"

#define LDSP __attribute__((address_space(3)))
#define GLBP __attribute__((address_space(1)))

// Cache-policy operand of global_load_lds for data read exactly once (the nt bit).
constexpr int kCachePolicyStream = 2;

// Workgroup barrier without the vmcnt(0) that __syncthreads implies: callers wait for
// their own direct-to-LDS loads with an explicit vmcnt first. The empty asm statements
// keep the compiler from moving LDS accesses across the barrier.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

namespace sdv {
namespace {

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline bf16x8 load8(const uint16_t *p) {
  return as_bf16x8(*reinterpret_cast<const u32x4 *>(p));
}

struct RowAcc {
  float t1, t2, sum;
  int arg;
};

__device__ inline RowAcc row_acc_init() { return RowAcc{-INFINITY, -INFINITY, 0.f, 0x7fffffff}; }

// The value lane l ^ off holds, off = 16 or 32, from gfx950's lane-swap instructions:
// v_permlane16/32_swap exchange the odd and even 16-lane (32-lane) halves of two
// registers, so lane l finds lane l ^ off's value in the first result when bit off of l
// is set and in the second otherwise. One VALU instruction each, no LDS crossbar.
__device__ inline uint32_t lane_xor_u32(uint32_t x, int off) {
  if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  }
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ inline float lane_xor(float x, int off) { return __uint_as_float(lane_xor_u32(__float_as_uint(x), off)); }
__device__ inline int lane_xor(int x, int off) { return (int)lane_xor_u32((uint32_t)x, off); }
__device__ inline double lane_xor(double x, int off) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t lo = lane_xor_u32((uint32_t)b, off), hi = lane_xor_u32((uint32_t)(b >> 32), off);
  return __longlong_as_double((long long)(lo | (hi << 32)));
}

// Lane i's value from lane i ^ 1 or i ^ 2 (quad permutes), or from lane (i + 4) or
// (i + 8) mod 16 of its row (row rotations): cross-lane moves in the VALU, no LDS.
__device__ inline uint32_t lane_dpp_u32(uint32_t x, int ctrl) {
  switch (ctrl) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
    case 4: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
  }
}

// Merge of disjoint sets' (max, runner-up, lowest id of the max): every lane of the wave
// ends with the triple of all 64 lanes. Quad permutes, then row rotations by 4 and 8
// (after the quads, lane i and lane i + 4 of a row hold different quads, then different
// halves), then the 16- and 32-lane swaps; every step merges two disjoint sets, and the
// merge is exact, so the result is the same triple whatever the order.
__device__ inline void wave_merge_top2(float &t1, float &t2, int &a1) {
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    float o1, o2;
    int oa;
    if (step < 4) {
      const int c = 1 << step;
      o1 = __uint_as_float(lane_dpp_u32(__float_as_uint(t1), c));
      o2 = __uint_as_float(lane_dpp_u32(__float_as_uint(t2), c));
      oa = (int)lane_dpp_u32((uint32_t)a1, c);
    } else {
      const int off = step == 4 ? 16 : 32;
      o1 = lane_xor(t1, off);
      o2 = lane_xor(t2, off);
      oa = lane_xor(a1, off);
    }
    if (beats(o1, oa, t1, a1)) { t2 = fmaxf(t1, o2); t1 = o1; a1 = oa; }
    else { t2 = fmaxf(t2, o1); }
  }
}

// Fold a tile's (t1, t2, arg, sum) into a running value; sums are relative to t1.
__device__ inline void row_acc_merge(RowAcc &r, const RowAcc &o, float scale_log2) {
  const bool win = beats(o.t1, o.arg, r.t1, r.arg);
  const float nt1 = win ? o.t1 : r.t1;
  float s = 0.f;
  if (scale_log2 > 0.f) {
    if (r.sum != 0.f) s += r.sum * exp2f((r.t1 - nt1) * scale_log2);
    if (o.sum != 0.f) s += o.sum * exp2f((o.t1 - nt1) * scale_log2);
  }
  if (win) { r.t2 = fmaxf(r.t1, o.t2); r.arg = o.arg; }
  else { r.t2 = fmaxf(r.t2, o.t1); }
  r.t1 = nt1;
  r.sum = s;
}

// Statistics of row `rr` of an fp32 tile in LDS over COLS columns, shared by the TPR
// consecutive threads of the row (all of them return the same value).
template <int ROWS, int COLS, int LDC>
__device__ RowAcc tile_row_stats(const float *Cs, int v0, int V, float scale_log2) {
  static_assert(256 % ROWS == 0, "rows must divide the workgroup");
  constexpr int TPR = 256 / ROWS;
  static_assert(COLS % TPR == 0 && TPR <= 64, "columns must split evenly");
  constexpr int CPT = COLS / TPR;
  const int rr = threadIdx.x / TPR, sub = threadIdx.x % TPR;
  const float *row = Cs + rr * LDC;
  float t1 = -INFINITY, t2 = -INFINITY;
  int a1 = 0x7fffffff;
#pragma unroll 4
  for (int i = 0; i < CPT; ++i) {
    const int c = sub + TPR * i;
    const int v = v0 + c;
    if (v < V) {
      const float z = row[c];
      if (beats(z, v, t1, a1)) { t2 = t1; t1 = z; a1 = v; }
      else if (z > t2) t2 = z;
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) {
    const float o1 = __shfl_xor(t1, off), o2 = __shfl_xor(t2, off);
    const int oa = __shfl_xor(a1, off);
    if (beats(o1, oa, t1, a1)) { t2 = fmaxf(t1, o2); t1 = o1; a1 = oa; }
    else { t2 = fmaxf(t2, o1); }
  }
  float s = 0.f;
  if (scale_log2 > 0.f) {
#pragma unroll 4
    for (int i = 0; i < CPT; ++i) {
      const int c = sub + TPR * i;
      if (v0 + c < V) s += exp2f((row[c] - t1) * scale_log2);
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  }
  return RowAcc{t1, t2, s, a1};
}

// fp32 logits of an LDS tile for rows m0.. < M and columns v0.. < V.
template <int ROWS, int COLS, int LDC>
__device__ void tile_store_logits(const float *Cs, float *logits, int m0, int v0, int M, int V) {
  for (int idx = threadIdx.x; idx < ROWS * COLS; idx += 256) {
    const int rr = idx / COLS, cc = idx - rr * COLS;
    const int m = m0 + rr, v = v0 + cc;
    if (m < M && v < V) logits[(size_t)m * V + v] = Cs[rr * LDC + cc];
  }
}

// Sum of a double over the workgroup (fixed order: wave butterflies, then waves 0..3).
__device__ inline double block_sum(double x, double *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ inline void write_stats(const VerifyArgs &a, int m, float t1, float t2, int arg,
                                   double lse, double zd) {
  int r, j;
  hidden_row(a.rm, m, &r, &j);
  sd_row_stats st;
  st.argmax = arg;
  st.top1 = t1;
  st.top2 = t2;
  st.pos = j;
  st.lse = lse;
  st.z_draft = zd;
  a.stats[m] = st;
}

// ------------------------------------------------------------- streaming regime
template <int MT, int BN, int KC>
__global__ __launch_bounds__(256) void k_gemm_stream(VerifyArgs a) {
  constexpr int CH = KC / 8;                 // 16-byte chunks per row per stage
  constexpr int ROWS = BN + 16 * MT;         // LM-head rows, then hidden rows
  constexpr int STAGE = ROWS * KC;           // bf16 elements per stage buffer
  constexpr int LOADS = ROWS * CH / 256;     // 16-byte loads per thread per stage
  constexpr int WN = BN / 16, SKW = 4 / WN;  // waves along vocabulary / along k
  constexpr int STEPS = KC / 32 / SKW;       // MFMA k-steps per wave per stage
  constexpr int CR = 16 * MT, LDC = BN + 4;
  static_assert(ROWS * CH % 256 == 0 && KC % (32 * SKW) == 0 && WN * SKW == 4, "shape");
  static_assert(CR * LDC * 4 <= STAGE * 2, "the output tile fits in one stage buffer");
  __shared__ __attribute__((aligned(16))) uint16_t S[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wk = wave / WN;
  const int G = gridDim.x, g = blockIdx.x;
  const int M = rows_total(a.rm);
  const int d = a.d, V = a.V;

  // This thread's loads: row r (< BN: LM head, else hidden row r - BN), chunk c.
  int l_row[LOADS], l_off[LOADS], l_k[LOADS];
  const uint16_t *l_hid[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int e = tid + 256 * i, r = e / CH, c = e % CH;
    l_row[i] = r;
    l_k[i] = 8 * c;
    l_off[i] = r * KC + 8 * (c ^ (r & 15));
    l_hid[i] = a.hidden;                        // rows past M read row 0; never used
    if (r >= BN) {
      const int m = r - BN;
      if (m < M) {
        int rq, j;
        const int hr = hidden_row(a.rm, m, &rq, &j);
        if (hr >= 0) l_hid[i] = a.hidden + (size_t)hr * d;
        else raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
      }
    }
  }
  const int nslab = (V + BN - 1) / BN;
  const int nst = (d + KC - 1) / KC;
  const int total = ((nslab - g + G - 1) / G) * nst;   // (slab, stage) pairs of this workgroup

  u32x4 R[LOADS];
  // Loads of pair t (clamped to the last pair). k beyond d loads a valid address and
  // keeps zeros, so the loop has no data-dependent branches around its loads.
  auto gload = [&](int t) {
    t = t < total ? t : total - 1;
    const int slab = g + (t / nst) * G, k0 = (t % nst) * KC;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int k = k0 + l_k[i];
      const bool ok = k < d;
      const int kk = ok ? k : d - 8;
      const uint16_t *row = l_row[i] < BN ? a.W + (size_t)min(slab * BN + l_row[i], V - 1) * d
                                          : l_hid[i];
      const u32x4 v = *reinterpret_cast<const u32x4 *>(row + kk);
      R[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) *reinterpret_cast<u32x4 *>(S + buf * STAGE + l_off[i]) = R[i];
  };

  f32x4 acc[MT], cacc[MT];                   // cacc: W12 corrected weights' products
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = cacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int br = 16 * wn + (lane & 15);
  RowAcc run = row_acc_init();                  // running stats of row tid / (256 / CR)

  gload(0);
  sstore(0);
  __syncthreads();
  for (int t = 0; t < total; ++t) {
    const int buf = t & 1;
    gload(t + 1);
    const uint16_t *Sb = S + buf * STAGE;
#pragma unroll
    for (int q = 0; q < STEPS; ++q) {
      const int c = 4 * (wk * STEPS + q) + (lane >> 4);
      const bf16x8 b = load8(Sb + br * KC + 8 * (c ^ (br & 15)));
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int ar = BN + 16 * i + (lane & 15);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            load8(Sb + ar * KC + 8 * (c ^ (ar & 15))), b, acc[i], 0, 0, 0);
      }
    }
    sstore(buf ^ 1);
    __syncthreads();
    if (t % nst == nst - 1) {
      // Slab finished: sum the k-split waves in a fixed order, then row statistics.
      // The tile lives in the stage buffer just consumed; the next store into it comes
      // after the barrier that ends this block.
      float *Cs = reinterpret_cast<float *>(S + buf * STAGE);
      const int v0 = (g + (t / nst) * G) * BN;
      for (int w = 0; w < SKW; ++w) {
        if (wk == w) {
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int rr = 16 * i + 4 * (lane >> 4) + q, cc = 16 * wn + (lane & 15);
              if (w == 0) Cs[rr * LDC + cc] = acc[i][q];
              else Cs[rr * LDC + cc] += acc[i][q];
            }
        }
        __syncthreads();
      }
      if (a.logits) tile_store_logits<CR, BN, LDC>(Cs, a.logits, 0, v0, M, V);
      const RowAcc ts = tile_row_stats<CR, BN, LDC>(Cs, v0, V, a.scale_log2);
      row_acc_merge(run, ts, a.scale_log2);
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
    }
  }

  // One partial per (row, workgroup); k_row_merge combines them.
  constexpr int TPR = 256 / CR;
  const int m = tid / TPR;
  if (tid % TPR == 0 && m < M) {
    TilePartial p;
    p.top1 = run.t1; p.top2 = run.t2; p.arg = run.arg; p.sum = run.sum;
    a.partials[(size_t)m * a.part_stride + g] = p;
  }
}

// ---------------------------------------------------------------- W12 decoding
// Eight bf16 weights of one W12 group (12 bytes: l0, l1 the low bytes of columns 0-3
// and 4-7, n the eight 4-bit codes, column j in bits 4j..4j+3). A code holds the sign
// in bit 3 and t in bits 0-2; the high byte is sign << 7 | lut[t], looked up four at a
// time with one byte permute (lut0 / lut1: the high bytes of t = 0..3 / 4..7), then
// interleaved with the low bytes into bf16 pairs. SpecPilot page, "Reasons": the
// weights travel as 4-bit planes and are rebuilt in the GEMM's registers.
__device__ inline u32x4 w12_decode8(uint32_t l0, uint32_t l1, uint32_t n, uint32_t lut0,
                                    uint32_t lut1) {
  const uint32_t y = n & 0x0F0F0F0Fu, z = (n >> 4) & 0x0F0F0F0Fu;
  const uint32_t x0 = __builtin_amdgcn_perm(z, y, 0x05010400u);   // codes of columns 0..3
  const uint32_t x1 = __builtin_amdgcn_perm(z, y, 0x07030602u);   // columns 4..7
  const uint32_t h0 = __builtin_amdgcn_perm(lut1, lut0, x0 & 0x07070707u) | ((x0 & 0x08080808u) << 4);
  const uint32_t h1 = __builtin_amdgcn_perm(lut1, lut0, x1 & 0x07070707u) | ((x1 & 0x08080808u) << 4);
  return u32x4{__builtin_amdgcn_perm(h0, l0, 0x05010400u), __builtin_amdgcn_perm(h0, l0, 0x07030602u),
               __builtin_amdgcn_perm(h1, l1, 0x05010400u), __builtin_amdgcn_perm(h1, l1, 0x07030602u)};
}

// Block permutation of a W12 stage row in LDS: the row's four 48-byte blocks (four
// 12-byte groups each) are stored at block b ^ w12_block_swz(row). A fragment read takes
// one group from each of 16 consecutive rows; with 192-byte rows those rows repeat every
// four in the 64 banks, and the permutation spreads them over all of them.
__device__ inline int w12_block_swz(int row) { return (row >> 2) & 3; }

// Byte offset of group c of LM-head row x in the region-blocked W12 layout.
__device__ inline size_t w12_group_offset(int x, int c, int nst) {
  return ((((size_t)(x >> 6) * nst + (c >> 4)) * 64 + (x & 63)) * 16 + (c & 15)) * 12;
}

// Part of the exact logit hidden . W[x] taken by thread t of nt: groups t, t + nt, ...
// of the LM-head row (bf16, or W12 codes plus that row's corrections).
__device__ inline double lm_head_dot_part(const VerifyArgs &a, const uint16_t *h, int x, int t,
                                          int nt) {
  const int ng = a.d / 8;
  double part = 0.0;
  if (a.w_blocked) {
    // Block (c / 16, x / 64) -- stage-major -- holds row x & 63 at 128 values per row;
    // chunk c & 15 sits at position (c & 15) ^ (x & 15).
    const size_t sstride = (size_t)((a.V + 63) / 64) * 8192;   // bf16 per stage of blocks
    const uint16_t *w = a.W + (size_t)(x >> 6) * 8192 + (size_t)(x & 63) * 128;
    for (int c = t; c < ng; c += nt)
      part += dot8_f64(*reinterpret_cast<const u32x4 *>(h + 8 * c),
                       *reinterpret_cast<const u32x4 *>(w + (size_t)(c >> 4) * sstride +
                                                        8 * ((c & 15) ^ (x & 15))));
    return part;
  }
  if (!a.w12_codes) {
    const uint16_t *w = a.W + (size_t)x * a.d;
    for (int c = t; c < ng; c += nt)
      part += dot8_f64(*reinterpret_cast<const u32x4 *>(h + 8 * c),
                       *reinterpret_cast<const u32x4 *>(w + 8 * c));
    return part;
  }
  const int nst = a.d / 128, rl = x & 63;
  for (int c = t; c < ng; c += nt) {
    const uint32_t *g = reinterpret_cast<const uint32_t *>(a.w12_codes + w12_group_offset(x, c, nst));
    part += dot8_f64(*reinterpret_cast<const u32x4 *>(h + 8 * c),
                     w12_decode8(g[0], g[1], g[2], a.w12_lut0, a.w12_lut1));
  }
  for (int s = t; s < nst; s += nt) {
    const uint32_t *slot = a.w12_corr + ((size_t)(x >> 6) * nst + s) * a.w12_cap;
    for (int e = 0; e < a.w12_cap; ++e) {
      const uint32_t ent = slot[e];
      if (ent != 0u && (int)((ent >> 7) & 63u) == rl)
        part += (double)bf16_to_f32(h[128 * s + (ent & 127u)]) * (double)__uint_as_float(ent & 0xffff0000u);
    }
  }
  return part;
}

// Statistics of verified row j of request r (packed row m) once lane `lane` of the wave
// holds its share (t1, t2, a1) of the row's merged partials: the wave reduces them, forms
// the drafted token's exact logit when the contraction left none (zx NaN or absent), and
// lane 0 writes the row's statistics and its argmax and drafted token to s_arg / s_x.
// The merge is exact (max with lowest-id ties, and a max for the runner-up), so any
// split of the partials over lanes gives the same bytes.
__device__ inline void greedy_row_finish(const VerifyArgs &a, int r, int j, int L, int m, int x,
                                         bool has_x, double zg, float t1, float t2, int a1,
                                         int lane, int *s_arg, int *s_x) {
  const bool need_dot = has_x && (!a.zx || zg != zg);
  double part = 0.0;
  if (need_dot) {
    part = lm_head_dot_part(a, a.hidden + ((size_t)r * (a.rm.gamma + 1) + j) * a.d, x, lane, 64);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  }
  wave_merge_top2(t1, t2, a1);
  if (lane == 0) {
    sd_row_stats st;
    st.argmax = a1;
    st.top1 = t1;
    st.top2 = t2;
    st.pos = j;
    st.lse = 0.0;
    st.z_draft = need_dot ? part : (has_x ? zg : 0.0);
    a.stats[m] = st;
    s_arg[j] = a1;
    if (j < L) s_x[j] = x;
  }
}

// Greedy acceptance of request r from its rows' argmaxes in s_arg and drafted tokens in
// s_x (LFM2.5-DSpark blog, "Quality parity"): a_r is the first row whose argmax differs
// from the draft (L_r when none does) and the next token is that row's argmax. Wave 0.
__device__ inline void greedy_decide(int r, int L, const int *s_arg, const int *s_x,
                                     int32_t *accept_len, int32_t *next_token,
                                     int64_t *counters, int lane) {
  const bool miss = lane < L && s_arg[lane] != s_x[lane];
  const unsigned long long mask = __ballot(miss);
  const int acc = mask ? (__ffsll((long long)mask) - 1) : L;
  if (lane == 0) {
    accept_len[r] = acc;
    next_token[r] = s_arg[acc];
    if (counters) {
      atomicAdd(reinterpret_cast<unsigned long long *>(counters), (unsigned long long)L);
      atomicAdd(reinterpret_cast<unsigned long long *>(counters + 1), (unsigned long long)acc);
    }
  }
}

// Greedy verify tail of request r, by the workgroup's nw waves (one wave per row):
// merges the n partials of each of its rows 0..L_r, writes their statistics with the
// drafted token's exact logit, then decides. s_arg[65] and s_x[64] are LDS; every
// thread of the workgroup calls it, and it returns with the workgroup converged (a
// request outside the rows the contraction computed returns early for all).
constexpr int kFusedPer = 8;    // loads in flight per lane

__device__ inline void merge_accept_greedy_request(
    const VerifyArgs &a, int r, int n, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ next_token, int64_t *__restrict__ counters, int nw, int *s_arg,
    int *s_x) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gamma = a.rm.gamma;
  // Two rounds of loads: the request's length, offset and the row count together, then
  // each row's drafted token, drafted-token logit and partials together.
  const int Lraw = a.verify_len ? a.verify_len[r] : gamma;
  const int base = a.rm.row_offsets ? a.rm.row_offsets[r] : r * (gamma + 1);
  const int M = rows_total(a.rm);
  const int L = clamp_len_value(Lraw, gamma, tid == 0 ? a.ws : nullptr);
  if (base < 0 || base + L >= M) {
    if (tid == 0) {
      raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
      accept_len[r] = 0;
      next_token[r] = -1;
    }
    return;
  }
  for (int j = wave; j <= L; j += nw) {
    const int m = base + j;
    // Only without a logit from the contraction (NaN or none) are the hidden and LM-head
    // rows read for the fp64 dot.
    const int xr = j < gamma ? a.draft_tokens[(size_t)r * gamma + j] : -1;
    const double zr = a.zx ? a.zx[m] : 0.0;
    const int x = j < L ? xr : -1;
    const bool has_x = x >= 0 && x < a.V;
    const double zg = has_x ? zr : 0.0;
    const TilePartial *P = a.partials + (size_t)m * a.part_stride;
    float t1 = -INFINITY, t2 = -INFINITY;
    int a1 = 0x7fffffff;
    for (int p0 = 0; p0 < n; p0 += 64 * kFusedPer) {
      TilePartial q[kFusedPer];
#pragma unroll
      for (int i = 0; i < kFusedPer; ++i) {
        const int p = p0 + lane + 64 * i;
        q[i] = p < n ? P[p] : TilePartial{-INFINITY, -INFINITY, 0x7fffffff, 0.f};
      }
#pragma unroll
      for (int i = 0; i < kFusedPer; ++i) {
        if (beats(q[i].top1, q[i].arg, t1, a1)) { t2 = fmaxf(t1, q[i].top2); t1 = q[i].top1; a1 = q[i].arg; }
        else { t2 = fmaxf(t2, q[i].top1); }
      }
    }
    greedy_row_finish(a, r, j, L, m, x, has_x, zg, t1, t2, a1, lane, s_arg, s_x);
  }
  __syncthreads();
  if (wave == 0) greedy_decide(r, L, s_arg, s_x, accept_len, next_token, counters, lane);
}

// ---------------------------------- greedy decision inside the streaming contraction
// Words of a published partial: the bits of (top1, top2) and of (arg, sum). A partial's
// arg is a vocabulary id or 0x7fffffff, never -1, so its second word is never kPubEmpty;
// the first would need two fp32 NaNs with every bit set, which no arithmetic result
// carries. A drafted-token logit is published as its fp64 bits: a computed value or a
// quiet NaN from arithmetic, never all ones either.
__device__ inline unsigned long long pub_word0(const TilePartial &p) {
  return (unsigned long long)__float_as_uint(p.top1) |
         ((unsigned long long)__float_as_uint(p.top2) << 32);
}
__device__ inline unsigned long long pub_word1(const TilePartial &p) {
  return (unsigned long long)(uint32_t)p.arg | ((unsigned long long)__float_as_uint(p.sum) << 32);
}
__device__ inline void pub_store(unsigned long long *w, unsigned long long v) {
  __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned long long pub_load(unsigned long long *w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Buffer e & 1 of the publication area.
__device__ inline unsigned long long *pub_buffer(const VerifyArgs &a, uint32_t e) {
  return a.pub + (size_t)(e & 1u) * kPubWords;
}
// Layout of a launch with M rows and n contraction workgroups: partial (m, g) at words
// 2 (m n + g) and 2 (m n + g) + 1, then the drafted-token logit of row m at 2 M n + m.
__host__ __device__ inline int pub_words_used(int M, int n) { return 2 * M * n + M; }

constexpr int kTailRowsPerWave = 3;                 // rows per wave: up to 12 per request
constexpr int kTailMaxRows = 4 * kTailRowsPerWave;
constexpr int kTailPerLane = kPubMaxGrid / 64;      // partials per lane and row
constexpr int kTailMaxRequests = 16;
constexpr int kTailSpinLimit = 1 << 20;

// Greedy verify of request r inside the streaming contraction's launch, by a workgroup
// appended to its grid; the n contraction workgroups publish every row's partial and
// the drafted-token logits into buffer pub_epoch & 1. Wave w takes rows w, w + 4 and
// w + 8 of the request, lane l the partials l + 64 i. The wave loads every word it needs,
// and loads them again (after a short sleep) until none is kPubEmpty; each word is
// written once per launch, so what it then holds is final. Rows are merged, finished and
// decided exactly as merge_accept_greedy_request does. The last deciding workgroup to
// finish (of B) records the words this launch published and moves the header to the
// other buffer; every workgroup of the launch read the header before that. A wait that
// runs out raises SD_FLAG_WAIT (the request's outputs are then not valid).
__device__ void greedy_decide_published(const VerifyArgs &a, int r, int n, int *s_arg, int *s_x) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gamma = a.rm.gamma;
  const uint32_t epoch = a.ws->pub_epoch;
  unsigned long long *buf = pub_buffer(a, epoch);
  const int M = rows_total(a.rm);
  const int L = clamp_len(a.verify_len, r, gamma, tid == 0 ? a.ws : nullptr);
  const int base = a.rm.row_offsets ? a.rm.row_offsets[r] : r * (gamma + 1);
  if (base < 0 || base + L >= M) {
    if (tid == 0) {
      raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
      a.greedy_accept_len[r] = 0;
      a.greedy_next_token[r] = -1;
    }
  } else {
    const int ipr = (n + 63) / 64;
    // zx[k]: whether the contraction publishes row k's drafted-token logit. It does for
    // a drafted row when it maps that packed row back to this request and position;
    // offsets that disagree with the lengths make it map the row elsewhere, and the
    // row then takes the fp64 dot here (flagged).
    int x[kTailRowsPerWave];
    bool hx[kTailRowsPerWave], zx[kTailRowsPerWave];
#pragma unroll
    for (int k = 0; k < kTailRowsPerWave; ++k) {
      const int j = wave + 4 * k;
      x[k] = j < L ? a.draft_tokens[(size_t)r * gamma + j] : -1;
      hx[k] = x[k] >= 0 && x[k] < a.V;
      int rq = -1, jj = -1;
      if (hx[k]) hidden_row(a.rm, base + j, &rq, &jj);
      zx[k] = hx[k] && rq == r && jj == j;
      if (hx[k] && !zx[k] && lane == 0) raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
    }
    unsigned long long w0[kTailRowsPerWave][kTailPerLane], w1[kTailRowsPerWave][kTailPerLane];
    unsigned long long zw[kTailRowsPerWave];
    for (int it = 0;; ++it) {
      // Every load is issued before any is tested. Rows past L_r, partials past n and
      // rows without a published logit load a word the request does publish (row L_r,
      // partial n - 1) and are left out of the merge.
#pragma unroll
      for (int k = 0; k < kTailRowsPerWave; ++k) {
        const size_t row = (size_t)(base + min(wave + 4 * k, L)) * n;
#pragma unroll
        for (int i = 0; i < kTailPerLane; ++i) {
          unsigned long long *w = buf + 2 * (row + min(lane + 64 * i, n - 1));
          w0[k][i] = pub_load(w);
          w1[k][i] = pub_load(w + 1);
        }
        zw[k] = pub_load(zx[k] ? buf + 2 * (size_t)M * n + base + wave + 4 * k : buf + 2 * row);
      }
      bool ok = true;
#pragma unroll
      for (int k = 0; k < kTailRowsPerWave; ++k) {
#pragma unroll
        for (int i = 0; i < kTailPerLane; ++i)
          ok &= (w0[k][i] != kPubEmpty) & (w1[k][i] != kPubEmpty);
        ok &= zw[k] != kPubEmpty;
      }
      if (__all(ok)) break;
      if (it == kTailSpinLimit) {
        if (lane == 0) raise_flag(a.ws, SD_FLAG_WAIT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int k = 0; k < kTailRowsPerWave; ++k) {
      const int j = wave + 4 * k;
      if (j > L) break;
      float t1 = -INFINITY, t2 = -INFINITY;
      int a1 = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kTailPerLane; ++i) {
        if (i < ipr && lane + 64 * i < n) {
          const float q1 = __uint_as_float((uint32_t)w0[k][i]);
          const float q2 = __uint_as_float((uint32_t)(w0[k][i] >> 32));
          const int qa = (int)(uint32_t)w1[k][i];
          if (beats(q1, qa, t1, a1)) { t2 = fmaxf(t1, q2); t1 = q1; a1 = qa; }
          else { t2 = fmaxf(t2, q1); }
        }
      }
      const double zg = zx[k] ? __longlong_as_double((long long)zw[k])
                      : hx[k] ? __longlong_as_double(0x7ff8000000000000ll) : 0.0;
      greedy_row_finish(a, r, j, L, base + j, x[k], hx[k], zg, t1, t2, a1, lane, s_arg, s_x);
    }
    __syncthreads();
    if (wave == 0)
      greedy_decide(r, L, s_arg, s_x, a.greedy_accept_len, a.greedy_next_token,
                    a.greedy_counters, lane);
  }
  if (tid == 0) {
    const uint32_t done = a.rm.B == 1 ? 0u : atomicAdd(&a.ws->pub_done, 1u);
    if (done == (uint32_t)(a.rm.B - 1)) {
      a.ws->pub_done = 0u;
      a.ws->pub_prev = (uint32_t)pub_words_used(M, n);
      a.ws->pub_epoch = epoch + 1u;
    }
  }
}

// Drafter chunk partials of every kept draft row, walked by the nw workgroups appended to
// the streaming contraction's grid (this one is number w): wave i of the walk takes items
// i, i + 4 nw, ... of the (draft row, chunk) list, so neighbouring waves read neighbouring
// chunks of one row. The bytes are those the standalone drafter-normaliser kernel writes.
__device__ void draft_partials_walk(const VerifyArgs &a, int w, int nw) {
  const int lane = threadIdx.x & 63, gamma = a.rm.gamma, C = a.dchunks;
  const int items = a.rm.B * gamma * C;
  for (int it = 4 * w + (threadIdx.x >> 6); it < items; it += 4 * nw) {
    const int rj = it / C, c = it - rj * C;
    const int r = rj / gamma, j = rj - r * gamma;
    const int L = clamp_len(a.verify_len, r, gamma, c == 0 && lane == 0 ? a.ws : nullptr);
    if (j >= L) continue;
    const uint16_t *row = a.draft_logits + (size_t)rj * a.V;
    const int x = a.draft_tokens[rj];
    const bool own_x = x >= 0 && x < a.V && x / kDraftChunk == c;
    const float lx = own_x ? bf16_to_f32(row[x]) : 0.f;
    const DraftPart p = draft_chunk_partial(row, a.V, c, lane, a.scale_log2);
    if (lane == 0) {
      a.dpart[(size_t)rj * C + c] = p;
      if (own_x) a.qx[rj] = lx;
    }
  }
}

// ------------------------------------------------- streaming regime, direct to LDS
// The streaming kernel for d % KC == 0. global_load_lds_dwordx4 moves every wave
// load's 1 KB (four 256-byte row segments for KC = 128) straight into one of NS LDS
// stage buffers, so NS-1 stages stay in flight per workgroup with no registers held.
// Wave w owns LM-head rows 16w..16w+15 of each 64-row slab over the full k range, so
// a slab's 16 x 16 output tiles are complete in registers and its row statistics are
// reduced with lane shuffles (no LDS round trip, no k-split reduction). The LM-head
// fragment is the MFMA's first operand, so a lane ends a slab holding one hidden row at
// four consecutive vocabulary ids: 16-byte logits stores, and two lane exchanges per
// statistic. A stage row
// holds KC/8 16-byte chunks; chunk j of row r holds logical chunk j ^ (r & 15).
// LM-head loads carry the streaming (non-temporal) cache policy: every byte is used
// once. Workgroup g walks the k stages of a slab starting at stage (g * kstride) mod
// nst (kstride coprime to nst), so concurrent workgroups read different offsets of
// their rows instead of all hitting the same column of power-of-two-strided rows.
// The blocked bf16 layout is stage-major, so workgroups that walk their stages in step
// (no offset) read one contiguous window of blocks at a time.
//
// With W12 the LM-head part of a stage is the slab's 64 rows of 12-byte groups (192
// bytes per row, stored in order) followed by the stage's correction slots; each
// fragment is decoded right before its MFMA, and a corrected weight (coded as a signed
// zero) gets its exact bits from the slot before the fragment enters the MFMA.
template <int MT, int KC, int NS, int FMT>
__global__ __launch_bounds__(256) void k_gemm_skinny(VerifyArgs a, int kstride) {
  constexpr bool W12 = FMT == kLmW12, BLK = FMT == kLmBlocked;
  constexpr int BN = 64;
  constexpr int CH = KC / 8;                 // 16-byte chunks per bf16 stage row
  constexpr int RPI = 64 / CH;               // bf16 stage rows per wave instruction
  static_assert((CH == 16 || CH == 32) && ((!W12 && !BLK) || KC == 128), "stage shape");
  // Stage layout in bytes: LM-head part, correction slots (W12), hidden rows.
  constexpr int WBYTES = W12 ? BN * KC * 3 / 2 : BN * KC * 2;
  constexpr int CBYTES = W12 ? 4 * kW12MaxCap : 0;
  constexpr int HOFF = WBYTES + CBYTES;
  constexpr int STAGE = (HOFF + 16 * MT * KC * 2) / 2;   // bf16 units per stage buffer
  constexpr int WI = WBYTES / (16 * 256);    // LM-head wave instructions per wave
  constexpr int CI = W12 ? 1 : 0;            // correction-slot instruction per wave
  constexpr int HI = MT * KC / 128;          // hidden wave instructions per wave
  constexpr int DPT = WI + CI + HI;
  constexpr int PEND = (NS - 2) * DPT;       // loads allowed in flight past the oldest stage
  static_assert(WBYTES % (16 * 256) == 0, "LM-head part fills whole loads");
  static_assert(PEND < 64, "vmcnt holds 6 bits");
  __shared__ __attribute__((aligned(16))) uint16_t S[NS * STAGE];

  // Workgroups past the contraction's grid normalise drafter rows instead (rejection
  // verify in one call); they share no data with the contraction's workgroups.
  if (a.dpart && (int)blockIdx.x >= a.g_main) {
    draft_partials_walk(a, (int)blockIdx.x - a.g_main, (int)gridDim.x - a.g_main);
    return;
  }
  // With a publication area, workgroups past the grid decide greedy acceptance, one
  // request each, from what the contraction's workgroups publish.
  if (a.pub && (int)blockIdx.x >= a.g_main) {
    int *s_i = reinterpret_cast<int *>(S);
    greedy_decide_published(a, (int)blockIdx.x - a.g_main, a.g_main, s_i, s_i + 72);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.g_main, g = blockIdx.x;
  const int M = rows_total(a.rm);
  const int d = a.d, V = a.V;
  // Publication buffer of this launch, and the words the previous publishing launch left
  // in the other one (this launch returns them to kPubEmpty).
  const uint32_t pub_epoch = a.pub ? a.ws->pub_epoch : 0u;
  const uint32_t pub_prev = a.pub ? a.ws->pub_prev : 0u;
  unsigned long long *const pbuf = a.pub ? pub_buffer(a, pub_epoch) : nullptr;

  // LM-head load i of this thread: bf16 rows r = RPI * (wave + 4 i) + lane / CH, stored
  // chunk lane % CH (swizzled); W12 16-byte piece u = 64 (wave + 4 i) + lane of the
  // slab's 12 KB, row u / 12. Hidden load j: rows RPI * (wave + 4 j) + lane / CH of the
  // hidden part.
  int w_row[WI], w_off[WI];
  const uint16_t *h_src[HI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    if (W12) {
      // LDS piece u (16 bytes) of the slab's 12 KB: row u / 12, piece u % 12 of its 192
      // bytes. Within a row, blocks of three pieces (four 12-byte groups) are permuted
      // by w12_block_swz, so the 16 rows a fragment read touches hit 64 different banks.
      const int u = 64 * (wave + 4 * i) + lane, row = u / 12, pc = u % 12;
      w_row[i] = 0;
      w_off[i] = 16 * (row * 12 + 3 * ((pc / 3) ^ w12_block_swz(row)) + pc % 3);
    } else if (BLK) {
      w_row[i] = 0;                           // the region is contiguous: piece u at 16 u
      w_off[i] = 16 * (64 * (wave + 4 * i) + lane);
    } else {
      const int r = RPI * (wave + 4 * i) + lane / CH;
      w_row[i] = r;
      w_off[i] = 8 * ((lane % CH) ^ (r & 15));
    }
  }
#pragma unroll
  for (int j = 0; j < HI; ++j) {
    const int m = RPI * (wave + 4 * j) + lane / CH;
    const uint16_t *src = a.hidden + 8 * ((lane % CH) ^ (m & 15));   // rows past M: row 0, unused
    if (m < M) {
      int rq, jj;
      const int hr = hidden_row(a.rm, m, &rq, &jj);
      if (hr >= 0) src += (size_t)hr * d;
      else raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
    }
    h_src[j] = src;
  }

  // Drafted token of packed row `lane` (M <= 16 MT <= 64), when the drafted-token
  // logits are produced here: LM-head row x passes through LDS while its slab streams,
  // so the workgroup owning that slab forms the exact fp64 dot of the bf16 hidden and
  // LM-head rows from the staged data. Wave w takes the w-th such row of a slab;
  // rows past the fourth of one slab are marked NaN and left to the merge.
  int zslab = -1, ztok = 0;
  if (a.zx && a.draft_tokens && lane < M) {
    int rq, jj;
    if (hidden_row(a.rm, lane, &rq, &jj) >= 0 && jj < clamp_len(a.verify_len, rq, a.rm.gamma, nullptr)) {
      const int x = a.draft_tokens[(size_t)rq * a.rm.gamma + jj];
      if (x >= 0 && x < V) { zslab = x / BN; ztok = x; }
    }
  }
  unsigned long long zmask = 0ull;
  int zrow = -1, zw = 0;
  double zacc = 0.0;

  const int nslab = (V + BN - 1) / BN;
  const int nst = d / KC;
  const int total = ((nslab - g + G - 1) / G) * nst;   // (slab, stage) pairs of this workgroup
  const int kshift = BLK ? 0 : (int)(((long long)g * kstride) % nst);
  const int cap = W12 ? a.w12_cap : 0;
  auto issue = [&](int t) {
    const int slab = g + (t / nst) * G, st = (t + kshift) % nst, k0 = st * KC;
    LDSP char *dst = (LDSP char *)S + (size_t)(t % NS) * STAGE * 2;
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const GLBP char *src =
          W12   ? (const GLBP char *)(a.w12_codes + ((size_t)slab * nst + st) * WBYTES + w_off[i])
          : BLK ? (const GLBP char *)a.W + ((size_t)st * nslab + slab) * WBYTES + w_off[i]
                : (const GLBP char *)(a.W + (size_t)min(slab * BN + w_row[i], V - 1) * d + w_off[i] + k0);
      __builtin_amdgcn_global_load_lds((const GLBP void *)src, (LDSP void *)(dst + (wave + 4 * i) * 1024),
                                       16, 0, kCachePolicyStream);
    }
    if (W12 && lane < 4) {
      // Slots 16 (4 wave + lane) .. + 3 of this (slab, stage); past CAP, a repeat of the
      // region's last 16 bytes (never read).
      const int ch = min(4 * wave + lane, cap / 4 - 1);
      const GLBP char *src = (const GLBP char *)(a.w12_corr + ((size_t)slab * nst + st) * cap) + 16 * ch;
      __builtin_amdgcn_global_load_lds((const GLBP void *)src, (LDSP void *)(dst + WBYTES + 64 * wave), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < HI; ++j)
      __builtin_amdgcn_global_load_lds((const GLBP void *)(h_src[j] + k0),
                                       (LDSP void *)(dst + HOFF + (wave + 4 * j) * 1024), 16, 0, 0);
  };

  f32x4 acc[MT], cacc[MT];                   // cacc: W12 corrected weights' products
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = cacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  RowAcc run[MT];                            // running statistics of row 16 i + fr
#pragma unroll
  for (int i = 0; i < MT; ++i) run[i] = row_acc_init();
  const int fr = lane & 15, fc = lane >> 4;
  const int br = 16 * wave + fr;

#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < total) issue(p);
  for (int t = 0; t < total; ++t) {
    // Stage t is complete once at most PEND newer loads of this thread are pending;
    // in the last NS-2 pairs fewer loads follow it, so wait for all of them.
    if (t + NS - 2 < total) {
      __builtin_amdgcn_s_waitcnt((PEND & 15) | (((PEND >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    lds_barrier();
    if (t + NS - 1 < total) issue(t + NS - 1);   // refills the buffer read in pair t - 1
    const LDSP uint16_t *Sb = (const LDSP uint16_t *)S + (t % NS) * STAGE;
    const LDSP uint16_t *Hb = Sb + HOFF / 2;                     // hidden rows
    const LDSP uint32_t *Wq = (const LDSP uint32_t *)Sb;          // W12 groups
    const LDSP uint32_t *Cb = (const LDSP uint32_t *)(Sb + WBYTES / 2);   // correction slots
    // W12 correction slots of this stage: lane l holds slot l.
    const uint32_t cent = W12 && lane < cap ? Cb[lane] : 0u;
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      const int c = 4 * s + fc;
      bf16x8 b;
      if (W12) {
        const int o = (br * KC * 3 / 2 + 12 * (c ^ (4 * w12_block_swz(br)))) / 4;
        b = __builtin_bit_cast(bf16x8, w12_decode8(Wq[o], Wq[o + 1], Wq[o + 2], a.w12_lut0, a.w12_lut1));
      } else {
        b = __builtin_bit_cast(bf16x8, *(const LDSP u32x4 *)(Sb + br * KC + 8 * (c ^ (br & 15))));
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int hr = 16 * i + fr;
        const bf16x8 av = __builtin_bit_cast(bf16x8, *(const LDSP u32x4 *)(Hb + hr * KC + 8 * (c ^ (hr & 15))));
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, av, acc[i], 0, 0, 0);
      }
    }
    if (W12) {
      // A corrected weight is coded as a signed zero, so the MFMAs left out its products;
      // they go into separate accumulators after the stage's MFMAs are issued, off the
      // MFMA operands' path. Each of this wave's slots (row_local / 16 == wave) adds
      // h[m][k] * w to z[m][v] in the lanes holding vocabulary row v, one hidden row each.
      for (unsigned long long mm = __ballot(cent != 0u && (int)((cent >> 11) & 3u) == wave); mm;
           mm &= mm - 1) {
        const uint32_t ent = (uint32_t)__builtin_amdgcn_readlane((int)cent, __ffsll((long long)mm) - 1);
        const int kl = ent & 127u, q = ent >> 7 & 3u;
        if ((int)((ent >> 9) & 3u) == fc) {
          const float w = __uint_as_float(ent & 0xffff0000u);
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const int hr = 16 * i + fr;
            const float h = bf16_to_f32(Hb[hr * KC + 8 * ((kl >> 3) ^ (hr & 15)) + (kl & 7)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) cacc[i][e] += e == q ? h * w : 0.f;
          }
        }
      }
    }
    if (t % nst == 0) {
      // First stage of a slab: which rows drafted a token of it.
      const int slab = g + (t / nst) * G;
      zmask = __ballot(zslab == slab);
      unsigned long long mm = zmask;
      for (int i = 0; i < wave && mm; ++i) mm &= mm - 1;
      zrow = mm ? __ffsll((long long)mm) - 1 : -1;
      zw = __shfl(ztok, zrow >= 0 ? zrow : 0) - slab * BN;
      zacc = 0.0;
    }
    if (zrow >= 0) {
      // Lane l < CH takes logical chunk l (8 values) of the staged hidden and LM-head
      // rows; with W12, lane 0 also adds the row's corrected weights of this stage.
      if (lane < CH) {
        const u32x4 hv = *(const LDSP u32x4 *)(Hb + zrow * KC + 8 * (lane ^ (zrow & 15)));
        u32x4 wv;
        if (W12) {
          const int o = (zw * KC * 3 / 2 + 12 * (lane ^ (4 * w12_block_swz(zw)))) / 4;
          wv = w12_decode8(Wq[o], Wq[o + 1], Wq[o + 2], a.w12_lut0, a.w12_lut1);
        } else {
          wv = *(const LDSP u32x4 *)(Sb + zw * KC + 8 * (lane ^ (zw & 15)));
        }
        zacc += dot8_f64(hv, wv);
      }
      if (W12) {
        // The row's corrected weights of this stage, one lane each.
        if (cent != 0u && (int)((cent >> 7) & 63u) == zw) {
          const int kl = cent & 127u;
          zacc += (double)bf16_to_f32(Hb[zrow * KC + 8 * ((kl >> 3) ^ (zrow & 15)) + (kl & 7)]) *
                  (double)__uint_as_float(cent & 0xffff0000u);
        }
      }
    }
    if (t % nst == nst - 1) {
      // Slab done. With the LM-head fragment as the MFMA's first operand, lane (fr, fc)
      // holds row 16 i + fr at the four consecutive vocabulary ids vb .. vb + 3; reduce
      // in registers, then over the four lanes that share fr.
      const int vb = (g + (t / nst) * G) * BN + 16 * wave + 4 * fc;
      if (W12) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          acc[i] += cacc[i];
          cacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = 16 * i + fr;
        if (a.logits && m < M) {
          float *dst = a.logits + (size_t)m * V;
          if ((V & 3) == 0 && vb + 4 <= V) {
            *reinterpret_cast<f32x4 *>(dst + vb) = acc[i];
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (vb + q < V) dst[vb + q] = acc[i][q];
          }
        }
        float t1 = -INFINITY, t2 = -INFINITY;
        int a1 = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float z = acc[i][q];
          if (vb + q < V) {
            if (beats(z, vb + q, t1, a1)) { t2 = t1; t1 = z; a1 = vb + q; }
            else if (z > t2) t2 = z;
          }
        }
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
          const float o1 = lane_xor(t1, off), o2 = lane_xor(t2, off);
          const int oa = lane_xor(a1, off);
          if (beats(o1, oa, t1, a1)) { t2 = fmaxf(t1, o2); t1 = o1; a1 = oa; }
          else { t2 = fmaxf(t2, o1); }
        }
        float s = 0.f;
        if (a.scale_log2 > 0.f) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (vb + q < V) s += exp2f((acc[i][q] - t1) * a.scale_log2);
          s += lane_xor(s, 16);
          s += lane_xor(s, 32);
        }
        row_acc_merge(run[i], RowAcc{t1, t2, s, a1}, a.scale_log2);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (zrow >= 0) {
        // Only lanes < CH hold parts of the dot, except W12's correction lanes.
        if constexpr (W12) {
          zacc += lane_xor(zacc, 32);
          zacc += lane_xor(zacc, 16);
        }
#pragma unroll
        for (int off = CH / 2; off >= 1; off >>= 1) zacc += __shfl_xor(zacc, off);
        if (lane == 0) {
          if (pbuf) pub_store(pbuf + 2 * (size_t)M * G + zrow, (unsigned long long)__double_as_longlong(zacc));
          else a.zx[zrow] = zacc;
        }
      }
      if (tid == 0 && zmask) {
        unsigned long long mm = zmask;
        for (int i = 0; i < 4 && mm; ++i) mm &= mm - 1;
        for (; mm; mm &= mm - 1) {
          const int zr = __ffsll((long long)mm) - 1;
          if (pbuf) pub_store(pbuf + 2 * (size_t)M * G + zr, 0x7ff8000000000000ull);
          else a.zx[zr] = __longlong_as_double(0x7ff8000000000000ll);
        }
      }
      zrow = -1;
    }
  }

  // Merge the four waves' running statistics in a fixed order; one partial per
  // (row, workgroup). Every load into LDS has landed (the last pairs waited for all).
  __syncthreads();
  RowAcc *X = reinterpret_cast<RowAcc *>(S);   // [4][16 MT]
  if (fc == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) X[wave * 16 * MT + 16 * i + fr] = run[i];
  }
  __syncthreads();
  if (tid < 16 * MT && tid < M) {
    RowAcc r0 = X[tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) row_acc_merge(r0, X[w * 16 * MT + tid], a.scale_log2);
    TilePartial p;
    p.top1 = r0.t1; p.top2 = r0.t2; p.arg = r0.arg; p.sum = r0.sum;
    if (pbuf) {
      unsigned long long *w = pbuf + 2 * ((size_t)tid * G + g);
      pub_store(w, pub_word0(p));
      pub_store(w + 1, pub_word1(p));
    } else {
      a.partials[(size_t)tid * a.part_stride + g] = p;
    }
  }
  if (pbuf) {
    unsigned long long *other = pub_buffer(a, pub_epoch + 1u);
    for (uint32_t w = (uint32_t)g * 256u + tid; w < pub_prev; w += (uint32_t)G * 256u)
      pub_store(other + w, kPubEmpty);
  }
}

// ----------------------------------------------------------------- tiled regime
// BM x BN output tiles; four waves in a 2 x 2 grid, each owning a (BM/2) x (BN/2)
// block of 16x16x32 MFMA tiles with its accumulators in registers. K advances in
// steps of 64 through double-buffered LDS: the global loads of step kt+1 are issued
// before step kt is computed and written to LDS after it. LDS rows are 128 bytes and
// a row's 16-byte chunk index is XORed with (row >> 1) & 7, so fragment reads of 16
// consecutive rows hit 16 different bank groups. Blocks are renumbered so the M-tiles
// of one vocabulary tile run back to back on the same XCD and share its L2.
template <int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_tile(VerifyArgs a, int n_mt, int n_nt) {
  constexpr int BK = 64, CH = BK / 8;
  constexpr int TM = BM / 32, TN = BN / 32;
  constexpr int A_LD = BM * CH / 256, B_LD = BN * CH / 256;
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
  static_assert(BM * 32 <= 2 * STAGE * 2, "epilogue exchange fits in the stage buffers");
  __shared__ __attribute__((aligned(16))) uint16_t S[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Hardware hands consecutive block ids to the 8 XCDs in turn; give each XCD a
  // contiguous range of logical tiles (M fastest).
  const int nb = n_mt * n_nt, hb = blockIdx.x;
  const int per = nb / 8, rem = nb % 8, xcd = hb % 8, pos = hb / 8;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + pos;
  const int mt = logical % n_mt, nt = logical / n_mt;
  const int m0 = mt * BM, v0 = nt * BN;
  const int M = rows_total(a.rm);
  const int d = a.d, V = a.V;
  if (m0 >= M) return;

  // Per-thread load sources (row start + chunk) and swizzled LDS offsets.
  const uint16_t *a_src[A_LD], *b_src[B_LD];
  int a_off[A_LD], b_off[B_LD], a_c[A_LD], b_c[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int e = tid + 256 * i, r = e / CH, c = e % CH;
    const int m = m0 + r;
    int hr = -1;
    if (m < M) {
      int rq, j;
      hr = hidden_row(a.rm, m, &rq, &j);
      if (hr < 0) raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
    }
    a_src[i] = a.hidden + (size_t)(hr >= 0 ? hr : 0) * d;   // rows past M: any valid row
    a_c[i] = 8 * c;
    a_off[i] = r * BK + 8 * (c ^ ((r >> 1) & 7));
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int e = tid + 256 * i, r = e / CH, c = e % CH;
    b_src[i] = a.W + (size_t)min(v0 + r, V - 1) * d;
    b_c[i] = 8 * c;
    b_off[i] = BM * BK + r * BK + 8 * (c ^ ((r >> 1) & 7));
  }

  u32x4 ra[A_LD], rb[B_LD];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int k = k0 + a_c[i];
      const u32x4 v = *reinterpret_cast<const u32x4 *>(a_src[i] + min(k, d - 8));
      ra[i] = k < d ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int k = k0 + b_c[i];
      const u32x4 v = *reinterpret_cast<const u32x4 *>(b_src[i] + min(k, d - 8));
      rb[i] = k < d ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
    uint16_t *Sb = S + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *reinterpret_cast<u32x4 *>(Sb + a_off[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *reinterpret_cast<u32x4 *>(Sb + b_off[i]) = rb[i];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (d + BK - 1) / BK;
  const int fr = lane & 15, fc = lane >> 4;
  // All fragments of one K step (two 32-wide substeps) are read before any MFMA of
  // the step, so LDS latency overlaps the first substep's MFMAs.
  bf16x8 af[2][TM], bfr[2][TN];
  auto read_frags = [&](int buf) {
    const uint16_t *Ab = S + buf * STAGE;
    const uint16_t *Bb = Ab + BM * BK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 4 * ks + fc;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + i * 16 + fr;
        af[ks][i] = load8(Ab + r * BK + 8 * (c ^ ((r >> 1) & 7)));
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * (BN / 2) + t * 16 + fr;
        bfr[ks][t] = load8(Bb + r * BK + 8 * (c ^ ((r >> 1) & 7)));
      }
    }
  };
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    read_frags(buf);
    gload(min(kt + 1, nk - 1));      // past the end: a harmless reload, stored to an unused buffer
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bfr[ks][t], acc[i][t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue from registers. Lane l holds rows wm*BM/2 + i*16 + 4*(l>>4) + q and
  // columns wn*BN/2 + t*16 + (l & 15).
  const int colb = v0 + wn * (BN / 2) + fr;
  if (a.logits) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * (BM / 2) + i * 16 + 4 * fc + q;
        if (m < M) {
          float *dst = a.logits + (size_t)m * V;
#pragma unroll
          for (int t = 0; t < TN; ++t)
            if (colb + t * 16 < V) dst[colb + t * 16] = acc[i][t][q];
        }
      }
  }
  // Row statistics over this wave's BN/2 columns, then across the two waves of a row.
  float *X = reinterpret_cast<float *>(S);   // [2][BM][4]: t1, t2, arg (bits), sum
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float t1 = -INFINITY, t2 = -INFINITY;
      int a1 = 0x7fffffff;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int v = colb + t * 16;
        const float z = acc[i][t][q];
        if (v < V) {
          if (beats(z, v, t1, a1)) { t2 = t1; t1 = z; a1 = v; }
          else if (z > t2) t2 = z;
        }
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        const float o1 = __shfl_xor(t1, off), o2 = __shfl_xor(t2, off);
        const int oa = __shfl_xor(a1, off);
        if (beats(o1, oa, t1, a1)) { t2 = fmaxf(t1, o2); t1 = o1; a1 = oa; }
        else { t2 = fmaxf(t2, o1); }
      }
      float s = 0.f;
      if (a.scale_log2 > 0.f) {
#pragma unroll
        for (int t = 0; t < TN; ++t)
          if (colb + t * 16 < V) s += exp2f((acc[i][t][q] - t1) * a.scale_log2);
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      }
      if (fr == 0) {
        const int rl = wm * (BM / 2) + i * 16 + 4 * fc + q;
        float *x = X + (wn * BM + rl) * 4;
        x[0] = t1; x[1] = t2; x[2] = __int_as_float(a1); x[3] = s;
      }
    }
  __syncthreads();
  for (int rl = tid; rl < BM; rl += 256) {
    const int m = m0 + rl;
    if (m >= M) continue;
    const float *x0 = X + rl * 4, *x1 = X + (BM + rl) * 4;
    RowAcc r0{x0[0], x0[1], x0[3], __float_as_int(x0[2])};
    const RowAcc r1{x1[0], x1[1], x1[3], __float_as_int(x1[2])};
    row_acc_merge(r0, r1, a.scale_log2);
    TilePartial p;
    p.top1 = r0.t1; p.top2 = r0.t2; p.arg = r0.arg; p.sum = r0.sum;
    a.partials[(size_t)m * a.part_stride + nt] = p;
  }
}

// ------------------------------------------------------ direct-to-LDS regime
// The tiled GEMM for d % BK == 0 and many rows. global_load_lds_dwordx4 moves each
// wave load's 1 KB straight into one of NS LDS stage buffers (no registers held), so
// NS-1 K steps are in flight per block. Each K step: wait for this thread's loads of
// the step (explicit vmcnt), one workgroup barrier, refill the buffer consumed in the
// previous step, then read fragments and run the MFMAs. NW = 8 waves (2 x 4) give
// two waves per SIMD, which hides LDS read latency behind the other wave's MFMAs.
// Rows of a stage are BK/8 16-byte chunks; chunk j of row r holds logical chunk
// j ^ swz(r), so the MFMA fragment reads of 16 rows spread over the bank groups.
// The LM-head fragment is the MFMA's first operand, so each lane ends with four
// consecutive vocabulary ids of one row: 16-byte logits stores, and per-row
// statistics that need two lane exchanges instead of four.
// Main loop of k_gemm_dma for a wave whose first NV of its TM row tiles hold verified rows
// (the rest are padding of the last row tile): the DMA issue and the barriers are the
// same for every NV, so the workgroup's waves stay in step; only the fragment reads and
// MFMAs of padding row tiles are left out.
// A wave raises its priority while it issues a k-step's MFMAs, so that of the two
// waves sharing a SIMD the one with matrix work ready issues first while the other
// reads its fragments.
template <int NV, int BM, int BN, int BK, int NS, int NW, int DPT>
__device__ __forceinline__ void dma_main_loop(uint16_t *S, const uint16_t *const (&src)[DPT], int nk,
                                              int wave, int lane, int wm, int wn,
                                              f32x4 (&acc)[BM / 32][BN / (NW / 2) / 16]) {
  constexpr int WNG = NW / 2, CH = BK / 8, STAGE = (BM + BN) * BK, TN = BN / WNG / 16;
  auto swz = [](int r) { return (r >> (CH == 4 ? 2 : 1)) & (CH - 1); };
  auto issue = [&](int kt) {
    const int kk = min(kt, nk - 1) * BK;            // past the end: reload the last step (unused)
    LDSP uint16_t *dst = (LDSP uint16_t *)S + (kt % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < DPT; ++i)
      __builtin_amdgcn_global_load_lds((const GLBP void *)(src[i] + kk),
                                       (LDSP void *)(dst + (wave + NW * i) * 512), 16, 0, 0);
  };
  const int fr = lane & 15, fc = lane >> 4;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p);
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt is complete once at most (NS-2)*DPT newer DMAs of this thread are pending.
    constexpr int PEND = (NS - 2) * DPT;
    __builtin_amdgcn_s_waitcnt((PEND & 15) | (((PEND >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
    lds_barrier();
    issue(kt + NS - 1);          // refills the buffer read in the previous iteration
    const LDSP uint16_t *Ab = (const LDSP uint16_t *)S + (kt % NS) * STAGE;
    const LDSP uint16_t *Bb = Ab + BM * BK;
    if constexpr (NV > 0) {
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int c = 4 * ks + fc;
        bf16x8 af[NV], bfr[TN];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int r = wm * (BM / 2) + i * 16 + fr;
          af[i] = __builtin_bit_cast(bf16x8, *(const LDSP u32x4 *)(Ab + r * BK + 8 * (c ^ swz(r))));
        }
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const int r = wn * (BN / WNG) + t * 16 + fr;
          bfr[t] = __builtin_bit_cast(bf16x8, *(const LDSP u32x4 *)(Bb + r * BK + 8 * (c ^ swz(r))));
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int t = 0; t < TN; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[t], af[i], acc[i][t], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
      }
    }
  }
}

template <int BM, int BN, int BK, int NS, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemm_dma(VerifyArgs a, int n_mt, int n_nt) {
  constexpr int NT = 64 * NW;                      // threads
  constexpr int WNG = NW / 2;                      // waves along N (2 along M)
  constexpr int CH = BK / 8;                       // 16-byte chunks per row per stage
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * BK;                 // bf16 per stage
  constexpr int DPT = ROWS * CH / NT;              // DMA instructions per thread per stage
  constexpr int RPI = 64 / CH;                     // rows per wave instruction
  constexpr int TM = BM / 32, TN = BN / WNG / 16;
  // 16 consecutive rows read at one chunk index land in 16 different bank groups.
  auto swz = [](int r) { return (r >> (CH == 4 ? 2 : 1)) & (CH - 1); };
  static_assert(ROWS * CH % NT == 0, "stage splits over the threads");
  __shared__ __attribute__((aligned(16))) uint16_t S[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WNG, wn = wave % WNG;
  const int nb = n_mt * n_nt, hb = blockIdx.x;
  const int per = nb / 8, rem = nb % 8, xcd = hb % 8, pos = hb / 8;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + pos;
  const int mt = logical % n_mt, nt = logical / n_mt;
  const int M = rows_total(a.rm);
  const int d = a.d, V = a.V;
  // The verified rows' 16-row tiles are dealt out as evenly as the row tiles allow (they
  // differ by at most one 16-row tile), so the row tiles that share an LM-head tile run at
  // one pace and keep reading it from L2 together. Row tile mt holds rows m0 .. m0 + mr - 1.
  const int rtiles = (M + 15) / 16, used = (rtiles + 2 * TM - 1) / (2 * TM);
  if (mt >= used) return;
  const int rt_base = rtiles / used, rt_extra = rtiles % used;
  const int m0 = 16 * (mt * rt_base + min(mt, rt_extra)), v0 = nt * BN;
  const int mr = min(16 * (rt_base + (mt < rt_extra ? 1 : 0)), M - m0);

  // DMA i of this thread: wave instruction w + 4 i covers rows RPI*(w + 4 i) .. + RPI - 1;
  // lane l fills LDS slot l: row r = base + l / CH, stored chunk j = l % CH, which holds
  // logical chunk j ^ swz(r).
  const uint16_t *src[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) {
    const int r = RPI * (wave + NW * i) + lane / CH, j = lane % CH;
    const int c = j ^ swz(r);
    const uint16_t *row;
    if (r < BM) {
      const int m = m0 + r;
      int hr = -1;
      if (r < mr) { int rq, jj; hr = hidden_row(a.rm, m, &rq, &jj); }
      row = a.hidden + (size_t)(hr >= 0 ? hr : 0) * d;
    } else {
      row = a.W + (size_t)min(v0 + r - BM, V - 1) * d;
    }
    src[i] = row + 8 * c;
  }
  const int nk = d / BK;                            // d % BK == 0 required
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row tiles of this wave that hold verified rows (wave-uniform).
  const int nv = __builtin_amdgcn_readfirstlane(max(0, min(TM, (mr - wm * (BM / 2) + 15) / 16)));
  static_assert(TM == 8, "one main-loop instance per count of verified row tiles");
  switch (nv) {
    case 8: dma_main_loop<8, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    case 7: dma_main_loop<7, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    case 6: dma_main_loop<6, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    case 5: dma_main_loop<5, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    case 4: dma_main_loop<4, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    case 3: dma_main_loop<3, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    case 2: dma_main_loop<2, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    case 1: dma_main_loop<1, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
    default: dma_main_loop<0, BM, BN, BK, NS, NW>(S, src, nk, wave, lane, wm, wn, acc); break;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): the trailing reloads land before LDS is reused
  __syncthreads();
  // Epilogue from registers. With the LM-head fragment as the MFMA's first operand,
  // lane (fr, fc) holds, for row tile i and vocabulary tile t, row
  // wm * BM/2 + 16 i + fr at the four consecutive ids 16 t + 4 fc .. + 3.
  const int fr = lane & 15, fc = lane >> 4;
  const int vb = v0 + wn * (BN / WNG) + 4 * fc;
  if (a.logits) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rl = wm * (BM / 2) + i * 16 + fr, m = m0 + rl;
      if (rl < mr) {
        float *dst = a.logits + (size_t)m * V;
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const int v = vb + t * 16;
          if ((V & 3) == 0 && v + 4 <= V) {
            *reinterpret_cast<f32x4 *>(dst + v) = acc[i][t];
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (v + q < V) dst[v + q] = acc[i][t][q];
          }
        }
      }
    }
  }
  float *X = reinterpret_cast<float *>(S);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float t1 = -INFINITY, t2 = -INFINITY;
    int a1 = 0x7fffffff;
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = vb + t * 16 + q;
        const float z = acc[i][t][q];
        if (v < V) {
          if (beats(z, v, t1, a1)) { t2 = t1; t1 = z; a1 = v; }
          else if (z > t2) t2 = z;
        }
      }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float o1 = lane_xor(t1, off), o2 = lane_xor(t2, off);
      const int oa = lane_xor(a1, off);
      if (beats(o1, oa, t1, a1)) { t2 = fmaxf(t1, o2); t1 = o1; a1 = oa; }
      else { t2 = fmaxf(t2, o1); }
    }
    float s = 0.f;
    if (a.scale_log2 > 0.f) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (vb + t * 16 + q < V) s += exp2f((acc[i][t][q] - t1) * a.scale_log2);
      s += lane_xor(s, 16);
      s += lane_xor(s, 32);
    }
    if (fc == 0) {
      const int rl = wm * (BM / 2) + i * 16 + fr;
      float *x = X + (wn * BM + rl) * 4;   // [WNG][BM][4]
      x[0] = t1; x[1] = t2; x[2] = __int_as_float(a1); x[3] = s;
    }
  }
  __syncthreads();
  for (int rl = tid; rl < mr; rl += NT) {
    const int m = m0 + rl;
    const float *x0 = X + rl * 4;
    RowAcc r0{x0[0], x0[1], x0[3], __float_as_int(x0[2])};
    for (int w = 1; w < WNG; ++w) {
      const float *x1 = X + (w * BM + rl) * 4;
      const RowAcc r1{x1[0], x1[1], x1[3], __float_as_int(x1[2])};
      row_acc_merge(r0, r1, a.scale_log2);
    }
    TilePartial p;
    p.top1 = r0.t1; p.top2 = r0.t2; p.arg = r0.arg; p.sum = r0.sum;
    a.partials[(size_t)m * a.part_stride + nt] = p;
  }
}

// One workgroup per verified row: merge the row's partials (loaded in one round of
// independent loads, kMergePer per thread) and write the drafted token's exact logit,
// an fp64 dot of the bf16 hidden and LM-head rows (bf16 x bf16 products are exact in
// fp64). The skinny contraction leaves that logit in a.zx; otherwise (or where it
// marked NaN) the rows are loaded right after the partials and dotted here.
constexpr int kMergePer = 16;   // partials per thread per round (n <= 4096 in one round)
constexpr int kDotPer = 4;      // 16-byte chunks per thread held for the dot (d <= 8192)

__global__ __launch_bounds__(256) void k_row_merge(VerifyArgs a, int n) {
  __shared__ double red[4];
  __shared__ float s_t1[4], s_t2[4];
  __shared__ int s_arg[4];
  const int m = blockIdx.x;
  const int M = rows_total(a.rm);
  if (m >= M) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = a.d / 8;

  int r, j;
  const int hr = hidden_row(a.rm, m, &r, &j);
  const uint16_t *hrow = a.hidden + (size_t)(hr >= 0 ? hr : 0) * a.d;
  int x = -1;
  if (hr >= 0 && a.draft_tokens &&
      j < clamp_len(a.verify_len, r, a.rm.gamma, tid == 0 ? a.ws : nullptr))
    x = a.draft_tokens[(size_t)r * a.rm.gamma + j];
  const bool has_x = x >= 0 && x < a.V;        // uniform across the workgroup
  // The drafted token's logit from the contraction, when it left one (NaN: not there).
  double zg = 0.0;
  if (has_x && a.zx) zg = a.zx[m];

  const TilePartial *P = a.partials + (size_t)m * a.part_stride;
  float t1 = -INFINITY, t2 = -INFINITY;
  int a1 = 0x7fffffff;
  TilePartial q[kMergePer];
  for (int base = 0; base < n; base += 256 * kMergePer) {
#pragma unroll
    for (int i = 0; i < kMergePer; ++i) {
      const int p = base + tid + 256 * i;
      q[i] = p < n ? P[p] : TilePartial{-INFINITY, -INFINITY, 0x7fffffff, 0.f};
    }
#pragma unroll
    for (int i = 0; i < kMergePer; ++i) {
      if (beats(q[i].top1, q[i].arg, t1, a1)) { t2 = fmaxf(t1, q[i].top2); t1 = q[i].top1; a1 = q[i].arg; }
      else { t2 = fmaxf(t2, q[i].top1); }
    }
  }
  // Without a logit from the contraction, the hidden and LM-head rows for the dot (read
  // here directly when the LM head is bf16 [V][d]).
  const bool need_dot = has_x && (!a.zx || zg != zg);
  const bool rowmajor = !a.w12_codes && !a.w_blocked;
  u32x4 hv[kDotPer];
#pragma unroll
  for (int i = 0; i < kDotPer; ++i) {
    const int c = tid + 256 * i;
    hv[i] = need_dot && rowmajor && c < nc ? *reinterpret_cast<const u32x4 *>(hrow + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }
  const uint16_t *wrow = rowmajor ? a.W + (size_t)(has_x ? x : 0) * a.d : nullptr;
  u32x4 wv[kDotPer];
#pragma unroll
  for (int i = 0; i < kDotPer; ++i) {
    const int c = tid + 256 * i;
    wv[i] = need_dot && rowmajor && c < nc ? *reinterpret_cast<const u32x4 *>(wrow + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }

#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o1 = __shfl_xor(t1, off), o2 = __shfl_xor(t2, off);
    const int oa = __shfl_xor(a1, off);
    if (beats(o1, oa, t1, a1)) { t2 = fmaxf(t1, o2); t1 = o1; a1 = oa; }
    else { t2 = fmaxf(t2, o1); }
  }
  if (lane == 0) { s_t1[wave] = t1; s_t2[wave] = t2; s_arg[wave] = a1; }
  __syncthreads();
  t1 = s_t1[0]; t2 = s_t2[0]; a1 = s_arg[0];
  for (int w = 1; w < 4; ++w) {
    if (beats(s_t1[w], s_arg[w], t1, a1)) { t2 = fmaxf(t1, s_t2[w]); t1 = s_t1[w]; a1 = s_arg[w]; }
    else { t2 = fmaxf(t2, s_t1[w]); }
  }
  double lse = 0.0;
  if (a.temperature > 0.f) {
    double S = 0.0;
    if (n <= 256 * kMergePer) {               // this thread's partials are still in q
#pragma unroll
      for (int i = 0; i < kMergePer; ++i)
        if (q[i].sum != 0.f) S += (double)q[i].sum * partial_weight(q[i].top1, t1, a.scale_log2);
    } else {
      for (int p = tid; p < n; p += 256) {
        const TilePartial o = P[p];
        if (o.sum != 0.f) S += (double)o.sum * partial_weight(o.top1, t1, a.scale_log2);
      }
    }
    S = block_sum(S, red);
    lse = (double)t1 * a.invT + log(S);
  }
  double zd = has_x ? zg : 0.0;
  if (need_dot) {
    double part = 0.0;
    if (!rowmajor) {
      part = lm_head_dot_part(a, hrow, x, tid, 256);
    } else {
#pragma unroll
      for (int i = 0; i < kDotPer; ++i) part += dot8_f64(hv[i], wv[i]);
      for (int c = tid + 256 * kDotPer; c < nc; c += 256)
        part += dot8_f64(*reinterpret_cast<const u32x4 *>(hrow + 8 * c), *reinterpret_cast<const u32x4 *>(wrow + 8 * c));
    }
    zd = block_sum(part, red);
  }
  if (tid == 0) write_stats(a, m, t1, t2, a1, lse, zd);
}

// Greedy verify tail in one kernel: one workgroup of kFusedWaves waves per request.
constexpr int kFusedWaves = 16;

__global__ __launch_bounds__(64 * kFusedWaves) void k_merge_accept_greedy(
    VerifyArgs a, int n, int32_t *__restrict__ accept_len, int32_t *__restrict__ next_token,
    int64_t *__restrict__ counters) {
  __shared__ int s_arg[65], s_x[64];
  merge_accept_greedy_request(a, blockIdx.x, n, accept_len, next_token, counters, kFusedWaves,
                              s_arg, s_x);
}

// Rejection verify's row merge and decision in one kernel (DSpark summary, "Problem
// definition": a draft survives iff u < min(1, p(x) / q(x)), and the first failure ends
// the accepted prefix). One workgroup of sixteen waves per request, 32 lanes per verified
// row, so requests of up to 32 rows (gamma <= kDecideMaxGamma), each lane holding sixteen
// partials in registers. A row's target partials are merged into its
// statistics -- argmax, top-2 and log sum exp(z / T) -- and written with the drafted
// token's exact logit; a kept draft row also merges its drafter chunk partials into
// log sum exp(l / T) and takes the acceptance test. A ballot over the rows gives a_r, and
// the request's draw record names the row the draw samples. The loads that do not need
// the request's offset go out first, the partials and drafted-token logits with it.
// Larger gamma takes the separate row merge and decision kernels.
constexpr int kDecideLanes = 32;
constexpr int kDecideHold = 16;   // target partials held per lane (n <= 512 in one round)
constexpr int kDecideThreads = 1024;
static_assert(kDecideMaxGamma + 1 == kDecideThreads / kDecideLanes, "one row slot per row");

__global__ __launch_bounds__(kDecideThreads) void k_merge_decide(VerifyArgs a, DecideArgs o, int n) {
  __shared__ int s_rej[64];
  __shared__ double s_lse[kDecideMaxGamma + 1], s_lseq[kDecideMaxGamma + 1];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int sub = tid & (kDecideLanes - 1), j = tid / kDecideLanes;   // row slot j
  const int gamma = a.rm.gamma, V = a.V, C = a.dchunks;
  // First round of loads: the request's length and offset, and everything of row j that
  // does not depend on them (its drafted token, uniform and drafter partials; rows past
  // the length are loaded and then ignored).
  const size_t rj = (size_t)r * gamma + min(j, gamma - 1);
  const int xl = a.draft_tokens[rj];
  const float u = o.u_accept[rj];
  const float lx = a.qx[rj];   // drafter logit of the token, left by the drafter normaliser
  if (o.pub)
    for (int k = tid; k < 2 * o.pub_chunks; k += kDecideThreads)
      o.pub[(size_t)r * 2 * o.pub_chunks + k] = kUnpublished;
  DraftPart dq[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) dq[i] = a.dpart[rj * C + min(sub + kDecideLanes * i, C - 1)];
  const int L = clamp_len(a.verify_len, r, gamma, tid == 0 ? a.ws : nullptr);
  const int cap = a.rm.B * (gamma + 1);
  const int base = a.rm.row_offsets ? a.rm.row_offsets[r] : r * (gamma + 1);
  if (base < 0 || base + L >= cap) {
    if (tid == 0) {
      raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
      o.rec[r] = draw_record(-1, 0, 0, -1, 0.0, 0.0, a.invT);
      o.accept_len[r] = 0;
      o.next_token[r] = -1;
    }
    return;
  }
  if (j <= L) {
    const int m = base + j;
    const bool drafted = j < L;
    const int x = drafted ? xl : -1;
    const bool has_x = x >= 0 && x < V;
    // Second round: the row's partials and drafted-token logit (they need the offset).
    const TilePartial *P = a.partials + (size_t)m * a.part_stride;
    TilePartial q[kDecideHold];
#pragma unroll
    for (int i = 0; i < kDecideHold; ++i) q[i] = P[min(sub + kDecideLanes * i, n - 1)];
    const double zg = a.zx[m];
    float t1 = -INFINITY, t2 = -INFINITY;
    int a1 = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kDecideHold; ++i) {
      if (sub + kDecideLanes * i >= n) q[i] = TilePartial{-INFINITY, -INFINITY, 0x7fffffff, 0.f};
      if (beats(q[i].top1, q[i].arg, t1, a1)) { t2 = fmaxf(t1, q[i].top2); t1 = q[i].top1; a1 = q[i].arg; }
      else { t2 = fmaxf(t2, q[i].top1); }
    }
    for (int p = sub + kDecideLanes * kDecideHold; p < n; p += kDecideLanes) {
      const TilePartial e = P[p];
      if (beats(e.top1, e.arg, t1, a1)) { t2 = fmaxf(t1, e.top2); t1 = e.top1; a1 = e.arg; }
      else { t2 = fmaxf(t2, e.top1); }
    }
#pragma unroll
    for (int off = kDecideLanes / 2; off >= 1; off >>= 1) {
      const float o1 = __shfl_xor(t1, off), o2 = __shfl_xor(t2, off);
      const int oa = __shfl_xor(a1, off);
      if (beats(o1, oa, t1, a1)) { t2 = fmaxf(t1, o2); t1 = o1; a1 = oa; }
      else { t2 = fmaxf(t2, o1); }
    }
    double S = 0.0;
#pragma unroll
    for (int i = 0; i < kDecideHold; ++i)
      if (q[i].sum != 0.f) S += (double)q[i].sum * partial_weight(q[i].top1, t1, a.scale_log2);
    for (int p = sub + kDecideLanes * kDecideHold; p < n; p += kDecideLanes) {
      const TilePartial e = P[p];
      if (e.sum != 0.f) S += (double)e.sum * partial_weight(e.top1, t1, a.scale_log2);
    }
    // The drafted token's logit comes from the contraction or the drafter-normaliser
    // launch; NaN marks a row neither formed (a crowded slab), whose dot is taken here.
    const bool need_dot = has_x && zg != zg;
    double part = 0.0;
    if (need_dot)
      part = lm_head_dot_part(a, a.hidden + ((size_t)r * (gamma + 1) + j) * a.d, x, sub, kDecideLanes);
    const DraftPart *Q = a.dpart + rj * C;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (!drafted || sub + kDecideLanes * i >= C) dq[i] = DraftPart{-INFINITY, 0.f, 0.0};
    float qm = fmaxf(dq[0].m, dq[1].m);
    for (int c = sub + 2 * kDecideLanes; drafted && c < C; c += kDecideLanes) qm = fmaxf(qm, Q[c].m);
#pragma unroll
    for (int off = kDecideLanes / 2; off >= 1; off >>= 1) {
      S += __shfl_xor(S, off);
      part += __shfl_xor(part, off);
      qm = fmaxf(qm, __shfl_xor(qm, off));
    }
    double qs = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (dq[i].s != 0.0) qs += dq[i].s * partial_weight(dq[i].m, qm, a.scale_log2);
    for (int c = sub + 2 * kDecideLanes; drafted && c < C; c += kDecideLanes) {
      const DraftPart e = Q[c];
      if (e.s != 0.0) qs += e.s * partial_weight(e.m, qm, a.scale_log2);
    }
#pragma unroll
    for (int off = kDecideLanes / 2; off >= 1; off >>= 1) qs += __shfl_xor(qs, off);
    if (sub == 0) {
      const double lse = (double)t1 * a.invT + log(S);
      s_lse[j] = lse;
      sd_row_stats st;
      st.argmax = a1;
      st.top1 = t1;
      st.top2 = t2;
      st.pos = j;
      st.lse = lse;
      st.z_draft = has_x ? (need_dot ? part : zg) : 0.0;
      a.stats[m] = st;
      if (drafted) {
        const double lse_q = (double)qm * a.invT + log(qs);
        o.lse_q[rj] = lse_q;
        s_lseq[j] = lse_q;
        int rej = 1;
        if (has_x) {
          const double logp = st.z_draft * a.invT - lse;
          const double logq = (double)lx * a.invT - lse_q;
          rej = !((double)u < fmin(1.0, exp(logp - logq)));
        }
        s_rej[j] = rej;
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    const unsigned long long mk = __ballot(tid < L && s_rej[tid]);
    if (tid == 0) {
      const int acc = mk ? (__ffsll((long long)mk) - 1) : L;
      o.rec[r] = draw_record(base, acc, L, r * gamma + acc, s_lse[acc], s_lseq[acc], a.invT);
      o.accept_len[r] = acc;
      if (o.counters) {
        atomicAdd(reinterpret_cast<unsigned long long *>(o.counters), (unsigned long long)L);
        atomicAdd(reinterpret_cast<unsigned long long *>(o.counters + 1), (unsigned long long)acc);
      }
    }
  }
}

// Resident workgroups per CU of each persistent kernel, cached per host thread for the
// device current on it (recomputed when that device changes), so concurrent callers on
// different threads never share the cache.
struct Occupancy {
  int device = -1, cus = 0;
  const void *fn[16] = {};
  int per_cu[16] = {};
};
thread_local Occupancy t_occ;

// Compute units of the current device.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (t_occ.device != dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 1;
    t_occ = Occupancy{};
    t_occ.cus = cus > 0 ? cus : 1;
    t_occ.device = dev;
  }
  return t_occ.cus;
}

int resident_blocks(const void *fn) {
  device_cus();
  int slot = 0;
  while (slot < 16 && t_occ.fn[slot] && t_occ.fn[slot] != fn) ++slot;
  if (slot < 16 && t_occ.fn[slot] == fn) return t_occ.cus * t_occ.per_cu[slot];
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 256, 0) != hipSuccess || n < 1) n = 1;
  if (slot < 16) { t_occ.fn[slot] = fn; t_occ.per_cu[slot] = n; }
  return t_occ.cus * n;
}

// Balanced persistent grid over BN-row slabs: at most one workgroup per resident slot
// and per partial column, and every workgroup gets `rounds` or `rounds - 1` slabs.
int persistent_grid(int nslab, int resident, int part_stride) {
  const int g0 = min(nslab, min(resident, part_stride));
  const int rounds = (nslab + g0 - 1) / g0;
  return (nslab + rounds - 1) / rounds;
}

template <int MT, int BN, int KC>
hipError_t launch_stream(const VerifyArgs &a, hipStream_t stream, int *n_part) {
  const void *fn = reinterpret_cast<const void *>(&k_gemm_stream<MT, BN, KC>);
  const int G = persistent_grid((a.V + BN - 1) / BN, resident_blocks(fn), a.part_stride);
  *n_part = G;
  hipLaunchKernelGGL((k_gemm_stream<MT, BN, KC>), dim3(G), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Smallest of a few small odd strides that is coprime to the stage count, so the
// start offsets of consecutive workgroups cover every stage evenly.
int stage_stride(int nst) {
  for (int s : {5, 7, 11, 13, 3}) {
    int x = nst, y = s;
    while (y) { const int t = x % y; x = y; y = t; }
    if (x == 1) return s;
  }
  return 1;
}

// Drafter-normaliser workgroups appended to a streaming contraction of G workgroups out of
// `resident` slots: the idle slots, up to one workgroup per four (row, chunk) items, and
// none unless every wave then takes at most kDraftItemsPerWave items (otherwise the
// walk would run long past the contraction and a separate launch does the work).
constexpr int kDraftItemsPerWave = 16;

int appended_draft_grid(const VerifyArgs &a, int G, int resident) {
  const long long items = (long long)a.rm.B * a.rm.gamma * a.dchunks;
  const int spare = resident - G;
  if (spare < 1 || items > 4LL * kDraftItemsPerWave * spare) return 0;
  return (int)min((long long)spare, (items + 3) / 4);
}

template <int MT, int KC, int NS, int FMT>
hipError_t launch_skinny_as(const VerifyArgs &a, hipStream_t stream, int *n_part,
                            bool *greedy_done, bool *draft_done) {
  const void *fn = reinterpret_cast<const void *>(&k_gemm_skinny<MT, KC, NS, FMT>);
  const int resident = resident_blocks(fn);
  const int G = persistent_grid((a.V + 63) / 64, resident, a.part_stride);
  *n_part = G;
  VerifyArgs k = a;
  k.g_main = G;
  // The greedy decision joins this launch when one deciding workgroup per request can
  // take its request's rows in one pass, the publication area holds the launch, and the
  // deciding workgroups get compute units of their own. Workgroups go out one per CU
  // before any CU takes a second; a decider that shares its CU with a streaming
  // workgroup waits behind that workgroup's loads (measured on a 512-workgroup grid:
  // 2-3 us per poll, a slower step than the separate launch).
  const int cap = a.rm.B * (a.rm.gamma + 1);
  const bool tail = a.pub && a.greedy_accept_len && a.rm.B <= kTailMaxRequests &&
                    a.rm.gamma + 1 <= kTailMaxRows && G + a.rm.B <= device_cus() &&
                    G <= kPubMaxGrid && pub_words_used(cap, G) <= kPubWords;
  if (!tail) {
    k.pub = nullptr;
    k.greedy_accept_len = nullptr;
  }
  if (greedy_done) *greedy_done = tail;
  const int extra = tail ? a.rm.B
                  : a.dpart && a.draft_logits ? appended_draft_grid(a, G, resident) : 0;
  if (tail || !extra) k.dpart = nullptr;
  if (draft_done) *draft_done = !tail && extra > 0;
  hipLaunchKernelGGL((k_gemm_skinny<MT, KC, NS, FMT>), dim3(G + extra), dim3(256), 0, stream, k,
                     stage_stride(a.d / KC));
  return hipGetLastError();
}

template <int MT, int KC, int NS>
hipError_t launch_skinny(const VerifyArgs &a, hipStream_t stream, int *n_part,
                         bool *greedy_done, bool *draft_done) {
  if constexpr (KC == 128) {
    if (a.w12_codes)
      return launch_skinny_as<MT, KC, NS, kLmW12>(a, stream, n_part, greedy_done, draft_done);
    if (a.w_blocked)
      return launch_skinny_as<MT, KC, NS, kLmBlocked>(a, stream, n_part, greedy_done, draft_done);
  }
  return launch_skinny_as<MT, KC, NS, kLmBf16>(a, stream, n_part, greedy_done, draft_done);
}

// Blocked copy of a bf16 LM head: block (st, s), stored stage-major at index
// st * ceil(V/64) + s, is 16 KB holding rows 64 s .. 64 s + 63 and columns
// 128 st .. 128 st + 127, row r's 16-byte chunk j at position j ^ (r & 15) -- the
// arrangement the streaming contraction keeps in LDS, so one stage is one contiguous
// read -- and rows past V zero. One workgroup per block; 16 lanes read one row's 256 bytes.
__global__ __launch_bounds__(256) void k_block_lm_head(const uint16_t *__restrict__ W, int V,
                                                       int d, uint16_t *__restrict__ out) {
  const int nst = d / 128, nslab = (V + 63) / 64;
  const size_t blk = blockIdx.x;
  const int s = (int)(blk / nst), st = (int)(blk % nst);
  uint16_t *dst = out + ((size_t)st * nslab + s) * 8192;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int u = threadIdx.x + 256 * q;      // 16-byte piece of the block
    const int r = u >> 4, j = (u & 15) ^ (r & 15);
    const int v = 64 * s + r;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (v < V) val = *reinterpret_cast<const u32x4 *>(W + (size_t)v * d + 128 * st + 8 * j);
    *reinterpret_cast<u32x4 *>(dst + 8 * u) = val;
  }
}

}  // namespace

hipError_t launch_block_lm_head(const uint16_t *W, int V, int d, uint16_t *out,
                                hipStream_t stream) {
  const size_t blocks = (size_t)((V + 63) / 64) * (d / 128);
  hipLaunchKernelGGL(k_block_lm_head, dim3((unsigned)blocks), dim3(256), 0, stream, W, V, d, out);
  return hipGetLastError();
}

size_t verify_workspace_layout(int B, int gamma, int V, size_t *part_off, int *part_stride,
                               size_t *zx_off) {
  const size_t cap = (size_t)B * (gamma + 1);
  const int stride = (V + kMinVocabTile - 1) / kMinVocabTile;
  const size_t po = sizeof(WsHeader) + kPubBytes;   // header, publication area, partials
  const size_t zo = po + align_up(cap * (size_t)stride * sizeof(TilePartial), 256);
  if (part_off) *part_off = po;
  if (part_stride) *part_stride = stride;
  if (zx_off) *zx_off = zo;
  return zo + align_up(cap * sizeof(double), 256);
}

hipError_t launch_contraction(const VerifyArgs &a, hipStream_t stream, int *n_part,
                              bool *zx_done, bool *greedy_done, bool *draft_done) {
  const int cap = a.rm.B * (a.rm.gamma + 1);
  *zx_done = false;
  if (greedy_done) *greedy_done = false;
  if (draft_done) *draft_done = false;
  if (a.d % 128 == 0 && cap <= 64) *zx_done = a.zx != nullptr && a.draft_tokens != nullptr;
  if (a.d % 128 == 0) {
    if (cap <= 16) return launch_skinny<1, 128, 4>(a, stream, n_part, greedy_done, draft_done);
    if (cap <= 32) return launch_skinny<2, 128, 3>(a, stream, n_part, greedy_done, draft_done);
    if (cap <= 64) return launch_skinny<4, 128, 2>(a, stream, n_part, greedy_done, draft_done);
  }
  if (cap <= 16) return launch_stream<1, 64, 256>(a, stream, n_part);
  if (cap <= 32) return launch_stream<2, 64, 128>(a, stream, n_part);
  if (cap <= 64) return launch_stream<4, 64, 128>(a, stream, n_part);
  constexpr int BM = 256;
  const int n_mt = (cap + BM - 1) / BM;
  if (a.d % 64 == 0) {
    // 320-wide vocabulary tiles: 15% fewer LDS bytes per flop than 256-wide ones and, on
    // the 151936-id vocabulary, 475 tiles per row tile (1.86 rounds of 256 CUs instead of
    // 2.32); measured 14-19% faster at 224-256 rows and even at 1024 rows.
    constexpr int BN = 320;
    *n_part = (a.V + BN - 1) / BN;
    hipLaunchKernelGGL((k_gemm_dma<BM, BN, 64, 2, 8>), dim3(n_mt * *n_part), dim3(512), 0, stream, a, n_mt, *n_part);
  } else if (cap <= 1024) {  // general d (register-staged K loop with a K tail)
    constexpr int BN = 128;
    *n_part = (a.V + BN - 1) / BN;
    hipLaunchKernelGGL((k_gemm_tile<BM, BN>), dim3(n_mt * *n_part), dim3(256), 0, stream, a, n_mt, *n_part);
  } else {
    constexpr int BN = 256;
    *n_part = (a.V + BN - 1) / BN;
    hipLaunchKernelGGL((k_gemm_tile<BM, BN>), dim3(n_mt * *n_part), dim3(256), 0, stream, a, n_mt, *n_part);
  }
  return hipGetLastError();
}

hipError_t launch_verify_greedy(const VerifyArgs &a, int32_t *accept_len, int32_t *next_token,
                                int64_t *counters, hipStream_t stream) {
  // A streaming contraction with few requests of few rows finishes the step in its own
  // launch (workgroups appended to its grid decide, from partials published in the
  // workspace's publication area); otherwise a separate launch does that.
  VerifyArgs f = a;
  if (a.zx && a.draft_tokens) {
    f.pub = reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(a.ws) + sizeof(WsHeader));
    f.greedy_accept_len = accept_len;
    f.greedy_next_token = next_token;
    f.greedy_counters = counters;
  }
  int n_part = 0;
  bool zx_done = false, greedy_done = false;
  hipError_t e = launch_contraction(f, stream, &n_part, &zx_done, &greedy_done);
  if (e != hipSuccess || greedy_done) return e;
  VerifyArgs m = a;
  if (!zx_done) m.zx = nullptr;
  hipLaunchKernelGGL(k_merge_accept_greedy, dim3(a.rm.B), dim3(64 * kFusedWaves), 0, stream, m,
                     n_part, accept_len, next_token, counters);
  return hipGetLastError();
}

hipError_t launch_merge_decide(const VerifyArgs &a, const DecideArgs &o, int n_part,
                               hipStream_t stream) {
  hipLaunchKernelGGL(k_merge_decide, dim3(a.rm.B), dim3(kDecideThreads), 0, stream, a, o, n_part);
  return hipGetLastError();
}

hipError_t launch_row_merge(const VerifyArgs &a, int n_part, bool zx_done, hipStream_t stream) {
  VerifyArgs m = a;
  if (!zx_done) m.zx = nullptr;
  hipLaunchKernelGGL(k_row_merge, dim3(a.rm.B * (a.rm.gamma + 1)), dim3(256), 0, stream, m, n_part);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream) {
  int n_part = 0;
  bool zx_done = false;
  hipError_t e = launch_contraction(a, stream, &n_part, &zx_done);
  if (e != hipSuccess) return e;
  return launch_row_merge(a, n_part, zx_done, stream);
}

int resident_workgroups(const void *fn) { return resident_blocks(fn); }

}  // namespace sdv
