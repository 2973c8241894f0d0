// LM-head verify contraction with fused row statistics (gfx950).
//
// z[m][v] = sum_k h[m][k] * W[v][k] for the M packed verified rows (LFM2.5-DSpark
// blog, "How DSpark works": the target checks the whole drafted block in one pass
// and shares one weight load across it; DSpark summary, "Production deployment":
// the LM head maps the d-vector to V logits, and variable-length requests are
// flattened rather than padded).
//
// Both operands are K-contiguous bf16 (hidden rows [M][d], LM head [V][d]); products
// run on the 16x16x32 bf16 MFMA with fp32 accumulation. Two regimes:
//   * streaming (M <= 64), k_gemm_stream: a persistent grid walks the vocabulary in
//     slabs of BN rows. Each stage moves KC k-values of the slab and of the hidden
//     rows into LDS with contiguous 512-byte row segments per wave load (W is read
//     from HBM exactly once); the LDS layout XORs each row's 16-byte chunk index
//     with (row & 15) so MFMA fragment reads from 16 rows hit 16 bank groups. Per
//     slab the fp32 tile is reduced to row statistics and merged into running
//     values, leaving one partial per (row, workgroup).
//   * tiled (M > 64), k_gemm_tile: BM x BN output tiles staged through LDS, one
//     partial per (row, vocabulary tile).
// k_row_merge then combines each row's partials (one workgroup per row).
// Row statistics: max, second max, lowest argmax and sum of exp((z - max) / T); the
// drafted token's logit is recomputed exactly as an fp64 dot of the bf16 inputs.
#include <math.h>

#include "sd_internal.h"

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

// Exact logit of row m's drafted token: an fp64 dot of the bf16 hidden row and LM-head
// row (bf16 x bf16 products are exact in fp64). 0 on bonus rows. All 256 threads call it.
__device__ double drafted_logit(const VerifyArgs &a, int m, double *red) {
  int r, j;
  const int hr = hidden_row(a.rm, m, &r, &j);
  int x = -1;
  if (hr >= 0 && a.draft_tokens &&
      j < clamp_len(a.verify_len, r, a.rm.gamma, threadIdx.x == 0 ? a.ws : nullptr))
    x = a.draft_tokens[(size_t)r * a.rm.gamma + j];
  if (x < 0 || x >= a.V) return 0.0;           // uniform across the workgroup
  const uint16_t *h = a.hidden + (size_t)hr * a.d;
  const uint16_t *w = a.W + (size_t)x * a.d;
  double part = 0.0;
  for (int c = threadIdx.x; c < a.d / 8; c += 256) {
    const u32x4 hv = *reinterpret_cast<const u32x4 *>(h + 8 * c);
    const u32x4 wv = *reinterpret_cast<const u32x4 *>(w + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      part += (double)__uint_as_float(hv[q] << 16) * (double)__uint_as_float(wv[q] << 16);
      part += (double)__uint_as_float(hv[q] & 0xffff0000u) *
              (double)__uint_as_float(wv[q] & 0xffff0000u);
    }
  }
  return block_sum(part, red);
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

  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
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

// ----------------------------------------------------------------- tiled regime
template <int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_tile(VerifyArgs a) {
  constexpr int BK = 64, LDK = BK + 8;
  constexpr int WM = 2, WN = 2;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int A_CH = BM * (BK / 8) / 256, B_CH = BN * (BK / 8) / 256;
  constexpr int LDC = BN + 4;
  constexpr int STAGE_BYTES = 2 * (BM + BN) * LDK * 2;
  constexpr int C_BYTES = BM * LDC * 4;
  constexpr int SMEM = STAGE_BYTES > C_BYTES ? STAGE_BYTES : C_BYTES;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  uint16_t *As = reinterpret_cast<uint16_t *>(smem);          // [2][BM][LDK]
  uint16_t *Bs = As + 2 * BM * LDK;                            // [2][BN][LDK]
  float *Cs = reinterpret_cast<float *>(smem);                 // [BM][LDC] after the K loop

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int v0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int M = rows_total(a.rm);
  const int d = a.d, V = a.V;
  if (m0 >= M) return;

  const uint16_t *asrc[A_CH];
  int a_lds[A_CH], a_k[A_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int ch = tid + 256 * c, rr = ch >> 3, kc = (ch & 7) * 8;
    a_lds[c] = rr * LDK + kc;
    a_k[c] = kc;
    asrc[c] = nullptr;
    const int m = m0 + rr;
    if (m < M) {
      int r, j;
      const int hr = hidden_row(a.rm, m, &r, &j);
      if (hr >= 0) asrc[c] = a.hidden + (size_t)hr * d;
      else raise_flag(a.ws, SD_FLAG_ROW_OFFSETS);
    }
  }
  const uint16_t *bsrc[B_CH];
  int b_lds[B_CH], b_k[B_CH];
#pragma unroll
  for (int c = 0; c < B_CH; ++c) {
    const int ch = tid + 256 * c, rr = ch >> 3, kc = (ch & 7) * 8;
    b_lds[c] = rr * LDK + kc;
    b_k[c] = kc;
    bsrc[c] = a.W + (size_t)min(v0 + rr, V - 1) * d;
  }

  u32x4 ra[A_CH], rb[B_CH];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int k = k0 + a_k[c];
      ra[c] = (asrc[c] && k < d) ? *reinterpret_cast<const u32x4 *>(asrc[c] + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int k = k0 + b_k[c];
      rb[c] = (k < d) ? *reinterpret_cast<const u32x4 *>(bsrc[c] + k) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c)
      *reinterpret_cast<u32x4 *>(As + buf * BM * LDK + a_lds[c]) = ra[c];
#pragma unroll
    for (int c = 0; c < B_CH; ++c)
      *reinterpret_cast<u32x4 *>(Bs + buf * BN * LDK + b_lds[c]) = rb[c];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (d + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t *Ab = As + buf * BM * LDK;
    const uint16_t *Bb = Bs + buf * BN * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = load8(Ab + (wm * TM * 16 + i * 16 + frag_row) * LDK + ks * 32 + frag_k);
#pragma unroll
      for (int t = 0; t < TN; ++t)
        bfr[t] = load8(Bb + (wn * TN * 16 + t * 16 + frag_row) * LDK + ks * 32 + frag_k);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[t], acc[i][t], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = wm * TM * 16 + i * 16 + 4 * (lane >> 4) + q;
        const int cc = wn * TN * 16 + t * 16 + (lane & 15);
        Cs[rr * LDC + cc] = acc[i][t][q];
      }
  __syncthreads();
  if (a.logits) tile_store_logits<BM, BN, LDC>(Cs, a.logits, m0, v0, M, V);
  const RowAcc ts = tile_row_stats<BM, BN, LDC>(Cs, v0, V, a.scale_log2);
  constexpr int TPR = 256 / BM;
  const int m = m0 + tid / TPR;
  if (tid % TPR == 0 && m < M) {
    TilePartial p;
    p.top1 = ts.t1; p.top2 = ts.t2; p.arg = ts.arg; p.sum = ts.sum;
    a.partials[(size_t)m * a.part_stride + blockIdx.x] = p;
  }
}

// One workgroup per verified row: merge the row's partials (loaded in one round of
// independent loads, kMergePer per thread) and compute the exact drafted-token logit.
constexpr int kMergePer = 16;   // partials per thread per round (n <= 4096 in one round)

__global__ __launch_bounds__(256) void k_row_merge(VerifyArgs a, int n) {
  __shared__ double red[4];
  __shared__ float s_t1[4], s_t2[4];
  __shared__ int s_arg[4];
  const int m = blockIdx.x;
  const int M = rows_total(a.rm);
  if (m >= M) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const TilePartial *P = a.partials + (size_t)m * a.part_stride;
  float t1 = -INFINITY, t2 = -INFINITY;
  int a1 = 0x7fffffff;
  for (int base = 0; base < n; base += 256 * kMergePer) {
    TilePartial q[kMergePer];
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
    for (int p = tid; p < n; p += 256) {      // second pass hits the cache
      const TilePartial q = P[p];
      if (q.sum != 0.f) S += (double)q.sum * exp(((double)q.top1 - (double)t1) * a.invT);
    }
    S = block_sum(S, red);
    lse = (double)t1 * a.invT + log(S);
  }
  const double zd = drafted_logit(a, m, red);
  if (tid == 0) write_stats(a, m, t1, t2, a1, lse, zd);
}

// Resident workgroups per CU for the streaming variants, cached for the current device.
struct Occupancy {
  int device = -1, cus = 0, per_cu[3] = {0, 0, 0};
};
Occupancy g_occ;

template <int MT, int BN, int KC>
hipError_t launch_stream(const VerifyArgs &a, int variant, hipStream_t stream) {
  if (g_occ.device < 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 1;
    g_occ.cus = cus > 0 ? cus : 1;
    g_occ.device = dev;
  }
  if (g_occ.per_cu[variant] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gemm_stream<MT, BN, KC>, 256, 0) !=
        hipSuccess)
      n = 1;
    g_occ.per_cu[variant] = n > 0 ? n : 1;
  }
  const int nslab = (a.V + BN - 1) / BN;
  const int resident = g_occ.cus * g_occ.per_cu[variant];
  // At most one workgroup per resident slot and per partial column.
  const int g0 = min(nslab, min(resident, a.part_stride));
  const int rounds = (nslab + g0 - 1) / g0;
  const int G = (nslab + rounds - 1) / rounds;   // every workgroup gets rounds or rounds-1 slabs
  hipLaunchKernelGGL((k_gemm_stream<MT, BN, KC>), dim3(G), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_row_merge, dim3(a.rm.B * (a.rm.gamma + 1)), dim3(256), 0, stream, a, G);
  return hipGetLastError();
}

}  // namespace

size_t verify_workspace_layout(int B, int gamma, int V, size_t *part_off, int *part_stride) {
  const size_t cap = (size_t)B * (gamma + 1);
  const int stride = (V + kMinVocabTile - 1) / kMinVocabTile;
  const size_t po = sizeof(WsHeader);
  if (part_off) *part_off = po;
  if (part_stride) *part_stride = stride;
  return po + align_up(cap * (size_t)stride * sizeof(TilePartial), 256);
}

hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream) {
  const int cap = a.rm.B * (a.rm.gamma + 1);
  if (cap <= 16) return launch_stream<1, 64, 256>(a, 0, stream);
  if (cap <= 32) return launch_stream<2, 64, 128>(a, 1, stream);
  if (cap <= 64) return launch_stream<4, 64, 128>(a, 2, stream);
  constexpr int BM = 128, BN = 128;
  const int nvt = (a.V + BN - 1) / BN;
  hipLaunchKernelGGL((k_gemm_tile<BM, BN>), dim3(nvt, (cap + BM - 1) / BM), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_row_merge, dim3(cap), dim3(256), 0, stream, a, nvt);
  return hipGetLastError();
}

}  // namespace sdv
