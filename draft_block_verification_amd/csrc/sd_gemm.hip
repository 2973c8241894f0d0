// LM-head verify contraction with a fused row-statistics epilogue (gfx950).
//
// z[m][v] = sum_k h[m][k] * W[v][k] for the M packed verified rows (LFM2.5-DSpark
// blog, "How DSpark works": the target checks the whole drafted block in one pass
// and shares one weight load across it; DSpark summary, "Production deployment":
// the LM head maps the d-vector to V logits, and variable-length requests are
// flattened rather than padded).
//
// Both operands are K-contiguous bf16 (hidden rows [M][d], LM head [V][d]); the
// products run on the 16x16x32 bf16 MFMA with fp32 accumulation. Two regimes:
//   * skinny (M <= 64): each workgroup owns 64 vocabulary rows; its four waves
//     split d and stream W straight from HBM into MFMA operand registers, so W
//     is read exactly once; the wave partials are summed in a fixed order.
//   * tiled (M > 64): BM x BN output tiles staged through LDS with a
//     double-buffered K loop.
// The epilogue of either regime turns the fp32 tile into, per (row, vocabulary
// tile): max, second max, lowest argmax and sum of exp((z - max) / T), and
// optionally stores the fp32 logits.
#include <math.h>

#include "sd_internal.h"

namespace sdv {
namespace {

__device__ inline bf16x8 load8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
__device__ inline bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

// Per (row, vocabulary tile) statistics of an fp32 tile held in LDS.
// All 256 threads take part; TPR consecutive threads share one row.
template <int ROWS, int COLS, int LDC>
__device__ void tile_epilogue(const float *Cs, int m0, int v0, int M, int V, float scale_log2,
                              float *logits, TilePartial *partials, int n_vtiles_cap, int vtile) {
  static_assert(256 % ROWS == 0, "rows must divide the workgroup");
  constexpr int TPR = 256 / ROWS;
  static_assert(COLS % TPR == 0, "columns must split evenly");
  constexpr int CPT = COLS / TPR;
  const int tid = threadIdx.x;

  if (logits) {
    for (int idx = tid; idx < ROWS * COLS; idx += 256) {
      const int rr = idx / COLS, cc = idx - rr * COLS;
      const int m = m0 + rr, v = v0 + cc;
      if (m < M && v < V) logits[(size_t)m * V + v] = Cs[rr * LDC + cc];
    }
  }

  const int rr = tid / TPR, sub = tid - rr * TPR;
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
  const int m = m0 + rr;
  if (sub == 0 && m < M) {
    TilePartial p;
    p.top1 = t1; p.top2 = t2; p.arg = a1; p.sum = s;
    partials[(size_t)m * n_vtiles_cap + vtile] = p;
  }
}

// ---------------------------------------------------------------- skinny regime
// MT 16-row MFMA tiles cover all M <= 16 * MT rows; NT = 4 column tiles give 64
// vocabulary rows per workgroup. Wave w handles the w-th quarter of d.
template <int MT>
__global__ __launch_bounds__(256) void k_gemm_skinny(const uint16_t *__restrict__ hidden,
                                                     const uint16_t *__restrict__ W, RowMap rm,
                                                     int d, int V, float scale_log2,
                                                     float *__restrict__ logits,
                                                     TilePartial *__restrict__ partials,
                                                     int n_vtiles_cap, WsHeader *ws) {
  constexpr int NT = 4, BN = 64, ROWS = 16 * MT, LDC = BN + 4, U = 2;
  __shared__ float Cs[ROWS * LDC];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v0 = blockIdx.x * BN;
  const int M = rows_total(rm);

  const uint16_t *arow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = 16 * i + (lane & 15);
    arow[i] = nullptr;
    if (m < M) {
      int r, j;
      const int hr = hidden_row(rm, m, &r, &j);
      if (hr >= 0) arow[i] = hidden + (size_t)hr * d;
      else raise_flag(ws, SD_FLAG_ROW_OFFSETS);
    }
  }
  const uint16_t *brow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int v = min(v0 + 16 * t + (lane & 15), V - 1);
    brow[t] = W + (size_t)v * d;
  }
  const int kq = (lane >> 4) * 8;
  const int nsteps = (d + 31) / 32;
  const int s_begin = wave * nsteps / 4, s_end = (wave + 1) * nsteps / 4;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 a_c[U][MT], b_c[U][NT];
  auto load_group = [&](int s0, bf16x8 (&a)[U][MT], bf16x8 (&b)[U][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u) * 32 + kq;
      const bool ok = (s0 + u) < s_end && k < d;
#pragma unroll
      for (int t = 0; t < NT; ++t) b[u][t] = ok ? load8(brow[t] + k) : zero8();
#pragma unroll
      for (int i = 0; i < MT; ++i) a[u][i] = (ok && arow[i]) ? load8(arow[i] + k) : zero8();
    }
  };
  if (s_begin < s_end) load_group(s_begin, a_c, b_c);
  for (int s = s_begin; s < s_end; s += U) {
    bf16x8 a_n[U][MT], b_n[U][NT];
    load_group(s + U, a_n, b_n);  // zeros, with no memory access, past s_end
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_c[u][i], b_c[u][t], acc[i][t], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < MT; ++i) a_c[u][i] = a_n[u][i];
#pragma unroll
      for (int t = 0; t < NT; ++t) b_c[u][t] = b_n[u][t];
    }
  }

  // Sum the four waves' partial products in a fixed order (wave 0 + 1 + 2 + 3).
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rr = 16 * i + 4 * (lane >> 4) + q, cc = 16 * t + (lane & 15);
            if (w == 0) Cs[rr * LDC + cc] = acc[i][t][q];
            else Cs[rr * LDC + cc] += acc[i][t][q];
          }
    }
    __syncthreads();
  }
  tile_epilogue<ROWS, BN, LDC>(Cs, 0, v0, M, V, scale_log2, logits, partials, n_vtiles_cap,
                               blockIdx.x);
}

// ----------------------------------------------------------------- tiled regime
template <int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_tile(const uint16_t *__restrict__ hidden,
                                                   const uint16_t *__restrict__ W, RowMap rm,
                                                   int d, int V, float scale_log2,
                                                   float *__restrict__ logits,
                                                   TilePartial *__restrict__ partials,
                                                   int n_vtiles_cap, WsHeader *ws) {
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
  const int M = rows_total(rm);
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
      const int hr = hidden_row(rm, m, &r, &j);
      if (hr >= 0) asrc[c] = hidden + (size_t)hr * d;
      else raise_flag(ws, SD_FLAG_ROW_OFFSETS);
    }
  }
  const uint16_t *bsrc[B_CH];
  int b_lds[B_CH], b_k[B_CH];
#pragma unroll
  for (int c = 0; c < B_CH; ++c) {
    const int ch = tid + 256 * c, rr = ch >> 3, kc = (ch & 7) * 8;
    b_lds[c] = rr * LDK + kc;
    b_k[c] = kc;
    bsrc[c] = W + (size_t)min(v0 + rr, V - 1) * d;
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
  tile_epilogue<BM, BN, LDC>(Cs, m0, v0, M, V, scale_log2, logits, partials, n_vtiles_cap,
                             blockIdx.x);
}

}  // namespace

int verify_gemm_vocab_tile(int max_rows) { return max_rows <= 64 ? 64 : 128; }

hipError_t launch_verify_gemm(const uint16_t *hidden, const uint16_t *W, const RowMap &rm, int d,
                              int V, float temperature, float *logits, TilePartial *partials,
                              int n_vtiles_cap, WsHeader *ws, int *n_vtiles_used,
                              hipStream_t stream) {
  const int cap = rm.B * (rm.gamma + 1);
  const float scale_log2 = temperature > 0.f ? (float)(1.4426950408889634 / (double)temperature) : 0.f;
  const dim3 block(256);
  if (cap <= 64) {
    const int nvt = (V + 63) / 64;
    *n_vtiles_used = nvt;
    const dim3 grid(nvt);
    if (cap <= 16)
      hipLaunchKernelGGL(k_gemm_skinny<1>, grid, block, 0, stream, hidden, W, rm, d, V, scale_log2, logits, partials, n_vtiles_cap, ws);
    else if (cap <= 32)
      hipLaunchKernelGGL(k_gemm_skinny<2>, grid, block, 0, stream, hidden, W, rm, d, V, scale_log2, logits, partials, n_vtiles_cap, ws);
    else
      hipLaunchKernelGGL(k_gemm_skinny<4>, grid, block, 0, stream, hidden, W, rm, d, V, scale_log2, logits, partials, n_vtiles_cap, ws);
  } else {
    constexpr int BM = 128, BN = 128;
    const int nvt = (V + BN - 1) / BN;
    *n_vtiles_used = nvt;
    const dim3 grid(nvt, (cap + BM - 1) / BM);
    hipLaunchKernelGGL((k_gemm_tile<BM, BN>), grid, block, 0, stream, hidden, W, rm, d, V, scale_log2, logits, partials, n_vtiles_cap, ws);
  }
  return hipGetLastError();
}

}  // namespace sdv
