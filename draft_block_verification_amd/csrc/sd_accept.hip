// Confidence truncation, row-statistics merge and acceptance kernels (gfx950).
//
// Truncation: DSpark summary (GeekNews), "Architecture": the confidence head
// scores each drafted position's survival and the scheduler keeps the confident
// prefix (E F G kept, H cut in the decode-round example).
// Greedy acceptance: LFM2.5-DSpark blog, "Quality parity": a draft survives only
// if it equals the target's choice; the first mismatch is replaced by the
// target's token.
// Rejection acceptance: DSpark summary, "Problem definition": rejection
// sampling accepts the longest prefix consistent with the target distribution
// without changing it; the correction token after the first rejection comes
// from the residual max(0, p - q), the bonus token after a fully accepted block
// from p.
#include <math.h>

#include "sd_internal.h"

namespace sdv {
namespace {

constexpr double kLog2e = 1.4426950408889634;

// First row of request r, or -1 when rows r .. r + L would leave the row capacity.
__device__ inline int request_base(const RowMap &rm, int r, int L, WsHeader *ws) {
  const int cap = rm.B * (rm.gamma + 1);
  const int base = rm.row_offsets ? rm.row_offsets[r] : r * (rm.gamma + 1);
  if (base < 0 || base + L >= cap) {
    raise_flag(ws, SD_FLAG_ROW_OFFSETS);
    return -1;
  }
  return base;
}

// ------------------------------------------------------------------ truncation
// One workgroup; thread t owns a contiguous run of requests, then a block scan
// turns the per-run row counts into packed row offsets.
__global__ __launch_bounds__(256) void k_truncate(const float *__restrict__ conf, int B, int gamma,
                                                  float threshold, int32_t *__restrict__ verify_len,
                                                  int32_t *__restrict__ row_offsets) {
  __shared__ int sums[256];
  const int tid = threadIdx.x;
  const int per = (B + 255) / 256;
  const int r0 = min(B, tid * per), r1 = min(B, r0 + per);
  int local = 0;
  for (int r = r0; r < r1; ++r) {
    const float *c = conf + (size_t)r * gamma;
    int L = 0;
    while (L < gamma && c[L] >= threshold) ++L;
    verify_len[r] = L;
    local += L + 1;
  }
  sums[tid] = local;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += v;
    __syncthreads();
  }
  int run = tid ? sums[tid - 1] : 0;
  for (int r = r0; r < r1; ++r) {
    row_offsets[r] = run;
    run += verify_len[r] + 1;
  }
  if (tid == 255) row_offsets[B] = sums[255];
}

// -------------------------------------------------------------- greedy accept
// One wave per request: lane j compares row j's argmax with draft j, a ballot finds
// the first mismatch, and the emitted token is the argmax of that row.
__global__ __launch_bounds__(256) void k_accept_greedy(const sd_row_stats *__restrict__ stats,
                                                       const int32_t *__restrict__ draft_tokens,
                                                       const int32_t *__restrict__ verify_len,
                                                       RowMap rm, int32_t *__restrict__ accept_len,
                                                       int32_t *__restrict__ next_token,
                                                       int64_t *__restrict__ counters) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rm.B) return;
  const int L = clamp_len(verify_len, r, rm.gamma, nullptr);
  const int base = request_base(rm, r, L, nullptr);
  if (base < 0) {
    if (lane == 0) { accept_len[r] = 0; next_token[r] = -1; }
    return;
  }
  const int am = lane <= L ? stats[base + lane].argmax : -1;
  const bool miss = lane < L && am != draft_tokens[(size_t)r * rm.gamma + lane];
  const unsigned long long mask = __ballot(miss);
  const int a = mask ? (__ffsll((long long)mask) - 1) : L;
  // Rows 0..L need L + 1 <= 65 lanes: with gamma = 64 the bonus row is read separately.
  const int tok = a < kWave ? __shfl(am, a) : stats[base + a].argmax;
  if (lane == 0) {
    accept_len[r] = a;
    next_token[r] = tok;
    if (counters) {
      atomicAdd(reinterpret_cast<unsigned long long *>(counters), (unsigned long long)L);
      atomicAdd(reinterpret_cast<unsigned long long *>(counters + 1), (unsigned long long)a);
    }
  }
}

// ------------------------------------------------------- draft-row normaliser
// One workgroup per kept draft row (r, j < L_r): lse_q = log sum_v exp(l_v / T)
// over the bf16 drafter logits, with an online max and an fp64 running sum.
__global__ __launch_bounds__(256) void k_draft_lse(const uint16_t *__restrict__ draft_logits,
                                                   const int32_t *__restrict__ verify_len, int B,
                                                   int gamma, int V, float temperature,
                                                   double *__restrict__ lse_q, WsHeader *ws) {
  __shared__ float sm[4];
  __shared__ double ss[4];
  const int r = blockIdx.x / gamma, j = blockIdx.x - r * gamma;
  const int L = clamp_len(verify_len, r, gamma, ws);
  if (j >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t *row = draft_logits + ((size_t)r * gamma + j) * V;
  const float sl = (float)(kLog2e / (double)temperature);
  const double invT = 1.0 / (double)temperature;

  float m = -INFINITY;
  double s = 0.0;
  auto absorb = [&](const float *x, int n) {
    float cm = x[0];
    for (int e = 1; e < n; ++e) cm = fmaxf(cm, x[e]);
    if (cm > m) {
      if (s != 0.0) s *= exp(((double)m - (double)cm) * invT);
      m = cm;
    }
    float part = 0.f;
    for (int e = 0; e < n; ++e) part += exp2f((x[e] - m) * sl);
    s += (double)part;
  };
  if ((V & 7) == 0) {
    const int nch = V >> 3;
    for (int c = tid; c < nch; c += 256) {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(row + (size_t)c * 8);
      float x[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[2 * q] = __uint_as_float(w[q] << 16);
        x[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
      absorb(x, 8);
    }
  } else {
    for (int v = tid; v < V; v += 256) {
      const float x = bf16_to_f32(row[v]);
      absorb(&x, 1);
    }
  }
  // Combine (max, sum) pairs: wave butterfly, then the four waves in order.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float om = __shfl_xor(m, off);
    const double os = __shfl_xor(s, off);
    const float nm = fmaxf(m, om);
    double ns = 0.0;
    if (s != 0.0) ns += s * exp(((double)m - (double)nm) * invT);
    if (os != 0.0) ns += os * exp(((double)om - (double)nm) * invT);
    m = nm;
    s = ns;
  }
  if (lane == 0) { sm[wave] = m; ss[wave] = s; }
  __syncthreads();
  if (tid == 0) {
    float M = sm[0];
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm[w]);
    double S = 0.0;
    for (int w = 0; w < 4; ++w)
      if (ss[w] != 0.0) S += ss[w] * exp(((double)sm[w] - (double)M) * invT);
    lse_q[(size_t)r * gamma + j] = (double)M * invT + log(S);
  }
}

// ----------------------------------------------------------- rejection accept
constexpr int kTileElems = 256 * 8;   // elements per scan tile (8 per thread)
constexpr int kMaxTiles = 1024;       // V <= 2^21 in the sampler

struct SampleRow {
  const float *z;         // target logits of the sampled row [V]
  const uint16_t *q;      // drafter logits of the row [V], or null for a plain p draw
  double lse_p, lse_q, invT;
};

// Weight of vocabulary id v: p_v for a plain draw, max(0, p_v - q_v) for a residual.
__device__ inline float draw_weight(const SampleRow &sr, int v) {
  const float p = expf((float)((double)sr.z[v] * sr.invT - sr.lse_p));
  if (!sr.q) return p;
  const float q = expf((float)((double)bf16_to_f32(sr.q[v]) * sr.invT - sr.lse_q));
  return fmaxf(p - q, 0.f);
}

// Inverse-CDF draw in ascending vocabulary id: the smallest v whose running weight
// exceeds u * S (S = total weight). All 256 threads call it and get the same id;
// -1 when the total weight is zero. If rounding leaves no such v, the last id with
// positive weight is taken.
//   Pass 1: per-thread sums of 8 consecutive ids per 2048-id tile, reduced to tile
//           totals in a fixed order; thread 0 finds the tile where the running
//           total crosses u * S.
//   Pass 2: an exclusive scan inside that tile locates the id.
__device__ int inverse_cdf_draw(const SampleRow &sr, int V, float u, double *tile_sum,
                                double *wave_part, double *scal, int *sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = (V + kTileElems - 1) / kTileElems;
  for (int t = 0; t < ntiles; ++t) {
    const int v0 = t * kTileElems + tid * 8;
    double part = 0.0;
    for (int e = 0; e < 8; ++e)
      if (v0 + e < V) part += (double)draw_weight(sr, v0 + e);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) wave_part[t * 4 + wave] = part;
  }
  __syncthreads();
  if (tid == 0) {
    double S = 0.0;
    for (int t = 0; t < ntiles; ++t) {
      tile_sum[t] = ((wave_part[4 * t] + wave_part[4 * t + 1]) + wave_part[4 * t + 2]) +
                    wave_part[4 * t + 3];
      S += tile_sum[t];
    }
    const double thresh = (double)u * S;
    int hit = -1, last_pos = 0;
    double carry = 0.0;
    if (S > 0.0) {
      for (int t = 0; t < ntiles; ++t) {
        if (carry + tile_sum[t] > thresh) { hit = t; break; }
        carry += tile_sum[t];
      }
      if (hit < 0) {
        last_pos = 1;
        for (int t = ntiles - 1; t >= 0; --t)
          if (tile_sum[t] > 0.0) { hit = t; break; }
      }
    }
    sel[0] = hit;
    sel[1] = last_pos;
    scal[0] = carry;
    scal[1] = thresh;
  }
  __syncthreads();
  const int hit = sel[0], last_pos = sel[1];
  if (hit < 0) return -1;
  const double carry = scal[0], thresh = scal[1];

  const int v0 = hit * kTileElems + tid * 8;
  float w[8];
  double mine = 0.0;
  for (int e = 0; e < 8; ++e) {
    w[e] = (v0 + e < V) ? draw_weight(sr, v0 + e) : 0.f;
    mine += (double)w[e];
  }
  double incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scal[2 + wave] = incl;
  __syncthreads();
  double before = 0.0;
  for (int q = 0; q < wave; ++q) before += scal[2 + q];
  const double base = carry + (before + (incl - mine));

  int cross = 0x7fffffff, lastp = -1;
  for (int e = 7; e >= 0; --e)
    if (w[e] > 0.f) { lastp = v0 + e; break; }
  if (!last_pos && base + mine > thresh) {
    double run = 0.0;
    for (int e = 0; e < 8; ++e) {
      run += (double)w[e];
      if (base + run > thresh) { cross = v0 + e; break; }
    }
    if (cross == 0x7fffffff && lastp >= 0) cross = lastp;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    cross = min(cross, __shfl_xor(cross, off));
    lastp = max(lastp, __shfl_xor(lastp, off));
  }
  if (lane == 0) { sel[2 + wave] = cross; sel[6 + wave] = lastp; }
  __syncthreads();
  int c = sel[2], l = sel[6];
  for (int q = 1; q < 4; ++q) { c = min(c, sel[2 + q]); l = max(l, sel[6 + q]); }
  __syncthreads();   // sel / scal are reused by the next call
  return (!last_pos && c != 0x7fffffff) ? c : l;
}

__global__ __launch_bounds__(256) void k_accept_rejection(
    const float *__restrict__ logits, const sd_row_stats *__restrict__ stats,
    const uint16_t *__restrict__ draft_logits, const int32_t *__restrict__ draft_tokens,
    const int32_t *__restrict__ verify_len, RowMap rm, const float *__restrict__ u_accept,
    const float *__restrict__ u_resample, int V, float temperature,
    const double *__restrict__ lse_q, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ next_token, int64_t *__restrict__ counters, WsHeader *ws) {
  __shared__ double tile_sum[kMaxTiles];
  __shared__ double wave_part[4 * kMaxTiles];
  __shared__ double scal[8];
  __shared__ int sel[12];
  __shared__ int s_a;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int gamma = rm.gamma;
  const int L = clamp_len(verify_len, r, gamma, tid == 0 ? ws : nullptr);
  const int base = request_base(rm, r, L, tid == 0 ? ws : nullptr);
  if (base < 0) {
    if (tid == 0) { accept_len[r] = 0; next_token[r] = -1; }
    return;
  }
  const double invT = 1.0 / (double)temperature;

  if (tid < kWave) {
    bool rejected = false;
    if (lane < L) {
      const sd_row_stats st = stats[base + lane];
      const int x = draft_tokens[(size_t)r * gamma + lane];
      if (x < 0 || x >= V) {
        rejected = true;
      } else {
        const size_t qrow = ((size_t)r * gamma + lane) * V;
        const double lx = (double)bf16_to_f32(draft_logits[qrow + x]);
        const double logp = st.z_draft * invT - st.lse;
        const double logq = lx * invT - lse_q[(size_t)r * gamma + lane];
        const double ratio = exp(logp - logq);
        rejected = !((double)u_accept[(size_t)r * gamma + lane] < fmin(1.0, ratio));
      }
    }
    const unsigned long long mask = __ballot(rejected);
    if (lane == 0) s_a = mask ? (__ffsll(mask) - 1) : L;
  }
  __syncthreads();
  const int a = s_a;

  SampleRow sr;
  sr.z = logits + (size_t)(base + a) * V;
  sr.lse_p = stats[base + a].lse;
  sr.invT = invT;
  sr.q = nullptr;
  sr.lse_q = 0.0;
  const float u = u_resample[(size_t)r * (gamma + 1) + a];
  int tok = -1;
  if (a < L) {
    sr.q = draft_logits + ((size_t)r * gamma + a) * V;
    sr.lse_q = lse_q[(size_t)r * gamma + a];
    tok = inverse_cdf_draw(sr, V, u, tile_sum, wave_part, scal, sel);
    if (tok < 0) {
      if (tid == 0) raise_flag(ws, SD_FLAG_NO_RESIDUAL);
      sr.q = nullptr;
    }
  }
  if (tok < 0) tok = inverse_cdf_draw(sr, V, u, tile_sum, wave_part, scal, sel);
  if (tok < 0) tok = stats[base + a].argmax;
  if (tid == 0) {
    accept_len[r] = a;
    next_token[r] = tok;
    if (counters) {
      atomicAdd(reinterpret_cast<unsigned long long *>(counters), (unsigned long long)L);
      atomicAdd(reinterpret_cast<unsigned long long *>(counters + 1), (unsigned long long)a);
    }
  }
}

}  // namespace

hipError_t launch_truncate(const float *conf, int B, int gamma, float threshold,
                           int32_t *verify_len, int32_t *row_offsets, hipStream_t stream) {
  hipLaunchKernelGGL(k_truncate, dim3(1), dim3(256), 0, stream, conf, B, gamma, threshold,
                     verify_len, row_offsets);
  return hipGetLastError();
}

hipError_t launch_accept_greedy(const sd_row_stats *stats, const int32_t *draft_tokens,
                                const int32_t *verify_len, const RowMap &rm,
                                int32_t *accept_len, int32_t *next_token, int64_t *counters,
                                hipStream_t stream) {
  hipLaunchKernelGGL(k_accept_greedy, dim3((rm.B + 3) / 4), dim3(256), 0, stream, stats, draft_tokens,
                     verify_len, rm, accept_len, next_token, counters);
  return hipGetLastError();
}

hipError_t launch_accept_rejection(const float *logits, const sd_row_stats *stats,
                                   const uint16_t *draft_logits, const int32_t *draft_tokens,
                                   const int32_t *verify_len, const RowMap &rm,
                                   const float *u_accept, const float *u_resample, int V,
                                   float temperature, int32_t *accept_len, int32_t *next_token,
                                   int64_t *counters, double *lse_q, WsHeader *ws,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(k_draft_lse, dim3(rm.B * rm.gamma), dim3(256), 0, stream, draft_logits,
                     verify_len, rm.B, rm.gamma, V, temperature, lse_q, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_accept_rejection, dim3(rm.B), dim3(256), 0, stream, logits, stats,
                     draft_logits, draft_tokens, verify_len, rm, u_accept, u_resample, V,
                     temperature, lse_q, accept_len, next_token, counters, ws);
  return hipGetLastError();
}

}  // namespace sdv
