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

#include "sd_launch.h"

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

// ----------------------------------------------------------- rejection accept
// Four wide kernels, each over chunks of kChunk vocabulary ids (grid x = chunk,
// grid y strides over rows or requests, so that concurrent workgroups stream
// neighbouring chunks of one row):
//   k_draft_partial   (chunk, draft row), one wave each: max and sum of
//                     exp((l - max) / T) of the drafter logits, for every kept draft row;
//   k_accept_decide   (request): merge those into log q-normalisers, then accept
//                     draft j iff u_accept < min(1, p_j(x_j) / q_j(x_j)) and take the
//                     first rejection a_r (or L_r);
//   k_draw_partial    (chunk, request): fp64 sums of the draw weights of row a_r --
//                     max(0, p - q) after a rejection, p for the bonus row;
//   k_draw_finalize   (request): find the chunk where the running sum crosses
//                     u_resample * S and scan it for the token.
constexpr int kChunk = 4096;            // vocabulary ids per chunk
constexpr int kPer = kChunk / 256;      // ids per thread per chunk

struct DraftPart {
  float m;       // max drafter logit of the chunk (raw, before / T)
  float pad;
  double s;      // sum over the chunk of exp((l - m) / T)
};

struct RejArgs {
  const float *logits;
  const sd_row_stats *stats;
  const uint16_t *draft_logits;
  const int32_t *draft_tokens;
  const int32_t *verify_len;
  RowMap rm;
  const float *u_accept, *u_resample;
  int V, C;                  // vocabulary size, chunks per row
  float sl;                  // log2(e) / T
  double invT;               // 1 / T
  int32_t *accept_len, *next_token;
  int64_t *counters;
  double *lse_q;             // [B][gamma]
  int32_t *acc_a;            // [B] accepted length, -1 for a request outside the row capacity
  DraftPart *dpart;          // [B][gamma][C]
  double *csum;              // [B][C][2]: residual (or bonus) weight sum, p weight sum
  double *rate_part;         // [B][gamma][C] acceptance-rate chunk sums, or null
  double *rate;              // [B][gamma] acceptance rate out, or null
  WsHeader *ws;
};

// 2^x by the hardware instruction. It returns no denormals: results below 2^-126 are 0,
// far below anything the sums and draws here resolve (each draw or sum is relative to a
// row whose weights add up to 1).
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline double block_sum_d(double x, double *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  const double r = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return r;
}

// Drafter-row normaliser, one wave per (chunk, kept draft row): the chunk's 4096 drafter
// logits arrive as eight 1 KB wave loads (load h gives lane l ids c * kChunk + 512 h + 8 l
// .. + 7; ids past V count as -inf), and the chunk's max and sum are reduced with lane
// exchanges only, with no workgroup barrier. Rows are 16-byte aligned when V % 8 == 0;
// otherwise the chunk is read one id at a time (two passes).
constexpr int kDraftWaves = 4;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Loads of chunk c of an aligned row (V % 8 == 0, so V >= 8 and v0 < V means v0 + 8 <= V).
// The address is clamped into the row, so every lane loads; past V the value is -inf.
__device__ inline void draft_chunk_load(const uint16_t *row, int V, int c, int lane, u32x4 (&w)[8]) {
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int v0 = c * kChunk + 512 * h + 8 * lane;
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

__device__ inline DraftPart draft_chunk_unaligned(const uint16_t *row, int V, int c, int lane,
                                                  float sl) {
  float m = -INFINITY;
#pragma unroll 1
  for (int h = 0; h < 8; ++h)
#pragma unroll 1
    for (int e = 0; e < 8; ++e) {
      const int v = c * kChunk + 512 * h + 8 * lane + e;
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
      const int v = c * kChunk + 512 * h + 8 * lane + e;
      if (v < V) sh[h] += exp2_hw((bf16_to_f32(row[v]) - m) * sl);
    }
  }
  return draft_part(m, sh);
}

// Full grid: a workgroup's waves take neighbouring chunks of one row; grid y strides over
// the rows.
__global__ __launch_bounds__(64 * kDraftWaves) void k_draft_partial(RejArgs a) {
  const int gamma = a.rm.gamma, lane = threadIdx.x & 63;
  const int c = blockIdx.x * kDraftWaves + (threadIdx.x >> 6);
  if (c >= a.C) return;
  const int V = a.V;
  for (int rj = blockIdx.y; rj < a.rm.B * gamma; rj += gridDim.y) {
    const int r = rj / gamma, j = rj - r * gamma;
    const int L = clamp_len(a.verify_len, r, gamma, c == 0 && lane == 0 ? a.ws : nullptr);
    if (j >= L) continue;
    const uint16_t *row = a.draft_logits + (size_t)rj * V;
    DraftPart p;
    if ((V & 7) == 0) {
      u32x4 w[8];
      draft_chunk_load(row, V, c, lane, w);
      p = draft_chunk_stats(w, a.sl);
    } else {
      p = draft_chunk_unaligned(row, V, c, lane, a.sl);
    }
    if (lane == 0) a.dpart[(size_t)rj * a.C + c] = p;
  }
}

// Bounded footprint, for running beside the contraction on another stream: a fixed grid
// of 16-wave workgroups whose waves walk the (draft row, chunk) items in row-major order
// with a stride of the grid's wave count, skipping rows past L_r, with the next item's
// loads in flight while the current one is reduced. Many waves per workgroup keep the
// work on few compute units (workgroups reach the XCDs in turn, so a grid of one per XCD
// holds one compute unit on each). Same partials, bit for bit, as k_draft_partial.
constexpr int kWalkWaves = 16;

__global__ __launch_bounds__(64 * kWalkWaves) void k_draft_partial_walk(RejArgs a) {
  const int gamma = a.rm.gamma, C = a.C, V = a.V, lane = threadIdx.x & 63;
  const int rows = a.rm.B * gamma;
  // The walk state is wave-uniform; readfirstlane keeps it in scalar registers, so the
  // kept-length lookups are scalar loads that do not wait on the vector loads in flight.
  const int nw = gridDim.x * kWalkWaves;
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * kWalkWaves + (threadIdx.x >> 6));
  const int dq = nw / C, dr = nw % C;
  int rj = gw / C, c = gw % C;
  int r_seen = -1, L_seen = 0;      // kept length of the last request looked up
  auto step = [&]() {
    rj += dq;
    c += dr;
    if (c >= C) { c -= C; ++rj; }
  };
  auto seek = [&]() {        // advance (rj, c) to the first item of a kept row, or rj >= rows
    while (rj < rows) {
      const int r = rj / gamma;
      if (r != r_seen) {
        r_seen = r;
        L_seen = clamp_len(a.verify_len, r, gamma, lane == 0 ? a.ws : nullptr);
      }
      if (rj - r * gamma < L_seen) return;
      step();
    }
  };
  seek();
  if ((V & 7) != 0) {
    while (rj < rows) {
      const DraftPart p = draft_chunk_unaligned(a.draft_logits + (size_t)rj * V, V, c, lane, a.sl);
      if (lane == 0) a.dpart[(size_t)rj * C + c] = p;
      step();
      seek();
    }
    return;
  }
  u32x4 w[8];
  if (rj < rows) draft_chunk_load(a.draft_logits + (size_t)rj * V, V, c, lane, w);
  while (rj < rows) {
    const int cur_rj = rj, cur_c = c;
    step();
    seek();
    // Next item's loads (past the end: the current item again, never used), issued on
    // every path so the wait before the reduction below leaves them in flight.
    const int nrj = rj < rows ? rj : cur_rj, nc = rj < rows ? c : cur_c;
    u32x4 wn[8];
    draft_chunk_load(a.draft_logits + (size_t)nrj * V, V, nc, lane, wn);
    const DraftPart p = draft_chunk_stats(w, a.sl);
    if (lane == 0) a.dpart[(size_t)cur_rj * C + cur_c] = p;
#pragma unroll
    for (int h = 0; h < 8; ++h) w[h] = wn[h];
  }
}

// One workgroup per request; 16 lanes per draft row (16 rows per pass). A row's
// token, statistics, uniform and chunk partials are loaded together, the drafted
// token's drafter logit as soon as its id is known.
constexpr int kDecideHold = 4;   // chunk partials held per lane (C <= 64 without reloads)

__global__ __launch_bounds__(256) void k_accept_decide(RejArgs a) {
  __shared__ int s_rej[64];
  const int r = blockIdx.x, tid = threadIdx.x, sub = tid & 15;
  const int gamma = a.rm.gamma;
  const int L = clamp_len(a.verify_len, r, gamma, tid == 0 ? a.ws : nullptr);
  const int base = request_base(a.rm, r, L, tid == 0 ? a.ws : nullptr);
  if (base < 0) {
    if (tid == 0) { a.acc_a[r] = -1; a.accept_len[r] = 0; a.next_token[r] = -1; }
    return;
  }
  for (int j0 = 0; j0 < L; j0 += 16) {
    const int j = j0 + (tid >> 4);
    const bool live = j < L;
    const size_t rj = (size_t)r * gamma + (live ? j : 0);
    const int x = live ? a.draft_tokens[rj] : -1;
    const bool xok = x >= 0 && x < a.V;
    double zx = 0.0, lse_p = 0.0;
    float u = 1.f;
    if (live && sub == 0) {
      zx = a.stats[base + j].z_draft;
      lse_p = a.stats[base + j].lse;
      u = a.u_accept[rj];
    }
    const DraftPart *P = a.dpart + rj * a.C;
    DraftPart hold[kDecideHold];
#pragma unroll
    for (int i = 0; i < kDecideHold; ++i) {
      const int c = sub + 16 * i;
      hold[i] = live && c < a.C ? P[c] : DraftPart{-INFINITY, 0.f, 0.0};
    }
    const float lx = xok ? bf16_to_f32(a.draft_logits[rj * a.V + x]) : 0.f;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kDecideHold; ++i) M = fmaxf(M, hold[i].m);
    for (int c = sub + 16 * kDecideHold; live && c < a.C; c += 16) M = fmaxf(M, P[c].m);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    double S = 0.0;
#pragma unroll
    for (int i = 0; i < kDecideHold; ++i)
      if (hold[i].s != 0.0) S += hold[i].s * exp(((double)hold[i].m - (double)M) * a.invT);
    for (int c = sub + 16 * kDecideHold; live && c < a.C; c += 16) {
      const DraftPart q = P[c];
      if (q.s != 0.0) S += q.s * exp(((double)q.m - (double)M) * a.invT);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) S += __shfl_xor(S, off);
    if (live && sub == 0) {
      const double lse = (double)M * a.invT + log(S);
      a.lse_q[rj] = lse;
      int rej = 1;
      if (xok) {
        const double logp = zx * a.invT - lse_p;
        const double logq = (double)lx * a.invT - lse;
        rej = !((double)u < fmin(1.0, exp(logp - logq)));
      }
      s_rej[j] = rej;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const unsigned long long m = __ballot(tid < L && s_rej[tid]);
    if (tid == 0) {
      const int acc = m ? (__ffsll((long long)m) - 1) : L;
      a.acc_a[r] = acc;
      a.accept_len[r] = acc;
      if (a.counters) {
        atomicAdd(reinterpret_cast<unsigned long long *>(a.counters), (unsigned long long)L);
        atomicAdd(reinterpret_cast<unsigned long long *>(a.counters + 1), (unsigned long long)acc);
      }
    }
  }
}

// The row being drawn from for request r: a_r after a rejection (residual), L_r otherwise.
// A row's probabilities softmax(l / T)_v = exp(l_v / T - lse) formed in fp32 as
// 2^((l_v - c) * sl) with c = lse * T and sl = log2(e) / T. For the ids that carry
// weight l_v - c is small and nearly exact, and the rounding of c scales every weight
// of the row by one common factor, which an inverse-CDF draw does not see.
struct ProbScale {
  float c, sl;
};

__device__ inline ProbScale prob_scale(double lse, const RejArgs &a) {
  return ProbScale{(float)(lse / a.invT), a.sl};
}

__device__ inline float prob_of(float l, ProbScale s) { return exp2_hw((l - s.c) * s.sl); }

struct DrawRow {
  const float *z;        // target logits of the row
  const uint16_t *q;     // drafter logits of the row (residual draws), else null
  ProbScale ps, qs;      // p and q of the row
};

__device__ inline bool draw_row(const RejArgs &a, int r, DrawRow *d, int *arow) {
  const int acc = a.acc_a[r];
  if (acc < 0) return false;
  const int gamma = a.rm.gamma;
  const int L = clamp_len(a.verify_len, r, gamma, nullptr);
  const int base = request_base(a.rm, r, L, nullptr);
  d->z = a.logits + (size_t)(base + acc) * a.V;
  d->ps = prob_scale(a.stats[base + acc].lse, a);
  d->q = nullptr;
  d->qs = prob_scale(0.0, a);
  if (acc < L) {
    d->q = a.draft_logits + ((size_t)r * gamma + acc) * a.V;
    d->qs = prob_scale(a.lse_q[(size_t)r * gamma + acc], a);
  }
  *arow = base + acc;
  return true;
}

// p_v, and max(0, p_v - q_v) when the row has drafter logits.
__device__ inline void draw_weights(const DrawRow &d, int v, float *p, float *res) {
  *p = prob_of(d.z[v], d.ps);
  *res = *p;
  if (d.q) *res = fmaxf(*p - prob_of(bf16_to_f32(d.q[v]), d.qs), 0.f);
}

// ------------------------------------------------------ analytic acceptance rate
// c*_j = sum_v min(p_j(v), q_j(v)) = 1 - TV(p_j, q_j): the probability that the
// rejection rule keeps position j when x_j is drawn from q_j (DSpark summary,
// "Architecture": the confidence head's training label). The chunk sums ride along
// in k_draw_partial's grid and k_draw_finalize adds them up in chunk order, so the
// value does not depend on scheduling.
__device__ void rate_chunk(const RejArgs &a, int rj, int c, double *red) {
  const int gamma = a.rm.gamma;
  const int r = rj / gamma, j = rj - r * gamma;
  const int L = clamp_len(a.verify_len, r, gamma, nullptr);
  if (j >= L) return;
  const int base = request_base(a.rm, r, L, nullptr);
  if (base < 0) return;
  const float *z = a.logits + (size_t)(base + j) * a.V;
  const uint16_t *q = a.draft_logits + (size_t)rj * a.V;
  const ProbScale ps = prob_scale(a.stats[base + j].lse, a), qs = prob_scale(a.lse_q[rj], a);
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kPer / 4; ++e) {
    const int v0 = c * kChunk + 4 * (threadIdx.x + 256 * e);
    float zf[4], ql[4];
    if ((a.V & 3) == 0 && v0 + 4 <= a.V) {
      const f32x4 zv = *reinterpret_cast<const f32x4 *>(z + v0);
      const uint2 qv = *reinterpret_cast<const uint2 *>(q + v0);
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[i] = zv[i];
      ql[0] = __uint_as_float(qv.x << 16); ql[1] = __uint_as_float(qv.x & 0xffff0000u);
      ql[2] = __uint_as_float(qv.y << 16); ql[3] = __uint_as_float(qv.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = v0 + i < a.V;
        zf[i] = in ? z[v0 + i] : 0.f;
        ql[i] = in ? bf16_to_f32(q[v0 + i]) : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (v0 + i < a.V) {
        s += (double)fminf(prob_of(zf[i], ps), prob_of(ql[i], qs));
      }
    }
  }
  s = block_sum_d(s, red);
  if (threadIdx.x == 0) a.rate_part[(size_t)rj * a.C + c] = s;
}

// Request r's rates: wave w sums rows w, w + 4, ...; lane l takes chunks l, l + 64, ...
// and a fixed butterfly adds the lanes. -1 marks positions that were not verified.
__device__ void rate_finalize(const RejArgs &a, int r) {
  const int gamma = a.rm.gamma, lane = threadIdx.x & 63;
  const int L = clamp_len(a.verify_len, r, gamma, nullptr);
  const bool ok = request_base(a.rm, r, L, nullptr) >= 0;
  for (int j = threadIdx.x >> 6; j < gamma; j += 4) {
    const size_t rj = (size_t)r * gamma + j;
    if (j < L && ok) {
      double s = 0.0;
      for (int c = lane; c < a.C; c += 64) s += a.rate_part[rj * a.C + c];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) a.rate[rj] = s;
    } else if (lane == 0) {
      a.rate[rj] = -1.0;
    }
  }
}

// Chunk sums of the draw weights: ids c*kChunk + 4*(tid + 256 e) + i (16-byte logit
// loads, each wave load 1 KB contiguous). Rows past B of k_draw_partial's row range
// compute acceptance-rate chunk sums of draft row (row - B).
__device__ void draw_chunk(const RejArgs &a, int r, int c, double *red) {
  DrawRow d;
  int arow;
  if (!draw_row(a, r, &d, &arow)) return;
  double sr = 0.0, sp = 0.0;
#pragma unroll
  for (int e = 0; e < kPer / 4; ++e) {
    const int v0 = c * kChunk + 4 * (threadIdx.x + 256 * e);
    float z[4], ql[4];
    if ((a.V & 3) == 0 && v0 + 4 <= a.V) {
      const f32x4 zv = *reinterpret_cast<const f32x4 *>(d.z + v0);
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = zv[i];
      if (d.q) {
        const uint2 qv = *reinterpret_cast<const uint2 *>(d.q + v0);
        ql[0] = __uint_as_float(qv.x << 16); ql[1] = __uint_as_float(qv.x & 0xffff0000u);
        ql[2] = __uint_as_float(qv.y << 16); ql[3] = __uint_as_float(qv.y & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = v0 + i < a.V;
        z[i] = in ? d.z[v0 + i] : -INFINITY;
        ql[i] = in && d.q ? bf16_to_f32(d.q[v0 + i]) : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (v0 + i < a.V) {
        const float p = prob_of(z[i], d.ps);
        float w = p;
        if (d.q) w = fmaxf(p - prob_of(ql[i], d.qs), 0.f);
        sr += (double)w;
        sp += (double)p;
      }
    }
  }
  sr = block_sum_d(sr, red);
  sp = block_sum_d(sp, red);
  if (threadIdx.x == 0) {
    a.csum[((size_t)r * a.C + c) * 2] = sr;
    a.csum[((size_t)r * a.C + c) * 2 + 1] = sp;
  }
}

__global__ __launch_bounds__(256) void k_draw_partial(RejArgs a, int rows) {
  __shared__ double red[4];
  const int c = blockIdx.x;
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    if (r < a.rm.B) draw_chunk(a, r, c, red);
    else rate_chunk(a, r - a.rm.B, c, red);
  }
}

__global__ __launch_bounds__(256) void k_draw_finalize(RejArgs a) {
  __shared__ double s_d[8];
  __shared__ int s_i[12];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.rate) rate_finalize(a, r);
  DrawRow d;
  int arow;
  if (!draw_row(a, r, &d, &arow)) return;
  const int gamma = a.rm.gamma;
  const int acc = a.acc_a[r];
  const double *cs = a.csum + (size_t)r * a.C * 2;
  // Chunk sums in chunk order: thread t owns chunks t*K .. t*K + K - 1 (K = ceil(C/256)),
  // an inclusive block scan gives every chunk's running sum.
  int use_p = 0;
  double S = 0.0, excl = 0.0, own = 0.0;
  const int K = (a.C + 255) / 256, c0 = tid * K;
  for (int pass = 0; pass < 2; ++pass) {
    own = 0.0;
    for (int k = 0; k < K; ++k)
      if (c0 + k < a.C) own += cs[2 * (c0 + k) + use_p];
    double incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) s_d[wave] = incl;
    __syncthreads();
    double before = 0.0;
    for (int q = 0; q < wave; ++q) before += s_d[q];
    excl = before + (incl - own);
    S = ((s_d[0] + s_d[1]) + s_d[2]) + s_d[3];
    __syncthreads();
    if (S != 0.0 || !d.q || pass == 1) break;
    // No residual mass (p == q at this row): draw from p instead.
    if (tid == 0) raise_flag(a.ws, SD_FLAG_NO_RESIDUAL);
    use_p = 1;
  }
  const double thresh = (double)a.u_resample[(size_t)r * (gamma + 1) + acc] * S;
  // First chunk whose running sum passes thresh; else (rounding) the last chunk with
  // positive weight.
  int first = 0x7fffffff, lastc = -1;
  if (S > 0.0) {
    double run = excl;
    for (int k = 0; k < K && c0 + k < a.C; ++k) {
      const double w = cs[2 * (c0 + k) + use_p];
      if (first == 0x7fffffff && run + w > thresh) first = c0 + k;
      run += w;
      if (w > 0.0) lastc = c0 + k;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    first = min(first, __shfl_xor(first, off));
    lastc = max(lastc, __shfl_xor(lastc, off));
  }
  if (lane == 0) { s_i[4 + wave] = first; s_i[8 + wave] = lastc; }
  __syncthreads();
  if (tid == 0) {
    int f = s_i[4], l = s_i[8];
    for (int q = 1; q < 4; ++q) { f = min(f, s_i[4 + q]); l = max(l, s_i[8 + q]); }
    const int hit = f != 0x7fffffff ? f : l;
    s_i[0] = hit; s_i[1] = f == 0x7fffffff ? 1 : 0; s_i[2] = use_p;
  }
  // Running sum before the hit chunk: the owner thread of that chunk knows it.
  __syncthreads();
  {
    const int h = s_i[0];
    if (h >= 0 && h >= c0 && h < c0 + K) {
      double run = excl;
      for (int c = c0; c < h; ++c) run += cs[2 * c + use_p];
      s_d[0] = run;
    }
  }
  __syncthreads();
  const int hit = s_i[0], last_pos = s_i[1], col = s_i[2];
  if (hit < 0) {                      // no weight at all: fall back to the target argmax
    if (tid == 0) a.next_token[r] = a.stats[arow].argmax;
    return;
  }
  if (col == 1) d.q = nullptr;
  const double carry = s_d[0];
  // Scan the crossing chunk: kPer consecutive ids per thread, exclusive scan of the
  // per-thread sums, then the crossing thread walks its ids.
  const int v0 = hit * kChunk + tid * kPer;
  float w[kPer];
  double mine = 0.0;
  if ((a.V & 7) == 0 && v0 + kPer <= a.V) {
#pragma unroll
    for (int h = 0; h < kPer / 4; ++h) {
      const f32x4 zv = *reinterpret_cast<const f32x4 *>(d.z + v0 + 4 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[4 * h + i] = prob_of(zv[i], d.ps);
    }
    if (d.q) {
#pragma unroll
      for (int h = 0; h < kPer / 8; ++h) {
        const u32x4 qv = *reinterpret_cast<const u32x4 *>(d.q + v0 + 8 * h);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float ql = __uint_as_float((i & 1) ? (qv[i >> 1] & 0xffff0000u) : (qv[i >> 1] << 16));
          w[8 * h + i] = fmaxf(w[8 * h + i] - prob_of(ql, d.qs), 0.f);
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      float p = 0.f, x = 0.f;
      if (v0 + e < a.V) draw_weights(d, v0 + e, &p, &x);
      w[e] = x;
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) mine += (double)w[e];
  double incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_d[2 + wave] = incl;
  __syncthreads();
  double before = 0.0;
  for (int q = 0; q < wave; ++q) before += s_d[2 + q];
  const double base = carry + (before + (incl - mine));
  int cross = 0x7fffffff, lastp = -1;
  for (int e = kPer - 1; e >= 0; --e)
    if (w[e] > 0.f) { lastp = v0 + e; break; }
  if (!last_pos && base + mine > thresh) {
    double run = 0.0;
    for (int e = 0; e < kPer; ++e) {
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
  if (lane == 0) { s_i[4 + wave] = cross; s_i[8 + wave] = lastp; }
  __syncthreads();
  if (tid == 0) {
    int c = s_i[4], l = s_i[8];
    for (int q = 1; q < 4; ++q) { c = min(c, s_i[4 + q]); l = max(l, s_i[8 + q]); }
    a.next_token[r] = (!last_pos && c != 0x7fffffff) ? c : l;
  }
}

// Second grid dimension for a row range (the hardware bounds it at 65535).
inline unsigned grid_rows(int rows) { return (unsigned)(rows < 65535 ? rows : 65535); }

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

size_t accept_workspace_layout(int B, int gamma, int V, AcceptLayout *lay) {
  const int C = (V + kChunk - 1) / kChunk;
  AcceptLayout l;
  l.chunks = C;
  l.lse_q = sizeof(WsHeader);
  l.acc_a = align_up(l.lse_q + (size_t)B * gamma * sizeof(double), 256);
  l.dpart = align_up(l.acc_a + (size_t)B * sizeof(int32_t), 256);
  l.csum = align_up(l.dpart + (size_t)B * gamma * C * sizeof(DraftPart), 256);
  const size_t total = align_up(l.csum + (size_t)B * C * 2 * sizeof(double), 256);
  if (lay) *lay = l;
  return total;
}

namespace {

// Arguments of the rejection kernels; the workspace regions come from the layout.
RejArgs rej_args(const uint16_t *draft_logits, const int32_t *verify_len, const RowMap &rm, int V,
                 float temperature, void *workspace) {
  AcceptLayout l;
  accept_workspace_layout(rm.B, rm.gamma, V, &l);
  char *w = reinterpret_cast<char *>(workspace);
  RejArgs a{};
  a.draft_logits = draft_logits;
  a.verify_len = verify_len;
  a.rm = rm;
  a.V = V;
  a.C = l.chunks;
  a.sl = (float)(kLog2e / (double)temperature);
  a.invT = 1.0 / (double)temperature;
  a.lse_q = reinterpret_cast<double *>(w + l.lse_q);
  a.acc_a = reinterpret_cast<int32_t *>(w + l.acc_a);
  a.dpart = reinterpret_cast<DraftPart *>(w + l.dpart);
  a.csum = reinterpret_cast<double *>(w + l.csum);
  a.ws = reinterpret_cast<WsHeader *>(workspace);
  return a;
}

}  // namespace

hipError_t launch_draft_normalizer(const uint16_t *draft_logits, const int32_t *verify_len,
                                   int B, int gamma, int V, float temperature, void *workspace,
                                   int workgroups, hipStream_t stream) {
  const RowMap rm{nullptr, B, gamma};
  const RejArgs a = rej_args(draft_logits, verify_len, rm, V, temperature, workspace);
  if (workgroups > 0)
    hipLaunchKernelGGL(k_draft_partial_walk, dim3(workgroups), dim3(64 * kWalkWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(k_draft_partial, dim3((a.C + kDraftWaves - 1) / kDraftWaves, grid_rows(B * gamma)),
                       dim3(64 * kDraftWaves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_accept_rejection(const float *logits, const sd_row_stats *stats,
                                   const uint16_t *draft_logits, const int32_t *draft_tokens,
                                   const int32_t *verify_len, const RowMap &rm,
                                   const float *u_accept, const float *u_resample, int V,
                                   float temperature, int32_t *accept_len, int32_t *next_token,
                                   int64_t *counters, double *accept_rate, void *workspace,
                                   bool normalized, hipStream_t stream) {
  RejArgs a = rej_args(draft_logits, verify_len, rm, V, temperature, workspace);
  a.logits = logits;
  a.stats = stats;
  a.draft_tokens = draft_tokens;
  a.u_accept = u_accept;
  a.u_resample = u_resample;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.counters = counters;
  // The drafter chunk partials are dead after k_accept_decide; their storage
  // ([B][gamma][C] entries of 16 bytes) holds the rate chunk sums.
  a.rate_part = accept_rate ? reinterpret_cast<double *>(a.dpart) : nullptr;
  a.rate = accept_rate;
  hipError_t e;
  if (!normalized) {
    hipLaunchKernelGGL(k_draft_partial,
                       dim3((a.C + kDraftWaves - 1) / kDraftWaves, grid_rows(rm.B * rm.gamma)),
                       dim3(64 * kDraftWaves), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_accept_decide, dim3(rm.B), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int draw_rows = rm.B + (accept_rate ? rm.B * rm.gamma : 0);
  hipLaunchKernelGGL(k_draw_partial, dim3(a.C, grid_rows(draw_rows)), dim3(256), 0, stream, a,
                     draw_rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_draw_finalize, dim3(rm.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sdv
