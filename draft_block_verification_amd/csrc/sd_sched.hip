// Hardware-aware prefix scheduler (gfx950): chooses how many drafted positions of
// each request the target verifies this step.
//
// DSpark summary, "Architecture" -> "Confidence-Scheduled Verification" ->
// "Hardware-Aware Prefix Scheduler": survival a[r][j] (running product of the
// per-position confidences) never grows along a block, so a global sort by survival
// admits each request's positions as a prefix; the admitted count K sets the target
// batch B = R + K, and the scheduler maximises tau * SPS(B), tau being the expected
// tokens of the step and SPS a steps-per-second table profiled once. "Engineering"
// -> "the scheduler in practice": the synchronous form stops at the first admission
// that lowers throughput; the asynchronous form picks K from two-step-old confidences
// by searching every K (no early stop) and admits the current top-K.
//
// One workgroup of 1024 threads. The confidences are staged in LDS and each
// request's survival is formed left to right in fp32. Survival falls along a block,
// so every request is already a sorted run; log2(R) levels of stable pairwise merges
// (each element finds its place by a binary search in the partner run) sort all
// R * gamma survivals, larger first, ties in (request, position) order. A block scan
// of fixed-point survivals gives tau along that order and a reduction picks K. The
// admitted set is then every candidate above the K-th sorted survival plus, among
// those equal to it, the first ones in (request, position) order; a block scan of the
// per-request counts gives the row offsets.
#include "sd_launch.h"

namespace sdv {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr double kFixScale = 1099511627776.0;   // 2^40 fixed-point units per token

// Confidence clamped into [0, 1]; NaN counts as 0.
__device__ inline float clamp_conf(float c) { return c > 0.f ? (c < 1.f ? c : 1.f) : 0.f; }

// Sort key of a survival a in [0, 1]: ascending keys are descending survivals.
__device__ inline unsigned survival_key(float a) { return ~__float_as_uint(a); }

__device__ inline float key_survival(unsigned k) { return __uint_as_float(~k); }

__device__ inline long long fixed_units(float a) { return (long long)((double)a * kFixScale); }

// Exclusive scan over the block of one 64-bit value per thread; *total gets the sum.
__device__ long long block_exclusive_scan(long long x, long long *red, long long *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  long long before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSchedWaves; ++w) {
    before += w < wave ? red[w] : 0;
    all += red[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

// Copies conf[R][gamma] into LDS (coalesced).
__device__ void stage_conf(const float *__restrict__ conf, int N, float *lds) {
  for (int i = threadIdx.x; i < N; i += kSchedThreads) lds[i] = conf[i];
  __syncthreads();
}

// Sorted survival keys of one confidence array; returns the buffer holding them
// (buf0 or buf1, N entries each).
__device__ unsigned *sorted_keys(const float *__restrict__ conf, int R, int gamma, unsigned *buf0,
                                 unsigned *buf1) {
  const int N = R * gamma;
  float *staged = reinterpret_cast<float *>(buf1);
  stage_conf(conf, N, staged);
  for (int r = threadIdx.x; r < R; r += kSchedThreads) {
    float run = 1.f;
    for (int j = 0; j < gamma; ++j) {
      run = run * clamp_conf(staged[r * gamma + j]);
      buf0[r * gamma + j] = survival_key(run);
    }
  }
  __syncthreads();
  unsigned *src = buf0, *dst = buf1;
  for (int len = gamma; len < N; len <<= 1) {
    for (int p = threadIdx.x; p < N; p += kSchedThreads) {
      const int a0 = (p / (2 * len)) * (2 * len);
      const int a1 = min(N, a0 + len), b1 = min(N, a0 + 2 * len);
      const unsigned x = src[p];
      int lo, hi, out;
      if (p < a1) {          // run A: B elements strictly below go first
        lo = a1; hi = b1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (src[mid] < x) lo = mid + 1; else hi = mid;
        }
        out = p + (lo - a1);
      } else {               // run B: A elements at or below go first (stable)
        lo = a0; hi = a1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (src[mid] <= x) lo = mid + 1; else hi = mid;
        }
        out = (p - a1) + lo;
      }
      dst[out] = x;
    }
    __syncthreads();
    unsigned *t = src; src = dst; dst = t;
  }
  return src;
}

// Sorted positions owned by this thread in choose_admitted: [k0, k1).
constexpr int kSegMax = kSchedMaxCandidates / kSchedThreads;

struct SpsSeg {
  float v[kSegMax + 1];   // SPS(R + k) for k = k0 .. k1
};

// Loads the SPS entries this thread needs, early, so the loads overlap the sort.
__device__ inline void load_sps(const float *__restrict__ sps, int R, int N, SpsSeg *s) {
  const int seg = (N + kSchedThreads - 1) / kSchedThreads;
  const int k0 = min(N, (int)threadIdx.x * seg), k1 = min(N, k0 + seg);
#pragma unroll
  for (int i = 0; i <= kSegMax; ++i) s->v[i] = k0 + i <= k1 ? sps[R + k0 + i] : 0.f;
}

// Admitted count K along the sorted keys. Thread t owns sorted positions
// [t * seg, t * seg + seg) and evaluates Theta at each of them (and at N for the
// last owner): Theta_K = (R * 2^40 + first K units) * SPS(R + K) in float64.
__device__ int choose_admitted(const unsigned *keys, int R, int N, const SpsSeg &sps,
                               int mode, long long *red_ll, double *red_d, int *red_i) {
  const int seg = (N + kSchedThreads - 1) / kSchedThreads;
  const int k0 = min(N, (int)threadIdx.x * seg), k1 = min(N, k0 + seg);
  long long mine = 0;
  for (int k = k0; k < k1; ++k) mine += fixed_units(key_survival(keys[k]));
  long long total;
  long long S = block_exclusive_scan(mine, red_ll, &total) + ((long long)R << 40);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int pick = N;             // early stop: first K whose admission lowers Theta
  double best = -1.0;       // global search: largest Theta, smallest K
  int best_k = N + 1;
  double th = (double)S * (double)sps.v[0];
#pragma unroll
  for (int i = 0; i < kSegMax; ++i) {
    const int k = k0 + i;
    if (k >= k1) break;
    S += fixed_units(key_survival(keys[k]));
    const double next = (double)S * (double)sps.v[i + 1];
    if (mode == SD_SCHED_EARLY_STOP) {
      if (next < th) { pick = k; break; }
    } else if (th > best) {
      best = th;
      best_k = k;
    }
    th = next;
  }
  // Theta_N (every candidate admitted): evaluated by the owner of the last position.
  if (mode != SD_SCHED_EARLY_STOP && k0 < k1 && k1 == N && th > best) {
    best = th;
    best_k = N;
  }
  if (mode == SD_SCHED_EARLY_STOP) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) pick = min(pick, __shfl_xor(pick, off));
    if (lane == 0) red_i[wave] = pick;
    __syncthreads();
    int K = N;
    for (int w = 0; w < kSchedWaves; ++w) K = min(K, red_i[w]);
    __syncthreads();
    return K;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ob = __shfl_xor(best, off);
    const int ok = __shfl_xor(best_k, off);
    if (ob > best || (ob == best && ok < best_k)) { best = ob; best_k = ok; }
  }
  if (lane == 0) { red_d[wave] = best; red_i[wave] = best_k; }
  __syncthreads();
  double b = red_d[0];
  int K = red_i[0];
  for (int w = 1; w < kSchedWaves; ++w)
    if (red_d[w] > b || (red_d[w] == b && red_i[w] < K)) { b = red_d[w]; K = red_i[w]; }
  __syncthreads();
  return K;
}

__global__ __launch_bounds__(kSchedThreads) void k_schedule(const float *__restrict__ conf,
                                                            const float *__restrict__ conf_stale,
                                                            int R, int gamma,
                                                            const float *__restrict__ sps,
                                                            int mode, int32_t *__restrict__ verify_len,
                                                            int32_t *__restrict__ row_offsets) {
  __shared__ unsigned buf0[kSchedMaxCandidates], buf1[kSchedMaxCandidates];
  __shared__ long long red_ll[kSchedWaves];
  __shared__ double red_d[kSchedWaves];
  __shared__ int red_i[kSchedWaves];
  __shared__ unsigned s_cut;
  const int N = R * gamma;
  // K from the stale confidences (asynchronous form) or the current ones.
  const bool stale = mode == SD_SCHED_TOP_K && conf_stale != nullptr;
  SpsSeg seg;
  load_sps(sps, R, N, &seg);
  const unsigned *keys = sorted_keys(stale ? conf_stale : conf, R, gamma, buf0, buf1);
  const int K = choose_admitted(keys, R, N, seg, mode, red_ll, red_d, red_i);
  if (stale) keys = sorted_keys(conf, R, gamma, buf0, buf1);
  if (threadIdx.x == 0) s_cut = K < N ? keys[K] : 0u;
  __syncthreads();
  const unsigned cut = s_cut;    // key of the first candidate left out
  // Per request: candidates strictly above the cut, and those equal to it.
  float *staged = reinterpret_cast<float *>(keys == buf0 ? buf1 : buf0);
  stage_conf(conf, N, staged);
  const int per = (R + kSchedThreads - 1) / kSchedThreads;
  const int r0 = min(R, (int)threadIdx.x * per), r1 = min(R, r0 + per);
  long long counts = 0;          // (above << 32) | equal over this thread's requests
  for (int r = r0; r < r1; ++r) {
    float run = 1.f;
    int above = 0, equal = 0;
    for (int j = 0; j < gamma; ++j) {
      run = run * clamp_conf(staged[r * gamma + j]);
      const unsigned k = survival_key(run);
      above += k < cut;
      equal += k == cut;
    }
    counts += ((long long)above << 32) | equal;
  }
  long long total;
  long long before = block_exclusive_scan(counts, red_ll, &total);
  // The first K - (all above) equal candidates in (request, position) order are admitted.
  const int take = K < N ? K - (int)(total >> 32) : 0;
  int eq_before = (int)(before & 0xffffffff);
  long long rows = 0;
  for (int r = r0; r < r1; ++r) {
    float run = 1.f;
    int above = 0, equal = 0;
    for (int j = 0; j < gamma; ++j) {
      run = run * clamp_conf(staged[r * gamma + j]);
      const unsigned k = survival_key(run);
      above += k < cut;
      equal += k == cut;
    }
    const int L = K < N ? above + min(equal, max(0, take - eq_before)) : gamma;
    eq_before += equal;
    verify_len[r] = L;
    rows += L + 1;
  }
  long long off = block_exclusive_scan(rows, red_ll, &total);
  for (int r = r0; r < r1; ++r) {
    row_offsets[r] = (int32_t)off;
    off += verify_len[r] + 1;
  }
  if (threadIdx.x == 0) row_offsets[R] = (int32_t)total;
}

}  // namespace

hipError_t launch_schedule(const float *conf, const float *conf_stale, int R, int gamma,
                           const float *sps, int mode, int32_t *verify_len, int32_t *row_offsets,
                           hipStream_t stream) {
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kSchedThreads), 0, stream, conf, conf_stale, R,
                     gamma, sps, mode, verify_len, row_offsets);
  return hipGetLastError();
}

}  // namespace sdv
