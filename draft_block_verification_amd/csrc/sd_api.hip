// C ABI of libsdverify: argument validation, workspace layout and kernel dispatch.
// Every check that can be made on the host runs before any GPU work is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include "sd_launch.h"

using namespace sdv;

// Scratch of sd_verify_greedy_noalloc: the verify workspace for callers that cannot
// allocate. One copy per GPU, at its own address on each; host code uses only the
// address looked up per device (scratch_address), never this name.
static __device__ __align__(256) uint8_t scratch[SD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int32_t kAbiVersion = 2;
constexpr int kMaxGamma = 64;        // one wavefront of draft positions per request
constexpr int kMaxVocab = 1 << 21;   // bound of the sampler's per-row tile table

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t check_sizes(int32_t B, int32_t gamma, int32_t d, int32_t V) {
  if (B < 1 || gamma < 1 || gamma > kMaxGamma || d < 8 || (d % 8) != 0 || V < 1 ||
      V > kMaxVocab)
    return SD_ESHAPE;
  // Row capacity, logits and partial arrays must stay addressable.
  const int64_t cap = (int64_t)B * (gamma + 1);
  if (cap > (int64_t)1 << 30 || cap * (int64_t)V > ((int64_t)1 << 46) ||
      (int64_t)V * d > ((int64_t)1 << 46))
    return SD_ESHAPE;
  return SD_OK;
}

size_t verify_ws_bytes(int32_t B, int32_t gamma, int32_t V) {
  return verify_workspace_layout(B, gamma, V, nullptr, nullptr, nullptr);
}

size_t accept_ws_bytes(int32_t B, int32_t gamma, int32_t V) {
  return accept_workspace_layout(B, gamma, V, nullptr);
}

int32_t launch_status(hipError_t e) { return e == hipSuccess ? SD_OK : SD_EDEVICE; }

// Clears n 32-bit words with a kernel (no memset node, so it is safe under graph capture).
__global__ void k_clear_words(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t clear_words(void *p, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_words, dim3((n + 63) / 64), dim3(64), 0, s,
                     reinterpret_cast<uint32_t *>(p), n);
  return hipGetLastError();
}

__global__ void k_copy_word(const uint32_t *src, uint32_t *dst) { *dst = *src; }

// Sets the publication area after a verify workspace's header to kPubEmpty words.
__global__ void k_fill_pub(unsigned long long *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = kPubEmpty;
}

// A new workspace's header cleared and, when it is large enough to hold one, its
// publication area emptied.
hipError_t init_workspace(void *ws, size_t bytes, hipStream_t s) {
  hipError_t e = clear_words(ws, sizeof(WsHeader) / 4, s);
  if (e != hipSuccess || bytes < sizeof(WsHeader) + kPubBytes) return e;
  const int n = 2 * kPubWords;
  hipLaunchKernelGGL(k_fill_pub, dim3((n + 255) / 256), dim3(256), 0, s,
                     reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(ws) + sizeof(WsHeader)), n);
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up on the first call made
// with that device current and kept for the process.
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// The first lookup on a device also prepares the scratch as sd_workspace_init prepares
// a workspace (enqueued on s); the address is kept only once that is enqueued.
hipError_t scratch_address(void **out, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    e = init_workspace(p, SD_NOALLOC_SCRATCH_BYTES, s);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t sd_abi_version(void) { return kAbiVersion; }

const char *sd_status_string(int32_t status) {
  switch (status) {
    case SD_OK: return "ok";
    case SD_EINVAL: return "invalid argument (null pointer, temperature or threshold)";
    case SD_ESHAPE: return "invalid sizes (B, gamma, d or V)";
    case SD_EALIGN: return "misaligned tensor pointer";
    case SD_EWORKSPACE: return "workspace missing or too small";
    case SD_EDEVICE: return "HIP launch or copy failed";
    case SD_ESCRATCH: return "problem exceeds the allocation-free scratch (SD_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t sd_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t d, int32_t V) {
  if (check_sizes(B, gamma, d, V) != SD_OK) return 0;
  return verify_ws_bytes(B, gamma, V);
}

size_t sd_accept_workspace_bytes(int32_t B, int32_t gamma, int32_t V) {
  if (check_sizes(B, gamma, 8, V) != SD_OK) return 0;
  return accept_ws_bytes(B, gamma, V);
}

int32_t sd_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
  if (!workspace || workspace_bytes < sizeof(WsHeader)) return SD_EWORKSPACE;
  if (!aligned(workspace, 256)) return SD_EALIGN;
  return launch_status(init_workspace(workspace, workspace_bytes, (hipStream_t)stream));
}

int32_t sd_device_flags(void *workspace, void *stream, uint32_t *flags, int32_t clear) {
  if (!workspace || !flags) return SD_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return SD_EDEVICE;
  uint32_t v = 0;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return SD_EDEVICE;
  *flags = v;
  if (clear) {
    if (clear_words(workspace, 1, s) != hipSuccess) return SD_EDEVICE;
    if (hipStreamSynchronize(s) != hipSuccess) return SD_EDEVICE;
  }
  return SD_OK;
}

int32_t sd_truncate_by_confidence(const float *conf, int32_t B, int32_t gamma, float threshold,
                                  int32_t *verify_len, int32_t *row_offsets, void *stream) {
  if (!conf || !verify_len || !row_offsets) return SD_EINVAL;
  if (!isfinite(threshold)) return SD_EINVAL;
  if (check_sizes(B, gamma, 8, 1) != SD_OK) return SD_ESHAPE;
  if (!aligned(conf, 4) || !aligned(verify_len, 4) || !aligned(row_offsets, 4)) return SD_EALIGN;
  return launch_status(launch_truncate(conf, B, gamma, threshold, verify_len, row_offsets,
                                       (hipStream_t)stream));
}

int32_t sd_schedule_prefix(const float *conf, const float *conf_stale, int32_t R, int32_t gamma,
                           const float *sps, int32_t n_sps, int32_t mode, int32_t *verify_len,
                           int32_t *row_offsets, void *stream) {
  static_assert(kSchedMaxCandidates == SD_SCHED_MAX_CANDIDATES, "candidate bound");
  if (!conf || !sps || !verify_len || !row_offsets) return SD_EINVAL;
  if (mode != SD_SCHED_EARLY_STOP && mode != SD_SCHED_TOP_K) return SD_EINVAL;
  if (mode == SD_SCHED_EARLY_STOP && conf_stale) return SD_EINVAL;
  if (R < 1 || gamma < 1 || gamma > kMaxGamma) return SD_ESHAPE;
  if ((int64_t)R * gamma > kSchedMaxCandidates) return SD_ESHAPE;
  if ((int64_t)n_sps < (int64_t)R * (gamma + 1) + 1) return SD_ESHAPE;
  if (!aligned(conf, 4) || !aligned(sps, 4) || !aligned(verify_len, 4) ||
      !aligned(row_offsets, 4) || (conf_stale && !aligned(conf_stale, 4)))
    return SD_EALIGN;
  return launch_status(launch_schedule(conf, conf_stale, R, gamma, sps, mode, verify_len,
                                       row_offsets, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Shared validation and argument set-up of the verify calls.
int32_t verify_setup(const uint16_t *hidden, const uint16_t *lm_head, const sd_w12 *w12,
                     bool blocked, const int32_t *draft_tokens, const int32_t *verify_len,
                     const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d, int32_t V,
                     float temperature, float *logits, sd_row_stats *stats, bool need_stats,
                     void *workspace, size_t workspace_bytes, VerifyArgs *out) {
  if (!hidden || (!lm_head && !w12) || (need_stats && !stats)) return SD_EINVAL;
  if (w12) {
    if (!w12->codes || !w12->corr) return SD_EINVAL;
    if (w12->b2 < 1 || w12->b2 > 121) return SD_EINVAL;
    // The W12 stream is read by the skinny contraction only.
    if (d % 128 != 0 || (int64_t)B * (gamma + 1) > 64 || w12->cap < 4 || w12->cap % 4 != 0 ||
        w12->cap > kW12MaxCap)
      return SD_ESHAPE;
    if (!aligned(w12->codes, 16) || !aligned(w12->corr, 16)) return SD_EALIGN;
  }
  // The blocked bf16 LM head, like W12, is read by the skinny contraction only.
  if (blocked && (d % 128 != 0 || (int64_t)B * (gamma + 1) > 64)) return SD_ESHAPE;
  if ((verify_len == nullptr) != (row_offsets == nullptr)) return SD_EINVAL;
  if (!isfinite(temperature) || temperature < 0.f) return SD_EINVAL;
  const int32_t sz = check_sizes(B, gamma, d, V);
  if (sz != SD_OK) return sz;
  if (!aligned(hidden, 16) || (lm_head && !aligned(lm_head, 16)) || (stats && !aligned(stats, 8)) ||
      (logits && !aligned(logits, 16)) || (draft_tokens && !aligned(draft_tokens, 4)) ||
      (verify_len && (!aligned(verify_len, 4) || !aligned(row_offsets, 4))))
    return SD_EALIGN;
  if (!workspace || workspace_bytes < verify_ws_bytes(B, gamma, V)) return SD_EWORKSPACE;
  if (!aligned(workspace, 256)) return SD_EALIGN;
  size_t part_off = 0, zx_off = 0;
  int part_stride = 0;
  verify_workspace_layout(B, gamma, V, &part_off, &part_stride, &zx_off);
  char *wsb = reinterpret_cast<char *>(workspace);
  *out = VerifyArgs{};
  VerifyArgs &a = *out;
  a.hidden = hidden;
  a.W = w12 ? nullptr : lm_head;
  a.w_blocked = blocked;
  a.w12_codes = w12 ? w12->codes : nullptr;
  a.w12_corr = w12 ? w12->corr : nullptr;
  a.w12_cap = w12 ? w12->cap : 0;
  a.w12_lut0 = a.w12_lut1 = 0u;
  if (w12) {
    // High byte of code t (sign clear): 0 for t = 0, b2 + t - 1 otherwise.
    for (int t = 1; t < 8; ++t) {
      const uint32_t hb = (uint32_t)(w12->b2 + t - 1) << (8 * (t & 3));
      if (t < 4) a.w12_lut0 |= hb; else a.w12_lut1 |= hb;
    }
  }
  a.draft_tokens = draft_tokens;
  a.verify_len = verify_len;
  a.rm = RowMap{row_offsets, B, gamma};
  a.d = d;
  a.V = V;
  a.temperature = temperature;
  a.scale_log2 = temperature > 0.f ? (float)(1.4426950408889634 / (double)temperature) : 0.f;
  a.invT = temperature > 0.f ? 1.0 / (double)temperature : 0.0;
  a.logits = logits;
  a.partials = reinterpret_cast<TilePartial *>(wsb + part_off);
  a.part_stride = part_stride;
  a.zx = reinterpret_cast<double *>(wsb + zx_off);
  a.stats = stats;
  a.ws = reinterpret_cast<WsHeader *>(workspace);
  return SD_OK;
}

// The three verify calls for any LM-head form: bf16 [V][d] (lm_head), W12 (w12) or the
// blocked bf16 copy (lm_head with blocked).
int32_t verify_logits_impl(const uint16_t *hidden, const uint16_t *lm_head, const sd_w12 *w12,
                           bool blocked, const int32_t *draft_tokens, const int32_t *verify_len,
                           const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                           int32_t V, float temperature, float *logits, sd_row_stats *stats,
                           void *workspace, size_t workspace_bytes, void *stream) {
  VerifyArgs a;
  const int32_t st = verify_setup(hidden, lm_head, w12, blocked, draft_tokens, verify_len,
                                  row_offsets, B, gamma, d, V, temperature, logits, stats, true,
                                  workspace, workspace_bytes, &a);
  if (st != SD_OK) return st;
  return launch_status(launch_verify(a, (hipStream_t)stream));
}

int32_t verify_contraction_impl(const uint16_t *hidden, const uint16_t *lm_head,
                                const sd_w12 *w12, bool blocked, const int32_t *verify_len,
                                const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                                int32_t V, float temperature, float *logits, void *workspace,
                                size_t workspace_bytes, void *stream) {
  VerifyArgs a;
  const int32_t st = verify_setup(hidden, lm_head, w12, blocked, nullptr, verify_len, row_offsets,
                                  B, gamma, d, V, temperature, logits, nullptr, false, workspace,
                                  workspace_bytes, &a);
  if (st != SD_OK) return st;
  int n_part = 0;
  bool zx_done = false;
  return launch_status(launch_contraction(a, (hipStream_t)stream, &n_part, &zx_done));
}

int32_t verify_greedy_impl(const uint16_t *hidden, const uint16_t *lm_head, const sd_w12 *w12,
                           bool blocked, const int32_t *draft_tokens, const int32_t *verify_len,
                           const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                           int32_t V, sd_row_stats *stats, int32_t *accept_len,
                           int32_t *next_token, int64_t *counters, void *workspace,
                           size_t workspace_bytes, void *stream) {
  if (!draft_tokens || !accept_len || !next_token) return SD_EINVAL;
  if (!aligned(accept_len, 4) || !aligned(next_token, 4) || (counters && !aligned(counters, 8)))
    return SD_EALIGN;
  VerifyArgs a;
  const int32_t st = verify_setup(hidden, lm_head, w12, blocked, draft_tokens, verify_len,
                                  row_offsets, B, gamma, d, V, 0.f, nullptr, stats, true,
                                  workspace, workspace_bytes, &a);
  if (st != SD_OK) return st;
  return launch_status(launch_verify_greedy(a, accept_len, next_token, counters,
                                            (hipStream_t)stream));
}

// Bytes of the blocked copy of a [V][d] LM head: ceil(V/64) * (d/128) blocks of 16 KB.
size_t blocked_bytes(int32_t V, int32_t d) {
  return (size_t)((V + 63) / 64) * (size_t)(d / 128) * 16384u;
}

}  // namespace

extern "C" {

int32_t sd_verify_logits(const uint16_t *hidden, const uint16_t *lm_head,
                         const int32_t *draft_tokens, const int32_t *verify_len,
                         const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                         int32_t V, float temperature, float *logits, sd_row_stats *stats,
                         void *workspace, size_t workspace_bytes, void *stream) {
  return verify_logits_impl(hidden, lm_head, nullptr, false, draft_tokens, verify_len,
                            row_offsets, B, gamma, d, V, temperature, logits, stats, workspace,
                            workspace_bytes, stream);
}

int32_t sd_verify_contraction(const uint16_t *hidden, const uint16_t *lm_head,
                              const int32_t *verify_len, const int32_t *row_offsets, int32_t B,
                              int32_t gamma, int32_t d, int32_t V, float temperature,
                              float *logits, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return verify_contraction_impl(hidden, lm_head, nullptr, false, verify_len, row_offsets, B,
                                 gamma, d, V, temperature, logits, workspace, workspace_bytes,
                                 stream);
}

int32_t sd_verify_greedy(const uint16_t *hidden, const uint16_t *lm_head,
                         const int32_t *draft_tokens, const int32_t *verify_len,
                         const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                         int32_t V, sd_row_stats *stats, int32_t *accept_len,
                         int32_t *next_token, int64_t *counters, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return verify_greedy_impl(hidden, lm_head, nullptr, false, draft_tokens, verify_len,
                            row_offsets, B, gamma, d, V, stats, accept_len, next_token, counters,
                            workspace, workspace_bytes, stream);
}

int32_t sd_verify_greedy_noalloc(const uint16_t *hidden, const uint16_t *lm_head,
                                 const int32_t *draft_tokens, const int32_t *verify_len,
                                 const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                                 int32_t V, sd_row_stats *stats, int32_t *accept_len,
                                 int32_t *next_token, int64_t *counters, uint32_t *flags,
                                 void *stream) {
  // Every host check before the scratch lookup, so bad arguments never touch the runtime.
  if (!lm_head || !draft_tokens || !accept_len || !next_token) return SD_EINVAL;
  const int32_t sz = check_sizes(B, gamma, d, V);
  if (sz != SD_OK) return sz;
  if (verify_ws_bytes(B, gamma, V) > SD_NOALLOC_SCRATCH_BYTES) return SD_ESCRATCH;
  if (!aligned(accept_len, 4) || !aligned(next_token, 4) || (counters && !aligned(counters, 8)) ||
      (flags && !aligned(flags, 4)))
    return SD_EALIGN;
  VerifyArgs a;
  // The setup checks run against a stand-in workspace address (never dereferenced on the
  // host); the real scratch address replaces it below.
  void *const probe = reinterpret_cast<void *>((uintptr_t)1 << 12);
  int32_t st = verify_setup(hidden, lm_head, nullptr, false, draft_tokens, verify_len, row_offsets,
                            B, gamma, d, V, 0.f, nullptr, stats, true, probe,
                            SD_NOALLOC_SCRATCH_BYTES, &a);
  if (st != SD_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  void *ws = nullptr;
  if (scratch_address(&ws, s) != hipSuccess) return SD_EDEVICE;
  st = verify_setup(hidden, lm_head, nullptr, false, draft_tokens, verify_len, row_offsets, B,
                    gamma, d, V, 0.f, nullptr, stats, true, ws, SD_NOALLOC_SCRATCH_BYTES, &a);
  if (st != SD_OK) return st;
  // The flag word starts every call at zero. The rest of the header and the publication
  // area carry over from the previous call, as in a workspace; partials and drafted-token
  // logits are written in full by the contraction before they are read.
  if (clear_words(ws, 1, s) != hipSuccess) return SD_EDEVICE;
  hipError_t e = launch_verify_greedy(a, accept_len, next_token, counters, s);
  if (e == hipSuccess && flags) {
    hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(1), 0, s, reinterpret_cast<const uint32_t *>(ws),
                       flags);
    e = hipGetLastError();
  }
  return launch_status(e);
}

int32_t sd_verify_logits_w12(const uint16_t *hidden, const sd_w12 *lm_head,
                             const int32_t *draft_tokens, const int32_t *verify_len,
                             const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                             int32_t V, float temperature, float *logits, sd_row_stats *stats,
                             void *workspace, size_t workspace_bytes, void *stream) {
  if (!lm_head) return SD_EINVAL;
  return verify_logits_impl(hidden, nullptr, lm_head, false, draft_tokens, verify_len,
                            row_offsets, B, gamma, d, V, temperature, logits, stats, workspace,
                            workspace_bytes, stream);
}

int32_t sd_verify_contraction_w12(const uint16_t *hidden, const sd_w12 *lm_head,
                                  const int32_t *verify_len, const int32_t *row_offsets, int32_t B,
                                  int32_t gamma, int32_t d, int32_t V, float temperature,
                                  float *logits, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  if (!lm_head) return SD_EINVAL;
  return verify_contraction_impl(hidden, nullptr, lm_head, false, verify_len, row_offsets, B,
                                 gamma, d, V, temperature, logits, workspace, workspace_bytes,
                                 stream);
}

int32_t sd_verify_greedy_w12(const uint16_t *hidden, const sd_w12 *lm_head,
                             const int32_t *draft_tokens, const int32_t *verify_len,
                             const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                             int32_t V, sd_row_stats *stats, int32_t *accept_len,
                             int32_t *next_token, int64_t *counters, void *workspace,
                             size_t workspace_bytes, void *stream) {
  if (!lm_head) return SD_EINVAL;
  return verify_greedy_impl(hidden, nullptr, lm_head, false, draft_tokens, verify_len,
                            row_offsets, B, gamma, d, V, stats, accept_len, next_token, counters,
                            workspace, workspace_bytes, stream);
}

size_t sd_lm_head_block_bytes(int32_t V, int32_t d) {
  if (V < 1 || d < 128 || d % 128 != 0) return 0;
  return blocked_bytes(V, d);
}

int32_t sd_lm_head_block(const uint16_t *lm_head, int32_t V, int32_t d, uint16_t *blocked,
                         size_t blocked_bytes_given, void *stream) {
  if (!lm_head || !blocked) return SD_EINVAL;
  if (V < 1 || d < 128 || d % 128 != 0) return SD_ESHAPE;
  if (!aligned(lm_head, 16) || !aligned(blocked, 16)) return SD_EALIGN;
  if (blocked_bytes_given < blocked_bytes(V, d)) return SD_EWORKSPACE;
  return launch_status(launch_block_lm_head(lm_head, V, d, blocked, (hipStream_t)stream));
}

int32_t sd_verify_logits_blocked(const uint16_t *hidden, const uint16_t *lm_head_blocked,
                                 const int32_t *draft_tokens, const int32_t *verify_len,
                                 const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                                 int32_t V, float temperature, float *logits,
                                 sd_row_stats *stats, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  return verify_logits_impl(hidden, lm_head_blocked, nullptr, true, draft_tokens, verify_len,
                            row_offsets, B, gamma, d, V, temperature, logits, stats, workspace,
                            workspace_bytes, stream);
}

int32_t sd_verify_contraction_blocked(const uint16_t *hidden, const uint16_t *lm_head_blocked,
                                      const int32_t *verify_len, const int32_t *row_offsets,
                                      int32_t B, int32_t gamma, int32_t d, int32_t V,
                                      float temperature, float *logits, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  return verify_contraction_impl(hidden, lm_head_blocked, nullptr, true, verify_len, row_offsets,
                                 B, gamma, d, V, temperature, logits, workspace, workspace_bytes,
                                 stream);
}

int32_t sd_verify_greedy_blocked(const uint16_t *hidden, const uint16_t *lm_head_blocked,
                                 const int32_t *draft_tokens, const int32_t *verify_len,
                                 const int32_t *row_offsets, int32_t B, int32_t gamma, int32_t d,
                                 int32_t V, sd_row_stats *stats, int32_t *accept_len,
                                 int32_t *next_token, int64_t *counters, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  return verify_greedy_impl(hidden, lm_head_blocked, nullptr, true, draft_tokens, verify_len,
                            row_offsets, B, gamma, d, V, stats, accept_len, next_token, counters,
                            workspace, workspace_bytes, stream);
}

int32_t sd_accept_greedy(const sd_row_stats *stats, const int32_t *draft_tokens,
                         const int32_t *verify_len, const int32_t *row_offsets, int32_t B,
                         int32_t gamma, int32_t *accept_len, int32_t *next_token,
                         int64_t *counters, void *stream) {
  if (!stats || !draft_tokens || !accept_len || !next_token) return SD_EINVAL;
  if ((verify_len == nullptr) != (row_offsets == nullptr)) return SD_EINVAL;
  if (check_sizes(B, gamma, 8, 1) != SD_OK) return SD_ESHAPE;
  if (!aligned(stats, 8) || !aligned(draft_tokens, 4) || !aligned(accept_len, 4) ||
      !aligned(next_token, 4) || (counters && !aligned(counters, 8)) ||
      (verify_len && (!aligned(verify_len, 4) || !aligned(row_offsets, 4))))
    return SD_EALIGN;
  RowMap rm{row_offsets, B, gamma};
  return launch_status(launch_accept_greedy(stats, draft_tokens, verify_len, rm, accept_len,
                                            next_token, counters, (hipStream_t)stream));
}

int32_t sd_accept_rejection(const float *logits, const sd_row_stats *stats,
                            const uint16_t *draft_logits, const int32_t *draft_tokens,
                            const int32_t *verify_len, const int32_t *row_offsets,
                            const float *u_accept, const float *u_resample, int32_t B,
                            int32_t gamma, int32_t V, float temperature, int32_t *accept_len,
                            int32_t *next_token, int64_t *counters, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return sd_accept_rejection_ex(logits, stats, draft_logits, draft_tokens, verify_len,
                                row_offsets, u_accept, u_resample, B, gamma, V, temperature,
                                accept_len, next_token, counters, nullptr, workspace,
                                workspace_bytes, stream);
}

int32_t sd_accept_rejection_ex(const float *logits, const sd_row_stats *stats,
                               const uint16_t *draft_logits, const int32_t *draft_tokens,
                               const int32_t *verify_len, const int32_t *row_offsets,
                               const float *u_accept, const float *u_resample, int32_t B,
                               int32_t gamma, int32_t V, float temperature, int32_t *accept_len,
                               int32_t *next_token, int64_t *counters, double *accept_rate,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (!logits || !stats || !draft_logits || !draft_tokens || !u_accept || !u_resample ||
      !accept_len || !next_token)
    return SD_EINVAL;
  if ((verify_len == nullptr) != (row_offsets == nullptr)) return SD_EINVAL;
  if (!isfinite(temperature) || !(temperature > 0.f)) return SD_EINVAL;
  if (check_sizes(B, gamma, 8, V) != SD_OK) return SD_ESHAPE;
  if (!aligned(logits, 16) || !aligned(stats, 8) || !aligned(draft_logits, 16) ||
      !aligned(draft_tokens, 4) || !aligned(u_accept, 4) || !aligned(u_resample, 4) ||
      !aligned(accept_len, 4) || !aligned(next_token, 4) || (counters && !aligned(counters, 8)) ||
      (accept_rate && !aligned(accept_rate, 8)) ||
      (verify_len && (!aligned(verify_len, 4) || !aligned(row_offsets, 4))))
    return SD_EALIGN;
  if (!workspace || workspace_bytes < accept_ws_bytes(B, gamma, V)) return SD_EWORKSPACE;
  if (!aligned(workspace, 256)) return SD_EALIGN;
  RowMap rm{row_offsets, B, gamma};
  return launch_status(launch_accept_rejection(logits, stats, draft_logits, draft_tokens,
                                               verify_len, rm, u_accept, u_resample, V,
                                               temperature, accept_len, next_token, counters,
                                               accept_rate, workspace, (hipStream_t)stream));
}


int32_t sd_verify_rejection(const uint16_t *hidden, const void *lm_head,
                            int32_t lm_head_layout, const uint16_t *draft_logits,
                            const int32_t *draft_tokens, const int32_t *verify_len,
                            const int32_t *row_offsets, const float *u_accept,
                            const float *u_resample, int32_t B, int32_t gamma, int32_t d,
                            int32_t V, float temperature, float *logits, sd_row_stats *stats,
                            int32_t *accept_len, int32_t *next_token, int64_t *counters,
                            double *accept_rate, void *verify_workspace,
                            size_t verify_workspace_bytes, void *accept_workspace,
                            size_t accept_workspace_bytes, void *stream) {
  if (lm_head_layout != SD_LM_HEAD_ROWS && lm_head_layout != SD_LM_HEAD_BLOCKED &&
      lm_head_layout != SD_LM_HEAD_W12)
    return SD_EINVAL;
  if (!lm_head || !logits || !stats || !draft_logits || !draft_tokens || !u_accept ||
      !u_resample || !accept_len || !next_token)
    return SD_EINVAL;
  if (!isfinite(temperature) || !(temperature > 0.f)) return SD_EINVAL;
  const bool w12 = lm_head_layout == SD_LM_HEAD_W12;
  VerifyArgs a;
  const int32_t st = verify_setup(
      hidden, w12 ? nullptr : static_cast<const uint16_t *>(lm_head),
      w12 ? static_cast<const sd_w12 *>(lm_head) : nullptr, lm_head_layout == SD_LM_HEAD_BLOCKED,
      draft_tokens, verify_len, row_offsets, B, gamma, d, V, temperature, logits, stats, true,
      verify_workspace, verify_workspace_bytes, &a);
  if (st != SD_OK) return st;
  if (!aligned(draft_logits, 16) || !aligned(u_accept, 4) || !aligned(u_resample, 4) ||
      !aligned(accept_len, 4) || !aligned(next_token, 4) || (counters && !aligned(counters, 8)) ||
      (accept_rate && !aligned(accept_rate, 8)))
    return SD_EALIGN;
  if (!accept_workspace || accept_workspace_bytes < accept_ws_bytes(B, gamma, V))
    return SD_EWORKSPACE;
  if (!aligned(accept_workspace, 256)) return SD_EALIGN;
  a.draft_logits = draft_logits;
  return launch_status(launch_verify_rejection(a, u_accept, u_resample, accept_len, next_token,
                                               counters, accept_rate, accept_workspace,
                                               (hipStream_t)stream));
}

}  // extern "C"
