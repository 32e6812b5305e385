// C ABI of libgqa: argument validation, workspace sizing and dispatch.
//
// Every check runs on the host before anything is enqueued, and none of them
// touches the HIP runtime, so the error paths can be exercised on a machine
// without a GPU.  See include/gqa.h for the contract of each entry point.
#include "gqa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "launch.hpp"
#include "paged_sched.hpp"
#include "prefill_sched.hpp"
#include "verify_sched.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kSupportedHq = 6;
constexpr int kSupportedHkv = 1;
constexpr int kSupportedD = 256;
constexpr int64_t kMaxBufferBytes = 0xFFFFFFFFll;  // 32-bit buffer offsets

gqa_status check_shape(int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0 || d <= 0) return GQA_ERR_INVALID;
  if (hq != kSupportedHq || hkv != kSupportedHkv || d != kSupportedD) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }

gqa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return GQA_OK;
  g_last_hip_error = (int)e;
  return GQA_ERR_HIP;
}

// Row-major [n][hkv][d] fp16 tensor of n rows fits the 32-bit buffer offsets.
bool rows_fit(int64_t n, int64_t row_bytes) { return n * row_bytes <= kMaxBufferBytes; }

gqa_status prefill_sizes(int32_t nq, int32_t n_kv, int32_t q_pos0, int32_t hq, int32_t hkv, int32_t d) {
  if (nq <= 0 || n_kv <= 0 || q_pos0 < 0) return GQA_ERR_INVALID;
  if ((int64_t)q_pos0 + nq > n_kv) return GQA_ERR_INVALID;
  gqa_status st = check_shape(hq, hkv, d);
  if (st != GQA_OK) return st;
  if (!rows_fit((int64_t)nq * hq, 2 * d) || !rows_fit(n_kv, 2 * d)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;   // created events, reused across sessions
  std::vector<hipEvent_t> marks;  // start/stop pairs of this session
  unsigned long long* clk = nullptr;  // device {cycles, wall ticks}, 16 bytes
  int clk_device = -1;
  double last_mhz = 0.0;              // average shader clock of the last session
};
thread_local Profiler g_prof;

hipEvent_t prof_event() {
  const size_t used = g_prof.marks.size();
  if (used < g_prof.pool.size()) return g_prof.pool[used];
  // timing only: no system-scope fence at record time (no cache write-back
  // and invalidation between the kernels being timed)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  g_prof.pool.push_back(e);
  return e;
}

}  // namespace

namespace gqa {
bool prof_events(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof.on) return false;
  hipEvent_t a = prof_event();
  if (!a) return false;
  g_prof.marks.push_back(a);
  hipEvent_t b = prof_event();
  if (!b) {
    g_prof.marks.pop_back();  // no pair: this launch goes untimed
    return false;
  }
  g_prof.marks.push_back(b);
  *start = a;
  *stop = b;
  return true;
}
unsigned long long* prof_clock() { return g_prof.on ? g_prof.clk : nullptr; }
}  // namespace gqa

extern "C" {

gqa_status gqa_profile_start(void) {
  g_prof.on = true;
  g_prof.marks.clear();
  g_prof.last_mhz = 0.0;
  // the clock accumulator is optional: without it only the times are kept
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess) {
    if (g_prof.clk && g_prof.clk_device != dev) {
      (void)hipFree(g_prof.clk);
      g_prof.clk = nullptr;
    }
    if (!g_prof.clk && hipMalloc((void**)&g_prof.clk, 2 * sizeof(unsigned long long)) == hipSuccess)
      g_prof.clk_device = dev;
    if (g_prof.clk && hipMemset(g_prof.clk, 0, 2 * sizeof(unsigned long long)) != hipSuccess) {
      (void)hipFree(g_prof.clk);
      g_prof.clk = nullptr;
    }
  }
  (void)hipGetLastError();  // a failure above leaves no error behind
  return GQA_OK;
}

gqa_status gqa_profile_stop(double* total_ms, int32_t* count) {
  if (!g_prof.on || !total_ms || !count) return GQA_ERR_INVALID;
  g_prof.on = false;
  double sum = 0.0;
  int32_t n = 0;
  for (size_t i = 0; i + 1 < g_prof.marks.size(); i += 2) {
    hipError_t e = hipEventSynchronize(g_prof.marks[i + 1]);
    if (e != hipSuccess) return hip_status(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_prof.marks[i], g_prof.marks[i + 1]);
    if (e != hipSuccess) return hip_status(e);
    sum += ms;
    ++n;
  }
  g_prof.marks.clear();
  if (g_prof.clk) {
    unsigned long long c[2] = {0, 0};
    int khz = 0;
    if (hipMemcpy(c, g_prof.clk, sizeof(c), hipMemcpyDeviceToHost) == hipSuccess && c[1] > 0 &&
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, g_prof.clk_device) == hipSuccess && khz > 0)
      g_prof.last_mhz = (double)c[0] / (double)c[1] * (double)khz * 1e-3;
    (void)hipGetLastError();
  }
  *total_ms = sum;
  *count = n;
  return GQA_OK;
}

gqa_status gqa_profile_clock_mhz(double* mhz) {
  if (!mhz) return GQA_ERR_INVALID;
  *mhz = g_prof.last_mhz;
  return GQA_OK;
}

const char* gqa_status_string(gqa_status status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID: return "GQA_ERR_INVALID: invalid argument";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: shape outside the supported family";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace smaller than required";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: HIP call failed";
  }
  return "unknown gqa_status";
}

int gqa_last_hip_error(void) { return g_last_hip_error; }

int gqa_abi_version(void) { return GQA_ABI_VERSION; }

// ------------------------------------------------------------ causal prefill
gqa_status gqa_prefill_causal_workspace_size(int32_t nq, int32_t n_kv, int32_t q_pos0, int32_t hq, int32_t hkv,
                                             int32_t d, size_t* bytes) {
  if (!bytes) return GQA_ERR_INVALID;
  gqa_status st = prefill_sizes(nq, n_kv, q_pos0, hq, hkv, d);
  if (st != GQA_OK) return st;
  const size_t w = gqa::prefill_any_workspace_bytes(nq, hq, q_pos0);
  if ((int64_t)w > kMaxBufferBytes) return GQA_ERR_UNSUPPORTED;
  *bytes = w;
  return GQA_OK;
}

gqa_status gqa_prefill_causal(const void* q, const void* k, const void* v, void* o, int32_t nq, int32_t n_kv,
                              int32_t q_pos0, int32_t hq, int32_t hkv, int32_t d, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return GQA_ERR_INVALID;
  if (!good_scale(scale)) return GQA_ERR_INVALID;
  size_t need = 0;
  gqa_status st = gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0, hq, hkv, d, &need);
  if (st != GQA_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need)) return GQA_ERR_WORKSPACE;
  return hip_status(gqa::launch_prefill_causal(q, k, v, o, nq, n_kv, q_pos0, hq, scale, workspace,
                                               (hipStream_t)stream));
}

// ------------------------------------------------------- E4M3 causal prefill
gqa_status gqa_prefill_causal_e4m3(const uint8_t* q_e4m3, float q_scale, const uint8_t* k_e4m3, float k_scale,
                                   const uint8_t* v_e4m3, float v_scale, void* o, int32_t nq, int32_t n_kv,
                                   int32_t q_pos0, int32_t hq, int32_t hkv, int32_t d, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!q_e4m3 || !k_e4m3 || !v_e4m3 || !o) return GQA_ERR_INVALID;
  if (!good_scale(scale) || !good_scale(q_scale) || !good_scale(k_scale) || !good_scale(v_scale))
    return GQA_ERR_INVALID;
  size_t need = 0;
  gqa_status st = gqa_prefill_causal_workspace_size(nq, n_kv, q_pos0, hq, hkv, d, &need);
  if (st != GQA_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need)) return GQA_ERR_WORKSPACE;
  return hip_status(gqa::launch_prefill_causal_e4m3(q_e4m3, q_scale, k_e4m3, k_scale, v_e4m3, v_scale, o, nq, n_kv,
                                                    q_pos0, hq, scale, workspace, (hipStream_t)stream));
}

// ------------------------------------------------------------ varlen prefill
namespace {
constexpr int32_t kMaxBatch = 1 << 20;

gqa_status varlen_sizes(int32_t batch, int32_t total_q, int32_t total_kv, int32_t hq, int32_t hkv, int32_t d) {
  if (batch <= 0 || total_q < 0 || total_kv < 0) return GQA_ERR_INVALID;
  gqa_status st = check_shape(hq, hkv, d);
  if (st != GQA_OK) return st;
  if (batch > kMaxBatch || !rows_fit((int64_t)total_q * hq, 2 * d) || !rows_fit(total_kv, 2 * d))
    return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}
}  // namespace

gqa_status gqa_prefill_causal_varlen_workspace_size(int32_t batch, int32_t total_q, int32_t hq, int32_t hkv,
                                                    int32_t d, size_t* bytes) {
  if (!bytes) return GQA_ERR_INVALID;
  gqa_status st = varlen_sizes(batch, total_q, 0, hq, hkv, d);
  if (st != GQA_OK) return st;
  const size_t w = gqa::prefill_varlen_workspace_bytes(gqa::prefill_varlen_schedule(batch, total_q));
  if ((int64_t)w > kMaxBufferBytes) return GQA_ERR_UNSUPPORTED;
  *bytes = w;
  return GQA_OK;
}

gqa_status gqa_prefill_causal_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                     const int32_t* cu_q, const int32_t* cu_kv, int32_t batch, int32_t total_q,
                                     int32_t total_kv, int32_t hq, int32_t hkv, int32_t d, float scale,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !cu_q || !cu_kv) return GQA_ERR_INVALID;
  if (!good_scale(scale)) return GQA_ERR_INVALID;
  gqa_status st = varlen_sizes(batch, total_q, total_kv, hq, hkv, d);
  if (st != GQA_OK) return st;
  size_t need = 0;
  st = gqa_prefill_causal_varlen_workspace_size(batch, total_q, hq, hkv, d, &need);
  if (st != GQA_OK) return st;
  if (!workspace || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  return hip_status(gqa::launch_prefill_causal_varlen(q, k, v, o, lse, cu_q, cu_kv, batch, total_q, total_kv, scale,
                                                      workspace, (hipStream_t)stream));
}

gqa_status gqa_prefill_causal_varlen_skipped(const void* workspace, int32_t* count, void* stream) {
  if (!workspace || !count) return GQA_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  int32_t hdr[4] = {0, 0, 0, 0};
  hipError_t e = hipMemcpyAsync(hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  *count = hdr[1];
  return GQA_OK;
}

// ------------------------------------------------------- paged block-sparse
namespace {
gqa_status paged_sizes(int32_t nq, int32_t n_block_ids, int32_t qblock_rows, int32_t kv_block_tokens, int32_t hq,
                       int32_t hkv, int32_t d) {
  if (nq <= 0 || n_block_ids < 0 || qblock_rows <= 0 || kv_block_tokens <= 0) return GQA_ERR_INVALID;
  gqa_status st = check_shape(hq, hkv, d);
  if (st != GQA_OK) return st;
  if (qblock_rows != gqa::kQBlockTokens || kv_block_tokens != gqa::kBlockTokens) return GQA_ERR_UNSUPPORTED;
  if (!rows_fit((int64_t)nq * hq, 2 * d) || (int64_t)n_block_ids * 8 > kMaxBufferBytes) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}
}  // namespace

gqa_status gqa_prefill_paged_sparse_workspace_size(int32_t nq, int32_t n_block_ids, int32_t qblock_rows,
                                                   int32_t kv_block_tokens, int32_t hq, int32_t hkv, int32_t d,
                                                   size_t* bytes) {
  if (!bytes) return GQA_ERR_INVALID;
  gqa_status st = paged_sizes(nq, n_block_ids, qblock_rows, kv_block_tokens, hq, hkv, d);
  if (st != GQA_OK) return st;
  const int nqb = (nq + gqa::kQBlockTokens - 1) / gqa::kQBlockTokens;
  const size_t w = gqa::paged_layout(nqb, n_block_ids).total;
  // the partials are addressed with 32-bit offsets from the workspace base
  if ((int64_t)w > kMaxBufferBytes) return GQA_ERR_UNSUPPORTED;
  *bytes = w;
  return GQA_OK;
}

gqa_status gqa_prefill_paged_sparse(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, int32_t n_table, int32_t n_pages, int32_t page_size,
                                    const int32_t* qblock_offsets, const int32_t* kv_block_ids, int32_t n_block_ids,
                                    int32_t qblock_rows, int32_t kv_block_tokens, int32_t nq, int32_t q_pos0,
                                    int32_t live_len, int32_t hq, int32_t hkv, int32_t d, float scale, void* o,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !page_table || !qblock_offsets || !o) return GQA_ERR_INVALID;
  if (n_block_ids > 0 && !kv_block_ids) return GQA_ERR_INVALID;
  if (!good_scale(scale)) return GQA_ERR_INVALID;
  if (n_table <= 0 || n_pages <= 0 || page_size <= 0 || q_pos0 < 0 || live_len <= 0) return GQA_ERR_INVALID;
  size_t need = 0;
  gqa_status st = gqa_prefill_paged_sparse_workspace_size(nq, n_block_ids, qblock_rows, kv_block_tokens, hq, hkv, d,
                                                          &need);
  if (st != GQA_OK) return st;
  if (page_size % gqa::kBlockTokens != 0 || page_size > gqa::kMaxPageSize) return GQA_ERR_UNSUPPORTED;
  if ((int64_t)q_pos0 + nq > live_len || (int64_t)live_len > (int64_t)n_table * page_size) return GQA_ERR_INVALID;
  // logical token positions (block id * 4) are int32 on the device
  if ((int64_t)n_table * page_size > INT32_MAX) return GQA_ERR_UNSUPPORTED;
  // the cache buffer plus the out-of-range marker offset must fit 32 bits
  if ((int64_t)n_pages * page_size * hkv * d * 2 > 0xFFFFFF00ll) return GQA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  return hip_status(gqa::launch_paged_sparse(q, k_cache, v_cache, page_table, n_table, n_pages, page_size, qblock_offsets,
                                             kv_block_ids, n_block_ids, nq, q_pos0, live_len, hq, scale, o, workspace,
                                             (hipStream_t)stream));
}

gqa_status gqa_prefill_paged_sparse_dropped(const void* workspace, int32_t* count, void* stream) {
  if (!workspace || !count) return GQA_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  int32_t hdr[4] = {0, 0, 0, 0};
  hipError_t e = hipMemcpyAsync(hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  if (hdr[0] != gqa::kPagedMagic || hdr[1] < 0) return GQA_ERR_INVALID;
  const gqa::PagedLayout L = gqa::paged_layout(hdr[1], hdr[2]);
  std::vector<int32_t> err((size_t)hdr[1]);
  if (!err.empty()) {
    e = hipMemcpyAsync(err.data(), (const char*)workspace + L.err, err.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e);
  }
  int64_t total = 0;
  for (int32_t x : err) total += x;
  *count = (int32_t)(total > 0x7FFFFFFF ? 0x7FFFFFFF : total);
  return GQA_OK;
}

// ------------------------------------------------------------ FP8 verifier
gqa_status gqa_verify_fp8kv_workspace_size(int32_t nq, int32_t n_kv, int32_t hq, int32_t hkv, int32_t d,
                                           size_t* bytes) {
  if (!bytes) return GQA_ERR_INVALID;
  if (nq <= 0 || n_kv <= 0 || nq > n_kv) return GQA_ERR_INVALID;
  gqa_status st = check_shape(hq, hkv, d);
  if (st != GQA_OK) return st;
  if (nq * hq > gqa::kVerifyMaxRows || n_kv > gqa::kVerifyMaxContext) return GQA_ERR_UNSUPPORTED;
  *bytes = gqa::verify_workspace_bytes(gqa::verify_schedule(nq, n_kv, hq));
  return GQA_OK;
}

gqa_status gqa_verify_fp8kv(const void* q, const uint8_t* k_e4m3, const uint8_t* v_e4m3, float k_scale,
                            float v_scale, void* o, int32_t nq, int32_t n_kv, int32_t hq, int32_t hkv, int32_t d,
                            float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_e4m3 || !v_e4m3 || !o) return GQA_ERR_INVALID;
  if (!good_scale(scale) || !good_scale(k_scale) || !good_scale(v_scale)) return GQA_ERR_INVALID;
  size_t need = 0;
  gqa_status st = gqa_verify_fp8kv_workspace_size(nq, n_kv, hq, hkv, d, &need);
  if (st != GQA_OK) return st;
  if (!workspace || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  return hip_status(gqa::launch_verify_fp8kv(q, k_e4m3, v_e4m3, k_scale, v_scale, o, nq, n_kv, hq, scale, workspace,
                                             (hipStream_t)stream));
}

gqa_status gqa_verify_fp8kv_noalloc(const void* q, const uint8_t* k_e4m3, const uint8_t* v_e4m3, float k_scale,
                                    float v_scale, void* o, int32_t nq, int32_t n_kv, int32_t hq, int32_t hkv,
                                    int32_t d, float scale, void* stream) {
  if (!q || !k_e4m3 || !v_e4m3 || !o) return GQA_ERR_INVALID;
  if (!good_scale(scale) || !good_scale(k_scale) || !good_scale(v_scale)) return GQA_ERR_INVALID;
  size_t need = 0;
  gqa_status st = gqa_verify_fp8kv_workspace_size(nq, n_kv, hq, hkv, d, &need);
  if (st != GQA_OK) return st;
  if (need > gqa::kVerifyScratchBytes) return GQA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  hipError_t e = gqa::verify_scratch(&ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(gqa::launch_verify_fp8kv(q, k_e4m3, v_e4m3, k_scale, v_scale, o, nq, n_kv, hq, scale, ws,
                                             (hipStream_t)stream));
}

}  // extern "C"
