// C ABI of libgqa: argument validation, workspace sizing and dispatch.
//
// Every check runs on the host before anything is enqueued, and none of them
// touches the HIP runtime, so the error paths can be exercised on a machine
// without a GPU.  See include/gqa.h for the contract of each entry point.
#include "gqa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.hpp"
#include "prefill_sched.hpp"

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

}  // namespace

extern "C" {

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
  const gqa::PrefillSched s = gqa::prefill_schedule(nq, hq, q_pos0);
  const size_t w = gqa::prefill_workspace_bytes(s);
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

}  // extern "C"
