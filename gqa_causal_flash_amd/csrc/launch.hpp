// Internal launchers behind the C ABI (one per entry point).  Arguments are
// already validated; each enqueues its kernels on `stream` and returns the
// first launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// Kernel timing hook (see gqa_profile_start): while profiling is on, hands out
// a start/stop event pair for the next main-kernel launch and returns true.
bool prof_events(hipEvent_t* start, hipEvent_t* stop);

// Launches a library kernel; the main attention kernel of each entry point goes
// through here.  While profiling, the launch is bracketed by a pair of events
// recorded on the stream (created without the system-scope fence, so a record
// does not write back and invalidate the caches).
template <class Kernel, class Params>
hipError_t launch_timed(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, const Params& p) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool timed = prof_events(&e0, &e1);
  hipError_t e = timed ? hipEventRecord(e0, stream) : hipSuccess;
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || !timed) return e;
  return hipEventRecord(e1, stream);
}

// Device accumulator {shader clock cycles, wall-clock ticks} that the prefill
// kernel adds its workgroups' lifetimes to while profiling is on, else null.
unsigned long long* prof_clock();

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, void* o, int nq, int n_kv, int q_pos0,
                                 int hq, float scale, void* workspace, hipStream_t stream);

hipError_t launch_prefill_causal_e4m3(const void* q, float q_scale, const void* k, float k_scale, const void* v,
                                      float v_scale, void* o, int nq, int n_kv, int q_pos0, int hq, float scale,
                                      void* workspace, hipStream_t stream);

hipError_t launch_prefill_causal_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int32_t* cu_q, const int32_t* cu_kv, int batch, int total_q,
                                        int total_kv, float scale, void* workspace, hipStream_t stream);

hipError_t launch_paged_sparse(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                               int n_table, int n_pages, int page_size, const int32_t* qblock_offsets,
                               const int32_t* kv_block_ids,
                               int n_block_ids, int nq, int q_pos0, int live_len, int hq, float scale, void* o,
                               void* workspace, hipStream_t stream);

hipError_t launch_verify_fp8kv(const void* q, const uint8_t* k, const uint8_t* v, float k_scale, float v_scale,
                               void* o, int nq, int n_kv, int hq, float scale, void* workspace, hipStream_t stream);

// Device address of the current device's fixed verifier scratch
// (kVerifyScratchBytes), looked up on the first call on each device.
hipError_t verify_scratch(void** ptr);

}  // namespace gqa
