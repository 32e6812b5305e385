// Internal launchers behind the C ABI (one per entry point).  Arguments are
// already validated; each enqueues its kernels on `stream` and returns the
// first launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, void* o, int nq, int n_kv, int q_pos0,
                                 int hq, float scale, void* workspace, hipStream_t stream);

}  // namespace gqa
