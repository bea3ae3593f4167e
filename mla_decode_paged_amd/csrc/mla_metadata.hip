// mla_get_metadata: the split-KV work plan (mla_plan.h) by one workgroup of
// 1024 threads.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_host.h"
#include "mla_plan.h"

namespace mla {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void mla_metadata_kernel(const int32_t* seqlens, int b, int n_slots,
                                                                    int F, int32_t* meta, int32_t* ns_out) {
  __shared__ int C[MLA_MAX_BATCH + 1];   // cost-line start of each sequence; C[b] = total
  __shared__ int NS[MLA_MAX_BATCH + 1];  // split prefix
  __shared__ int wave_sums[kPlanThreads / 64 + 1];
  plan_block<kPlanThreads>(seqlens, b, n_slots, F, meta, ns_out, C, NS, wave_sums);
}

}  // namespace mla

extern "C" int mla_get_metadata(const int32_t* cache_seqlens, int b, int num_slots, int split_overhead,
                                int32_t* tile_meta, int32_t* num_splits, void* stream) {
  const char* fn = "mla_get_metadata";
  if (int rc = mla::check_plan_args(fn, cache_seqlens, b, num_slots, split_overhead, tile_meta, num_splits))
    return rc;
  hipLaunchKernelGGL(mla::mla_metadata_kernel, dim3(1), dim3(mla::kPlanThreads), 0,
                     static_cast<hipStream_t>(stream), cache_seqlens, b, num_slots, split_overhead, tile_meta,
                     num_splits);
  if (hipError_t e = hipGetLastError(); e != hipSuccess)
    return mla::set_error(MLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return mla::clear_error();
}

extern "C" const char* mla_last_error(void) { return mla::error_buffer(); }
