// Next-weight prefetch: one streaming read of a buffer whose values are discarded, so that
// the bytes sit in the caches (the MI355X Infinity Cache holds 256 MB) when the next call
// reads them. A caller issues it for layer i + 1's weight on a second stream while layer i
// runs, as the pages prefetch weight rows into L2 ahead of the gemv calls that read them
// (bloomery issue #565, section 4, "Remaining Round 1 items"; and the later rounds' plan
// of an L2 prefetch of the next weights while a gather waits).
//
// The grid is capped (a few workgroups per CU), so the prefetch shares the chip with the
// call it overlaps instead of displacing it; each thread keeps kLoads 16-byte loads in
// flight per trip through a grid-stride loop.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr int kLoads = 8;

__global__ __launch_bounds__(256) void prefetch_kernel(const uint8_t* buf, uint32_t bytes) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), 0, (int)bytes,
                                                   0x00020000);
  const uint32_t stride = gridDim.x * 256u * 16u;  // one trip: every thread's first load
  for (uint32_t o = (blockIdx.x * 256u + threadIdx.x) * 16u; o < bytes; o += kLoads * stride) {
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; u++) {
      // past the end: the descriptor's size bound reads zeros without touching memory
      const uint32_t ou = o + u * stride;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, ou < bytes ? ou : 0x80000000u, 0, 0);
    }
    // the loaded values are only kept live until they arrive
#pragma unroll
    for (int u = 0; u < kLoads; u++) __asm__ volatile("" ::"v"(v[u]));
  }
}

}  // namespace

hipError_t launch_prefetch(const void* buf, int64_t bytes, int workgroups, hipStream_t stream) {
  const int64_t per_wg = (int64_t)kLoads * 256 * 16;
  int64_t g = (bytes + per_wg - 1) / per_wg;
  if (g > workgroups) g = workgroups;
  hipLaunchKernelGGL(prefetch_kernel, dim3((uint32_t)(g < 1 ? 1 : g)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(buf), (uint32_t)bytes);
  return hipGetLastError();
}

}  // namespace nvfp4
