// Measurement support, not part of the NVFP4 layer: a plain streaming read of one buffer
// in one launch. It is the measured single-launch read roof that the weight-streaming
// kernels are compared against (the pages quote their own decode paths against a
// measured local roof next to the nominal one: Rocket engineering log, entry "A GDN
// decode path on GB10 ...", roofline table).
//
// Each workgroup reads a contiguous run of U * 4 KiB: load u of thread i reads bytes
// 4096 u + 16 i of the run, so every load instruction of a workgroup covers 4 KiB of
// whole 128-byte lines. Loads are raw buffer loads (bytes past the end read as zero
// without touching memory). The loaded words are XOR-folded and stored only when the
// fold hits a fixed value, which keeps the loads live and writes next to nothing.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr uint32_t kFoldMark = 0x9E3779B9u;

template <int U>
__global__ __launch_bounds__(256) void read_probe(const uint8_t* buf, uint32_t bytes,
                                                  uint32_t* sink) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), 0, (int)bytes,
                                                   0x00020000);
  const uint32_t base = (uint32_t)blockIdx.x * (4096u * U) + 16u * threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; u++) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + 4096u * u, 0, 0);
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < U; u++) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (x == kFoldMark) sink[0] = x;
}

template <int U>
hipError_t launch_u(const uint8_t* buf, uint32_t bytes, uint32_t* sink, hipStream_t stream) {
  const uint32_t per_wg = 4096u * U;
  hipLaunchKernelGGL((read_probe<U>), dim3((bytes + per_wg - 1) / per_wg), dim3(256), 0, stream,
                     buf, bytes, sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, int loads_per_thread, uint32_t* sink,
                             hipStream_t stream) {
  const auto* b = static_cast<const uint8_t*>(buf);
  const uint32_t n = (uint32_t)bytes;
  switch (loads_per_thread) {
    case 1: return launch_u<1>(b, n, sink, stream);
    case 2: return launch_u<2>(b, n, sink, stream);
    case 4: return launch_u<4>(b, n, sink, stream);
    case 8: return launch_u<8>(b, n, sink, stream);
    case 16: return launch_u<16>(b, n, sink, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4
