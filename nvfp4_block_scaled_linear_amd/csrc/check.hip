// Check mode of the linear calls (NVFP4_F_CHECK): scans of the operands' data that OR a
// fault bit into the caller's word, enqueued before the product only when the flag is set,
// so the product kernels are the same with and without it. The pages' engine refuses NaN
// E4M3 scale bytes and values that overflow once scaled (bloomery issue #565, section 10
// "Other PRs", PRs #597 and #710).
//
// E4M3FN has one NaN pattern per sign, S.1111.111 (0x7F, 0xFF). For a 32-bit word v,
// ((v & 0x7F7F7F7F) + 0x01010101) & 0x80808080 is non-zero exactly when one of its bytes
// is such a pattern: a byte's low seven bits plus one reach 0x80 only from 0x7F, and no
// byte carries into the next.
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr int kCheckThreads = 256;
constexpr int64_t kCheckMaxBlocks = 2048;

__device__ __forceinline__ uint32_t nan_e4m3_bytes(uint32_t v) {
  return ((v & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

// bytes [0, n) of p, n even, p 2-byte aligned; 16-byte pieces when p and n allow
__global__ __launch_bounds__(kCheckThreads) void scan_scale_bytes(const uint8_t* p, int64_t n,
                                                                  uint32_t* faults) {
  const int64_t tid = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * kCheckThreads;
  uint32_t hit = 0u;
  if (((uintptr_t)p & 15u) == 0 && (n & 15) == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    for (int64_t i = tid; i < (n >> 4); i += nthr) {
      const uint4 v = q[i];
      hit |= nan_e4m3_bytes(v.x) | nan_e4m3_bytes(v.y) | nan_e4m3_bytes(v.z) |
             nan_e4m3_bytes(v.w);
    }
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    for (int64_t i = tid; i < (n >> 1); i += nthr) hit |= nan_e4m3_bytes(q[i]);
  }
  if (hit) atomicOr(faults, (uint32_t)NVFP4_FAULT_NAN_SCALE);
}

// fp32 tensor scales [0, n): NaN or infinite
__global__ __launch_bounds__(kCheckThreads) void scan_tensor_scales(const float* ts, int64_t n,
                                                                    uint32_t* faults) {
  const int64_t tid = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * kCheckThreads;
  bool bad = false;
  for (int64_t i = tid; i < n; i += nthr)
    bad = bad || (__float_as_uint(ts[i]) & 0x7F800000u) == 0x7F800000u;
  if (bad) atomicOr(faults, (uint32_t)NVFP4_FAULT_NAN_SCALE);
}

// BF16 rows [rows][ld], K values each (K even, ld even): NaN or infinite values
__global__ __launch_bounds__(kCheckThreads) void scan_bf16_rows(const uint16_t* x, int64_t ld,
                                                                int64_t rows, int64_t K,
                                                                uint32_t* faults) {
  const int64_t tid = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * kCheckThreads;
  const int64_t pairs = K >> 1;
  uint32_t hit = 0u;
  for (int64_t i = tid; i < rows * pairs; i += nthr) {
    const int64_t r = i / pairs, c = i % pairs;
    const uint32_t v = *reinterpret_cast<const uint32_t*>(x + r * ld + 2 * c);
    hit |= ((v & 0x7F80u) == 0x7F80u) | ((v & 0x7F800000u) == 0x7F800000u);
  }
  if (hit) atomicOr(faults, (uint32_t)NVFP4_FAULT_NONFINITE);
}

uint32_t check_blocks(int64_t items) {
  const int64_t b = (items + kCheckThreads - 1) / kCheckThreads;
  return (uint32_t)(b < 1 ? 1 : (b > kCheckMaxBlocks ? kCheckMaxBlocks : b));
}

}  // namespace

hipError_t launch_check_scales(const uint8_t* scales, int64_t bytes, const float* ts,
                               int64_t n_ts, uint32_t* faults, hipStream_t stream) {
  if (bytes > 0) {
    hipLaunchKernelGGL(scan_scale_bytes, dim3(check_blocks(bytes / 16 + 1)), dim3(kCheckThreads),
                       0, stream, scales, bytes, faults);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_ts > 0) {
    hipLaunchKernelGGL(scan_tensor_scales, dim3(check_blocks(n_ts)), dim3(kCheckThreads), 0,
                       stream, ts, n_ts, faults);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_check_bf16(const void* x, int64_t ld, int64_t rows, int64_t K,
                             uint32_t* faults, hipStream_t stream) {
  hipLaunchKernelGGL(scan_bf16_rows, dim3(check_blocks(rows * (K / 2) / 4 + 1)),
                     dim3(kCheckThreads), 0, stream, static_cast<const uint16_t*>(x), ld, rows,
                     K, faults);
  return hipGetLastError();
}

}  // namespace nvfp4
