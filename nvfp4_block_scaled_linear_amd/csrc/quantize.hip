// NVFP4 quantizer on the device, bit-exact with the rule stated in nvfp4.h: per-row
// tensor scales for W4A4 activations (bloomery issue #565, section 4, PR #687: 4-bit
// activations on the prompt GEMM) and a per-tensor scale for weights (one tensor scale
// per matrix, PR #490). Every step is one correctly rounded fp32 operation in the stated
// order (this file is compiled without fast-math, and the divisions are IEEE divisions),
// and the E4M3 / E2M1 roundings are the bit-level encoders of device.hpp. Non-finite
// inputs set a fault bit (the pages' quantizers refuse them: section 10, PR #597).
#include "device.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

template <int IN>
__device__ __forceinline__ void load16(const void* x, int64_t off, float v[16]) {
  if (IN == 0) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + off);
    const u32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      v[8 + 2 * i] = __uint_as_float(b[i] << 16);
      v[8 + 2 * i + 1] = __uint_as_float(b[i] & 0xFFFF0000u);
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + off);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const u32x4 a = p[q];
#pragma unroll
      for (int i = 0; i < 4; i++) v[4 * q + i] = __uint_as_float(a[i]);
    }
  }
}

// amax of 16 values, and whether all are finite
__device__ __forceinline__ float amax16(const float v[16], bool& finite) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    finite = finite && is_finite(v[i]);
    m = fmaxf(m, __builtin_fabsf(v[i]));
  }
  return m;
}

// one 16-block with tensor scale t -> 8 code bytes + 1 scale byte
__device__ __forceinline__ void quantize_block(const float v[16], float t, uint8_t* codes8,
                                               uint8_t* scale1) {
  uint32_t lo, hi;
  const uint32_t s = quantize16(v, t, lo, hi);
  *reinterpret_cast<uint2*>(codes8) = make_uint2(lo, hi);
  *scale1 = (uint8_t)s;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// One workgroup per row: row amax -> ts[row], then the row's blocks.
template <int IN>
__global__ __launch_bounds__(256) void quantize_rows(const void* x, int64_t ldx, int64_t K,
                                                     uint8_t* codes, uint8_t* scales, float* ts,
                                                     uint32_t* faults) {
  __shared__ float wmax[4];
  __shared__ float ts_sh;
  const int64_t row = blockIdx.x;
  const int64_t nb = K >> 4;
  const int64_t base = row * ldx;
  bool finite = true;
  float m = 0.0f;
  // rows of at most one block per thread (K <= 4096) keep their block in registers for
  // the second pass instead of loading it again
  const bool one = nb <= (int64_t)blockDim.x;  // uniform
  float keep[16];
  if (one) {
    if ((int64_t)threadIdx.x < nb) {
      load16<IN>(x, base + 16 * (int64_t)threadIdx.x, keep);
      m = amax16(keep, finite);
    }
  } else {
    for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
      float v[16];
      load16<IN>(x, base + 16 * b, v);
      m = fmaxf(m, amax16(v, finite));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = wmax[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); w++) r = fmaxf(r, wmax[w]);
    const float t = r / 2688.0f;
    ts_sh = t;
    ts[row] = t;
  }
  __syncthreads();
  const float t = ts_sh;
  if (one) {
    const int64_t b = threadIdx.x;
    if (b < nb) quantize_block(keep, t, codes + row * (K >> 1) + 8 * b, scales + row * nb + b);
  } else {
    for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
      float v[16];
      load16<IN>(x, base + 16 * b, v);
      quantize_block(v, t, codes + row * (K >> 1) + 8 * b, scales + row * nb + b);
    }
  }
  if (!finite && faults) atomicOr(faults, (uint32_t)NVFP4_FAULT_NONFINITE);
}

// Per-tensor form: (1) clear the amax word (ts[0] holds amax bits while the call runs),
// (2) block amax folded in with an unsigned max on the bit pattern (exact for
// non-negative floats, order-independent), (3) ts = amax / 2688, (4) blocks.
__global__ void amax_clear(float* ts) { *reinterpret_cast<uint32_t*>(ts) = 0u; }

template <int IN>
__global__ __launch_bounds__(256) void amax_tensor(const void* x, int64_t ldx, int64_t M,
                                                   int64_t K, float* ts, uint32_t* faults) {
  __shared__ float wmax[4];
  const int64_t nb = K >> 4;
  const int64_t total = M * nb;
  bool finite = true;
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / nb, b = i - row * nb;
    float v[16];
    load16<IN>(x, row * ldx + 16 * b, v);
    m = fmaxf(m, amax16(v, finite));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = wmax[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); w++) r = fmaxf(r, wmax[w]);
    atomicMax(reinterpret_cast<uint32_t*>(ts), __float_as_uint(r));
  }
  if (!finite && faults) atomicOr(faults, (uint32_t)NVFP4_FAULT_NONFINITE);
}

__global__ void ts_finalize(float* ts) {
  const float amax = __uint_as_float(*reinterpret_cast<const uint32_t*>(ts));
  ts[0] = amax / 2688.0f;
}

template <int IN>
__global__ __launch_bounds__(256) void quantize_blocks(const void* x, int64_t ldx, int64_t M,
                                                       int64_t K, uint8_t* codes,
                                                       uint8_t* scales, const float* ts) {
  const int64_t nb = K >> 4;
  const int64_t total = M * nb;
  const float t = ts[0];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / nb, b = i - row * nb;
    float v[16];
    load16<IN>(x, row * ldx + 16 * b, v);
    quantize_block(v, t, codes + row * (K >> 1) + 8 * b, scales + i);
  }
}

template <int IN>
hipError_t launch_in(const void* x, int64_t ldx, int64_t M, int64_t K, int ts_mode,
                     uint8_t* codes, uint8_t* scales, float* ts, uint32_t* faults,
                     hipStream_t stream) {
  if (ts_mode == 0) {
    hipLaunchKernelGGL((quantize_rows<IN>), dim3((uint32_t)M), dim3(256), 0, stream, x, ldx, K,
                       codes, scales, ts, faults);
    return hipGetLastError();
  }
  const int64_t total = M * (K >> 4);
  int64_t grid = (total + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(amax_clear, dim3(1), dim3(1), 0, stream, ts);
  hipLaunchKernelGGL((amax_tensor<IN>), dim3((uint32_t)grid), dim3(256), 0, stream, x, ldx, M,
                     K, ts, faults);
  hipLaunchKernelGGL(ts_finalize, dim3(1), dim3(1), 0, stream, ts);
  hipLaunchKernelGGL((quantize_blocks<IN>), dim3((uint32_t)grid), dim3(256), 0, stream, x, ldx,
                     M, K, codes, scales, ts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int in_type, const void* x, int64_t ldx, int64_t M, int64_t K,
                           int ts_mode, uint8_t* codes, uint8_t* scales, float* ts,
                           uint32_t* faults, hipStream_t stream) {
  return in_type == 0 ? launch_in<0>(x, ldx, M, K, ts_mode, codes, scales, ts, faults, stream)
                      : launch_in<1>(x, ldx, M, K, ts_mode, codes, scales, ts, faults, stream);
}

}  // namespace nvfp4
