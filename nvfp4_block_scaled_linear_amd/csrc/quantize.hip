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

// Per-row form. Workgroup (row, c) takes 16-blocks 64c + [0, 64) of its row, and further
// runs of 64 blocks C apart for C workgroups per row (C is chosen so that small batches
// spread each row over several workgroups and large ones keep one per row): it first
// finds the amax of the whole row (each of the row's workgroups reads the row, which
// stays in L2) and so ts[row] = amax / 2688, then quantizes its blocks with four lanes per
// block, four values per lane: the block amax over the four lanes (max is exact in any
// order), the block scale and divisor computed alike in the four lanes, and each lane's
// four quotients and codes. Every value is the one quantize16 computes.
constexpr int kRowChunkBlocks = 64;  // 16-blocks per workgroup: 4 lanes per block, 256 threads

template <int IN>
__device__ __forceinline__ void load4(const void* x, int64_t off, float v[4]) {
  if (IN == 0) {
    const uint2 a = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + off);
    v[0] = __uint_as_float(a.x << 16);
    v[1] = __uint_as_float(a.x & 0xFFFF0000u);
    v[2] = __uint_as_float(a.y << 16);
    v[3] = __uint_as_float(a.y & 0xFFFF0000u);
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = __uint_as_float(a[i]);
  }
}

template <int IN>
__global__ __launch_bounds__(256) void quantize_rows(const void* x, int64_t ldx, int64_t K,
                                                     uint8_t* codes, uint8_t* scales, float* ts,
                                                     uint32_t* faults) {
  __shared__ float wmax[4];
  const int64_t row = blockIdx.x;
  const int64_t nb = K >> 4;
  const int64_t base = row * ldx;
  // (1) the row's amax and finiteness
  bool finite = true;
  float m = 0.0f;
  for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
    float v[16];
    load16<IN>(x, base + 16 * b, v);
    m = fmaxf(m, amax16(v, finite));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float t = amax / 2688.0f;
  if (blockIdx.y == 0) {
    if (threadIdx.x == 0) ts[row] = t;
    if (!finite && faults) atomicOr(faults, (uint32_t)NVFP4_FAULT_NONFINITE);
  }
  // (2) this workgroup's blocks: lane j (0..3) of block b holds values 4j..4j+3; whole
  // blocks (all four lanes) take the same trips through the loop
  const int j = threadIdx.x & 3;
  for (int64_t b = (int64_t)blockIdx.y * kRowChunkBlocks + (threadIdx.x >> 2); b < nb;
       b += (int64_t)gridDim.y * kRowChunkBlocks) {
    float v[4];
    load4<IN>(x, base + 16 * b + 4 * j, v);
    float amax_b = fmaxf(fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                         fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
    amax_b = fmaxf(amax_b, __shfl_xor(amax_b, 1, 4));
    amax_b = fmaxf(amax_b, __shfl_xor(amax_b, 2, 4));
    const float ratio = (t == 0.0f) ? 0.0f : (amax_b / 6.0f) / t;
    const uint32_t s = e4m3_rne(ratio);
    const float den = e4m3_value(s) * t;
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; i++) q[i] = (den == 0.0f) ? __builtin_copysignf(0.0f, v[i]) : v[i] / den;
    // four codes (16 bits, low nibble first) per lane; lanes 2i and 2i + 1 join theirs into
    // the block's code dword i
    uint32_t c = e2m1_rne2<1>(e2m1_rne2<0>(0u, q[0], q[1]), q[2], q[3]);
    c |= (uint32_t)__shfl_xor((int)c, 1, 4) << 16;
    if ((j & 1) == 0) *reinterpret_cast<uint32_t*>(codes + row * (K >> 1) + 8 * b + 2 * j) = c;
    if (j == 0) scales[row * nb + b] = (uint8_t)s;
  }
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
    // about 1024 workgroups or more in all, at most one per 64 blocks of a row
    const int64_t per_row = ((K >> 4) + kRowChunkBlocks - 1) / kRowChunkBlocks;
    const int64_t want = (1024 + M - 1) / M;
    const int64_t chunks = want < per_row ? want : per_row;
    hipLaunchKernelGGL((quantize_rows<IN>), dim3((uint32_t)M, (uint32_t)chunks), dim3(256), 0,
                       stream, x, ldx, K, codes, scales, ts, faults);
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
