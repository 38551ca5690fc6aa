// Tiled NVFP4 GEMM on the BF16 matrix cores for prompt-sized M (M > 16).
//
// The pages' prompt GEMMs run a pipelined 128x128 tile and copy their operands through
// a multi-stage pipeline in 128-value K steps (bloomery issue #565, section 4: PRs #696,
// #754 and #822), with activations rounded once rather than in every tile (PR #761).
// That design targets GB10 tensor cores; on gfx950 we keep the ideas that still hold and
// shape the rest for CDNA4:
//  - Workgroup tile 128 (M) x 256 (N) x 64 (K), four wave64s side by side along N, each
//    computing 128 x 64 with the 32x32x16 BF16 MFMA (8 accumulator tiles of 32x32).
//  - Activations (BF16, or NVFP4 decoded once per tile) are staged through LDS, double
//    buffered with one barrier per K step, rows padded by 16 bytes against bank
//    conflicts; all four waves read them.
//  - The weight never goes through LDS: each wave loads its own 64 columns' nibbles
//    (16 B per lane per K step) straight into registers and decodes them to exact BF16
//    operands, so every weight element is decoded once per workgroup.
//  - Workgroups are numbered so that each XCD (blockIdx % 8) owns a contiguous run of
//    tiles that share activation rows (A-stationary), keeping the reused operand in its
//    own L2.
// The fp32 accumulator is scaled once by the tensor scale(s) in the epilogue.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int LDA = BK + 8;  // bf16 per LDS row: 64 values + 16-byte pad

template <int ACT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t M = a.M, N = a.N, K = a.K;

  // XCD-aware tile order: consecutive tiles of one XCD share the same M rows.
  const int64_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int64_t total = nbm * nbn;
  const int64_t bid = blockIdx.x;
  int64_t lin = bid;
  if (total % 8 == 0) lin = (bid % 8) * (total / 8) + bid / 8;
  const int64_t m0 = (lin / nbn) * BM;
  const int64_t n0 = (lin % nbn) * BN;

  // weight columns of this lane: two 32-column subtiles, K half h of each 64-k step
  const int col = lane & 31;
  const int h = lane >> 5;
  const int64_t kb = K >> 1, sb = K >> 4;
  const uint8_t* wrow[2];
  const uint8_t* srow[2];
  bool nok[2];
#pragma unroll
  for (int st = 0; st < 2; st++) {
    const int64_t n = n0 + 64 * wave + 32 * st + col;
    nok[st] = n < N;
    const int64_t nn = nok[st] ? n : 0;
    wrow[st] = a.w_codes + nn * kb;
    srow[st] = a.w_scales + nn * sb;
  }

  const int KT = (int)((K + BK - 1) / BK);

  // activation staging registers
  u32x4 areg[4];
  uint32_t asc = 0;
  // weight registers: next step's loads and the current step's values
  u32x4 bnext[2], bcur[2];
  uint32_t snext[2], scur[2];

  auto load_step = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    if (ACT == 0) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int c = tid + 256 * q;
        const int row = c >> 3, ch = c & 7;
        const int64_t gm = m0 + row, gk = k0 + 8 * ch;
        areg[q] = (gm < M && gk < K)
                      ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) +
                                                         gm * a.ldx + gk)
                      : u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      const int row = tid >> 1, half = tid & 1;
      const int64_t gm = m0 + row, gk = k0 + 32 * half;
      if (gm < M && gk < K) {
        areg[0] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.x) + gm * kb +
                                                  (gk >> 1));
        asc = *reinterpret_cast<const uint16_t*>(a.x_scales + gm * sb + (gk >> 4));
      } else {
        areg[0] = u32x4{0u, 0u, 0u, 0u};
        asc = 0u;
      }
    }
#pragma unroll
    for (int st = 0; st < 2; st++) {
      const int64_t gk = k0 + 32 * h;
      if (nok[st] && gk < K) {
        bnext[st] = *reinterpret_cast<const u32x4*>(wrow[st] + (gk >> 1));
        snext[st] = *reinterpret_cast<const uint16_t*>(srow[st] + (gk >> 4));
      } else {
        bnext[st] = u32x4{0u, 0u, 0u, 0u};
        snext[st] = 0u;
      }
    }
  };

  auto store_a = [&](int buf) {
    uint16_t* dst = As[buf];
    if (ACT == 0) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int c = tid + 256 * q;
        const int row = c >> 3, ch = c & 7;
        *reinterpret_cast<u32x4*>(dst + row * LDA + 8 * ch) = areg[q];
      }
    } else {
      const int row = tid >> 1, half = tid & 1;
      const float s0 = e4m3_to_f32<0>(asc), s1 = e4m3_to_f32<1>(asc);
      u32x4* p = reinterpret_cast<u32x4*>(dst + row * LDA + 32 * half);
      p[0] = decode8(areg[0][0], s0);
      p[1] = decode8(areg[0][1], s0);
      p[2] = decode8(areg[0][2], s1);
      p[3] = decode8(areg[0][3], s1);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][st][r] = 0.f;

  load_step(0);
  store_a(0);
#pragma unroll
  for (int st = 0; st < 2; st++) {
    bcur[st] = bnext[st];
    scur[st] = snext[st];
  }

  for (int kt = 0; kt < KT; kt++) {
    if (kt + 1 < KT) load_step(kt + 1);
    __syncthreads();
    const uint16_t* src = As[kt & 1];
    float ws[2][2];
#pragma unroll
    for (int st = 0; st < 2; st++) {
      ws[st][0] = e4m3_to_f32<0>(scur[st]);
      ws[st][1] = e4m3_to_f32<1>(scur[st]);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      u32x4 B[2];
#pragma unroll
      for (int st = 0; st < 2; st++) B[st] = decode8(bcur[st][j], ws[st][j >> 1]);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const u32x4 A =
            *reinterpret_cast<const u32x4*>(src + (32 * mt + col) * LDA + 32 * h + 8 * j);
#pragma unroll
        for (int st = 0; st < 2; st++) acc[mt][st] = mfma32(A, B[st], acc[mt][st]);
      }
    }
    if (kt + 1 < KT) {
      store_a((kt + 1) & 1);
#pragma unroll
      for (int st = 0; st < 2; st++) {
        bcur[st] = bnext[st];
        scur[st] = snext[st];
      }
    }
  }

  const float ts = a.w_ts[0];
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t row = m0 + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= M) continue;
      const float f = (ACT == 0) ? ts : a.x_ts[row] * ts;
#pragma unroll
      for (int st = 0; st < 2; st++) {
        const int64_t n = n0 + 64 * wave + 32 * st + col;
        if (n < N) a.y[row * a.ldy + n] = acc[mt][st][r] * f;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int act_kind, hipStream_t stream) {
  const int64_t blocks = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (act_kind == 0)
    hipLaunchKernelGGL((gemm_kernel<0>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<1>), dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
