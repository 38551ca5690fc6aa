// Weight-streaming NVFP4 linear for a few activation rows (M <= 16): decode rows, MTP
// verify (4 rows) and the routed-expert rows of a MoE decode step.
//
// Each weight byte is read from HBM exactly once for all rows of the pass — the fix the
// pages apply to multi-row verify (bloomery issue #565, section 4 "Round 1": a run of
// several tokens dots each selected expert's rows for all its slots in one pass, PR
// #808; several rows as one multi-column walk, PR #652) — and many loads are kept in
// flight per lane (the m-column walk keeping eight chunks in flight, section 9, PR
// #511).
//
// gfx950 mapping. A workgroup owns 16*TN weight rows (n) and splits K over its waves;
// within a wave the four 16-lane groups take four contiguous K ranges. Each lane streams
// 16-byte code loads (32 nibbles of one row) plus the two E4M3 scale bytes that cover
// them, decodes them in registers to exact BF16 (device.hpp), and feeds the 16x16x32 BF16
// MFMA with the activation rows (padded to 16) as the A operand. Partial sums of the
// waves meet in LDS and are added in a fixed order (no atomics), then scaled by the
// tensor scale and stored as fp32.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr int kUnroll = 4;  // 32-k pieces per lane whose loads are issued together

template <int TN, int ACT>
__device__ __forceinline__ void stream_pass(const StreamArgs& a, const uint8_t* wc,
                                            const uint8_t* ws, int64_t n0, const void* xrow,
                                            const uint8_t* xsrow, bool row_ok,
                                            f32x4 (&acc)[TN]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int col = lane & 15;
  const int slot = wave * 4 + (lane >> 4);
  const int64_t K = a.K;
  const int Kc = (int)(K >> 5);  // 32-k pieces per row
  const int S = 4 * W;
  const int P = (Kc + S - 1) / S;
  const int p_begin = slot * P;
  const int64_t kb = K >> 1;
  const int64_t sb = K >> 4;

#pragma unroll
  for (int t = 0; t < TN; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* wrow[TN];
  const uint8_t* srow[TN];
  bool nok[TN];
#pragma unroll
  for (int t = 0; t < TN; t++) {
    const int64_t n = n0 + 16 * t + col;
    nok[t] = n < a.N;
    const int64_t nn = nok[t] ? n : 0;
    wrow[t] = wc + nn * kb;
    srow[t] = ws + nn * sb;
  }

  for (int s0 = 0; s0 < P; s0 += kUnroll) {
    u32x4 cw[kUnroll][TN];
    uint32_t sc[kUnroll][TN];
    u32x4 xa[kUnroll][ACT == 0 ? 4 : 1];
    uint32_t xsc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int piece = p_begin + s0 + u;
      const bool pv = (s0 + u < P) && (piece < Kc);
#pragma unroll
      for (int t = 0; t < TN; t++) {
        if (pv && nok[t]) {
          cw[u][t] = *reinterpret_cast<const u32x4*>(wrow[t] + (int64_t)piece * 16);
          sc[u][t] = *reinterpret_cast<const uint16_t*>(srow[t] + (int64_t)piece * 2);
        } else {
          cw[u][t] = u32x4{0u, 0u, 0u, 0u};
          sc[u][t] = 0u;
        }
      }
      if (ACT == 0) {
#pragma unroll
        for (int d = 0; d < (ACT == 0 ? 4 : 1); d++) {
          xa[u][d] = (pv && row_ok)
                         ? reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(xrow) +
                                                          (int64_t)piece * 32)[d]
                         : u32x4{0u, 0u, 0u, 0u};
        }
        xsc[u] = 0u;
      } else {
        if (pv && row_ok) {
          xa[u][0] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(xrow) +
                                                     (int64_t)piece * 16);
          xsc[u] = *reinterpret_cast<const uint16_t*>(xsrow + (int64_t)piece * 2);
        } else {
          xa[u][0] = u32x4{0u, 0u, 0u, 0u};
          xsc[u] = 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      u32x4 A[4];
      if (ACT == 0) {
#pragma unroll
        for (int d = 0; d < 4; d++) A[d] = xa[u][ACT == 0 ? d : 0];
      } else {
        const float xs0 = e4m3_to_f32<0>(xsc[u]);
        const float xs1 = e4m3_to_f32<1>(xsc[u]);
        A[0] = decode8(xa[u][0][0], xs0);
        A[1] = decode8(xa[u][0][1], xs0);
        A[2] = decode8(xa[u][0][2], xs1);
        A[3] = decode8(xa[u][0][3], xs1);
      }
#pragma unroll
      for (int t = 0; t < TN; t++) {
        const float s0v = e4m3_to_f32<0>(sc[u][t]);
        const float s1v = e4m3_to_f32<1>(sc[u][t]);
        acc[t] = mfma16(A[0], decode8(cw[u][t][0], s0v), acc[t]);
        acc[t] = mfma16(A[1], decode8(cw[u][t][1], s0v), acc[t]);
        acc[t] = mfma16(A[2], decode8(cw[u][t][2], s1v), acc[t]);
        acc[t] = mfma16(A[3], decode8(cw[u][t][3], s1v), acc[t]);
      }
    }
  }
}

// Adds the waves' partial tiles in wave order and hands each (row, n, sum) to `store`.
template <int TN, typename Store>
__device__ __forceinline__ void reduce_store(const f32x4 (&acc)[TN], float* red, int64_t n0,
                                             Store store) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
#pragma unroll
  for (int t = 0; t < TN; t++)
#pragma unroll
    for (int r = 0; r < 4; r++) red[((wave * TN + t) * 4 + r) * 64 + lane] = acc[t][r];
  __syncthreads();
  for (int o = threadIdx.x; o < TN * 256; o += blockDim.x) {
    const int t = o >> 8, mm = (o >> 4) & 15, cc = o & 15;
    const int src = cc + 16 * (mm >> 2), r = mm & 3;
    float s = 0.f;
    for (int w = 0; w < W; w++) s += red[((w * TN + t) * 4 + r) * 64 + src];
    store(mm, n0 + 16 * t + cc, s);
  }
  __syncthreads();
}

template <int TN, int ACT>
__global__ __launch_bounds__(512) void stream_dense(StreamArgs a) {
  extern __shared__ float red[];
  const int64_t n0 = (int64_t)blockIdx.x * 16 * TN;
  const int m = threadIdx.x & 15;
  const bool row_ok = m < a.M;
  const int mr = row_ok ? m : 0;
  const void* xrow;
  const uint8_t* xsrow = nullptr;
  if (ACT == 0) {
    xrow = static_cast<const uint16_t*>(a.x) + (int64_t)mr * a.ldx;
  } else {
    xrow = static_cast<const uint8_t*>(a.x) + (int64_t)mr * (a.K >> 1);
    xsrow = a.x_scales + (int64_t)mr * (a.K >> 4);
  }
  f32x4 acc[TN];
  stream_pass<TN, ACT>(a, a.w_codes, a.w_scales, n0, xrow, xsrow, row_ok, acc);
  const float ts = a.apply_ts ? a.w_ts[0] : 1.0f;
  reduce_store<TN>(acc, red, n0, [&](int mm, int64_t n, float s) {
    if (mm < a.M && n < a.N) {
      const float f = (ACT == 0) ? ts : a.x_ts[mm] * ts;
      a.y[(int64_t)mm * a.ldy + n] = s * f;
    }
  });
}

template <int TN, int ACT>
__global__ __launch_bounds__(512) void stream_grouped(StreamArgs a) {
  extern __shared__ float red[];
  const int slot = blockIdx.y;
  if (slot >= *a.n_active) return;  // uniform over the workgroup
  const int e = a.active[slot];
  const int beg = a.offsets[e], end = a.offsets[e + 1];
  const uint8_t* wc = a.w_codes + (int64_t)e * a.N * (a.K >> 1);
  const uint8_t* ws = a.w_scales + (int64_t)e * a.N * (a.K >> 4);
  const float ts = a.apply_ts ? a.w_ts[e] : 1.0f;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * TN;
  for (int c0 = beg; c0 < end; c0 += 16) {
    const int rows = min(16, end - c0);
    const int m = threadIdx.x & 15;
    const bool row_ok = m < rows;
    const int r = a.sorted[c0 + (row_ok ? m : 0)];
    const int64_t xr = a.rows_per_token ? r / a.top_k : r;
    const void* xrow;
    const uint8_t* xsrow = nullptr;
    if (ACT == 0) {
      xrow = static_cast<const uint16_t*>(a.x) + xr * a.ldx;
    } else {
      xrow = static_cast<const uint8_t*>(a.x) + xr * (a.K >> 1);
      xsrow = a.x_scales + xr * (a.K >> 4);
    }
    f32x4 acc[TN];
    stream_pass<TN, ACT>(a, wc, ws, n0, xrow, xsrow, row_ok, acc);
    reduce_store<TN>(acc, red, n0, [&](int mm, int64_t n, float s) {
      if (mm < rows && n < a.N) {
        const int rr = a.sorted[c0 + mm];
        float f = ts;
        if (ACT != 0) {
          const int64_t xrr = a.rows_per_token ? rr / a.top_k : rr;
          f = a.x_ts[xrr] * ts;
        }
        a.y[(int64_t)rr * a.ldy + n] = s * f;
      }
    });
  }
}

template <int TN, int ACT>
hipError_t launch_tn(const StreamArgs& a, bool grouped, int max_active, int W,
                     hipStream_t stream) {
  const dim3 block(64 * W);
  const size_t lds = (size_t)W * TN * 4 * 64 * sizeof(float);
  const int64_t groups = (a.N + 16 * TN - 1) / (16 * TN);
  if (grouped) {
    hipLaunchKernelGGL((stream_grouped<TN, ACT>), dim3((uint32_t)groups, (uint32_t)max_active),
                       block, lds, stream, a);
  } else {
    hipLaunchKernelGGL((stream_dense<TN, ACT>), dim3((uint32_t)groups), block, lds, stream, a);
  }
  return hipGetLastError();
}

// Picks 16-row tiles per workgroup so that whole rounds of workgroups fill the 256 CUs:
// estimated time ~ rounds * TN; ties go to the larger tile (fewer activation re-reads).
int pick_tn(int64_t N) {
  int best = 1;
  int64_t best_cost = -1;
  for (int tn = 1; tn <= 4; tn++) {
    const int64_t groups = (N + 16 * tn - 1) / (16 * tn);
    const int64_t cost = ((groups + 255) / 256) * tn;
    if (best_cost < 0 || cost <= best_cost) {
      best = tn;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace

hipError_t launch_stream(const StreamArgs& a, int act_kind, bool grouped, int max_active,
                         hipStream_t stream) {
  const int64_t Kc = a.K / 32;
  int W = (int)((Kc + 15) / 16);
  W = W < 1 ? 1 : (W > 8 ? 8 : W);
  const int tn = grouped ? 1 : pick_tn(a.N);
#define NVFP4_TN_CASE(TNV)                                                       \
  case TNV:                                                                      \
    return act_kind == 0 ? launch_tn<TNV, 0>(a, grouped, max_active, W, stream)  \
                         : launch_tn<TNV, 1>(a, grouped, max_active, W, stream);
  switch (tn) {
    NVFP4_TN_CASE(1)
    NVFP4_TN_CASE(2)
    NVFP4_TN_CASE(3)
    NVFP4_TN_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef NVFP4_TN_CASE
}

}  // namespace nvfp4
