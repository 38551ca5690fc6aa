// Weight-streaming NVFP4 linear for a few activation rows (M <= 16): decode rows, MTP
// verify (4 rows) and the routed-expert rows of a MoE decode step.
//
// Each weight byte is read from HBM exactly once for all rows of the pass — the fix the
// pages apply to multi-row verify (bloomery issue #565, section 4 "Round 1": a run of
// several tokens dots each selected expert's rows for all its slots in one pass, PR
// #808; several rows as one multi-column walk, PR #652) — and several steps of loads
// stay in flight per lane (the m-column walk keeping eight chunks in flight, section 9,
// PR #511).
//
// gfx950 mapping: post-block-scaled 4x4x4 MFMAs.
//  - The E2M1 codes decode *unscaled* to BF16 with v_cvt_scalef32_pk_bf16_fp4 at scale
//    1.0 (exact, two values per instruction). Each group of four MFMAs covers exactly one
//    16-value scale block, and its fp32 partial is multiplied by that block's E4M3 scale
//    once (one FMA per output), so the scale never touches the per-element path.
//  - v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4x4x4 products. Lane l = 4b + j
//    (block b, column j) is weight row n = 4*(b % 4) + j of a 16-row tile at k-group
//    g = l / 16, so a lane holds whole 16-k blocks of its own row: its 16-byte code load
//    is 32 consecutive k. The four blocks with the same g share their A (the
//    activations): CBSZ = 2 broadcasts the A of block ABID of each group of four, so each
//    lane supplies one 16-byte piece of activations per step (row j, piece b % 4).
//  - Memory requests are shaped for the vector L1, which is the narrow point of this
//    stream: each wave takes a contiguous run of 128-k steps, so the two 64-byte halves
//    of every 128-byte weight line are requested by one wave in consecutive loads, and
//    activations are loaded row-contiguous (16 lanes read 256 bytes of one row) and
//    moved into the operand layout above through a small wave-private LDS buffer.
//  - The workgroup's scale rows are one contiguous block; it is copied into LDS once
//    with 16-byte loads and each lane reads its two scale bytes from there.
//  - Activation rows are padded to sets of four (R sets for M <= 4R); a workgroup owns
//    16*TN weight rows and W waves, with a ring of a few steps of loads in flight per
//    wave.
//  - Loads are raw buffer loads: out-of-range offsets read as zero without touching
//    memory, so bounds and predication need no branches (a branch around a load forces a
//    wait for it at the join and serializes the stream).
//  - Partial sums of the lane groups and waves meet in LDS and are added in a fixed order
//    (no atomics), then scaled by the tensor scale and stored as fp32.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

// Steps of loads in flight per wave (measured at K=4096): the dense kernel keeps eight for
// one row set, where few loads per step leave the memory pipe short of work (M=4, N=4096
// NVFP4 activations: 10.3 us with quantize against 10.7 us at depth four; M=1, K=N=2048:
// 4.4 against 4.7 us); four for two row sets (M=8, N=12288: 10.3 us against 10.8 us at
// eight); two for more, where each step already holds TN + R 16-byte loads per lane (M=16:
// 13.9 us against 14.7 us at four). The grouped kernels stream one expert's tile per
// workgroup and keep four (two from three row sets).
__host__ __device__ constexpr int dense_ring_depth(int R) {
  return R == 1 ? 8 : (R == 2 ? 4 : 2);
}
__host__ __device__ constexpr int grouped_ring_depth(int R) { return R >= 3 ? 2 : 4; }
constexpr uint32_t kOOB = 0x80000000u;
// Activation transpose buffer: one 16-byte piece per lane, rows of 16 pieces padded to
// 288 bytes so that both the row-contiguous writes and the operand-layout reads are free
// of bank conflicts.
constexpr uint32_t kXRow = 288;
constexpr uint32_t kXSet = 4 * kXRow;  // one set of four activation rows

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// kOOB when chunk start `k` is at or past K (offsets stay below 2^31 otherwise)
__device__ __forceinline__ uint32_t past(uint32_t K, uint32_t k) {
  return ((K - 1u - k) >> 31) << 31;
}

template <int TN, int R, int ACT>
struct StepBuf {
  u32x4 w[TN];       // 32 codes of this lane's row (per tile)
  u32x4 x[R];        // BF16: 8 k of activation row 4r + lane/16 at k0 + 8*(lane%16);
                     // NVFP4: x[r][0] the same piece as 8 codes, x[r][1] its scale byte
};

// MFMA 4x4x4 over one 4-k slice: A from block ABID of each group of four blocks
template <int ABID>
__device__ __forceinline__ f32x4 mfma4(uint32_t a01, uint32_t a23, uint32_t b01, uint32_t b23,
                                       f32x4 c) {
  const uint32_t av[2] = {a01, a23};
  const uint32_t bv[2] = {b01, b23};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4, av),
                                                __builtin_bit_cast(bf16x4, bv), c, 2, ABID, 0);
}

// Two BF16 values of byte SEL of `codes`, unscaled (exact)
template <int SEL>
__device__ __forceinline__ uint32_t cvt2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, SEL));
}

// Descriptor offsets of this lane's activation row (row 4r + lane/16) in each row set
// (kOOB for padding rows).
struct RowMap {
  uint32_t off[4];   // activation row
  uint32_t soff[4];  // NVFP4 activations: scale row
};

// Row stride (bytes) of the tile's scales in LDS: K/16 plus 4, so the 16 rows a wave
// reads together fall in different banks.
__host__ __device__ __forceinline__ uint32_t lds_scale_stride(int64_t K) {
  return (uint32_t)(K >> 4) + 4u;
}

// LDS bytes of the tile's scales (0 without SLDS): rows, 16 spare bytes, rounded to 16
__host__ __device__ __forceinline__ uint32_t lds_scale_bytes(int TN, int64_t K, bool slds) {
  return slds ? ((16u * TN * lds_scale_stride(K) + 31u) & ~15u) : 0u;
}

// In-call quantized activations (ACT == 2): the four rows' exact BF16 values stay in LDS
// for the whole stream, rows padded to whole 128-k steps plus 32 bytes (no bank
// conflicts between the four rows of an operand read); then the rows' amax bits, a
// non-finite flag per row and the rows' tensor scales.
__host__ __device__ __forceinline__ uint32_t xq_row_bytes(int64_t K) {
  return (uint32_t)(((K + 127) / 128) * 256 + 32);
}
__host__ __device__ __forceinline__ uint32_t xq_bytes(int64_t K) {
  return 4u * xq_row_bytes(K) + 48u;
}

// LDS layout of a workgroup: [scales | transpose buffers of the W waves, or the quantized
// rows | the waves' partial sums]. The partial sums have their own bytes, so a wave can
// write them while another still streams.
__host__ __device__ __forceinline__ uint32_t lds_red_offset(int TN, int R, int W, int64_t K,
                                                            bool slds, int act = 0) {
  const uint32_t stream =
      lds_scale_bytes(TN, K, slds) + (act == 2 ? xq_bytes(K) : (uint32_t)(W * R) * kXSet);
  return (stream + 15u) & ~15u;
}
// one wave's partials: 16 weight rows x 4 activation rows per (tile, row set)
__host__ __device__ __forceinline__ size_t lds_bytes(int TN, int R, int W, int64_t K, bool slds,
                                                     int act = 0) {
  return lds_red_offset(TN, R, W, K, slds, act) + (size_t)W * TN * R * 16 * 4 * sizeof(float);
}

// Waves splitting K: about eight 128-k steps per wave, one to four waves. The in-call
// quantization sizes its loops from this rule rather than from blockDim, whose read from
// the dispatch packet after the weight ring is issued would wait for the whole ring.
__host__ __device__ constexpr int waves_for_k(int64_t K) {
  const int64_t w = ((K + 127) / 128 + 7) / 8;
  return w < 1 ? 1 : (w > 4 ? 4 : (int)w);
}

// In-call activation quantization (ACT == 2): the workgroup quantizes the a.M <= 4 BF16
// rows by the per-row rule (row amax -> ts_row = amax / 2688 -> per 16-block E4M3 scale
// and E2M1 codes, the quantizer's own quantize16) and keeps their exact decoded BF16
// values e2m1 * e4m3 in LDS (rows past a.M and k past K are zero), so the stream
// multiplies exactly what nvfp4_quantize_act followed by the W4A4 call would. A row with
// a NaN or Inf gets a NaN tensor scale (its outputs are NaN). LDS: rows at xq, then
// amax bits [4], non-finite flags [4], ts_row [4].
//
// The rows' BF16 values are loaded first (xq_issue, before the weight ring, so that
// waiting for them does not wait for the ring), kQBlocks 16-blocks per thread: K <= 8192
// keeps a.M * K/16 within kQBlocks * 64 * waves_for_k(K) for every K.
constexpr int kQBlocks = 8;

struct XqRegs {
  u32x4 v[kQBlocks][2];
};

__device__ __forceinline__ void xq_issue(const StreamArgs& a, XqRegs& r) {
  const int nthr = 64 * waves_for_k(a.K);
  const int nb = (int)(a.K >> 4);
  const auto xr = make_rsrc(a.x, (uint32_t)(((a.x_rows - 1) * a.ldx + a.K) * 2));
#pragma unroll
  for (int u = 0; u < kQBlocks; u++) {
    const int j = threadIdx.x + u * nthr;
    const int m = j / nb, b = j % nb;
    const uint32_t off = j < a.M * nb ? (uint32_t)((m * a.ldx + 16 * b) * 2) : kOOB;
    r.v[u][0] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
    r.v[u][1] = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16u, 0, 0);
  }
}

__device__ __forceinline__ void unpack16(const u32x4& lo, const u32x4& hi, float v[16]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = __uint_as_float(lo[i] << 16);
    v[2 * i + 1] = __uint_as_float(lo[i] & 0xFFFF0000u);
    v[8 + 2 * i] = __uint_as_float(hi[i] << 16);
    v[8 + 2 * i + 1] = __uint_as_float(hi[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void xq_finish(const StreamArgs& a, const XqRegs& r, uint8_t* xq) {
  const int nthr = 64 * waves_for_k(a.K);
  const uint32_t rb = xq_row_bytes(a.K);
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(xq + 4 * rb);
  uint32_t* bad = amax_bits + 4;
  float* ts_row = reinterpret_cast<float*>(bad + 4);
  const int nb = (int)(a.K >> 4);         // 16-blocks per row
  const int nbp = (int)(rb - 32u) >> 5;  // 16-blocks per padded row
  if (threadIdx.x < 8) amax_bits[threadIdx.x] = 0u;  // amax bits and flags
  // rows and padding past the data are zero (stores after the barrier below fill the rest)
  for (int j = threadIdx.x; j < 4 * nbp; j += nthr) {
    const int m = j / nbp, b = j % nbp;
    if (m >= a.M || b >= nb) {
      u32x4* d = reinterpret_cast<u32x4*>(xq + m * rb + 32u * b);
      d[0] = u32x4{0u, 0u, 0u, 0u};
      d[1] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  // (1) row amax: per thread, then per wave (max is exact in any order), then one LDS
  // atomic max per wave and row on the bits of the non-negative float
  float pm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t badm = 0u;  // bit m: row m holds a NaN or Inf
#pragma unroll
  for (int u = 0; u < kQBlocks; u++) {
    const int j = threadIdx.x + u * nthr;
    if (j < a.M * nb) {
      float v[16];
      unpack16(r.v[u][0], r.v[u][1], v);
      float mx = 0.0f;
      bool fin = true;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        fin = fin && is_finite(v[i]);
        mx = fmaxf(mx, __builtin_fabsf(v[i]));
      }
      const int m = j / nb;
#pragma unroll
      for (int rr = 0; rr < 4; rr++) pm[rr] = (m == rr) ? fmaxf(pm[rr], mx) : pm[rr];
      if (!fin) badm |= 1u << m;
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; rr++) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) pm[rr] = fmaxf(pm[rr], __shfl_xor(pm[rr], off, 64));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) badm |= (uint32_t)__shfl_xor((int)badm, off, 64);
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      if (rr < a.M) atomicMax(&amax_bits[rr], __float_as_uint(pm[rr]));
      if ((badm >> rr) & 1u) bad[rr] = 1u;
    }
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const float t = __uint_as_float(amax_bits[threadIdx.x]) / 2688.0f;
    ts_row[threadIdx.x] = bad[threadIdx.x] ? __builtin_nanf("") : t;
  }
  // (2) blocks: codes and scale (quantize16, the quantizer's own arithmetic), then their
  // exact BF16 values (decode8, as the W4A4 stream decodes stored codes)
#pragma unroll
  for (int u = 0; u < kQBlocks; u++) {
    const int j = threadIdx.x + u * nthr;
    if (j < a.M * nb) {
      const int m = j / nb, b = j % nb;
      float v[16];
      unpack16(r.v[u][0], r.v[u][1], v);
      uint32_t lo, hi;
      const uint32_t sc = quantize16(v, __uint_as_float(amax_bits[m]) / 2688.0f, lo, hi);
      const float sd = e4m3_value(sc);
      u32x4* d = reinterpret_cast<u32x4*>(xq + m * rb + 32u * b);
      d[0] = decode8(lo, sd);
      d[1] = decode8(hi, sd);
    }
  }
}

// Tile t of the workgroup is weight rows n0 + t * tstride + [0, 16), of which the first
// lim[t] exist (rows past them read as zero).
template <int TN, int R, int ACT, bool SLDS, int kDepth>
__device__ __forceinline__ void pass4(const StreamArgs& a, const uint8_t* wc, const uint8_t* ws,
                                      int64_t n0, int64_t tstride, const int (&lim)[TN],
                                      const RowMap& rm, uint8_t* lds, f32x4 (&acc)[TN][R]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: uniform guards
  const int W = blockDim.x >> 6;
  const int g = lane >> 4;             // k-group of the lane (32 k of the 128-k step)
  const int bp = (lane >> 2) & 3;      // block within the group: activation piece index
  const int q = lane & 15;             // activation piece loaded by the lane (row-contiguous)
  const int nl = 4 * bp + (lane & 3);  // weight row of the lane within a 16-row tile
  const uint32_t K = (uint32_t)a.K;
  const uint32_t kb = K >> 1, sb = K >> 4;
  const int NS = (int)((K + 127u) >> 7);
  // an even number of steps per wave, so that each wave's scale bytes (8 per step and row)
  // start on a 16-byte boundary
  const int per_wave = 2 * ((NS + 2 * W - 1) / (2 * W));
  const int first = wave * per_wave;
  const int NSW = first < NS ? min(per_wave, NS - first) : 0;  // uniform over the wave

#pragma unroll
  for (int t = 0; t < TN; t++)
#pragma unroll
    for (int r = 0; r < R; r++) acc[t][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // descriptors over the rows the tiles span (up to the end of the matrix)
  int64_t span = (TN - 1) * tstride + 16;
  span = (a.N - n0) < span ? (a.N - n0) : span;
  const auto wr = make_rsrc(wc + n0 * kb, (uint32_t)(span * kb));
  const auto sr = make_rsrc(ws + n0 * sb, (uint32_t)(span * sb));
  uint32_t wrow[TN], srow[TN];
#pragma unroll
  for (int t = 0; t < TN; t++) {
    const bool ok = nl < lim[t];
    wrow[t] = ok ? (uint32_t)((t * tstride + nl) * kb) : kOOB;
    srow[t] = ok ? (uint32_t)((t * tstride + nl) * sb) : kOOB;
  }
  __amdgpu_buffer_rsrc_t xr, xsr;
  if (ACT != 1) {
    xr = make_rsrc(a.x, (uint32_t)(((a.x_rows - 1) * a.ldx + a.K) * 2));  // last row: K values
    xsr = xr;
  } else {
    xr = make_rsrc(a.x, (uint32_t)(a.x_rows * kb));
    xsr = make_rsrc(a.x_scales, (uint32_t)(a.x_rows * sb));
  }

  static_assert(ACT != 2 || (TN == 1 && R == 1), "in-call quantization: one row set, one tile");
  uint8_t* lds_s = lds;
  uint8_t* xbuf = lds + lds_scale_bytes(TN, a.K, SLDS) + (ACT == 2 ? 0u : (uint32_t)wave * R * kXSet);
  const uint32_t sls = lds_scale_stride(a.K);
  const uint32_t xw = kXRow * g + 16u * q;                 // this lane's piece (write)
  const uint32_t xrd = kXRow * (lane & 3) + 16u * (4 * g + bp);  // operand piece (read)

  // Step i of this wave. Every load is issued unconditionally; a step past the wave's
  // last one and chunks past K get out-of-range offsets and read zeros. With SLDS the
  // scale offset is kept for the LDS read at compute time.
  uint32_t kstep[kDepth];
  auto load = [&](int i, StepBuf<TN, R, ACT>& b, uint32_t& kg_out) {
    const uint32_t k0 = (uint32_t)((first + i) * 128);
    const uint32_t step_out = i < NSW ? 0u : kOOB;  // uniform
    const uint32_t kg = k0 + 32u * g;                // this lane's 32 weight k
    const uint32_t out_g = step_out | past(K, kg);
    kg_out = kg;
#pragma unroll
    for (int t = 0; t < TN; t++)
      b.w[t] = __builtin_amdgcn_raw_buffer_load_b128(wr, (wrow[t] + (kg >> 1)) | out_g, 0, 0);
    const uint32_t kp = k0 + 8u * q;  // this lane's activation piece: 8 k
    const uint32_t out_p = step_out | past(K, kp);
#pragma unroll
    for (int r = 0; r < R; r++) {
      if (ACT == 2) {
        // in-call quantized activations are read from LDS at compute time
      } else if (ACT == 0) {
        b.x[r] = __builtin_amdgcn_raw_buffer_load_b128(xr, (rm.off[r] + 2u * kp) | out_p, 0, 0);
      } else {
        b.x[r][0] = __builtin_amdgcn_raw_buffer_load_b32(xr, (rm.off[r] + (kp >> 1)) | out_p, 0, 0);
        b.x[r][1] = __builtin_amdgcn_raw_buffer_load_b8(xsr, (rm.soff[r] + (kp >> 4)) | out_p, 0, 0);
      }
    }
  };
  // without SLDS: the two scale bytes of each tile straight from memory, per ring slot
  uint32_t sreg_fallback[kDepth][TN];
  auto load_scales = [&](int i, int slot) {
    if (SLDS) return;
    const uint32_t k0 = (uint32_t)((first + i) * 128);
    const uint32_t step_out = i < NSW ? 0u : kOOB;
    const uint32_t kg = k0 + 32u * g;
    const uint32_t out_g = step_out | past(K, kg);
#pragma unroll
    for (int t = 0; t < TN; t++)
      sreg_fallback[slot][t] =
          __builtin_amdgcn_raw_buffer_load_b16(sr, (srow[t] + (kg >> 4)) | out_g, 0, 0);
  };

  auto compute = [&](StepBuf<TN, R, ACT>& b, uint32_t kg, int slot) {
    // activations: row-contiguous pieces -> LDS -> operand layout
    u32x4 A[R];
    if (ACT == 2) {
      // the quantized rows in LDS: row lane & 3, 8 k at k0 + 8 * (4g + bp)
      const uint32_t k0 = kg - 32u * g;
      A[0] = *reinterpret_cast<const u32x4*>(xbuf + (lane & 3) * xq_row_bytes(a.K) +
                                             2u * (k0 + 8u * (4 * g + bp)));
    } else {
#pragma unroll
      for (int r = 0; r < R; r++) {
        u32x4 v = b.x[r];
        if (ACT != 0) v = decode8(b.x[r][0], e4m3_to_f32<0>(b.x[r][1]));  // exact BF16
        *reinterpret_cast<u32x4*>(xbuf + r * kXSet + xw) = v;
      }
#pragma unroll
      for (int r = 0; r < R; r++) A[r] = *reinterpret_cast<const u32x4*>(xbuf + r * kXSet + xrd);
    }
#pragma unroll
    for (int t = 0; t < TN; t++) {
      uint32_t sc;
      if (SLDS) {
        // past-K chunks read a real scale here but their codes are zero
        sc = *reinterpret_cast<const uint16_t*>(lds_s + (16 * t + nl) * sls + (kg >> 4));
      } else {
        sc = sreg_fallback[slot][t];
      }
      const float s0 = e4m3_to_f32<0>(sc);
      const float s1 = e4m3_to_f32<1>(sc);
      // unscaled BF16 weights: dword d holds k = 8d .. 8d+7 of the lane's 32
      uint32_t wb[16];
#pragma unroll
      for (int d = 0; d < 4; d++) {
        wb[4 * d + 0] = cvt2<0>(b.w[t][d]);
        wb[4 * d + 1] = cvt2<1>(b.w[t][d]);
        wb[4 * d + 2] = cvt2<2>(b.w[t][d]);
        wb[4 * d + 3] = cvt2<3>(b.w[t][d]);
      }
      // Scale block 0 (k 0..15 of the lane's 32, activation pieces 0, 1) and block 1 (k
      // 16..31, pieces 2, 3) of every row set: 2R independent chains of four MFMAs, issued
      // round-robin so that no MFMA waits on the one before it, then each chain's
      // partial times its block's scale into the accumulator (block 0, then block 1).
      f32x4 c0[R], c1[R];
#pragma unroll
      for (int r = 0; r < R; r++) {
        c0[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        c1[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int r = 0; r < R; r++) c0[r] = mfma4<0>(A[r][0], A[r][1], wb[0], wb[1], c0[r]);
#pragma unroll
      for (int r = 0; r < R; r++) c1[r] = mfma4<2>(A[r][0], A[r][1], wb[8], wb[9], c1[r]);
#pragma unroll
      for (int r = 0; r < R; r++) c0[r] = mfma4<0>(A[r][2], A[r][3], wb[2], wb[3], c0[r]);
#pragma unroll
      for (int r = 0; r < R; r++) c1[r] = mfma4<2>(A[r][2], A[r][3], wb[10], wb[11], c1[r]);
#pragma unroll
      for (int r = 0; r < R; r++) c0[r] = mfma4<1>(A[r][0], A[r][1], wb[4], wb[5], c0[r]);
#pragma unroll
      for (int r = 0; r < R; r++) c1[r] = mfma4<3>(A[r][0], A[r][1], wb[12], wb[13], c1[r]);
#pragma unroll
      for (int r = 0; r < R; r++) c0[r] = mfma4<1>(A[r][2], A[r][3], wb[6], wb[7], c0[r]);
#pragma unroll
      for (int r = 0; r < R; r++) c1[r] = mfma4<3>(A[r][2], A[r][3], wb[14], wb[15], c1[r]);
#pragma unroll
      for (int r = 0; r < R; r++) {
#pragma unroll
        for (int qq = 0; qq < 4; qq++) acc[t][r][qq] = __builtin_fmaf(s0, c0[r][qq], acc[t][r][qq]);
#pragma unroll
        for (int qq = 0; qq < 4; qq++) acc[t][r][qq] = __builtin_fmaf(s1, c1[r][qq], acc[t][r][qq]);
      }
    }
  };

  // With SLDS each wave copies the scale bytes of its own steps (8 per 128-k step and
  // weight row: bytes [8 first, 8 (first + NSW)) of each tile row) into the workgroup's
  // scale rows in LDS and reads back only those, so no wave waits for another. Lane L
  // copies 16-byte piece L % 4 (+ 4j) of row L / 4 of each tile, so one load per lane and
  // tile covers eight steps; that first round is issued before the weight ring, so its
  // latency overlaps the ring's. Pieces past the wave's steps, and rows past N, read as
  // zero; the former go to a spare slot after the scale rows.
  const uint32_t s_pieces = (uint32_t)(NSW + 1) >> 1;  // 16-byte pieces per row (uniform)
  const int srow_l = lane >> 2;                        // tile row of the lane's pieces
  auto piece_src = [&](int t, uint32_t p) -> uint32_t {
    const bool ok = p < s_pieces && srow_l < lim[t];
    return ok ? (uint32_t)((t * tstride + srow_l) * sb) + 8u * (uint32_t)first + 16u * p : kOOB;
  };
  auto piece_put = [&](int t, uint32_t p, u32x4 v) {
    const uint32_t at = p < s_pieces ? (16u * t + srow_l) * sls + 8u * (uint32_t)first + 16u * p
                                     : 16u * TN * sls;
    uint32_t* d = reinterpret_cast<uint32_t*>(lds_s + at);  // rows are 4-byte aligned
    d[0] = v[0];
    d[1] = v[1];
    d[2] = v[2];
    d[3] = v[3];
  };
  u32x4 sreg[TN];
  if (SLDS) {
#pragma unroll
    for (int t = 0; t < TN; t++)
      sreg[t] = __builtin_amdgcn_raw_buffer_load_b128(sr, piece_src(t, lane & 3), 0, 0);
  }
  XqRegs xq_regs;
  if constexpr (ACT == 2) {
    xq_issue(a, xq_regs);  // before the ring, so that waiting for them does not wait for it
    __builtin_amdgcn_sched_barrier(0);
  }
  StepBuf<TN, R, ACT> buf[kDepth];
#pragma unroll
  for (int j = 0; j < kDepth; j++) {
    load(j, buf[j], kstep[j]);
    load_scales(j, j);
  }
  // In-call quantization of the (up to four) BF16 rows while the weight ring is in flight;
  // every wave reads all of them, hence the barrier.
  if constexpr (ACT == 2) {
    xq_finish(a, xq_regs, xbuf);
    __syncthreads();
  }
  if (SLDS) {
#pragma unroll
    for (int t = 0; t < TN; t++) piece_put(t, lane & 3, sreg[t]);
    // runs longer than eight steps: the further pieces, loaded and stored directly
    const uint32_t s_rounds = (s_pieces + 3u) & ~3u;  // uniform trip count
    for (uint32_t p = (uint32_t)(lane & 3) + 4u; p < s_rounds; p += 4u) {
#pragma unroll
      for (int t = 0; t < TN; t++)
        piece_put(t, p, __builtin_amdgcn_raw_buffer_load_b128(sr, piece_src(t, p), 0, 0));
    }
  }
  // Rounds of kDepth steps; every round but the last refills the ring, the last one only
  // drains it (a peeled round rather than guarded loads, which would make the compiler
  // wait for every load in flight where the guarded paths join).
  const int rounds = (NSW + kDepth - 1) / kDepth;  // uniform
  for (int c = 0; c + 1 < rounds; c++) {
#pragma unroll
    for (int j = 0; j < kDepth; j++) {
      compute(buf[j], kstep[j], j);
      load((c + 1) * kDepth + j, buf[j], kstep[j]);
      load_scales((c + 1) * kDepth + j, j);
      __builtin_amdgcn_sched_barrier(0);  // refill the slot now, not at the end of the round
    }
  }
  // (a wave with no steps computes nothing: its ring read zeros, but its scale rows in
  // LDS were never written)
  const int last = (rounds - 1) * kDepth;
#pragma unroll
  for (int j = 0; j < kDepth; j++)
    if (rounds > 0 && last + j < NSW) compute(buf[j], kstep[j], j);
}

// The fixed order in which partial sums meet: a wave's four k-groups in registers,
// (g0 + g2) + (g1 + g3), then the waves in order in LDS, starting from zero.
//
// group_sum: the sum over the k-groups of lane i's partial (lane 16g + i holds group g's),
// left in every lane. v_permlane32_swap with v as both operands returns the rows (0, 1,
// 0, 1) and (2, 3, 2, 3) of v; v_permlane16_swap with s as both returns (0, 0, 2, 2) and
// (1, 1, 3, 3) of s.
__device__ __forceinline__ float group_sum(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc[t][r][q] of lane (g, i) is the partial of weight row 16t + i and activation row
// 4r + q over k-group g of this wave's steps. The k-groups' sums go to
// red[wave][t][r][i][q] (lanes 0..15 write them).
template <int TN, int R>
__device__ __forceinline__ void write_partials(const f32x4 (&acc)[TN][R], float* red) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < TN; t++)
#pragma unroll
    for (int r = 0; r < R; r++) {
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; q++) v[q] = group_sum(acc[t][r][q]);
      if (lane < 16) *reinterpret_cast<f32x4*>(red + (((wave * TN + t) * R + r) * 16 + lane) * 4) = v;
    }
}

// the sum over the W waves, in order, of output (tile t, row set r, weight row i, act row q)
template <int TN, int R>
__device__ __forceinline__ float wave_sum(const float* red, int W, int t, int r, int i, int q) {
  float s = 0.f;
  for (int w = 0; w < W; w++) s += red[(((w * TN + t) * R + r) * 16 + i) * 4 + q];
  return s;
}

// Adds the partials in the fixed order and hands each (x row m, weight row n, sum) to
// `store`. red: the workgroup's partial-sum bytes (lds_red_offset), which no stream step
// uses, so only the one barrier between the writes and the reads is needed.
template <int TN, int R, typename Store>
__device__ __forceinline__ void reduce_store(const f32x4 (&acc)[TN][R], float* red, int64_t n0,
                                             Store store) {
  const int W = blockDim.x >> 6;
  write_partials<TN, R>(acc, red);
  __syncthreads();
  // one output per (t, r, q, i)
  for (int o = threadIdx.x; o < TN * R * 64; o += blockDim.x) {
    const int i = o & 15, q = (o >> 4) & 3, r = (o >> 6) % R, t = (o >> 6) / R;
    store(4 * r + q, n0 + 16 * t + i, wave_sum<TN, R>(red, W, t, r, i, q));
  }
}

template <int TN, int R, int ACT, bool SLDS>
__global__ __launch_bounds__(256) void stream_dense(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds + lds_red_offset(TN, R, blockDim.x >> 6, a.K, SLDS, ACT));
  // Row split: S workgroups share a weight tile, split s taking activation rows
  // [4R s, 4R (s + 1)). A row's arithmetic does not depend on the other rows of its
  // workgroup, so the split changes no result. The S splits of a tile are S apart in
  // steps of eight workgroups, which puts them on the same XCD (workgroup b runs on XCD
  // b % 8) and lets all but one read the tile from that XCD's L2.
  const int S = a.rsplit > 1 ? a.rsplit : 1;
  const int64_t bid = blockIdx.x;
  const int64_t tile = S == 1 ? bid : (bid % 8) + 8 * (bid / (8 * S));
  const int m0 = S == 1 ? 0 : (int)((bid / 8) % S) * 4 * R;
  const int64_t n0 = tile * 16 * TN;
  if (n0 >= a.N) return;  // padding of the split grid to whole groups of eight (uniform)
  const int i = (threadIdx.x >> 4) & 3;  // the x row this lane loads within a set of four
  RowMap rm;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int m = m0 + 4 * r + i;
    const bool ok = r < R && m < a.M;
    if (ACT == 0) {
      rm.off[r] = ok ? (uint32_t)(m * a.ldx * 2) : kOOB;
      rm.soff[r] = kOOB;
    } else {
      rm.off[r] = ok ? (uint32_t)(m * (a.K >> 1)) : kOOB;
      rm.soff[r] = ok ? (uint32_t)(m * (a.K >> 4)) : kOOB;
    }
  }
  int lim[TN];
#pragma unroll
  for (int t = 0; t < TN; t++) {
    const int64_t left = a.N - n0 - 16 * t;
    lim[t] = left < 0 ? 0 : (left > 16 ? 16 : (int)left);
  }
  f32x4 acc[TN][R];
  pass4<TN, R, ACT, SLDS, dense_ring_depth(R)>(a, a.w_codes, a.w_scales, n0, 16, lim, rm, lds, acc);
  const float ts = a.apply_ts ? a.w_ts[0] : 1.0f;
  float ts_q[4] = {0.f, 0.f, 0.f, 0.f};  // in-call quantized rows' tensor scales
  if (ACT == 2) {
    const float* tq = reinterpret_cast<const float*>(lds + lds_scale_bytes(TN, a.K, SLDS) +
                                                     4 * xq_row_bytes(a.K) + 32);
#pragma unroll
    for (int m = 0; m < 4; m++) ts_q[m] = tq[m];
  }
  reduce_store<TN, R>(acc, red, n0, [&](int mr, int64_t n, float s) {
    const int m = m0 + mr;
    if (m < a.M && n < a.N) {
      const float f = (ACT == 0) ? ts : (ACT == 2 ? ts_q[m & 3] * ts : a.x_ts[m] * ts);
      a.y[(int64_t)m * a.ldy + n] = s * f;
    }
  });
}

// The routes of a grouped workgroup's expert, from its slot record: the first ones come
// with the record (read together with its header), later ones from `sorted`.
struct SlotRoutes {
  int e, beg, count, n;
  int4 q[kSlotRoutes / 4];
  __device__ __forceinline__ explicit SlotRoutes(const StreamArgs& a) {
    const int4* rec = reinterpret_cast<const int4*>(a.slots + kSlotInts * blockIdx.y);
    const int4 h = rec[0];
#pragma unroll
    for (int j = 0; j < kSlotRoutes / 4; j++) q[j] = rec[1 + j];
    e = h.x, beg = h.y, count = h.z - h.y, n = h.w;
  }
  // route c (0 <= c < count) of the expert
  __device__ __forceinline__ int route(const StreamArgs& a, int c) const {
    int v = q[0].x;
#pragma unroll
    for (int j = 0; j < kSlotRoutes / 4; j++) {
      v = c == 4 * j + 0 ? q[j].x : v;
      v = c == 4 * j + 1 ? q[j].y : v;
      v = c == 4 * j + 2 ? q[j].z : v;
      v = c == 4 * j + 3 ? q[j].w : v;
    }
    if (c >= n) v = a.sorted[beg + c];
    return v;
  }
};

template <int R, int ACT, bool SLDS>
__global__ __launch_bounds__(256) void stream_grouped(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds + lds_red_offset(1, R, blockDim.x >> 6, a.K, SLDS));
  const SlotRoutes sr(a);
  const int e = sr.e;
  if (e < 0) return;  // a slot past the active experts (uniform over the workgroup)
  const uint8_t* wc = a.w_codes + (int64_t)e * a.N * (a.K >> 1);
  const uint8_t* ws = a.w_scales + (int64_t)e * a.N * (a.K >> 4);
  const float ts = a.apply_ts ? a.w_ts[e] : 1.0f;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int i = (threadIdx.x >> 4) & 3;
  for (int c0 = 0; c0 < sr.count; c0 += 4 * R) {
    const int rows = min(4 * R, sr.count - c0);
    RowMap rm;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int m = 4 * r + i;
      const bool ok = r < R && m < rows;
      const int route = sr.route(a, c0 + (ok ? m : 0));
      const int64_t xrow = a.rows_per_token ? route / a.top_k : route;
      if (ACT == 0) {
        rm.off[r] = ok ? (uint32_t)(xrow * a.ldx * 2) : kOOB;
        rm.soff[r] = kOOB;
      } else {
        rm.off[r] = ok ? (uint32_t)(xrow * (a.K >> 1)) : kOOB;
        rm.soff[r] = ok ? (uint32_t)(xrow * (a.K >> 4)) : kOOB;
      }
    }
    f32x4 acc[1][R];
    const int lim[1] = {(int)((a.N - n0) < 16 ? (a.N - n0) : 16)};
    pass4<1, R, ACT, SLDS, grouped_ring_depth(R)>(a, wc, ws, n0, 16, lim, rm, lds, acc);
    reduce_store<1, R>(acc, red, n0, [&](int m, int64_t n, float s) {
      if (m < rows && n < a.N) {
        const int rr = sr.route(a, c0 + m);
        float f = ts;
        if (ACT != 0) {
          const int64_t xrr = a.rows_per_token ? rr / a.top_k : rr;
          f = a.x_ts[xrr] * ts;
        }
        a.y[(int64_t)rr * a.ldy + n] = s * f;
      }
    });
    __syncthreads();  // the next pass writes its partials over these
  }
}

// Grouped gate_up with the SwiGLU epilogue: the workgroup streams gate rows n0 + [0, 16)
// and the matching up rows N/2 + n0 + [0, 16) of its expert as two tiles, reduces both in
// the same fixed order as reduce_store, and writes a = bf16_rne(silu(g) * u) where g and
// u are exactly the per-route rows' fp32 values (sum times the same scale factor) and
// silu is device.hpp's.
template <int R, int ACT, bool SLDS>
__global__ __launch_bounds__(256) void stream_grouped_swiglu(StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds + lds_red_offset(2, R, blockDim.x >> 6, a.K, SLDS));
  const SlotRoutes sr(a);
  const int e = sr.e;
  if (e < 0) return;  // a slot past the active experts (uniform over the workgroup)
  const uint8_t* wc = a.w_codes + (int64_t)e * a.N * (a.K >> 1);
  const uint8_t* ws = a.w_scales + (int64_t)e * a.N * (a.K >> 4);
  const float ts = a.w_ts[e];
  const int64_t half = a.N >> 1;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int vr = (int)((half - n0) < 16 ? (half - n0) : 16);
  const int lim[2] = {vr, vr};
  const int i = (threadIdx.x >> 4) & 3;
  const int W = blockDim.x >> 6;
  for (int c0 = 0; c0 < sr.count; c0 += 4 * R) {
    const int rows = min(4 * R, sr.count - c0);
    RowMap rm;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int m = 4 * r + i;
      const bool ok = r < R && m < rows;
      const int route = sr.route(a, c0 + (ok ? m : 0));
      const int64_t xrow = a.rows_per_token ? route / a.top_k : route;
      if (ACT == 0) {
        rm.off[r] = ok ? (uint32_t)(xrow * a.ldx * 2) : kOOB;
        rm.soff[r] = kOOB;
      } else {
        rm.off[r] = ok ? (uint32_t)(xrow * (a.K >> 1)) : kOOB;
        rm.soff[r] = ok ? (uint32_t)(xrow * (a.K >> 4)) : kOOB;
      }
    }
    f32x4 acc[2][R];
    pass4<2, R, ACT, SLDS, grouped_ring_depth(R)>(a, wc, ws, n0, half, lim, rm, lds, acc);
    write_partials<2, R>(acc, red);
    __syncthreads();
    for (int o = threadIdx.x; o < R * 64; o += blockDim.x) {
      const int nl = o & 15, q = (o >> 4) & 3, r = o >> 6;
      const float sg = wave_sum<2, R>(red, W, 0, r, nl, q);
      const float su = wave_sum<2, R>(red, W, 1, r, nl, q);
      const int m = 4 * r + q;
      const int64_t n = n0 + nl;
      if (m < rows && n < half) {
        const int rr = sr.route(a, c0 + m);
        float f = ts;
        if (ACT != 0) {
          const int64_t xrr = a.rows_per_token ? rr / a.top_k : rr;
          f = a.x_ts[xrr] * ts;
        }
        const float g = sg * f;
        const float u = su * f;
        const float sg = silu(g);
        a.a_out[(int64_t)rr * half + n] = (uint16_t)f32_to_bf16_rne(sg * u);
      }
    }
    __syncthreads();
  }
}

template <int R, int ACT>
hipError_t launch_grouped_swiglu(const StreamArgs& a, int max_active, int W, bool slds,
                                 hipStream_t stream) {
  const size_t lds = lds_bytes(2, R, W, a.K, slds);
  const int64_t groups = ((a.N >> 1) + 15) / 16;
  if (slds)
    hipLaunchKernelGGL((stream_grouped_swiglu<R, ACT, true>),
                       dim3((uint32_t)groups, (uint32_t)max_active), dim3(64 * W), lds, stream, a);
  else
    hipLaunchKernelGGL((stream_grouped_swiglu<R, ACT, false>),
                       dim3((uint32_t)groups, (uint32_t)max_active), dim3(64 * W), lds, stream, a);
  return hipGetLastError();
}

template <int TN, int R, int ACT>
hipError_t launch_dense(const StreamArgs& a, int W, bool slds, hipStream_t stream) {
  const size_t lds = lds_bytes(TN, R, W, a.K, slds, ACT);
  const int64_t tiles = (a.N + 16 * TN - 1) / (16 * TN);
  const int64_t groups = a.rsplit > 1 ? (tiles + 7) / 8 * 8 * a.rsplit : tiles;
  if (slds)
    hipLaunchKernelGGL((stream_dense<TN, R, ACT, true>), dim3((uint32_t)groups), dim3(64 * W), lds,
                       stream, a);
  else
    hipLaunchKernelGGL((stream_dense<TN, R, ACT, false>), dim3((uint32_t)groups), dim3(64 * W),
                       lds, stream, a);
  return hipGetLastError();
}

template <int R, int ACT>
hipError_t launch_grouped(const StreamArgs& a, int max_active, int W, bool slds,
                          hipStream_t stream) {
  const size_t lds = lds_bytes(1, R, W, a.K, slds);
  const int64_t groups = (a.N + 15) / 16;
  if (slds)
    hipLaunchKernelGGL((stream_grouped<R, ACT, true>), dim3((uint32_t)groups, (uint32_t)max_active),
                       dim3(64 * W), lds, stream, a);
  else
    hipLaunchKernelGGL((stream_grouped<R, ACT, false>),
                       dim3((uint32_t)groups, (uint32_t)max_active), dim3(64 * W), lds, stream, a);
  return hipGetLastError();
}

// Wider tiles are chosen only for three or more row sets (launch_stream), so only those
// combinations are built.
template <int TN, int ACT>
hipError_t dense_r(const StreamArgs& a, int R, int W, bool slds, hipStream_t stream) {
  if constexpr (TN == 1) {
    if (R == 1) return launch_dense<1, 1, ACT>(a, W, slds, stream);
    if (R == 2) return launch_dense<1, 2, ACT>(a, W, slds, stream);
  }
  if (R == 3) return launch_dense<TN, 3, ACT>(a, W, slds, stream);
  if (R == 4) return launch_dense<TN, 4, ACT>(a, W, slds, stream);
  return hipErrorInvalidValue;
}

template <int ACT>
hipError_t dense_tn(const StreamArgs& a, int tn, int R, int W, bool slds, hipStream_t stream) {
  switch (tn) {
    case 1: return dense_r<1, ACT>(a, R, W, slds, stream);
    case 2: return dense_r<2, ACT>(a, R, W, slds, stream);
    case 3: return dense_r<3, ACT>(a, R, W, slds, stream);
    case 4: return dense_r<4, ACT>(a, R, W, slds, stream);
    default: return hipErrorInvalidValue;
  }
}

// The scale copy needs whole 16-byte chunks per row (K % 256 == 0; then every tile's and
// expert's scale block starts 16-byte aligned when the scales do) and a modest LDS
// footprint.
bool use_lds_scales(const StreamArgs& a, int tn) {
  if (a.K % 256 != 0 || (uintptr_t)a.w_scales % 16 != 0) return false;
  return lds_scale_bytes(tn, a.K, true) <= 32768;
}

// Picks 16-row tiles per workgroup so that whole rounds of workgroups fill the 256 CUs:
// estimated time ~ rounds * TN; ties go to the larger tile (fewer activation re-reads).
int pick_tn(int64_t N) {
  int best = 1;
  int64_t best_cost = -1;
  for (int tn : {1, 2, 3, 4}) {
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

hipError_t launch_stream_cfg(const StreamArgs& a_in, int act_kind, bool grouped, int max_active,
                             int tn, int W, int rsets, hipStream_t stream) {
  StreamArgs a = a_in;
  if (W < 1 || W > 4) return hipErrorInvalidValue;
  // activation kinds: 0 BF16, 1 NVFP4 (both forms), 2 BF16 quantized in the call (dense
  // only); anything else is refused rather than taken by one of the templates
  if (act_kind != 0 && act_kind != 1 && !(act_kind == 2 && !grouped)) return hipErrorInvalidValue;
  if (grouped && a.a_out) {
    const bool slds = use_lds_scales(a, 2);
    const int R = a.M > 0 ? (a.M + 3) / 4 : 1;
    switch (R) {
      case 1: return act_kind == 0 ? launch_grouped_swiglu<1, 0>(a, max_active, W, slds, stream)
                                   : launch_grouped_swiglu<1, 1>(a, max_active, W, slds, stream);
      case 2: return act_kind == 0 ? launch_grouped_swiglu<2, 0>(a, max_active, W, slds, stream)
                                   : launch_grouped_swiglu<2, 1>(a, max_active, W, slds, stream);
      default: return act_kind == 0 ? launch_grouped_swiglu<4, 0>(a, max_active, W, slds, stream)
                                    : launch_grouped_swiglu<4, 1>(a, max_active, W, slds, stream);
    }
  }
  const bool slds = use_lds_scales(a, grouped ? 1 : tn);
  if (grouped) {
    // rows of one expert pass in sets of four: one set covers decode-sized loads
    const int R = a.M > 0 ? (a.M + 3) / 4 : 1;
    switch (R) {
      case 1: return act_kind == 0 ? launch_grouped<1, 0>(a, max_active, W, slds, stream)
                                   : launch_grouped<1, 1>(a, max_active, W, slds, stream);
      case 2: return act_kind == 0 ? launch_grouped<2, 0>(a, max_active, W, slds, stream)
                                   : launch_grouped<2, 1>(a, max_active, W, slds, stream);
      default: return act_kind == 0 ? launch_grouped<4, 0>(a, max_active, W, slds, stream)
                                    : launch_grouped<4, 1>(a, max_active, W, slds, stream);
    }
  }
  const int sets = (a.M + 3) / 4;
  // default: one workgroup per tile takes every row, except on launches of at most 256
  // tiles (one workgroup per CU) with three or more row sets, where two workgroups share a
  // tile (W4A4 M=16, N=4096: 8.0 against 8.8 us); the split changes no result
  if (rsets <= 0 && tn == 1 && (a.N + 15) / 16 <= 256 && sets >= 3) rsets = (sets + 1) / 2;
  const int R = rsets > 0 && rsets < sets ? rsets : sets;
  a.rsplit = (sets + R - 1) / R;
  if (act_kind == 2) {  // in-call quantized activations: one row set, 16-row tiles
    if (R != 1 || tn != 1 || W != waves_for_k(a.K)) return hipErrorInvalidValue;
    if (a.M * (a.K >> 4) > (int64_t)kQBlocks * 64 * W) return hipErrorInvalidValue;
    return launch_dense<1, 1, 2>(a, W, slds, stream);
  }
  return act_kind == 0 ? dense_tn<0>(a, tn, R, W, slds, stream)
                       : dense_tn<1>(a, tn, R, W, slds, stream);
}

hipError_t launch_stream(const StreamArgs& a, int act_kind, bool grouped, int max_active,
                         hipStream_t stream) {
  const int W = waves_for_k(a.K);
  // up to two row sets: 16-row tiles keep the most workgroups in flight (M=8 at K=4096,
  // N=12288: 10.2 us against 10.6 us with 48-row tiles); more row sets: wider tiles share
  // each activation load among more weight rows
  const int tn = (grouped || a.M <= 8) ? 1 : pick_tn(a.N);
  return launch_stream_cfg(a, act_kind, grouped, max_active, tn, W, 0, stream);
}

}  // namespace nvfp4
