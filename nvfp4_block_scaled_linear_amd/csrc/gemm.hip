// Tiled NVFP4 GEMM on the BF16 matrix cores for prompt-sized M (M > 16).
//
// The pages' prompt GEMMs run a pipelined 128x128 tile and copy their operands through
// a multi-stage pipeline in 128-value K steps (bloomery issue #565, section 4: PRs #696,
// #754 and #822), with activations rounded once rather than in every tile (PR #761).
// That design targets GB10 tensor cores; on gfx950 we keep the ideas that still hold and
// shape the rest for CDNA4:
//  - Large M: a 256 (M) x 256 (N) x 64 (K) tile on twelve wave64s with split roles:
//    eight consumer waves (two along M, four along N, each 128 x 64 with the 32x32x16
//    BF16 MFMA) only read LDS and run MFMAs; four producer waves only load, decode the
//    weight tile once per workgroup and write both operands to LDS (gemm_wide below).
//    With more such tiles than CUs (BF16 activations), one workgroup per CU takes its
//    XCD's tiles in turn as a persistent pipeline, the next tile's loads issued while
//    the current one's last steps and stores run (gemm_wide_grouped_p's dense form).
//  - Smaller M: a 32*MT (M) x 256 (N) tile on four wave64s side by side along N, each
//    computing 32*MT x 64 and decoding its own weight columns in registers; two
//    workgroups per CU.
//  - Activations (BF16, or NVFP4 decoded once per tile) are staged through LDS, double
//    buffered with one barrier per K step, rows padded by 16 bytes against bank
//    conflicts; all four waves read them.
//  - The weight never goes through LDS: each wave loads its own 64 columns' nibbles
//    (16 B per lane per K step) straight into registers and decodes them to exact BF16
//    operands (e2m1 * e4m3 in f32, high halves), so every weight element is decoded once
//    per workgroup.
//  - Global loads run two K steps ahead in two register sets; they are raw buffer loads
//    (out-of-range offsets read zeros), so no branch guards a load and the compiler
//    waits only for the step it needs.
//  - Workgroups are numbered per XCD (blockIdx % 8) so that the operand an XCD reuses
//    stays in its own L2: the 256-row tiles share activation rows (A-stationary); the
//    smaller-M kernels take an eighth of the weight's columns per XCD (weight-stationary).
// The fp32 accumulator is scaled once by the tensor scale(s) in the epilogue; with BF16
// activations the results leave through branch-free buffer stores.
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int LDA = BK + 8;  // bf16 per LDS row: 64 values + 16-byte pad
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)b, 0x00020000);
}

// kOOB when k is at or past K
__device__ __forceinline__ uint32_t past(uint32_t K, uint32_t k) {
  return ((K - 1u - k) >> 31) << 31;
}

template <int MT, int ACT>
struct RegA {  // one K step of this thread's activation loads
  u32x4 v[ACT == 0 ? MT : 1];
  uint32_t c[ACT == 0 ? 1 : MT];   // NVFP4: 8 codes per piece
  uint32_t s[ACT == 0 ? 1 : MT];   // NVFP4: the piece's scale byte
};
struct RegB {  // one K step of this lane's weight loads (two 32-column subtiles)
  u32x4 c[2];
  uint32_t s[2];
};

// GROUPED: the expert-grouped form. A workgroup takes tile blockIdx.x / nbn of the route
// grouping's tile list (tile_rows = BM routes of one expert), gathers those routes'
// activation rows through a row table in LDS, multiplies them by that expert's weight and
// writes each result to its route's output row; the per-row arithmetic (k order, MFMA
// shape, epilogue) is the dense form's, so a route's row equals the dense product of its
// activation row with the expert's weight.
//
// SWIGLU (grouped only): the tile's 256 columns are 128 gate columns and the matching 128
// up columns N/2 + ...; wave w takes gate columns 32w + [0, 32) of the block as its first
// 32-column subtile and the matching up columns as its second, so each lane holds g and u
// of the same outputs and writes bf16_rne(silu(g) * u) to a_out, g and u being exactly the
// per-route rows' values.
//
// SB: the weight scales come in 16-byte pieces, four 64-k steps of one column per load
// (K a multiple of 256, scale rows 16-byte aligned). A per-step 2-byte scale load touches
// a cache line per column for 2 bytes, as many line lookups in the vector L1 as the code
// loads themselves; the 16-byte piece serves four steps with one.
template <int MT, int ACT, bool GROUPED = false, bool SWIGLU = false, bool SB = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(GemmArgs a) {
  constexpr int BM = 32 * MT;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_a[];  // [2][BM * LDA]
  __shared__ int32_t row_x[GROUPED ? BM : 1];      // x row of each tile row (-1: none)
  __shared__ __attribute__((aligned(16))) int32_t row_route[GROUPED ? BM : 4];  // route of each tile row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t M = a.M, N = a.N, K = a.K;
  const uint32_t Ku = (uint32_t)K;
  const int64_t half = N >> 1;
  const int64_t nbn = SWIGLU ? (half + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;

  int64_t m0 = 0, n0, rows_m;
  // grouped: tile tile_of and column block cb_of of this workgroup. XCD x (blockIdx % 8)
  // takes the x-th eighth of the tile list, each tile with all its column blocks: a
  // tile's gathered activation rows are fetched into one XCD's L2, and so, mostly, are
  // the weights of an expert (its tiles are consecutive)
  const int64_t bx = blockIdx.x;
  const int64_t per_xcd = GROUPED ? (*a.n_tiles + 7) / 8 : 0;  // tiles per XCD
  const int64_t tile_of = (bx / 8) / nbn < per_xcd ? (bx % 8) * per_xcd + (bx / 8) / nbn
                                                   : INT64_MAX;  // past this XCD's share
  const int64_t cb_of = (bx / 8) % nbn;
  const uint8_t* wcodes = a.w_codes;
  const uint8_t* wscales = a.w_scales;
  float ts = a.w_ts[0];
  if (GROUPED) {
    const int64_t tile = tile_of;
    if (tile >= *a.n_tiles) return;  // uniform over the workgroup
    const int e = a.tiles[2 * tile];
    const int32_t beg = a.tiles[2 * tile + 1];
    const int32_t end = a.offsets[e + 1];
    rows_m = (end - beg) < BM ? (end - beg) : BM;
    n0 = cb_of * BN;
    wcodes += (int64_t)e * N * (K >> 1);
    wscales += (int64_t)e * N * (K >> 4);
    ts = a.apply_ts ? a.w_ts[e] : 1.0f;
    for (int i = tid; i < BM; i += 256) {
      const int32_t route = i < rows_m ? a.sorted[beg + i] : -1;
      row_route[i] = route;
      row_x[i] = route < 0 ? -1 : (a.rows_per_token ? route / a.top_k : route);
    }
    __syncthreads();
  } else {
    // XCD-aware tile order, weight-stationary: XCD x (blockIdx % 8) takes the column
    // tiles [x * nbn / 8, (x + 1) * nbn / 8) for every row tile, so it fetches an eighth
    // of the weight and all of the (here smaller) activation rows; otherwise consecutive
    // tiles of one XCD share the same rows.
    const int64_t nbm = (M + BM - 1) / BM;
    const int64_t total = nbm * nbn;
    const int64_t bid = blockIdx.x;
    if (nbn % 8 == 0) {
      const int64_t per = nbn / 8, j = bid / 8;
      m0 = (j / per) * BM;
      n0 = ((bid % 8) * per + j % per) * BN;
    } else {
      int64_t lin = bid;
      if (total % 8 == 0) lin = (bid % 8) * (total / 8) + bid / 8;
      m0 = (lin / nbn) * BM;
      n0 = (lin % nbn) * BN;
    }
    rows_m = (M - m0) < BM ? (M - m0) : BM;
  }
  const int64_t rows_n = (N - n0) < BN ? (N - n0) : BN;
  // this wave's weight column of subtile st and lane column col: n0 + 64 * wave + 32 st
  // + col, or for SwiGLU gate column cb * 128 + 32 * wave + col (st = 0) and the matching
  // up column N/2 + ... (st = 1)
  const int64_t scol0 = SWIGLU ? cb_of * (BN / 2) + 32 * wave : 0;  // SwiGLU gate column base
  auto wcol = [&](int st, int c) -> int64_t {
    return SWIGLU ? (st ? half : 0) + scol0 + c : n0 + 64 * wave + 32 * st + c;
  };
  auto wcol_ok = [&](int st, int c) -> bool {
    return SWIGLU ? scol0 + c < half : wcol(st, c) < N;
  };

  // activation descriptors: this tile's rows (dense) or all of x (grouped)
  __amdgpu_buffer_rsrc_t xr, xsr;
  {
    const int64_t xrow0 = GROUPED ? 0 : m0;
    const int64_t nrows = GROUPED ? a.x_rows : rows_m;
    if (ACT == 0) {
      xr = rsrc(static_cast<const uint16_t*>(a.x) + xrow0 * a.ldx, ((nrows - 1) * a.ldx + K) * 2);
      xsr = xr;
    } else {
      xr = rsrc(static_cast<const uint8_t*>(a.x) + xrow0 * (K >> 1), nrows * (K >> 1));
      xsr = rsrc(a.x_scales + xrow0 * (K >> 4), nrows * (K >> 4));
    }
  }
  // x row read for tile row `row` (relative to the descriptor), or -1
  auto xrow_of = [&](int row) -> int64_t {
    if (GROUPED) return row_x[row];
    return row < rows_m ? row : -1;
  };
  // weight descriptors over this tile's columns; lane (col, h): two 32-column subtiles,
  // K half h of each 64-k step
  const int col = lane & 31;
  const int h = lane >> 5;
  // descriptors over this tile's columns (dense) or the whole expert (grouped: its codes
  // fit 32-bit offsets)
  const int64_t wbase = GROUPED ? 0 : n0;
  const int64_t wrows = GROUPED ? N : rows_n;
  const auto wr = rsrc(wcodes + wbase * (K >> 1), wrows * (K >> 1));
  const auto sr = rsrc(wscales + wbase * (K >> 4), wrows * (K >> 4));
  uint32_t woff[2], soff[2];
#pragma unroll
  for (int st = 0; st < 2; st++) {
    const int64_t nl = wcol(st, col) - wbase;
    woff[st] = wcol_ok(st, col) ? (uint32_t)(nl * (K >> 1)) : kOOB;
    soff[st] = wcol_ok(st, col) ? (uint32_t)(nl * (K >> 4)) : kOOB;
  }

  const int KT = (int)((K + BK - 1) / BK);
  const int KT2 = KT + (KT & 1);  // even step count: an odd tail step reads zeros

  auto issue = [&](int kt, RegA<MT, ACT>& ra, RegB& rb) {
    const uint32_t k0 = (uint32_t)kt * BK;
    if (ACT == 0) {
#pragma unroll
      for (int q = 0; q < MT; q++) {
        const int c = tid + 256 * q;
        const int row = c >> 3, ch = c & 7;
        const uint32_t k = k0 + 8u * ch;
        const int64_t xrow = xrow_of(row);
        const uint32_t off = xrow < 0 ? kOOB : (uint32_t)(xrow * a.ldx * 2) + 2u * k;
        ra.v[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, off | past(Ku, k), 0, 0);
      }
    } else {
#pragma unroll
      for (int q = 0; q < MT; q++) {
        const int p = tid + 256 * q;
        const int row = p >> 3, j = p & 7;
        const uint32_t k = k0 + 8u * j;
        const int64_t xrow = xrow_of(row);
        const uint32_t oc = xrow < 0 ? kOOB : (uint32_t)(xrow * (K >> 1)) + (k >> 1);
        const uint32_t os = xrow < 0 ? kOOB : (uint32_t)(xrow * (K >> 4)) + (k >> 4);
        ra.c[q] = __builtin_amdgcn_raw_buffer_load_b32(xr, oc | past(Ku, k), 0, 0);
        ra.s[q] = __builtin_amdgcn_raw_buffer_load_b8(xsr, os | past(Ku, k), 0, 0);
      }
    }
    const uint32_t kh = k0 + 32u * h;
#pragma unroll
    for (int st = 0; st < 2; st++) {
      rb.c[st] = __builtin_amdgcn_raw_buffer_load_b128(wr, (woff[st] + (kh >> 1)) | past(Ku, kh), 0, 0);
      if (!SB)
        rb.s[st] = __builtin_amdgcn_raw_buffer_load_b16(sr, (soff[st] + (kh >> 4)) | past(Ku, kh), 0, 0);
    }
  };
  // SB: the scales of steps [kt, kt + 4) (kt a multiple of 4): 4 bytes per step, this
  // lane's two at byte 2h of each. The next piece is loaded once the current one's last
  // step is decoded.
  u32x4 sblk[2];  // [st]
  auto issue_sb = [&](int kt) {
    const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
    for (int st = 0; st < 2; st++)
      sblk[st] = __builtin_amdgcn_raw_buffer_load_b128(sr, (soff[st] + (k0 >> 4)) | past(Ku, k0), 0, 0);
  };
  const uint32_t hsh = 16u * h;

  auto write_a = [&](const RegA<MT, ACT>& ra, int buf) {
    uint16_t* dst = lds_a + buf * (BM * LDA);
    if (ACT == 0) {
#pragma unroll
      for (int q = 0; q < MT; q++) {
        const int c = tid + 256 * q;
        const int row = c >> 3, ch = c & 7;
        *reinterpret_cast<u32x4*>(dst + row * LDA + 8 * ch) = ra.v[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < MT; q++) {
        const int p = tid + 256 * q;
        const int row = p >> 3, j = p & 7;
        *reinterpret_cast<u32x4*>(dst + row * LDA + 8 * j) =
            decode8(ra.c[q], e4m3_to_f32<0>(ra.s[q]));  // exact BF16 activations
      }
    }
  };

  f32x16 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][st][r] = 0.f;

  // sw[st]: the step's two scale bytes in bytes 0 and 1 (SB: picked from the piece)
  auto decode = [&](const RegB& rb, const uint32_t (&sw)[2], u32x4 (&Bd)[2][4]) {
#pragma unroll
    for (int st = 0; st < 2; st++) {
      const float s0 = e4m3_to_f32<0>(sw[st]);
      const float s1 = e4m3_to_f32<1>(sw[st]);
#pragma unroll
      for (int j = 0; j < 4; j++) Bd[st][j] = decode8(rb.c[st][j], j < 2 ? s0 : s1);
    }
  };
  // the scale words of step kt: without SB the step's own loads; with SB dword kt % 4 of
  // the piece (compile-time in the unrolled loop)
  auto scales = [&](const RegB& rb, auto stepc, uint32_t (&sw)[2]) {
    constexpr int j = decltype(stepc)::value;
#pragma unroll
    for (int st = 0; st < 2; st++) sw[st] = SB ? sblk[st][j & 3] >> hsh : rb.s[st];
  };

  // One K step: refill the freed register sets with step kt + 2, multiply from LDS
  // buffer kt & 1 with this step's decoded weights while decoding step kt + 1's (the
  // decode's VALU work fills the MFMA pipeline's shadow), stage step kt + 1's
  // activations into the other buffer.
  // jc: kt % 4 as a compile-time constant (it selects the scale word with SB)
  auto body = [&](auto jc, int kt, RegA<MT, ACT>& ra_free, RegB& rb_free, RegA<MT, ACT>& ra_next,
                  const RegB& rb_next, const u32x4 (&Bd)[2][4], u32x4 (&Bd_next)[2][4]) {
    constexpr int j4 = decltype(jc)::value;
    issue(kt + 2, ra_free, rb_free);
    // 32-route tiles: the loads stay at the step's top, a whole step ahead of their decode
    if constexpr (MT == 1) __builtin_amdgcn_sched_barrier(0);
    const uint16_t* src = lds_a + (kt & 1) * (BM * LDA);
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const u32x4 A =
            *reinterpret_cast<const u32x4*>(src + (32 * mt + col) * LDA + 32 * h + 8 * j);
#pragma unroll
        for (int st = 0; st < 2; st++) acc[mt][st] = mfma32(A, Bd[st][j], acc[mt][st]);
      }
    }
    uint32_t sw[2];
    scales(rb_next, std::integral_constant<int, (j4 + 1) & 3>{}, sw);
    decode(rb_next, sw, Bd_next);
    // step kt + 1 was the piece's last: load the next one (steps kt + 2 ... kt + 5)
    if constexpr (SB && j4 == 2) issue_sb(kt + 2);
    // interleave: each MFMA followed by a share of the decode's VALU work, with the LDS
    // operand reads spread between them (NVFP4 activations: a smaller share per MFMA,
    // which keeps the 128-row grouped form within its 256 registers, no scratch)
    constexpr int kValuShare = ACT == 0 ? 160 / (8 * MT) + 1 : 4;
#pragma unroll
    for (int i = 0; i < 8 * MT; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // one MFMA
      if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, kValuShare, 0);  // VALU
    }
    write_a(ra_next, (kt + 1) & 1);
    // Keep the next step's decode below the barrier: the scheduler otherwise lifts that
    // pure VALU work into this step, where it must first wait for the loads issued here
    // (measured: the 32- and 128-route grouped forms 2-3 % faster; the dense 64-row form
    // is faster without it).
    if constexpr (MT != 2) __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    if constexpr (MT != 2) __builtin_amdgcn_sched_barrier(0);
  };

  RegA<MT, ACT> ra0, ra1;
  RegB rb0, rb1;
  u32x4 Bd0[2][4], Bd1[2][4];
  using I0 = std::integral_constant<int, 0>;
  if (SB) issue_sb(0);
  issue(0, ra0, rb0);
  issue(1, ra1, rb1);
  {
    uint32_t sw[2];
    scales(rb0, I0{}, sw);
    decode(rb0, sw, Bd0);
  }
  write_a(ra0, 0);
  __syncthreads();
  if constexpr (SB) {
    // K is whole 4-step pieces (KT2 = KT, a multiple of 4)
    for (int kt = 0; kt < KT2; kt += 4) {
      body(I0{}, kt, ra0, rb0, ra1, rb1, Bd0, Bd1);
      body(std::integral_constant<int, 1>{}, kt + 1, ra1, rb1, ra0, rb0, Bd1, Bd0);
      body(std::integral_constant<int, 2>{}, kt + 2, ra0, rb0, ra1, rb1, Bd0, Bd1);
      body(std::integral_constant<int, 3>{}, kt + 3, ra1, rb1, ra0, rb0, Bd1, Bd0);
    }
  } else {
    for (int kt = 0; kt < KT2; kt += 2) {
      body(I0{}, kt, ra0, rb0, ra1, rb1, Bd0, Bd1);
      body(std::integral_constant<int, 1>{}, kt + 1, ra1, rb1, ra0, rb0, Bd1, Bd0);
    }
  }

  // BF16 activations: branch-free stores through one descriptor over the output (grouped:
  // every route's row; dense: the tile's rows), rows without a route, rows past M and
  // columns past the end at out-of-range offsets, while the output fits 32-bit offsets
  if (ACT == 0) {
    const int64_t nroutes = a.rows_per_token ? a.x_rows * a.top_k : a.x_rows;
    const int64_t span = SWIGLU ? nroutes * half * 2
                                : (GROUPED ? nroutes * a.ldy * 4 : rows_m * a.ldy * 4);
    if (span < ((int64_t)1 << 31)) {
      const auto yr = SWIGLU ? rsrc(a.a_out, span) : rsrc(GROUPED ? a.y : a.y + m0 * a.ldy, span);
      const uint32_t pitch = SWIGLU ? (uint32_t)half : (uint32_t)a.ldy;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int g4 = 0; g4 < 4; g4++) {
          const int lrow0 = 32 * mt + 8 * g4 + 4 * h;
          int4 rt = make_int4(lrow0, lrow0 + 1, lrow0 + 2, lrow0 + 3);
          if (GROUPED) rt = *reinterpret_cast<const int4*>(&row_route[lrow0]);
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int r = 4 * g4 + q;
            const int32_t row = q == 0 ? rt.x : q == 1 ? rt.y : q == 2 ? rt.z : rt.w;
            if (SWIGLU) {
              const uint32_t off = row < 0 || !wcol_ok(0, col)
                                       ? kOOB : ((uint32_t)row * pitch + (uint32_t)(scol0 + col)) * 2u;
              const float g = acc[mt][0][r] * ts;
              const float u = acc[mt][1][r] * ts;
              __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(silu(g) * u), yr, off,
                                                    0, 0);
            } else {
#pragma unroll
              for (int st = 0; st < 2; st++) {
                const int64_t n = n0 + 64 * wave + 32 * st + col;
                const uint32_t off = row < 0 || n >= N ? kOOB : ((uint32_t)row * pitch + (uint32_t)n) * 4u;
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(uint32_t, acc[mt][st][r] * ts), yr, off, 0, 0);
              }
            }
          }
        }
      return;
    }
  }
  if (SWIGLU) {
    // g in subtile 0, u in subtile 1 of the same lane
    if (!wcol_ok(0, col)) return;
    const int64_t n = scol0 + col;
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int lrow = 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t route = row_route[lrow];
        if (route < 0) continue;
        const int64_t xrow = row_x[lrow];
        const float f = (ACT == 0) ? ts : a.x_ts[xrow] * ts;
        const float g = acc[mt][0][r] * f;
        const float u = acc[mt][1][r] * f;
        a.a_out[route * half + n] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
      }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int lrow = 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
      int64_t row, xrow;
      if (GROUPED) {
        row = row_route[lrow];
        xrow = row_x[lrow];
        if (row < 0) continue;
      } else {
        row = m0 + lrow;
        xrow = row;
        if (row >= M) continue;
      }
      const float f = (ACT == 0) ? ts : a.x_ts[xrow] * ts;
#pragma unroll
      for (int st = 0; st < 2; st++) {
        const int64_t n = n0 + 64 * wave + 32 * st + col;
        if (n < N) a.y[row * a.ldy + n] = acc[mt][st][r] * f;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// gemm_wide: 256 x 256 tiles, wave-specialized. Eight consumer waves (two along M, four
// along N, each 128 x 64) only read LDS and run MFMAs; four producer waves only load,
// decode and write LDS, so no wave both waits on global loads and feeds the MFMA pipe.
// Both operand stages are double buffered in LDS (147 KB) with one workgroup barrier per 64-k
// step: between barriers the producers write step kt + 1's stage while the consumers
// multiply step kt's. The producers hold two register sets of loads, issued two steps
// ahead. Each output element sums its K products in the same order as the 64-row kernel
// (the same 32x32x16 MFMA chain over the same k), so rows do not depend on the tiling.
// ---------------------------------------------------------------------------------------
constexpr int kWideBM = 256;

template <int ACT>
struct RegAP {  // one K step of a producer lane's activation loads (8 chunks)
  u32x4 v[ACT == 0 ? 8 : 1];
  uint32_t c[ACT == 0 ? 1 : 8];
  uint32_t s[ACT == 0 ? 1 : 8];
};
struct RegBP {  // one K step of a producer lane's weight chunks (two of 32 codes)
  u32x4 c[2];
  uint32_t s[2];
};

template <int ACT, bool SB = false>
__global__ __launch_bounds__(768) void gemm_wide(GemmArgs a) {
  constexpr int BM = kWideBM;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* As = lds;                 // [2][BM * LDA]  activations [row][k]
  uint16_t* Bs = lds + 2 * BM * LDA;  // [2][BN * LDA]  decoded weight [column][k]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: the role branch is uniform
  const int64_t M = a.M, N = a.N, K = a.K;
  const uint32_t Ku = (uint32_t)K;

  const int64_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int64_t total = nbm * nbn;
  const int64_t bid = blockIdx.x;
  int64_t lin = bid;
  if (total % 8 == 0) lin = (bid % 8) * (total / 8) + bid / 8;
  const int64_t m0 = (lin / nbn) * BM;
  const int64_t n0 = (lin % nbn) * BN;
  const int64_t rows_m = (M - m0) < BM ? (M - m0) : BM;
  const int64_t rows_n = (N - n0) < BN ? (N - n0) : BN;
  const int KT = (int)((K + BK - 1) / BK);
  const int KT2 = KT + (KT & 1);  // whole rounds of the two register sets

  if (wave >= 8) {
    // descriptors from values made explicitly scalar (the role branch would otherwise leave
    // them in vector registers, and every load would loop over the lanes' descriptors)
    auto uni = [](const void* p) -> const void* {
      const uint64_t v = (uint64_t)(uintptr_t)p;
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    };
    auto uni64 = [](int64_t v) -> int64_t {
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
      return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    __amdgpu_buffer_rsrc_t xr, xsr;
    if (ACT == 0) {
      xr = rsrc(uni(static_cast<const uint16_t*>(a.x) + m0 * a.ldx), uni64(((rows_m - 1) * a.ldx + K) * 2));
      xsr = xr;
    } else {
      xr = rsrc(uni(static_cast<const uint8_t*>(a.x) + m0 * (K >> 1)), uni64(rows_m * (K >> 1)));
      xsr = rsrc(uni(a.x_scales + m0 * (K >> 4)), uni64(rows_m * (K >> 4)));
    }
    const auto wr = rsrc(uni(a.w_codes + n0 * (K >> 1)), uni64(rows_n * (K >> 1)));
    const auto sr = rsrc(uni(a.w_scales + n0 * (K >> 4)), uni64(rows_n * (K >> 4)));
    // ---------------- producers: 256 lanes ----------------
    const int pt = tid - 512;
    uint32_t bwoff[2], bsoff[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int bc = (pt + 256 * q) >> 1;
      bwoff[q] = bc < rows_n ? (uint32_t)(bc * (K >> 1)) : kOOB;
      bsoff[q] = bc < rows_n ? (uint32_t)(bc * (K >> 4)) : kOOB;
    }
    auto issue = [&](int kt, RegAP<ACT>& ra, RegBP& rb) {
      const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const uint32_t kh = k0 + 32u * ((pt + 256 * q) & 1);
        if (!SB)
          rb.s[q] = __builtin_amdgcn_raw_buffer_load_b16(sr, (bsoff[q] + (kh >> 4)) | past(Ku, kh), 0, 0);
        rb.c[q] = __builtin_amdgcn_raw_buffer_load_b128(wr, (bwoff[q] + (kh >> 1)) | past(Ku, kh), 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int c = pt + 256 * q;
        const int row = c >> 3, j = c & 7;
        const uint32_t k = k0 + 8u * j;
        if (ACT == 0) {
          const uint32_t off = (uint32_t)(row * a.ldx * 2) + 2u * k;
          ra.v[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, off | past(Ku, k), 0, 0);
        } else {
          ra.c[q] = __builtin_amdgcn_raw_buffer_load_b32(
              xr, ((uint32_t)(row * (K >> 1)) + (k >> 1)) | past(Ku, k), 0, 0);
          ra.s[q] = __builtin_amdgcn_raw_buffer_load_b8(
              xsr, ((uint32_t)(row * (K >> 4)) + (k >> 4)) | past(Ku, k), 0, 0);
        }
      }
    };
    auto write_stage = [&](const RegAP<ACT>& ra, const RegBP& rb, const uint32_t (&sw)[2], int buf) {
      uint16_t* da = As + buf * (BM * LDA);
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int c = pt + 256 * q;
        const int row = c >> 3, j = c & 7;
        u32x4 v;
        if (ACT == 0) v = ra.v[q];
        else v = decode8(ra.c[q], e4m3_to_f32<0>(ra.s[q]));  // exact BF16 activations
        *reinterpret_cast<u32x4*>(da + row * LDA + 8 * j) = v;
      }
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const int c = pt + 256 * q;
        const int bc = c >> 1, bh = c & 1;
        uint16_t* db = Bs + buf * (BN * LDA) + bc * LDA + 32 * bh;
        const float s0 = e4m3_to_f32<0>(sw[q]), s1 = e4m3_to_f32<1>(sw[q]);
#pragma unroll
        for (int d = 0; d < 4; d++)
          *reinterpret_cast<u32x4*>(db + 8 * d) = decode8(rb.c[q][d], d < 2 ? s0 : s1);
      }
    };
    // SB: the scales of steps [kt, kt + 4) (kt a multiple of 4), 4 bytes per step, this
    // lane's two at byte 2 * (lane's K half) of each. The next piece is loaded once the
    // current one's last step is staged.
    u32x4 sblk[2];  // [q]
    auto issue_sb = [&](int kt) {
      const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
      for (int q = 0; q < 2; q++)
        sblk[q] = __builtin_amdgcn_raw_buffer_load_b128(sr, (bsoff[q] + (k0 >> 4)) | past(Ku, k0), 0, 0);
    };
    const uint32_t hsh = 16u * (pt & 1);
    // the scale words of step j (mod 4, compile-time)
    auto scales = [&](const RegBP& rb, auto stepc, uint32_t (&sw)[2]) {
      constexpr int j = decltype(stepc)::value;
#pragma unroll
      for (int q = 0; q < 2; q++) sw[q] = SB ? sblk[q][j & 3] >> hsh : rb.s[q];
    };
    RegAP<ACT> ra[2];
    RegBP rb[2];
    using I0 = std::integral_constant<int, 0>;
    if (SB) issue_sb(0);
    issue(0, ra[0], rb[0]);
    issue(1, ra[1], rb[1]);
    {
      uint32_t sw[2];
      scales(rb[0], I0{}, sw);
      write_stage(ra[0], rb[0], sw, 0);
    }
    issue(2, ra[0], rb[0]);
    __syncthreads();  // stage 0 ready
    // step kt: write step kt + 1's stage from set (kt + 1) % 2, refill that set with step
    // kt + 3; one barrier per step, matched by the consumers'
    // jc: kt % 4 as a compile-time constant (it selects the scale word with SB)
    auto pstep = [&](auto jc, int kt, RegAP<ACT>& ran, RegBP& rbn) {
      constexpr int j4 = decltype(jc)::value;
      uint32_t sw[2];
      scales(rbn, std::integral_constant<int, (j4 + 1) & 3>{}, sw);
      write_stage(ran, rbn, sw, (kt + 1) & 1);
      // step kt + 1 was the piece's last: load the next one (steps kt + 2 ... kt + 5)
      if constexpr (SB && j4 == 2) issue_sb(kt + 2);
      issue(kt + 3, ran, rbn);
      __syncthreads();
    };
    if constexpr (SB) {
      // K is whole 4-step pieces (KT2 = KT, a multiple of 4)
      for (int kt = 0; kt < KT2; kt += 4) {
        pstep(I0{}, kt, ra[1], rb[1]);
        pstep(std::integral_constant<int, 1>{}, kt + 1, ra[0], rb[0]);
        pstep(std::integral_constant<int, 2>{}, kt + 2, ra[1], rb[1]);
        pstep(std::integral_constant<int, 3>{}, kt + 3, ra[0], rb[0]);
      }
    } else {
      for (int kt = 0; kt < KT2; kt += 2) {
        pstep(I0{}, kt, ra[1], rb[1]);
        pstep(std::integral_constant<int, 1>{}, kt + 1, ra[0], rb[0]);
      }
    }
    return;
  }

  // ---------------- consumers: 8 waves ----------------
  const int wm = wave >> 2, wn = wave & 3;
  const int col = lane & 31;
  const int h = lane >> 5;
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][st][r] = 0.f;
  __syncthreads();  // stage 0 ready
  for (int kt = 0; kt < KT2; kt++) {
    const uint16_t* sa = As + (kt & 1) * (BM * LDA) + (128 * wm + col) * LDA + 32 * h;
    const uint16_t* sb = Bs + (kt & 1) * (BN * LDA) + (64 * wn + col) * LDA + 32 * h;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      u32x4 B[2];
#pragma unroll
      for (int st = 0; st < 2; st++)
        B[st] = *reinterpret_cast<const u32x4*>(sb + 32 * st * LDA + 8 * j);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const u32x4 A = *reinterpret_cast<const u32x4*>(sa + 32 * mt * LDA + 8 * j);
#pragma unroll
        for (int st = 0; st < 2; st++) acc[mt][st] = mfma32(A, B[st], acc[mt][st]);
      }
    }
    __syncthreads();
  }

  const float ts = a.w_ts[0];
  if (ACT == 0 && rows_m * a.ldy * 4 < ((int64_t)1 << 31)) {
    // Branch-free stores through a descriptor over the tile's rows: rows past M fall
    // outside its range, columns past N take an out-of-range offset.
    const auto yr = rsrc(a.y + m0 * a.ldy, rows_m * a.ldy * 4);
    const uint32_t ldy = (uint32_t)a.ldy;
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const uint32_t lrow = 128 * wm + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int st = 0; st < 2; st++) {
          const int64_t n = n0 + 64 * wn + 32 * st + col;
          const uint32_t off = n < N ? (lrow * ldy + (uint32_t)n) * 4u : kOOB;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[mt][st][r] * ts),
                                                yr, off, 0, 0);
        }
      }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t row = m0 + 128 * wm + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= M) continue;
      const float f = (ACT == 0) ? ts : a.x_ts[row] * ts;
#pragma unroll
      for (int st = 0; st < 2; st++) {
        const int64_t n = n0 + 64 * wn + 32 * st + col;
        if (n < N) a.y[row * a.ldy + n] = acc[mt][st][r] * f;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// gemm_wide_grouped: the wide wave-specialized tile on an expert's routes. Workgroup
// (tile t, column block cb) takes active expert t's first routes (up to 256; the rest of
// the expert's routes are in the grouping's tile list, for the 64-row grouped kernel),
// gathers their activation rows through a row table in LDS and multiplies them by that
// expert's weight. Operands, stages, MFMA chain and k order are gemm_wide's, and the
// epilogue is the grouped 64/128-row kernel's, so a route's row is the dense product bit
// for bit.
//
// SWIGLU: the tile's 256 columns are 128 gate columns and the matching 128 up columns
// N/2 + ...: consumer wave wn takes gate columns 32 wn + [0, 32) of the block as its first
// 32-column subtile and the matching up columns as its second, so each lane holds g and u
// of the same outputs and writes bf16_rne(silu(g) * u).
// ---------------------------------------------------------------------------------------
template <int ACT, bool SWIGLU, bool SB = false>
__global__ __launch_bounds__(768) void gemm_wide_grouped(GemmArgs a) {
  constexpr int BM = kWideBM;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* As = lds;                 // [2][BM * LDA]  activations [row][k]
  uint16_t* Bs = lds + 2 * BM * LDA;  // [2][BN * LDA]  decoded weight [column][k]
  __shared__ int32_t row_x[BM];       // x row of each tile row (-1: none)
  __shared__ int32_t row_route[BM];   // route of each tile row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = a.N, K = a.K;
  const uint32_t Ku = (uint32_t)K;
  const int64_t half = N >> 1;
  const int64_t nbn = SWIGLU ? (half + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;

  // XCD x (blockIdx % 8) takes the x-th eighth of the active list, each expert with all
  // its column blocks: the gathered rows of a tile are fetched into one XCD's L2
  const int64_t bx = blockIdx.x;
  const int64_t n_act = *a.n_active;
  const int64_t per_xcd = (n_act + 7) / 8;
  const int64_t t = (bx / 8) / nbn < per_xcd ? (bx % 8) * per_xcd + (bx / 8) / nbn : INT64_MAX;
  if (t >= n_act) return;  // uniform over the workgroup, before any barrier
  const int64_t cb = (bx / 8) % nbn;
  const int e = a.active[t];
  const int32_t beg = a.offsets[e];
  const int32_t cnt = a.offsets[e + 1] - beg;
  const int rows_m = cnt < BM ? cnt : BM;
  const float ts = a.apply_ts ? a.w_ts[e] : 1.0f;
  for (int i = tid; i < BM; i += 768) {
    const int32_t route = i < rows_m ? a.sorted[beg + i] : -1;
    row_route[i] = route;
    row_x[i] = route < 0 ? -1 : (a.rows_per_token ? route / a.top_k : route);
  }
  __syncthreads();  // row table ready

  const int KT = (int)((K + BK - 1) / BK);
  const int KT2 = KT + (KT & 1);  // whole rounds of the two register sets

  if (wave >= 8) {
    auto uni = [](const void* p) -> const void* {
      const uint64_t v = (uint64_t)(uintptr_t)p;
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    };
    auto uni64 = [](int64_t v) -> int64_t {
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
      return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    // all of x (rows gathered by the row table) and all of expert e's weight
    __amdgpu_buffer_rsrc_t xr, xsr;
    if (ACT == 0) {
      xr = rsrc(uni(a.x), uni64(((a.x_rows - 1) * a.ldx + K) * 2));
      xsr = xr;
    } else {
      xr = rsrc(uni(a.x), uni64(a.x_rows * (K >> 1)));
      xsr = rsrc(uni(a.x_scales), uni64(a.x_rows * (K >> 4)));
    }
    const auto wr = rsrc(uni(a.w_codes + (int64_t)e * N * (K >> 1)), uni64(N * (K >> 1)));
    const auto sr = rsrc(uni(a.w_scales + (int64_t)e * N * (K >> 4)), uni64(N * (K >> 4)));
    // ---------------- producers: 256 lanes ----------------
    const int pt = tid - 512;
    // this lane's 8 activation chunks: tile row (pt + 256 q) / 8, 16 bytes at chunk pt % 8
    uint32_t xoff[8], xsoff[ACT == 0 ? 1 : 8];
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const int32_t xrow = row_x[(pt + 256 * q) >> 3];
      if (ACT == 0) {
        xoff[q] = xrow < 0 ? kOOB : (uint32_t)(xrow * a.ldx * 2);
      } else {
        xoff[q] = xrow < 0 ? kOOB : (uint32_t)(xrow * (K >> 1));
        xsoff[q] = xrow < 0 ? kOOB : (uint32_t)(xrow * (K >> 4));
      }
    }
    // this lane's 2 weight chunks: tile column (pt + 256 q) / 2, K half (pt + 256 q) % 2
    uint32_t bwoff[2], bsoff[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int bc = (pt + 256 * q) >> 1;
      int64_t wrow;
      bool ok;
      if (SWIGLU) {
        // tile column bc = 64 wn + 32 st + j: gate (st = 0) or up (st = 1) column
        // cb * 128 + 32 wn + j
        const int64_t c = cb * (BN / 2) + 32 * (bc >> 6) + (bc & 31);
        wrow = ((bc >> 5) & 1 ? half : 0) + c;
        ok = c < half;
      } else {
        wrow = cb * BN + bc;
        ok = wrow < N;
      }
      bwoff[q] = ok ? (uint32_t)(wrow * (K >> 1)) : kOOB;
      bsoff[q] = ok ? (uint32_t)(wrow * (K >> 4)) : kOOB;
    }
    auto issue = [&](int kt, RegAP<ACT>& ra, RegBP& rb) {
      const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const uint32_t kh = k0 + 32u * ((pt + 256 * q) & 1);
        if (!SB)
          rb.s[q] = __builtin_amdgcn_raw_buffer_load_b16(sr, (bsoff[q] + (kh >> 4)) | past(Ku, kh), 0, 0);
        rb.c[q] = __builtin_amdgcn_raw_buffer_load_b128(wr, (bwoff[q] + (kh >> 1)) | past(Ku, kh), 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int j = (pt + 256 * q) & 7;
        const uint32_t k = k0 + 8u * j;
        if (ACT == 0) {
          ra.v[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (xoff[q] + 2u * k) | past(Ku, k), 0, 0);
        } else {
          ra.c[q] = __builtin_amdgcn_raw_buffer_load_b32(xr, (xoff[q] + (k >> 1)) | past(Ku, k), 0, 0);
          ra.s[q] = __builtin_amdgcn_raw_buffer_load_b8(xsr, (xsoff[q] + (k >> 4)) | past(Ku, k), 0, 0);
        }
      }
    };
    auto write_stage = [&](const RegAP<ACT>& ra, const RegBP& rb, const uint32_t (&sw)[2], int buf) {
      uint16_t* da = As + buf * (BM * LDA);
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int c = pt + 256 * q;
        const int row = c >> 3, j = c & 7;
        u32x4 v;
        if (ACT == 0) v = ra.v[q];
        else v = decode8(ra.c[q], e4m3_to_f32<0>(ra.s[q]));  // exact BF16 activations
        *reinterpret_cast<u32x4*>(da + row * LDA + 8 * j) = v;
      }
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const int c = pt + 256 * q;
        const int bc = c >> 1, bh = c & 1;
        uint16_t* db = Bs + buf * (BN * LDA) + bc * LDA + 32 * bh;
        const float s0 = e4m3_to_f32<0>(sw[q]), s1 = e4m3_to_f32<1>(sw[q]);
#pragma unroll
        for (int d = 0; d < 4; d++)
          *reinterpret_cast<u32x4*>(db + 8 * d) = decode8(rb.c[q][d], d < 2 ? s0 : s1);
      }
    };
    // SB: the scales of steps [kt, kt + 4) (kt a multiple of 4), 4 bytes per step, this
    // lane's two at byte 2 * (lane's K half) of each. The next piece is loaded once the
    // current one's last step is staged.
    u32x4 sblk[2];  // [q]
    auto issue_sb = [&](int kt) {
      const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
      for (int q = 0; q < 2; q++)
        sblk[q] = __builtin_amdgcn_raw_buffer_load_b128(sr, (bsoff[q] + (k0 >> 4)) | past(Ku, k0), 0, 0);
    };
    const uint32_t hsh = 16u * (pt & 1);
    // the scale words of step j (mod 4, compile-time)
    auto scales = [&](const RegBP& rb, auto stepc, uint32_t (&sw)[2]) {
      constexpr int j = decltype(stepc)::value;
#pragma unroll
      for (int q = 0; q < 2; q++) sw[q] = SB ? sblk[q][j & 3] >> hsh : rb.s[q];
    };
    RegAP<ACT> ra[2];
    RegBP rb[2];
    using I0 = std::integral_constant<int, 0>;
    if (SB) issue_sb(0);
    issue(0, ra[0], rb[0]);
    issue(1, ra[1], rb[1]);
    {
      uint32_t sw[2];
      scales(rb[0], I0{}, sw);
      write_stage(ra[0], rb[0], sw, 0);
    }
    issue(2, ra[0], rb[0]);
    __syncthreads();  // stage 0 ready
    // jc: kt % 4 as a compile-time constant (it selects the scale word with SB)
    auto pstep = [&](auto jc, int kt, RegAP<ACT>& ran, RegBP& rbn) {
      constexpr int j4 = decltype(jc)::value;
      uint32_t sw[2];
      scales(rbn, std::integral_constant<int, (j4 + 1) & 3>{}, sw);
      write_stage(ran, rbn, sw, (kt + 1) & 1);
      // step kt + 1 was the piece's last: load the next one (steps kt + 2 ... kt + 5)
      if constexpr (SB && j4 == 2) issue_sb(kt + 2);
      issue(kt + 3, ran, rbn);
      __syncthreads();
    };
    if constexpr (SB) {
      // K is whole 4-step pieces (KT2 = KT, a multiple of 4)
      for (int kt = 0; kt < KT2; kt += 4) {
        pstep(I0{}, kt, ra[1], rb[1]);
        pstep(std::integral_constant<int, 1>{}, kt + 1, ra[0], rb[0]);
        pstep(std::integral_constant<int, 2>{}, kt + 2, ra[1], rb[1]);
        pstep(std::integral_constant<int, 3>{}, kt + 3, ra[0], rb[0]);
      }
    } else {
      for (int kt = 0; kt < KT2; kt += 2) {
        pstep(I0{}, kt, ra[1], rb[1]);
        pstep(std::integral_constant<int, 1>{}, kt + 1, ra[0], rb[0]);
      }
    }
    return;
  }

  // ---------------- consumers: 8 waves ----------------
  const int wm = wave >> 2, wn = wave & 3;
  const int col = lane & 31;
  const int h = lane >> 5;
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][st][r] = 0.f;
  __syncthreads();  // stage 0 ready
  for (int kt = 0; kt < KT2; kt++) {
    const uint16_t* sa = As + (kt & 1) * (BM * LDA) + (128 * wm + col) * LDA + 32 * h;
    const uint16_t* sb = Bs + (kt & 1) * (BN * LDA) + (64 * wn + col) * LDA + 32 * h;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      u32x4 B[2];
#pragma unroll
      for (int st = 0; st < 2; st++)
        B[st] = *reinterpret_cast<const u32x4*>(sb + 32 * st * LDA + 8 * j);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const u32x4 A = *reinterpret_cast<const u32x4*>(sa + 32 * mt * LDA + 8 * j);
#pragma unroll
        for (int st = 0; st < 2; st++) acc[mt][st] = mfma32(A, B[st], acc[mt][st]);
      }
    }
    __syncthreads();
  }

  if (SWIGLU) {
    // g in subtile 0, u in subtile 1 of the same lane
    const int64_t n = cb * (BN / 2) + 32 * wn + col;
    if (n >= half) return;
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int lrow = 128 * wm + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t route = row_route[lrow];
        if (route < 0) continue;
        const int64_t xrow = row_x[lrow];
        const float f = (ACT == 0) ? ts : a.x_ts[xrow] * ts;
        const float g = acc[mt][0][r] * f;
        const float u = acc[mt][1][r] * f;
        a.a_out[route * half + n] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
      }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int lrow = 128 * wm + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
      const int64_t route = row_route[lrow];
      if (route < 0) continue;
      const int64_t xrow = row_x[lrow];
      const float f = (ACT == 0) ? ts : a.x_ts[xrow] * ts;
#pragma unroll
      for (int st = 0; st < 2; st++) {
        const int64_t n = cb * BN + 64 * wn + 32 * st + col;
        if (n < N) a.y[route * a.ldy + n] = acc[mt][st][r] * f;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// gemm_wide_grouped_p: the wide grouped form as a persistent pipeline. One workgroup per
// CU takes its XCD's tiles in turn: tile j = blockIdx / 8 + i * (gridDim / 8) of XCD
// blockIdx % 8's share (gridDim a multiple of 8), the order of gemm_wide_grouped, so a
// workgroup's tiles stay on its XCD. The producers' steps run on from one tile into the
// next: the next tile's first loads are issued three steps before the current tile ends,
// its row table is written during the current tile's first steps, and its operand
// offsets are read back from that table just before its first loads.
// The consumers store a tile's results while the producers stage the next tile, so the
// stores at the end of a tile overlap the next tile's steps instead of ending a round of
// workgroups together. Per tile the arithmetic (MFMA chain, k order, epilogue) is
// gemm_wide_grouped's, so every result is the same bits.
// DENSE: the plain product of gemm_wide (BF16 activations, rows [M] of x and y): the
// tiles of the 256 x 256 grid in gemm_wide's order, XCD x taking the x-th eighth of them
// (for the prefill shape one row block each), and the identity as each tile's row table.
// ---------------------------------------------------------------------------------------
constexpr int kPersistMaxTiles = 256;  // tiles per workgroup: one header per producer lane

template <int ACT>
struct PState {  // a tile's operand offsets for the producer lane
  uint32_t xoff[8];
  uint32_t xsoff[ACT == 0 ? 1 : 8];
  uint32_t bwoff[2], bsoff[2];
  __amdgpu_buffer_rsrc_t wr, sr;
};

template <int ACT, bool SWIGLU, bool SB, bool DENSE = false>
__global__ __launch_bounds__(768) void gemm_wide_grouped_p(GemmArgs a) {
  constexpr int BM = kWideBM;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* As = lds;                 // [2][BM * LDA]  activations [row][k]
  uint16_t* Bs = lds + 2 * BM * LDA;  // [2][BN * LDA]  decoded weight [column][k]
  __shared__ int32_t row_x[2][BM];    // per tile parity: x row of each tile row (-1: none)
  __shared__ int32_t row_route[2][BM];
  __shared__ int4 hdr[kPersistMaxTiles];  // per tile: expert, first route, routes, column block
  __shared__ float hts[kPersistMaxTiles];  // per tile: the expert's tensor scale (or 1)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = a.N, K = a.K;
  const uint32_t Ku = (uint32_t)K;
  const int64_t half = N >> 1;
  const int64_t nbn = SWIGLU ? (half + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;

  const int64_t xcd = blockIdx.x % 8, jb = blockIdx.x / 8, jstep = gridDim.x / 8;
  // this XCD's share: active experts (each with its column blocks), or dense tiles
  const int64_t n_units = DENSE ? ((a.M + BM - 1) / BM) * nbn : *a.n_active;
  const int64_t per_xcd = (n_units + 7) / 8;
  const int64_t tx = n_units - xcd * per_xcd;  // units in this XCD's share
  const int64_t J = (DENSE ? 1 : nbn) * (tx <= 0 ? 0 : (tx < per_xcd ? tx : per_xcd));
  const int ntiles = jb < J ? (int)((J - jb + jstep - 1) / jstep) : 0;
  if (ntiles == 0) return;  // uniform over the workgroup, before any barrier

  const int KT = (int)((K + BK - 1) / BK);
  const int KT2 = KT + (KT & 1);  // whole rounds of the two register sets (>= 8 here)

  if (wave >= 8 && tid - 512 < ntiles) {
    const int i = tid - 512;
    const int64_t j = jb + (int64_t)i * jstep;
    if (DENSE) {
      // header: expert 0, first row, rows, column block
      const int64_t lin = xcd * per_xcd + j;
      const int64_t m0 = (lin / nbn) * BM;
      hdr[i] = make_int4(0, (int)m0, (int)(a.M - m0 < BM ? a.M - m0 : BM), (int)(lin % nbn));
      hts[i] = a.w_ts[0];
    } else {
      const int e = a.active[xcd * per_xcd + j / nbn];
      const int32_t beg = a.offsets[e];
      const int32_t cnt = a.offsets[e + 1] - beg;
      hdr[i] = make_int4(e, beg, cnt < BM ? cnt : BM, (int)(j % nbn));
      // read here, before any store: once the kernel has stored, a load of w_ts may no
      // longer be a scalar load, and a vector load in the epilogue would make the
      // compiler wait for all earlier stores at each of its joins
      hts[i] = a.apply_ts ? a.w_ts[e] : 1.0f;
    }
  }
  __syncthreads();  // headers ready
  // tile 0's row table (each producer lane writes its row pt)
  if (wave >= 8) {
    const int pt = tid - 512;
    const int4 h0 = hdr[0];
    const int32_t route = pt < h0.z ? (DENSE ? h0.y + pt : a.sorted[h0.y + pt]) : -1;
    row_route[0][pt] = route;
    row_x[0][pt] = route < 0 ? -1 : (a.rows_per_token ? route / a.top_k : route);
  }
  __syncthreads();  // tile 0's row table ready

  if (wave >= 8) {
    auto uni = [](const void* p) -> const void* {
      const uint64_t v = (uint64_t)(uintptr_t)p;
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    };
    auto uni64 = [](int64_t v) -> int64_t {
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
      return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    __amdgpu_buffer_rsrc_t xr, xsr;
    if (ACT == 0) {
      xr = rsrc(uni(a.x), uni64(((a.x_rows - 1) * a.ldx + K) * 2));
      xsr = xr;
    } else {
      xr = rsrc(uni(a.x), uni64(a.x_rows * (K >> 1)));
      xsr = rsrc(uni(a.x_scales), uni64(a.x_rows * (K >> 4)));
    }
    const int pt = tid - 512;
    // tiles past the last have no rows
    const int4 nohdr = make_int4(0, 0, 0, 0);
    auto tile_hdr = [&](int i) -> int4 { return i < ntiles ? hdr[i] : nohdr; };
    // a tile's operand offsets from its header and its row table (parity buf)
    auto make_state = [&](const int4& h, PState<ACT>& st, int buf) {
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int64_t xrow = row_x[buf][(pt >> 3) + 32 * q];
        if (ACT == 0) {
          st.xoff[q] = xrow < 0 ? kOOB : (uint32_t)(xrow * a.ldx * 2);
        } else {
          st.xoff[q] = xrow < 0 ? kOOB : (uint32_t)(xrow * (K >> 1));
          st.xsoff[q] = xrow < 0 ? kOOB : (uint32_t)(xrow * (K >> 4));
        }
      }
      const int e = h.x;
      const int64_t cb = h.w;
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const int bc = (pt + 256 * q) >> 1;
        int64_t wrow;
        bool ok;
        if (SWIGLU) {
          const int64_t c = cb * (BN / 2) + 32 * (bc >> 6) + (bc & 31);
          wrow = ((bc >> 5) & 1 ? half : 0) + c;
          ok = c < half && h.z > 0;
        } else {
          wrow = cb * BN + bc;
          ok = wrow < N && h.z > 0;
        }
        st.bwoff[q] = ok ? (uint32_t)(wrow * (K >> 1)) : kOOB;
        st.bsoff[q] = ok ? (uint32_t)(wrow * (K >> 4)) : kOOB;
      }
      st.wr = rsrc(uni(a.w_codes + (int64_t)e * N * (K >> 1)), uni64(N * (K >> 1)));
      st.sr = rsrc(uni(a.w_scales + (int64_t)e * N * (K >> 4)), uni64(N * (K >> 4)));
    };
    auto issue = [&](const PState<ACT>& st, int kt, RegAP<ACT>& ra, RegBP& rb) {
      const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const uint32_t kh = k0 + 32u * ((pt + 256 * q) & 1);
        if (!SB)
          rb.s[q] = __builtin_amdgcn_raw_buffer_load_b16(st.sr, (st.bsoff[q] + (kh >> 4)) | past(Ku, kh), 0, 0);
        rb.c[q] = __builtin_amdgcn_raw_buffer_load_b128(st.wr, (st.bwoff[q] + (kh >> 1)) | past(Ku, kh), 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int j = (pt + 256 * q) & 7;
        const uint32_t k = k0 + 8u * j;
        if (ACT == 0) {
          ra.v[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (st.xoff[q] + 2u * k) | past(Ku, k), 0, 0);
        } else {
          ra.c[q] = __builtin_amdgcn_raw_buffer_load_b32(xr, (st.xoff[q] + (k >> 1)) | past(Ku, k), 0, 0);
          ra.s[q] = __builtin_amdgcn_raw_buffer_load_b8(xsr, (st.xsoff[q] + (k >> 4)) | past(Ku, k), 0, 0);
        }
      }
    };
    auto write_stage = [&](const RegAP<ACT>& ra, const RegBP& rb, const uint32_t (&sw)[2], int buf) {
      uint16_t* da = As + buf * (BM * LDA);
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int c = pt + 256 * q;
        const int row = c >> 3, j = c & 7;
        u32x4 v;
        if (ACT == 0) v = ra.v[q];
        else v = decode8(ra.c[q], e4m3_to_f32<0>(ra.s[q]));  // exact BF16 activations
        *reinterpret_cast<u32x4*>(da + row * LDA + 8 * j) = v;
      }
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const int c = pt + 256 * q;
        const int bc = c >> 1, bh = c & 1;
        uint16_t* db = Bs + buf * (BN * LDA) + bc * LDA + 32 * bh;
        const float s0 = e4m3_to_f32<0>(sw[q]), s1 = e4m3_to_f32<1>(sw[q]);
#pragma unroll
        for (int d = 0; d < 4; d++)
          *reinterpret_cast<u32x4*>(db + 8 * d) = decode8(rb.c[q][d], d < 2 ? s0 : s1);
      }
    };
    u32x4 sblk[2];  // SB: the scales of a 4-step piece (see gemm_wide_grouped)
    auto issue_sb = [&](const PState<ACT>& st, int kt) {
      const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
      for (int q = 0; q < 2; q++)
        sblk[q] = __builtin_amdgcn_raw_buffer_load_b128(st.sr, (st.bsoff[q] + (k0 >> 4)) | past(Ku, k0), 0, 0);
    };
    const uint32_t hsh = 16u * (pt & 1);
    auto scales = [&](const RegBP& rb, auto stepc, uint32_t (&sw)[2]) {
      constexpr int j = decltype(stepc)::value;
#pragma unroll
      for (int q = 0; q < 2; q++) sw[q] = SB ? sblk[q][j & 3] >> hsh : rb.s[q];
    };

    RegAP<ACT> ra[2];
    RegBP rb[2];
    // the tile whose loads are being issued: the current one, and from three steps before
    // its end the next one (the current tile needs no more loads by then)
    PState<ACT> st;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    make_state(tile_hdr(0), st, 0);
    if (SB) issue_sb(st, 0);
    issue(st, 0, ra[0], rb[0]);
    issue(st, 1, ra[1], rb[1]);
    {
      uint32_t sw[2];
      scales(rb[0], I0{}, sw);
      write_stage(ra[0], rb[0], sw, 0);
    }
    issue(st, 2, ra[0], rb[0]);
    __syncthreads();  // stage 0 of tile 0 ready
    // step kt + j of the current tile: stage the next step (or the next tile's first),
    // issue step (kt + j + 3) % KT2 of the issue tile, and with SB at j = 2 the piece of
    // steps (kt + 4) % KT2 ...
    auto pstep = [&](auto jc, int kt, RegAP<ACT>& ran, RegBP& rbn) {
      constexpr int j4 = decltype(jc)::value;
      uint32_t sw[2];
      scales(rbn, std::integral_constant<int, (j4 + 1) & 3>{}, sw);
      write_stage(ran, rbn, sw, (kt + j4 + 1) & 1);
      if constexpr (SB && j4 == 2) issue_sb(st, kt + 4 < KT2 ? kt + 4 : kt + 4 - KT2);
      const int ik = kt + j4 + 3;
      issue(st, ik < KT2 ? ik : ik - KT2, ran, rbn);
      __syncthreads();
    };
    // the routes, for the next tiles' row tables: loaded without a branch (a lane past the
    // tile's routes reads zero), so that no load in flight is waited for early
    const int64_t nroutes = a.rows_per_token ? a.x_rows * a.top_k : a.x_rows;
    const auto rr = rsrc(uni(DENSE ? nullptr : a.sorted), uni64(DENSE ? 0 : nroutes * 4));
    for (int i = 0; i < ntiles; i++) {
      // this lane's row of the next tile's row table, in flight during the first round
      const int4 hn = tile_hdr(i + 1);
      const bool has = pt < hn.z;
      int32_t rl = hn.y + pt;  // DENSE: the identity
      if (!DENSE)
        rl = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rr, has ? (uint32_t)(hn.y + pt) * 4u : kOOB,
                                                           0, 0);
      // rounds of four steps (SB: one scale piece each) or two
      for (int kt = 0; kt < KT2; kt += SB ? 4 : 2) {
        pstep(I0{}, kt, ra[1], rb[1]);
        if (kt == KT2 - 4) {
          // the current tile's loads are all issued: the next tile's offsets, from its
          // row table (written at least one barrier ago, see below) and header
          make_state(hn, st, (i + 1) & 1);
        }
        pstep(I1{}, kt, ra[0], rb[0]);
        if constexpr (SB) {
          pstep(I2{}, kt, ra[1], rb[1]);
          pstep(I3{}, kt, ra[0], rb[0]);
        }
        if (kt == 0) {
          // the next tile's row table, parity (i + 1) & 1, one row per lane: the consumers
          // read parity i & 1 for the current tile, and the other parity's last reader
          // (tile i - 1's epilogue) ran before this tile's first barrier. The empty asm
          // keeps the route's use here: lifted to the top of the tile, it would wait there
          // for every load in flight
          asm volatile("" : "+v"(rl));
          const int32_t rn = has ? rl : -1;
          row_route[(i + 1) & 1][pt] = rn;
          row_x[(i + 1) & 1][pt] = rn < 0 ? -1 : (a.rows_per_token ? rn / a.top_k : rn);
        }
      }
    }
    return;
  }

  // ---------------- consumers: 8 waves ----------------
  const int wm = wave >> 2, wn = wave & 3;
  const int col = lane & 31;
  const int h = lane >> 5;
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mt][st][r] = 0.f;
  __syncthreads();  // stage 0 of tile 0 ready
  // the output: BF16 rows [routes][N/2] (SwiGLU) or fp32 rows [routes][ldy]
  const int64_t nroutes = a.rows_per_token ? a.x_rows * a.top_k : a.x_rows;
  const auto yr = SWIGLU ? rsrc(a.a_out, nroutes * half * 2) : rsrc(a.y, nroutes * a.ldy * 4);
  for (int i = 0; i < ntiles; i++) {
    for (int kt = 0; kt < KT2; kt++) {
      const uint16_t* sa = As + (kt & 1) * (BM * LDA) + (128 * wm + col) * LDA + 32 * h;
      const uint16_t* sb = Bs + (kt & 1) * (BN * LDA) + (64 * wn + col) * LDA + 32 * h;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        u32x4 B[2];
#pragma unroll
        for (int st = 0; st < 2; st++)
          B[st] = *reinterpret_cast<const u32x4*>(sb + 32 * st * LDA + 8 * j);
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          const u32x4 A = *reinterpret_cast<const u32x4*>(sa + 32 * mt * LDA + 8 * j);
#pragma unroll
          for (int st = 0; st < 2; st++) acc[mt][st] = mfma32(A, B[st], acc[mt][st]);
        }
      }
      __syncthreads();
    }
    // the tile's results (row table parity i & 1), while the producers stage the next tile
    const int64_t cb = __builtin_amdgcn_readfirstlane(hdr[i].w);
    const float ts = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                   __builtin_bit_cast(int, hts[i])));
    const int buf = i & 1;
    // Branch-free stores: buffer stores with out-of-range offsets for the rows without a
    // route and the columns past the end (the host takes this form only while the output
    // fits 32-bit offsets). The lane's rows come four at a time (one 16-byte LDS read).
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int lrow0 = 128 * wm + 32 * mt + 8 * g4 + 4 * h;
        const int4 rt = *reinterpret_cast<const int4*>(&row_route[buf][lrow0]);
        int4 xr4 = make_int4(0, 0, 0, 0);
        if (ACT != 0) xr4 = *reinterpret_cast<const int4*>(&row_x[buf][lrow0]);
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int r = 4 * g4 + q;
          const int32_t route = q == 0 ? rt.x : q == 1 ? rt.y : q == 2 ? rt.z : rt.w;
          float f = ts;
          if (ACT != 0) {
            const int32_t xrow = q == 0 ? xr4.x : q == 1 ? xr4.y : q == 2 ? xr4.z : xr4.w;
            f = a.x_ts[xrow < 0 ? 0 : xrow] * ts;
          }
          if (SWIGLU) {
            const uint32_t n = (uint32_t)(cb * (BN / 2) + 32 * wn + col);
            const uint32_t off = route < 0 || n >= (uint32_t)half
                                     ? kOOB : ((uint32_t)route * (uint32_t)half + n) * 2u;
            const float gg = acc[mt][0][r] * f;
            const float u = acc[mt][1][r] * f;
            __builtin_amdgcn_raw_buffer_store_b16(
                (uint16_t)f32_to_bf16_rne(silu(gg) * u), yr, off, 0, 0);
          } else {
#pragma unroll
            for (int st = 0; st < 2; st++) {
              const uint32_t n = (uint32_t)(cb * BN + 64 * wn + 32 * st + col);
              const uint32_t off = route < 0 || n >= (uint32_t)N
                                       ? kOOB : ((uint32_t)route * (uint32_t)a.ldy + n) * 4u;
              __builtin_amdgcn_raw_buffer_store_b32(
                  __builtin_bit_cast(uint32_t, acc[mt][st][r] * f), yr, off, 0, 0);
            }
          }
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int st = 0; st < 2; st++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[mt][st][r] = 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// gemm_splitk: problems whose 64 x 256 tiles leave most CUs idle (e.g. M = 512, N = 4096:
// 128 tiles). A 64 (M) x 128 (N) tile on sixteen waves: four groups of four waves take
// the four quarters of K, each wave computing 64 x 32 (two 32x32x16 subtiles) with its
// own 32 weight columns decoded in registers, and each group staging its quarter's
// activations through its own LDS buffers. The groups' partial tiles meet in LDS and are
// added in a fixed order (quarter 0 + 1 + 2 + 3) before the one store. One workgroup per
// CU and four waves per SIMD, so one wave's MFMAs overlap the others' decode work; no
// workspace and no atomics.
// ---------------------------------------------------------------------------------------
constexpr int kSkBM = 64, kSkBN = 128, kSkSplit = 4;

template <int ACT>
struct SkRegA {  // one K step of this thread's activation loads (two 16-byte pieces)
  u32x4 v[ACT == 0 ? 2 : 1];
  uint32_t c[ACT == 0 ? 1 : 2];
};
struct SkRegB {  // one K step of this lane's weight column: 32 codes
  u32x4 c;
};

template <int ACT>
__global__ __launch_bounds__(1024) void gemm_splitk(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_k[];  // [4][4][BM * LDA]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wave >> 2, wn = wave & 3;  // K quarter, 32-column group
  const int gt = tid & 255;                 // thread within the quarter's group
  const int64_t M = a.M, N = a.N, K = a.K;
  const uint32_t Ku = (uint32_t)K;

  const int64_t nbn = (N + kSkBN - 1) / kSkBN;
  // XCD-aware order, weight-stationary: here the weight is the larger operand (W4A4
  // M = 512, N = K = 4096: 9.4 MB against 1.1 MB), so XCD x (blockIdx % 8) takes the
  // column tiles [x * nbn / 8, (x + 1) * nbn / 8) for every row tile and fetches only its
  // eighth of the weight, rather than all of it for one row tile
  const int64_t lin = blockIdx.x;
  int64_t mi, ni;
  if (nbn % 8 == 0) {
    const int64_t per = nbn / 8, j = lin / 8;
    mi = j / per;
    ni = (lin % 8) * per + j % per;
  } else {
    mi = lin / nbn;
    ni = lin % nbn;
  }
  const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)mi) * kSkBM;
  const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((int)ni) * kSkBN;
  const int64_t rows_m = (M - m0) < kSkBM ? (M - m0) : kSkBM;
  const int64_t rows_n = (N - n0) < kSkBN ? (N - n0) : kSkBN;

  // this quarter's steps: kbeg .. kbeg + KTs - 1, in whole rounds of four (padding steps
  // and steps past K read zeros). Quarters start on a round (KTs a multiple of four) and
  // K is whole rounds (K % 256 == 0), so no round crosses K: a round's 16-byte scale
  // pieces lie inside their rows or wholly past K.
  const int KT = (int)((K + BK - 1) / BK);
  const int KTs = (((KT + kSkSplit - 1) / kSkSplit) + 3) & ~3;
  const int kbeg = ks * KTs;
  const int KT4 = KTs;

  __amdgpu_buffer_rsrc_t xr, xsr;
  if (ACT == 0) {
    xr = rsrc(static_cast<const uint16_t*>(a.x) + m0 * a.ldx, ((rows_m - 1) * a.ldx + K) * 2);
    xsr = xr;
  } else {
    xr = rsrc(static_cast<const uint8_t*>(a.x) + m0 * (K >> 1), rows_m * (K >> 1));
    xsr = rsrc(a.x_scales + m0 * (K >> 4), rows_m * (K >> 4));
  }
  // weights: lane (col, h) holds column n0 + 32 wn + col, K half h of each 64-k step
  const int col = lane & 31;
  const int h = lane >> 5;
  const auto wr = rsrc(a.w_codes + n0 * (K >> 1), rows_n * (K >> 1));
  const auto sr = rsrc(a.w_scales + n0 * (K >> 4), rows_n * (K >> 4));
  const int nl = 32 * wn + col;
  const uint32_t woff = nl < rows_n ? (uint32_t)(nl * (K >> 1)) : kOOB;
  const uint32_t soff = nl < rows_n ? (uint32_t)(nl * (K >> 4)) : kOOB;
  uint16_t* as = lds_k + ks * 4 * (kSkBM * LDA);  // this quarter's four buffers

  // Offsets: the per-thread part is fixed over the steps and carries the row's
  // out-of-range bit; a step adds its k0 part and one uniform out-of-range term. K is
  // whole 64-k steps here, so every k of a step lies below K exactly when k0 does, and
  // the sums stay below 2^31 before the out-of-range bit (no carry into it).
  uint32_t xo[2], xso[2];
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int c = gt + 256 * q;
    const int row = c >> 3, ch = c & 7;
    const uint32_t rowok = row < rows_m ? 0u : kOOB;
    if (ACT == 0) {
      xo[q] = ((uint32_t)(row * a.ldx * 2) + 16u * ch) | rowok;
      xso[q] = 0;
    } else {
      xo[q] = ((uint32_t)(row * (K >> 1)) + 4u * ch) | rowok;
      // the row's scales, loaded a round (16 bytes) at a time; the piece's byte is picked
      // at staging
      xso[q] = (uint32_t)(row * (K >> 4)) | rowok;
    }
  }
  const uint32_t wo = woff + 16u * h;  // this lane's K half of each step's 32 code bytes

  auto issue = [&](int kt, SkRegA<ACT>& ra, SkRegB& rb) {
    const uint32_t k0 = (uint32_t)(kbeg + kt) * BK;
    // padding steps and steps past K (uniform)
    const uint32_t out = (kt < KTs ? 0u : kOOB) | past(Ku, k0);
#pragma unroll
    for (int q = 0; q < 2; q++) {
      if (ACT == 0)
        ra.v[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (xo[q] + 2u * k0) | out, 0, 0);
      else
        ra.c[q] = __builtin_amdgcn_raw_buffer_load_b32(xr, (xo[q] + (k0 >> 1)) | out, 0, 0);
    }
    rb.c = __builtin_amdgcn_raw_buffer_load_b128(wr, (wo + (k0 >> 1)) | out, 0, 0);
  };
  // Scales come four steps at a time: one 16-byte piece per weight column (each step's
  // dword holds its four scale bytes, both K halves) and per activation row, i.e. a
  // quarter of the cache lines that a load per step would touch. Slot 0 holds the
  // current round of four steps, slot 1 the next. A round lies wholly inside the quarter
  // and below K, or it reads zeros; a step outside the quarter or past K also takes zero
  // scales explicitly (live), as its codes are zero.
  u32x4 wsc[2];
  u32x4 xsc[2][ACT == 0 ? 1 : 2];
  auto issue_scales = [&](int kt, u32x4& w, u32x4 (&x)[ACT == 0 ? 1 : 2]) {
    const uint32_t k0 = (uint32_t)(kbeg + kt) * BK;
    const uint32_t out = (kt < KTs ? 0u : kOOB) | past(Ku, k0);
    if (ACT != 0) {
#pragma unroll
      for (int q = 0; q < 2; q++)
        x[q] = __builtin_amdgcn_raw_buffer_load_b128(xsr, (xso[q] + (k0 >> 4)) | out, 0, 0);
    }
    w = __builtin_amdgcn_raw_buffer_load_b128(sr, (soff + (k0 >> 4)) | out, 0, 0);
  };
  const int KTq = KT - kbeg;  // steps of this quarter below K
  auto live = [&](int kt) { return kt < KTs && kt < KTq; };  // uniform
  auto write_a = [&](const SkRegA<ACT>& ra, uint32_t xs0, uint32_t xs1, int buf) {
    uint16_t* dst = as + buf * (kSkBM * LDA);
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int c = gt + 256 * q;
      const int ch = c & 7;
      const int row = c >> 3;
      u32x4 v;
      if (ACT == 0) v = ra.v[q];
      else v = decode8(ra.c[q], e4m3_to_f32<0>((q ? xs1 : xs0) >> (8 * (ch >> 1))));  // exact BF16
      *reinterpret_cast<u32x4*>(dst + row * LDA + 8 * ch) = v;
    }
  };
  auto decode = [&](const SkRegB& rb, uint32_t sdw, u32x4 (&bd)[4]) {
    const uint32_t sw = sdw >> (16 * h);
    const float s0 = e4m3_to_f32<0>(sw), s1 = e4m3_to_f32<1>(sw);
#pragma unroll
    for (int j = 0; j < 4; j++) bd[j] = decode8(rb.c[j], j < 2 ? s0 : s1);
  };
  // the step's scale dwords: step kt of the current round (slot 0) or the next (slot 1)
  auto wscale = [&](int slot, int j, int kt) { return live(kt) ? wsc[slot][j] : 0u; };
  auto xscale = [&](int slot, int j, int q, int kt) {
    if constexpr (ACT == 0) return 0u;
    else return live(kt) ? xsc[slot][q][j] : 0u;
  };

  f32x16 acc[2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[mt][r] = 0.f;

  // Loads run four steps ahead in a ring of four register sets (the steps are short: a
  // wave's step is eight MFMAs). Step kt multiplies LDS buffer kt & 3 with its decoded
  // weights while decoding step kt + 1's weights and staging step kt + 2's activations
  // into buffer (kt + 2) & 3, then refills the set it freed with step kt + 4. Staging two
  // steps ahead into four buffers needs a workgroup barrier only after every second step:
  // a buffer read in steps kt - 2 or kt - 1 is rewritten in step kt or kt + 1, after the
  // barrier that ends step kt - 1 (kt even).
  SkRegA<ACT> ra[4];
  SkRegB rb[4];
  u32x4 bd[2][4];
  auto step = [&](auto ic, int kt) {
    constexpr int I = decltype(ic)::value;
    constexpr int J = (I + 1) & 3;
    const uint16_t* src = as + (kt & 3) * (kSkBM * LDA);
    u32x4 af[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      af[i] = *reinterpret_cast<const u32x4*>(src + (32 * (i & 1) + col) * LDA + 32 * h + 8 * (i >> 1));
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i & 1] = mfma32(af[i], bd[I & 1][i >> 1], acc[i & 1]);
    constexpr int SD = (I + 1) >> 2, JD = (I + 1) & 3;  // slot and index of step kt + 1
    decode(rb[J], wscale(SD, JD, kt + 1), bd[J & 1]);
    // interleave: operand reads two ahead of their MFMA, the next step's decode between
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
      if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);                 // VALU
    }
    constexpr int SA = (I + 2) >> 2, JA = (I + 2) & 3;  // slot and index of step kt + 2
    write_a(ra[(I + 2) & 3], xscale(SA, JA, 0, kt + 2), xscale(SA, JA, 1, kt + 2), (kt + 2) & 3);
    __builtin_amdgcn_sched_barrier(0);
    issue(kt + 4, ra[I], rb[I]);
    if (I == 0) issue_scales(kt + 4, wsc[1], xsc[1]);  // the next round's
    __builtin_amdgcn_sched_barrier(0);
    if (I & 1) __syncthreads();
    if (I == 3) {  // the next round becomes the current one
      wsc[0] = wsc[1];
      if constexpr (ACT != 0) {
        xsc[0][0] = xsc[1][0];
        xsc[0][1] = xsc[1][1];
      }
    }
  };

  issue_scales(0, wsc[0], xsc[0]);
#pragma unroll
  for (int i = 0; i < 4; i++) issue(i, ra[i], rb[i]);
  decode(rb[0], wscale(0, 0, 0), bd[0]);
  write_a(ra[0], xscale(0, 0, 0, 0), xscale(0, 0, 1, 0), 0);
  write_a(ra[1], xscale(0, 1, 0, 1), xscale(0, 1, 1, 1), 1);
  __syncthreads();
  for (int kt = 0; kt < KT4; kt += 4) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
    step(std::integral_constant<int, 2>{}, kt + 2);
    step(std::integral_constant<int, 3>{}, kt + 3);
  }

  // quarters 1..3 hand their partial tiles to quarter 0 through LDS (over the staging
  // buffers: the loop ended with a barrier), which adds them in order
  float* red = reinterpret_cast<float*>(lds_k);  // [3][4 wn][2 mt][16][64 lanes]
  if (ks > 0) {
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        red[((((ks - 1) * 4 + wn) * 2 + mt) * 16 + r) * 64 + lane] = acc[mt][r];
  }
  __syncthreads();
  if (ks == 0) {
    const float ts = a.w_ts[0];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        float v = acc[mt][r];
#pragma unroll
        for (int q = 0; q < kSkSplit - 1; q++) v += red[(((q * 4 + wn) * 2 + mt) * 16 + r) * 64 + lane];
        const int64_t row = m0 + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t n = n0 + nl;
        if (row < M && n < N) {
          const float f = (ACT == 0) ? ts : a.x_ts[row] * ts;
          a.y[row * a.ldy + n] = v * f;
        }
      }
  }
}

template <int ACT>
hipError_t launch_splitk(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = ((a.M + kSkBM - 1) / kSkBM) * ((a.N + kSkBN - 1) / kSkBN);
  const size_t stage = (size_t)kSkSplit * 4 * kSkBM * LDA * sizeof(uint16_t);
  const size_t red = (size_t)(kSkSplit - 1) * 4 * 2 * 16 * 64 * sizeof(float);
  hipLaunchKernelGGL((gemm_splitk<ACT>), dim3((uint32_t)blocks), dim3(1024),
                     stage > red ? stage : red, stream, a);
  return hipGetLastError();
}

// Weight scales in 16-byte pieces of four 64-k steps: K whole pieces and the scale rows
// 16-byte aligned (with K a multiple of 256 every row is, once the base is).
bool scale_pieces(const GemmArgs& a) {
  return a.K % (4 * BK) == 0 && (uintptr_t)a.w_scales % 16 == 0;
}

template <int MT, int ACT>
hipError_t launch_mt(const GemmArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * MT;
  const int64_t blocks = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const size_t lds = 2 * (size_t)BM * LDA * sizeof(uint16_t);
  if (scale_pieces(a))
    hipLaunchKernelGGL((gemm_kernel<MT, ACT, false, false, true>), dim3((uint32_t)blocks), dim3(256),
                       lds, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<MT, ACT>), dim3((uint32_t)blocks), dim3(256), lds, stream, a);
  return hipGetLastError();
}

// CUs of the current device, rounded down to a multiple of eight (0 if unknown): the grid
// of the persistent wide grouped form, one workgroup per CU
int persist_grid() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = n / 8 * 8;
  }
  return cached[dev];
}

template <int ACT>
hipError_t launch_wide(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = ((a.M + kWideBM - 1) / kWideBM) * ((a.N + BN - 1) / BN);
  const size_t lds = 2 * (size_t)(kWideBM + BN) * LDA * sizeof(uint16_t);
  if constexpr (ACT == 0) {
    // more tiles than CUs: the persistent pipeline (gemm_wide_grouped_p's dense form), on
    // the conditions of its grouped use: eight steps per tile or more, at most
    // kPersistMaxTiles tiles per workgroup, and x, the weight codes and the output within
    // 32-bit offsets from their bases
    const int grid = persist_grid();
    const int64_t KT = (a.K + BK - 1) / BK;
    constexpr int64_t kLim = (int64_t)1 << 31;
    if (grid >= 8 && blocks > grid && KT + (KT & 1) >= 8 && a.M * a.ldy * 4 < kLim &&
        ((a.M - 1) * a.ldx + a.K) * 2 < kLim && a.N * (a.K >> 1) < kLim &&
        ((blocks + 7) / 8 + grid / 8 - 1) / (grid / 8) <= kPersistMaxTiles) {
      GemmArgs d = a;
      d.x_rows = a.M;
      d.rows_per_token = 0;
      d.top_k = 1;
      if (scale_pieces(a))
        hipLaunchKernelGGL((gemm_wide_grouped_p<0, false, true, true>), dim3((uint32_t)grid),
                           dim3(768), lds, stream, d);
      else
        hipLaunchKernelGGL((gemm_wide_grouped_p<0, false, false, true>), dim3((uint32_t)grid),
                           dim3(768), lds, stream, d);
      return hipGetLastError();
    }
  }
  if (scale_pieces(a))
    hipLaunchKernelGGL((gemm_wide<ACT, true>), dim3((uint32_t)blocks), dim3(768), lds, stream, a);
  else
    hipLaunchKernelGGL((gemm_wide<ACT>), dim3((uint32_t)blocks), dim3(768), lds, stream, a);
  return hipGetLastError();
}

// Tile choice: 256 x 256 tiles (each decoded weight element feeds 256 rows) when they give
// at least one workgroup per CU; otherwise 64-row tiles, whose two workgroups per CU keep
// more of the chip busy on smaller problems.
bool use_wide(int64_t M, int64_t N) {
  return ((M + kWideBM - 1) / kWideBM) * ((N + BN - 1) / BN) >= 256;
}

// grouped form: 128-route tiles, two workgroups per CU; 64-route tiles for the routes
// past each expert's first 256 when the wide grouped form takes those
constexpr int kGroupedMT = 4;
constexpr int kGroupedRestMT = 1;

template <int MT, int ACT>
hipError_t launch_grouped_mt(const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  constexpr int BM = 32 * MT;
  const size_t lds = 2 * (size_t)BM * LDA * sizeof(uint16_t);
  // whole groups of eight tiles (the tiles past the list's end return at once)
  const int64_t tiles8 = (max_tiles + 7) / 8 * 8;
  // (the 128-route form has no registers to spare for the pieces)
  constexpr bool kSB = MT <= 2;
  const bool sb = kSB && scale_pieces(a);
  if (a.a_out) {
    const int64_t blocks = tiles8 * (((a.N >> 1) + BN / 2 - 1) / (BN / 2));
    if (sb)
      hipLaunchKernelGGL((gemm_kernel<MT, ACT, true, true, kSB>), dim3((uint32_t)blocks),
                         dim3(256), lds, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<MT, ACT, true, true>), dim3((uint32_t)blocks),
                         dim3(256), lds, stream, a);
  } else {
    const int64_t blocks = tiles8 * ((a.N + BN - 1) / BN);
    if (sb)
      hipLaunchKernelGGL((gemm_kernel<MT, ACT, true, false, kSB>), dim3((uint32_t)blocks),
                         dim3(256), lds, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<MT, ACT, true>), dim3((uint32_t)blocks), dim3(256),
                         lds, stream, a);
  }
  return hipGetLastError();
}


template <int ACT, bool SWIGLU>
hipError_t launch_grouped_wide_p(const GemmArgs& a, int grid, size_t lds, bool sb,
                                 hipStream_t stream) {
  if (sb)
    hipLaunchKernelGGL((gemm_wide_grouped_p<ACT, SWIGLU, true>), dim3((uint32_t)grid), dim3(768),
                       lds, stream, a);
  else
    hipLaunchKernelGGL((gemm_wide_grouped_p<ACT, SWIGLU, false>), dim3((uint32_t)grid), dim3(768),
                       lds, stream, a);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_grouped_wide(const GemmArgs& a, int64_t max_active, hipStream_t stream) {
  const size_t lds = 2 * (size_t)(kWideBM + BN) * LDA * sizeof(uint16_t);
  const int64_t act8 = (max_active + 7) / 8 * 8;
  const bool sb = scale_pieces(a);
  // the persistent form: at least eight steps per tile (a round of four before the next
  // tile's offsets are built, four after), at most kPersistMaxTiles tiles per workgroup,
  // and an output its stores reach with 32-bit offsets
  {
    const int64_t KT = (a.K + BK - 1) / BK;
    const int64_t nbn = a.a_out ? ((a.N >> 1) + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
    const int64_t nroutes = a.rows_per_token ? a.x_rows * a.top_k : a.x_rows;
    const int64_t out_bytes = a.a_out ? nroutes * (a.N >> 1) * 2 : nroutes * a.ldy * 4;
    const int grid = persist_grid();
    if (KT + (KT & 1) >= 8 && grid >= 8 && out_bytes < ((int64_t)1 << 31) &&
        (act8 / 8 * nbn + grid / 8 - 1) / (grid / 8) <= kPersistMaxTiles)
      return a.a_out ? launch_grouped_wide_p<ACT, true>(a, grid, lds, sb, stream)
                     : launch_grouped_wide_p<ACT, false>(a, grid, lds, sb, stream);
  }
  if (a.a_out) {
    const int64_t blocks = act8 * (((a.N >> 1) + BN / 2 - 1) / (BN / 2));
    if (sb)
      hipLaunchKernelGGL((gemm_wide_grouped<ACT, true, true>), dim3((uint32_t)blocks), dim3(768),
                         lds, stream, a);
    else
      hipLaunchKernelGGL((gemm_wide_grouped<ACT, true>), dim3((uint32_t)blocks), dim3(768), lds,
                         stream, a);
  } else {
    const int64_t blocks = act8 * ((a.N + BN - 1) / BN);
    if (sb)
      hipLaunchKernelGGL((gemm_wide_grouped<ACT, false, true>), dim3((uint32_t)blocks), dim3(768),
                         lds, stream, a);
    else
      hipLaunchKernelGGL((gemm_wide_grouped<ACT, false>), dim3((uint32_t)blocks), dim3(768), lds,
                         stream, a);
  }
  return hipGetLastError();
}

}  // namespace

int gemm_grouped_tile_rows(bool wide) { return 32 * (wide ? kGroupedRestMT : kGroupedMT); }

hipError_t launch_gemm_grouped(const GemmArgs& a, int act_kind, int64_t max_tiles,
                               hipStream_t stream) {
  switch (act_kind) {
    case 0: return launch_grouped_mt<kGroupedMT, 0>(a, max_tiles, stream);
    case 1: return launch_grouped_mt<kGroupedMT, 1>(a, max_tiles, stream);
    default: return hipErrorInvalidValue;
  }
}

// the wide grouped form: each active expert's first routes in 256-route tiles, then the
// rest of the routes (the tile list) in 64-route tiles
hipError_t launch_gemm_grouped_wide(const GemmArgs& a, int act_kind, int64_t max_active,
                                    int64_t max_tiles, hipStream_t stream) {
  if (act_kind != 0 && act_kind != 1) return hipErrorInvalidValue;
  // the short launch of the remaining routes first: the rows a following combine reads
  // are then the wide launch's, written last
  hipError_t e = act_kind == 0 ? launch_grouped_mt<kGroupedRestMT, 0>(a, max_tiles, stream)
                               : launch_grouped_mt<kGroupedRestMT, 1>(a, max_tiles, stream);
  if (e != hipSuccess) return e;
  return act_kind == 0 ? launch_grouped_wide<0>(a, max_active, stream)
                       : launch_grouped_wide<1>(a, max_active, stream);
}

// Largest activation row pitch (elements) the GEMM's 32-bit buffer offsets can address
// for a 256-row tile.
int64_t gemm_max_ldx() { return ((int64_t)1 << 31) / (2 * 256) - 1; }

// K split four ways when the 64 x 256 tiles would not give every CU a workgroup, the K
// quarters stay at least four steps long and K is whole rounds of four 64-k steps. Its
// scales come as 16-byte pieces (four steps of one column or row), so the scale bases
// must be 16-byte aligned (the ABI guarantees 2); otherwise the 64-row kernel runs.
bool use_splitk(const GemmArgs& a, int act_kind) {
  const bool aligned16 = (uintptr_t)a.w_scales % 16 == 0 &&
                         (act_kind == 0 || (uintptr_t)a.x_scales % 16 == 0);
  return aligned16 && ((a.M + 63) / 64) * ((a.N + BN - 1) / BN) < 256 &&
         a.K >= 4 * kSkSplit * BK && a.K % (4 * BK) == 0;
}

hipError_t launch_gemm(const GemmArgs& a, int act_kind, hipStream_t stream) {
  if (act_kind != 0 && act_kind != 1) return hipErrorInvalidValue;
  if (use_wide(a.M, a.N))
    return act_kind == 0 ? launch_wide<0>(a, stream) : launch_wide<1>(a, stream);
  if (use_splitk(a, act_kind))
    return act_kind == 0 ? launch_splitk<0>(a, stream) : launch_splitk<1>(a, stream);
  return act_kind == 0 ? launch_mt<2, 0>(a, stream) : launch_mt<2, 1>(a, stream);
}

}  // namespace nvfp4
