// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

// Rows of one weight-streaming pass: up to 16 activation rows against one weight.
struct StreamArgs {
  // activations: BF16 bits [rows][ldx], or NVFP4 codes [rows][K/2] + scales + row ts
  const void* x;
  const uint8_t* x_scales;
  const float* x_ts;
  int64_t ldx;      // BF16: elements per row
  // weight (for the grouped form: expert 0; expert e is offset by e * N * K/2 etc.)
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_ts;
  int64_t N, K;
  // output fp32 [rows][ldy]
  float* y;
  int64_t ldy;
  int64_t x_rows;   // rows in x (bounds the activation reads)
  int32_t M;        // dense: number of rows (<= 16); grouped: rows per expert pass hint
  int32_t apply_ts; // multiply the accumulator by the weight's tensor scale
  int32_t rsplit;   // dense: workgroups sharing one weight tile, each taking its own sets
                    // of four rows (0 or 1: one workgroup takes every row)
  // grouped form (NULL for dense)
  const int32_t* slots;      // [grid y] slot records (RouteWorkspace::slots)
  const int32_t* sorted;     // route ids grouped by expert
  int32_t rows_per_token;    // x row of route r: r / top_k (1) or r (0)
  int32_t top_k;
  // grouped gate_up with the SwiGLU epilogue (NULL otherwise): a[route][n] =
  // bf16(silu(h[n]) * h[n + N/2]) for n < N/2, BF16 rows of N/2 values
  uint16_t* a_out;
};

hipError_t launch_stream(const StreamArgs& a, int act_kind, bool grouped, int max_active,
                         hipStream_t stream);
// the same with an explicit launch shape: tn 16-row tiles per workgroup, W waves splitting
// K, rsets sets of four activation rows per workgroup (dense; 0: all rows in one)
hipError_t launch_stream_cfg(const StreamArgs& a, int act_kind, bool grouped, int max_active,
                             int tn, int W, int rsets, hipStream_t stream);

struct GemmArgs {
  const void* x;
  const uint8_t* x_scales;
  const float* x_ts;
  int64_t ldx;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_ts;
  int64_t M, N, K;
  float* y;
  int64_t ldy;
  // grouped form (NULL tiles for dense): tiles of tile_rows routes of one expert, rows
  // gathered from x by route, written to y row = route; w_* point at expert 0
  const int32_t* tiles;      // [n_tiles][2] (expert, first slot in sorted)
  const int32_t* n_tiles;    // [1]
  const int32_t* offsets;    // [E+1]
  const int32_t* sorted;     // route ids grouped by expert
  int64_t x_rows;            // rows in x
  int32_t rows_per_token;    // x row of route r: r / top_k (1) or r (0)
  int32_t top_k;
  int32_t apply_ts;          // multiply by the expert's tensor scale
  // grouped SwiGLU form (NULL otherwise): BF16 rows [routes][N/2] of
  // bf16(silu(h[n]) * h[n + N/2])
  uint16_t* a_out;
  // grouped wide form: the active experts, one 256-route tile each (their first routes)
  const int32_t* active;     // [E]
  const int32_t* n_active;   // [1]
};

hipError_t launch_gemm(const GemmArgs& a, int act_kind, hipStream_t stream);
// grouped form: max_tiles bounds the tile list the route grouping writes
hipError_t launch_gemm_grouped(const GemmArgs& a, int act_kind, int64_t max_tiles,
                               hipStream_t stream);
// routes per tile of the grouped GEMM's tile list: with `wide`, the routes past each
// expert's first kWideGroupedRows, which the wide grouped form takes
int gemm_grouped_tile_rows(bool wide);
// grouped wide form: each active expert's first routes (up to its tile of 256) in one
// 256 x 256-tile workgroup per column block, then the grouping's tile list of the rest;
// max_active bounds the active list, max_tiles the tile list
constexpr int kWideGroupedRows = 256;
hipError_t launch_gemm_grouped_wide(const GemmArgs& a, int act_kind, int64_t max_active,
                                    int64_t max_tiles, hipStream_t stream);
// largest BF16 activation row pitch (elements) the GEMM's buffer offsets address
int64_t gemm_max_ldx();

hipError_t launch_quantize(int in_type, const void* x, int64_t ldx, int64_t M, int64_t K,
                           int ts_mode, uint8_t* codes, uint8_t* scales, float* ts,
                           uint32_t* faults, hipStream_t stream);

// grouped-call helpers
struct RouteWorkspace {
  int32_t* offsets;       // [E+1]
  int32_t* active;        // [E]
  int32_t* n_active;      // [1]
  int32_t* route_expert;  // [R] expert of route r, or -1 when dropped
  int32_t* sorted;        // [R]
  float* rows;            // [R][N] fp32 per-route rows (combine form; SwiGLU on the GEMM path)
  int32_t* tiles;         // GEMM path: [n_tiles][2] (expert, first slot in `sorted`)
  int32_t* n_tiles;       // [1]
  int32_t tile_rows;      // GEMM path: routes per tile (0: no tile list)
  int32_t main_rows;      // GEMM path: routes at the start of each expert's group that the
                          // tile list leaves out (taken by the wide grouped form; 0: none)
  int32_t* chunk_counts;  // chunked grouping: [chunks][E] counts, then first slots
  int32_t* slots;         // [max_slots][kSlotInts] slot records, one per active expert in
                          // ascending id: (expert, begin, end, n, the expert's first n
                          // routes of `sorted`, n <= kSlotRoutes); expert -1 in the slots
                          // past the last one
  int32_t max_slots;      // min(routes, experts)
};
constexpr int kSlotInts = 16;
constexpr int kSlotRoutes = kSlotInts - 4;

// int32 entries of the chunked grouping's count table for this route set (0 when the
// route set is grouped by a single workgroup)
int64_t route_chunk_ints(int64_t T, int top_k, int E);

// also zeroes output row r (zero_row_bytes bytes of zero_out, when not NULL) of every
// dropped route
hipError_t launch_route_sort(const int32_t* topk_ids, int64_t T, int top_k, int E,
                             const RouteWorkspace& ws, uint32_t* faults, void* zero_out,
                             int64_t zero_row_bytes, hipStream_t stream);
hipError_t launch_combine(const float* rows, const int32_t* route_expert,
                          const float* topk_w, const float* w_ts, int64_t T, int top_k,
                          int64_t N, float* y, hipStream_t stream);

// check mode: E4M3 NaN scale bytes [0, bytes) and non-finite tensor scales [0, n_ts) set
// NVFP4_FAULT_NAN_SCALE; non-finite BF16 values of rows [rows][ld] (K each) set
// NVFP4_FAULT_NONFINITE
hipError_t launch_check_scales(const uint8_t* scales, int64_t bytes, const float* ts,
                               int64_t n_ts, uint32_t* faults, hipStream_t stream);
hipError_t launch_check_bf16(const void* x, int64_t ld, int64_t rows, int64_t K,
                             uint32_t* faults, hipStream_t stream);

// next-weight prefetch: a streaming read of [buf, buf + bytes), values discarded, on at most
// `workgroups` workgroups
hipError_t launch_prefetch(const void* buf, int64_t bytes, int workgroups, hipStream_t stream);

// measurement support: one streaming read of `bytes` bytes (loads_per_thread 16-byte loads
// per thread, 1/2/4/8/16)
hipError_t launch_read_probe(const void* buf, int64_t bytes, int loads_per_thread, uint32_t* sink,
                             hipStream_t stream);

}  // namespace nvfp4
