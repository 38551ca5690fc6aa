// Helpers of the expert-grouped call: route grouping and the ordered combine (the SwiGLU
// to BF16 is the streaming kernel's epilogue).
//
// Routes are grouped expert-ascending ("true rows, expert-ascending" with expert-first
// offsets: Rocket log entry "Rank-local E256 MoE misses the Qwen K1 and K4 step
// budgets", and run_moe_grouped in the entry "The expert split decodes the same
// tokens; ..."), so one workgroup can stream an expert's weight once for all its
// routes. The combine accumulates each token's routes in fp32 in ascending expert order
// with the expert's tensor scale folded into the router weight (same entry, section
// "Why rows and not partial sums"), which keeps it deterministic: no atomics touch
// floating-point data anywhere in this file.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

constexpr int kSortThreads = 1024;

// Zeroes `bytes` bytes (even) of output row r of a dropped route; dword stores when the
// row allows them.
__device__ __forceinline__ void zero_route_row(void* out, int64_t bytes, int64_t r) {
  if (!out) return;
  char* row = static_cast<char*>(out) + r * bytes;
  if ((bytes & 3) == 0 && ((uintptr_t)row & 3) == 0) {
    for (int64_t b = 0; b < bytes; b += 4) *reinterpret_cast<uint32_t*>(row + b) = 0u;
  } else {
    for (int64_t b = 0; b < bytes; b += 2) *reinterpret_cast<uint16_t*>(row + b) = 0u;
  }
}

// Tile list of the GEMM path: expert e's routes sorted[off, off + cnt) split into tiles
// of ws.tile_rows routes; tile_off is e's first tile. With ws.main_rows, the list holds
// only the routes past each expert's first main_rows (the wide grouped form takes those).
__device__ __forceinline__ void write_tiles(const RouteWorkspace& ws, int e, int32_t off,
                                            int32_t cnt, int32_t tile_off) {
  const int32_t nt = (cnt + ws.tile_rows - 1) / ws.tile_rows;
  for (int32_t i = 0; i < nt; i++) {
    ws.tiles[2 * (tile_off + i)] = e;
    ws.tiles[2 * (tile_off + i) + 1] = off + i * ws.tile_rows;
  }
}

// Exclusive prefix sum over the block: a shuffle scan inside each wave, then the wave
// totals through LDS (two barriers). `wsum` holds blockDim.x / 64 entries.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* wsum, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int32_t base = 0, tot = 0;
  for (int w = 0; w < nw; w++) {
    const int32_t sw = wsum[w];
    base += w < wave ? sw : 0;
    tot += sw;
  }
  *total = tot;
  __syncthreads();  // wsum is reused by the next scan
  return base + x - v;
}

// Offsets, the active list, the slot record headers and the tile list from the per-expert
// counts in cnt[E] (LDS); afterwards cnt[e] holds expert e's first slot in `sorted`. A
// slot record gives a streaming workgroup its expert, its route range and (when the
// caller fills them: slot_of != NULL, then slot_of[e] is e's slot) its first routes in
// one 64-byte read, without the dependent reads of the active list, offsets and routes.
// write = false: only cnt becomes each expert's first slot (no workspace writes)
__device__ __forceinline__ void expert_scans(const RouteWorkspace& ws, int E, int32_t* cnt,
                                             int32_t* wsum, int32_t* slot_of = nullptr,
                                             bool write = true) {
  const int tid = threadIdx.x, nt = blockDim.x;
  int32_t run = 0, act_run = 0, tile_run = 0;
  for (int e0 = 0; e0 < E; e0 += nt) {
    const int e = e0 + tid;
    const int32_t c = e < E ? cnt[e] : 0;
    const int32_t rest = c > ws.main_rows ? c - ws.main_rows : 0;  // routes in the tile list
    const int32_t ntile = ws.tile_rows > 0 ? (rest + ws.tile_rows - 1) / ws.tile_rows : 0;
    int32_t tot, tot_a, tot_t;
    const int32_t o = block_exclusive_scan(c, wsum, &tot) + run;
    const int32_t a = block_exclusive_scan(c > 0 ? 1 : 0, wsum, &tot_a) + act_run;
    const int32_t to = block_exclusive_scan(ntile, wsum, &tot_t) + tile_run;
    if (e < E && write) {
      ws.offsets[e] = o;
      if (c > 0) {
        ws.active[a] = e;
        const int32_t n = slot_of ? (c < kSlotRoutes ? c : kSlotRoutes) : 0;
        *reinterpret_cast<int4*>(ws.slots + kSlotInts * a) = make_int4(e, o, o + c, n);
        if (slot_of) slot_of[e] = a;
      }
      if (ntile > 0) write_tiles(ws, e, o + (c - rest), rest, to);
    }
    if (e < E) cnt[e] = o;
    run += tot;
    act_run += tot_a;
    tile_run += tot_t;
  }
  for (int s = act_run + tid; write && s < ws.max_slots; s += nt) ws.slots[kSlotInts * s] = -1;
  if (tid == 0 && write) {
    ws.offsets[E] = run;
    *ws.n_active = act_run;
    if (ws.tile_rows > 0) *ws.n_tiles = tile_run;
  }
  __syncthreads();
}

// Single workgroup, any number of routes. The same offsets, active list and tile list as
// route_sort_fast; the order of routes within one expert's group is
// unspecified here (atomic cursors), which no output depends on: every route's row is
// computed from its own activation row and its expert alone.
__global__ __launch_bounds__(kSortThreads) void route_sort(const int32_t* ids, int64_t T,
                                                           int top_k, int E, RouteWorkspace ws,
                                                           uint32_t* faults, void* zero_out,
                                                           int64_t zero_row_bytes) {
  extern __shared__ int32_t sh[];
  int32_t* wsum = sh;       // [16]
  int32_t* cnt = sh + 16;   // [E] routes per expert, then the scatter cursors
  const int64_t R = T * top_k;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortThreads) cnt[e] = 0;
  __syncthreads();

  // (1) validate: id in range and not repeated earlier in its token; dropped -> -1
  bool bad = false;
  for (int64_t r = tid; r < R; r += kSortThreads) {
    const int32_t e = ids[r];
    bool ok = (e >= 0 && e < E);
    const int64_t t0 = (r / top_k) * top_k;
    for (int64_t rr = t0; rr < r; rr++) ok = ok && (ids[rr] != e);
    ws.route_expert[r] = ok ? e : -1;
    if (!ok) zero_route_row(zero_out, zero_row_bytes, r);
    if (ok) atomicAdd(&cnt[e], 1);  // integer count: order-independent
    bad = bad || !ok;
  }
  if (bad && faults) atomicOr(faults, (uint32_t)NVFP4_FAULT_BAD_ROUTE);
  __threadfence();  // route_expert is read back below by other threads
  __syncthreads();

  // (2) offsets, active list, tile list; cnt becomes the scatter cursors
  expert_scans(ws, E, cnt, wsum);

  // (3) scatter
  for (int64_t r = tid; r < R; r += kSortThreads) {
    const int32_t e = ws.route_expert[r];
    if (e >= 0) ws.sorted[atomicAdd(&cnt[e], 1)] = (int32_t)r;
  }
}

// Route sets beyond one workgroup's quick reach (more than kFastRoutes routes, top_k <=
// kRegTopK) are grouped by chunks of kChunkTokens tokens, one workgroup each, one token
// per thread with its ids in registers:
//  (1) route_count_chunks validates its tokens' routes and counts them per expert into
//      chunk_counts[chunk][E];
//  (2) route_scan_chunks (one workgroup) turns the counts into the offsets, the active
//      list, the tile list and, in place, each chunk's first slot per expert;
//  (3) route_scatter_chunks places its routes from those slots.
// Chunks keep ascending token order within an expert's group; inside a chunk the order is
// unspecified (LDS atomic cursors), which no output depends on: every route's row is
// computed from its own activation row and its expert alone.
constexpr int kRegTopK = 16;
constexpr int kChunkTokens = 256;

// a token's ids and validity (in range, not repeated earlier in the token)
template <int KREG>
__device__ __forceinline__ void load_token(const int32_t* ids, int64_t t, int top_k, int E,
                                           int32_t (&e)[KREG], bool (&ok)[KREG]) {
#pragma unroll
  for (int j = 0; j < KREG; j++) e[j] = j < top_k ? ids[t * top_k + j] : -1;
#pragma unroll
  for (int j = 0; j < KREG; j++) {
    bool v = j < top_k && e[j] >= 0 && e[j] < E;
#pragma unroll
    for (int jj = 0; jj < j; jj++) v = v && e[jj] != e[j];
    ok[j] = v;
  }
}

// KREG: the exact top_k (fully unrolled), or kRegTopK with top_k <= kRegTopK read at run time
template <int KREG>
__global__ __launch_bounds__(kChunkTokens) void route_count_chunks(const int32_t* ids, int64_t T,
                                                                   int top_k_rt, int E,
                                                                   RouteWorkspace ws,
                                                                   uint32_t* faults,
                                                                   void* zero_out,
                                                                   int64_t zero_row_bytes) {
  const int top_k = KREG == kRegTopK ? top_k_rt : KREG;
  extern __shared__ int32_t cnt[];  // [E]
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kChunkTokens) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kChunkTokens + tid;
  bool bad = false;
  if (t < T) {
    int32_t e[KREG];
    bool ok[KREG];
    load_token<KREG>(ids, t, top_k, E, e, ok);
#pragma unroll
    for (int j = 0; j < KREG; j++) {
      if (j >= top_k) break;
      const int64_t r = t * top_k + j;
      ws.route_expert[r] = ok[j] ? e[j] : -1;
      if (ok[j]) {
        atomicAdd(&cnt[e[j]], 1);  // integer count: order-independent
      } else {
        zero_route_row(zero_out, zero_row_bytes, r);
        bad = true;
      }
    }
  }
  if (bad && faults) atomicOr(faults, (uint32_t)NVFP4_FAULT_BAD_ROUTE);
  __syncthreads();
  int32_t* cc = ws.chunk_counts + (int64_t)blockIdx.x * E;
  for (int e = tid; e < E; e += kChunkTokens) cc[e] = cnt[e];
}

__global__ __launch_bounds__(kSortThreads) void route_scan_chunks(int E, int64_t nchunks,
                                                                  RouteWorkspace ws) {
  extern __shared__ int32_t sh[];
  int32_t* wsum = sh;      // [16]
  int32_t* cnt = sh + 16;  // [E] routes per expert, then each expert's first slot
  const int tid = threadIdx.x;
  // (the chunk loops are unrolled so that their loads are in flight together rather than
  // one round trip per chunk)
  for (int e = tid; e < E; e += kSortThreads) {
    int32_t c = 0;
#pragma unroll 8
    for (int64_t k = 0; k < nchunks; k++) c += ws.chunk_counts[k * E + e];
    cnt[e] = c;
  }
  __syncthreads();
  expert_scans(ws, E, cnt, wsum);
  // chunk k's first slot for expert e: e's first slot plus the earlier chunks' counts
  for (int e = tid; e < E; e += kSortThreads) {
    int32_t run = cnt[e];
    for (int64_t k0 = 0; k0 < nchunks; k0 += 8) {  // eight counts loaded, then stored
      int32_t c[8];
#pragma unroll
      for (int j = 0; j < 8; j++) c[j] = k0 + j < nchunks ? ws.chunk_counts[(k0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (k0 + j < nchunks) ws.chunk_counts[(k0 + j) * E + e] = run;
        run += c[j];
      }
    }
  }
}

template <int KREG>
__global__ __launch_bounds__(kChunkTokens) void route_scatter_chunks(const int32_t* ids, int64_t T,
                                                                     int top_k_rt, int E,
                                                                     RouteWorkspace ws) {
  const int top_k = KREG == kRegTopK ? top_k_rt : KREG;
  extern __shared__ int32_t cur[];  // [E] this chunk's next slot per expert
  const int tid = threadIdx.x;
  const int32_t* cc = ws.chunk_counts + (int64_t)blockIdx.x * E;
  for (int e = tid; e < E; e += kChunkTokens) cur[e] = cc[e];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kChunkTokens + tid;
  if (t >= T) return;
  int32_t e[KREG];
  bool ok[KREG];
  load_token<KREG>(ids, t, top_k, E, e, ok);
#pragma unroll
  for (int j = 0; j < KREG; j++) {
    if (j >= top_k) break;
    if (ok[j]) ws.sorted[atomicAdd(&cur[e[j]], 1)] = (int32_t)(t * top_k + j);
  }
}

// route_scan_chunks and route_scatter_chunks in one launch, for up to kFusedScanChunks
// chunks: every workgroup sums the chunks' counts itself (its own chunk's first slot per
// expert: the expert's first slot plus the earlier chunks' counts), workgroup 0 also
// writes the offsets, the active list, the slot records and the tile list, and each then
// places its chunk's routes. The same grouping as the three launches.
constexpr int64_t kFusedScanChunks = 32;

template <int KREG>
__global__ __launch_bounds__(kChunkTokens) void route_scan_scatter_chunks(const int32_t* ids,
                                                                          int64_t T, int top_k_rt,
                                                                          int E, int64_t nchunks,
                                                                          RouteWorkspace ws) {
  const int top_k = KREG == kRegTopK ? top_k_rt : KREG;
  extern __shared__ int32_t sh[];
  int32_t* wsum = sh;        // [16] wave totals of a scan
  int32_t* cnt = sh + 16;    // [E] routes per expert, then each expert's first slot
  int32_t* cur = cnt + E;    // [E] this chunk's next slot per expert
  const int tid = threadIdx.x;
  const int64_t ch = blockIdx.x;
  for (int e = tid; e < E; e += kChunkTokens) {
    int32_t c = 0, before = 0;
#pragma unroll 8
    for (int64_t k = 0; k < nchunks; k++) {
      const int32_t v = ws.chunk_counts[k * E + e];
      before += k < ch ? v : 0;
      c += v;
    }
    cnt[e] = c;
    cur[e] = before;
  }
  __syncthreads();
  expert_scans(ws, E, cnt, wsum, nullptr, ch == 0);
  for (int e = tid; e < E; e += kChunkTokens) cur[e] += cnt[e];
  __syncthreads();
  const int64_t t = ch * kChunkTokens + tid;
  if (t >= T) return;
  int32_t e[KREG];
  bool ok[KREG];
  load_token<KREG>(ids, t, top_k, E, e, ok);
#pragma unroll
  for (int j = 0; j < KREG; j++) {
    if (j >= top_k) break;
    if (ok[j]) ws.sorted[atomicAdd(&cur[e[j]], 1)] = (int32_t)(t * top_k + j);
  }
}

// Decode-sized route sets (R <= kFastRoutes): the same result as route_sort, computed in
// LDS with no dependent global-memory round trips. One route per thread (the block is
// sized to R); the expert offsets and the active-expert list come from block-wide scans;
// a route's place among its expert's routes is the number of earlier routes with the
// same expert (stable, counted with 16-byte LDS reads).
constexpr int kFastRoutes = kSortThreads;

__global__ __launch_bounds__(kSortThreads) void route_sort_fast(const int32_t* ids, int64_t T,
                                                                int top_k, int E,
                                                                RouteWorkspace ws,
                                                                uint32_t* faults, void* zero_out,
                                                                int64_t zero_row_bytes) {
  extern __shared__ __attribute__((aligned(16))) int32_t sh[];
  const int nt = blockDim.x;                // >= R, a multiple of 64
  int32_t* ids_s = sh;                      // [nt]
  int32_t* rexp = sh + nt;                  // [nt] expert of each route, -1 dropped/padding
  int32_t* wsum = sh + 2 * nt;              // [16] wave totals of a scan
  int32_t* cnt = sh + 2 * nt + 16;          // [E] routes per expert
  int32_t* slot_of = cnt + E;               // [E] slot of each active expert
  const int R = (int)(T * top_k);
  const int tid = threadIdx.x;

  ids_s[tid] = tid < R ? ids[tid] : -1;
  for (int e = tid; e < E; e += nt) cnt[e] = 0;
  __syncthreads();

  // validate: in range and not repeated earlier in its token
  int32_t my_e = -1;
  if (tid < R) {
    const int32_t e = ids_s[tid];
    bool ok = (e >= 0 && e < E);
    const int t0 = (tid / top_k) * top_k;
    for (int r = t0; r < tid; r++) ok = ok && (ids_s[r] != e);
    my_e = ok ? e : -1;
    ws.route_expert[tid] = my_e;
    if (!ok) zero_route_row(zero_out, zero_row_bytes, tid);
    if (!ok && faults) atomicOr(faults, (uint32_t)NVFP4_FAULT_BAD_ROUTE);
    if (ok) atomicAdd(&cnt[e], 1);  // integer count: order-independent
  }
  rexp[tid] = my_e;
  __syncthreads();

  // offsets, active list, slot records, tile list; cnt becomes each expert's first slot
  expert_scans(ws, E, cnt, wsum, slot_of);

  if (my_e >= 0) {
    // stable place among the expert's routes
    int rank = 0;
    const int full = tid & ~3;
    for (int r = 0; r < full; r += 4) {
      const int4 v = *reinterpret_cast<const int4*>(rexp + r);
      rank += (v.x == my_e) + (v.y == my_e) + (v.z == my_e) + (v.w == my_e);
    }
    for (int r = full; r < tid; r++) rank += (rexp[r] == my_e);
    ws.sorted[cnt[my_e] + rank] = tid;
    if (rank < kSlotRoutes) ws.slots[kSlotInts * slot_of[my_e] + 4 + rank] = tid;
  }
}

// y[t][n] = sum over the token's routes in ascending expert id of (w * ts_e) * row[n]
// One workgroup per (token, 1024 columns). The first top_k threads read their route's
// expert and router weight together, rank the route among the token's kept routes by
// expert id in LDS and stage its row index and weight r * ts_e at that rank; each thread
// then loads its four columns of every route row before summing them with fmaf in that
// order, starting from zero. (Three dependent memory round trips per workgroup: routes,
// tensor scales, rows.)
constexpr int kCombineMaxK = 64;

__global__ __launch_bounds__(256) void combine_kernel(const float* rows,
                                                      const int32_t* route_expert,
                                                      const float* topk_w,
                                                      const float* w_ts, int64_t T, int top_k,
                                                      int64_t N, float* y) {
  __shared__ int32_t ex[kCombineMaxK];
  __shared__ int32_t rr[kCombineMaxK];
  __shared__ float wr[kCombineMaxK];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t e = -1;
  float w = 0.f;
  if (tid < top_k) {
    e = route_expert[t * top_k + tid];
    w = topk_w[t * top_k + tid];
    ex[tid] = e;
  }
  __syncthreads();
  int n_routes = 0;  // kept routes of the token (ids are distinct within a token)
  for (int j = 0; j < top_k; j++) n_routes += ex[j] >= 0;
  if (e >= 0) {
    int slot = 0;
    for (int j = 0; j < top_k; j++) slot += (ex[j] >= 0 && ex[j] < e);
    rr[slot] = (int32_t)(t * top_k + tid);
    wr[slot] = w * w_ts[e];
  }
  __syncthreads();
  const int64_t n0 = (int64_t)blockIdx.y * 1024 + 4 * threadIdx.x;
  if (n0 >= N) return;
  const bool vec = n0 + 4 <= N && (N & 3) == 0;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int kBatch = 8;  // route rows in flight per thread
  for (int q0 = 0; q0 < n_routes; q0 += kBatch) {
    float v[kBatch][4];
#pragma unroll
    for (int q = 0; q < kBatch; q++) {
      if (q0 + q < n_routes) {
        const float* src = rows + (int64_t)rr[q0 + q] * N + n0;
        if (vec) {
          const float4 f = *reinterpret_cast<const float4*>(src);
          v[q][0] = f.x; v[q][1] = f.y; v[q][2] = f.z; v[q][3] = f.w;
        } else {
#pragma unroll
          for (int c = 0; c < 4; c++) v[q][c] = n0 + c < N ? src[c] : 0.f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; q++) {
      if (q0 + q < n_routes) {
        const float w = wr[q0 + q];
#pragma unroll
        for (int c = 0; c < 4; c++) acc[c] = __builtin_fmaf(w, v[q][c], acc[c]);
      }
    }
  }
  float* dst = y + t * N + n0;
  if (vec) {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; c++)
      if (n0 + c < N) dst[c] = acc[c];
  }
}

int64_t grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  return g < 1 ? 1 : (g > 8192 ? 8192 : g);
}

}  // namespace

hipError_t launch_route_sort(const int32_t* topk_ids, int64_t T, int top_k, int E,
                             const RouteWorkspace& ws, uint32_t* faults, void* zero_out,
                             int64_t zero_row_bytes, hipStream_t stream) {
  if (T * top_k <= kFastRoutes) {
    const int nt = (int)((T * top_k + 63) / 64 * 64);
    const size_t lds = sizeof(int32_t) * ((size_t)2 * nt + 16 + 2 * (size_t)E);
    hipLaunchKernelGGL(route_sort_fast, dim3(1), dim3(nt), lds, stream, topk_ids, T, top_k, E,
                       ws, faults, zero_out, zero_row_bytes);
    return hipGetLastError();
  }
  const size_t lds = sizeof(int32_t) * (16 + (size_t)E);
  if (top_k <= kRegTopK) {
    const int64_t nchunks = (T + kChunkTokens - 1) / kChunkTokens;
    const size_t lds_c = sizeof(int32_t) * (size_t)E;
    auto kc = top_k == 1 ? route_count_chunks<1>
            : top_k == 2 ? route_count_chunks<2>
            : top_k == 4 ? route_count_chunks<4>
            : top_k == 8 ? route_count_chunks<8>
                         : route_count_chunks<kRegTopK>;
    auto ks = top_k == 1 ? route_scatter_chunks<1>
            : top_k == 2 ? route_scatter_chunks<2>
            : top_k == 4 ? route_scatter_chunks<4>
            : top_k == 8 ? route_scatter_chunks<8>
                         : route_scatter_chunks<kRegTopK>;
    hipLaunchKernelGGL(kc, dim3((uint32_t)nchunks), dim3(kChunkTokens), lds_c, stream, topk_ids, T,
                       top_k, E, ws, faults, zero_out, zero_row_bytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nchunks <= kFusedScanChunks) {
      auto kf = top_k == 1 ? route_scan_scatter_chunks<1>
              : top_k == 2 ? route_scan_scatter_chunks<2>
              : top_k == 4 ? route_scan_scatter_chunks<4>
              : top_k == 8 ? route_scan_scatter_chunks<8>
                           : route_scan_scatter_chunks<kRegTopK>;
      hipLaunchKernelGGL(kf, dim3((uint32_t)nchunks), dim3(kChunkTokens),
                         sizeof(int32_t) * (16 + 2 * (size_t)E), stream, topk_ids, T, top_k, E,
                         nchunks, ws);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(route_scan_chunks, dim3(1), dim3(kSortThreads), lds, stream, E, nchunks, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ks, dim3((uint32_t)nchunks), dim3(kChunkTokens), lds_c, stream, topk_ids, T,
                       top_k, E, ws);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_sort, dim3(1), dim3(kSortThreads), lds, stream, topk_ids, T, top_k, E,
                     ws, faults, zero_out, zero_row_bytes);
  return hipGetLastError();
}

int64_t route_chunk_ints(int64_t T, int top_k, int E) {
  if (T * top_k <= kFastRoutes || top_k > kRegTopK) return 0;
  return (T + kChunkTokens - 1) / kChunkTokens * (int64_t)E;
}

hipError_t launch_combine(const float* rows, const int32_t* route_expert, const float* topk_w,
                          const float* w_ts, int64_t T, int top_k, int64_t N, float* y,
                          hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)T, (uint32_t)((N + 1023) / 1024)), dim3(256),
                     0, stream, rows, route_expert, topk_w, w_ts, T, top_k, N, y);
  return hipGetLastError();
}

}  // namespace nvfp4
