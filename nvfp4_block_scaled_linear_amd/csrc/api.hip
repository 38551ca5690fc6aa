// C ABI of libnvfp4 (declared and documented in include/nvfp4.h): argument checks on the
// host, then kernel dispatch on the caller's stream. Nothing here allocates memory or
// synchronizes; the only state kept between calls is each device's address of the
// no-allocation call's fixed scratch array.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "kernels.hpp"
#include "nvfp4.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // sizes must fit the kernels' int indices
constexpr int64_t kMaxK = (int64_t)1 << 22;    // a 64-row weight block stays under 2^31 bytes
constexpr int64_t kMaxBufferBytes = ((int64_t)1 << 31) - 1;  // 32-bit buffer offsets
constexpr int kMaxExperts = 4096;               // route grouping keeps per-expert counters in LDS
constexpr int kStreamMaxRows = 16;              // rows of one weight-streaming pass

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

nvfp4_status launch_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH; }

// checks shared by the weight operand and the activation operand of linear/grouped calls
nvfp4_status check_act(int32_t act_kind, const void* x, const uint8_t* x_scales,
                       const float* x_ts, int64_t ldx, int64_t K) {
  if (act_kind != NVFP4_ACT_BF16 && act_kind != NVFP4_ACT_NVFP4 &&
      act_kind != NVFP4_ACT_BF16_QUANTIZE)
    return NVFP4_ERR_ARG;
  if (!x) return NVFP4_ERR_NULL;
  if (!aligned(x, 16)) return NVFP4_ERR_ALIGN;
  if (act_kind != NVFP4_ACT_NVFP4) {
    if (x_scales || x_ts) return NVFP4_ERR_ARG;
    if (ldx < K || ldx > kMaxDim) return NVFP4_ERR_SHAPE;
    if (ldx % 8 != 0) return NVFP4_ERR_ALIGN;
  } else {
    if (!x_scales || !x_ts) return NVFP4_ERR_NULL;
    if (!aligned(x_scales, 2) || !aligned(x_ts, 4)) return NVFP4_ERR_ALIGN;
  }
  return NVFP4_OK;
}

nvfp4_status check_flags(uint32_t flags, const uint32_t* faults) {
  if (flags & ~(uint32_t)NVFP4_F_CHECK) return NVFP4_ERR_ARG;
  if ((flags & NVFP4_F_CHECK) && !faults) return NVFP4_ERR_NULL;
  if (faults && !aligned(faults, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// check mode: the activation operand's data (rows x rows of K values)
hipError_t check_act_data(int32_t act_kind, const void* x, const uint8_t* x_scales,
                          const float* x_ts, int64_t ldx, int64_t rows, int64_t K,
                          uint32_t* faults, hipStream_t s) {
  if (act_kind == NVFP4_ACT_NVFP4) return launch_check_scales(x_scales, rows * (K / 16), x_ts, rows, faults, s);
  return launch_check_bf16(x, ldx, rows, K, faults, s);
}

nvfp4_status check_weight(const uint8_t* w_codes, const uint8_t* w_scales, const float* w_ts) {
  if (!w_codes || !w_scales || !w_ts) return NVFP4_ERR_NULL;
  if (!aligned(w_codes, 16) || !aligned(w_scales, 2) || !aligned(w_ts, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

nvfp4_status check_k(int64_t K) {
  if (K <= 0 || K > kMaxK || K % 32 != 0) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

// The grouped call takes the MFMA GEMM path when its routes average at least this many per
// active expert (prompt-sized batches); below it, the weight-streaming kernel.
constexpr int64_t kGroupedGemmRoutes = 32;

bool grouped_uses_gemm(int64_t T, int top_k, int E) {
  const int64_t R = T * top_k;
  const int64_t active = R < E ? R : E;
  return R >= kGroupedGemmRoutes * active;
}

// The GEMM path's wide form (each expert's first 256 routes in one 256-route tile, the
// rest in 64-route tiles) when the experts hold at least this many routes on average;
// below it most of a 256-route tile would be padding. Depends on the route set only, so
// that both calls of a layer agree on the workspace's grouping.
constexpr int64_t kGroupedWideRoutes = 192;
bool grouped_uses_wide(int64_t T, int top_k, int E) {
  const int64_t R = T * top_k;
  const int64_t active = R < E ? R : E;
  return grouped_uses_gemm(T, top_k, E) && R >= kGroupedWideRoutes * active;
}

// grouped-call workspace layout: 256-byte aligned regions
struct Layout {
  size_t offsets, active, n_active, route_expert, sorted, slots, rows, tiles, n_tiles, chunks, total;
  int64_t max_tiles;
};

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout grouped_layout(int64_t T, int top_k, int E, int64_t N, int32_t out_mode) {
  Layout L;
  const size_t R = (size_t)T * (size_t)top_k;
  const bool gemm = grouped_uses_gemm(T, top_k, E);
  const int64_t tr = gemm_grouped_tile_rows(grouped_uses_wide(T, top_k, E));
  L.max_tiles = gemm ? ((int64_t)R + tr - 1) / tr + E : 0;  // one partial tile per expert
  size_t o = 0;
  L.offsets = o; o = up256(o + sizeof(int32_t) * ((size_t)E + 1));
  L.active = o; o = up256(o + sizeof(int32_t) * (size_t)E);
  L.n_active = o; o = up256(o + sizeof(int32_t));
  L.route_expert = o; o = up256(o + sizeof(int32_t) * R);
  L.sorted = o; o = up256(o + sizeof(int32_t) * R);
  L.slots = o; o = up256(o + kSlotInts * sizeof(int32_t) * (R < (size_t)E ? R : (size_t)E));
  L.tiles = o; o = up256(o + sizeof(int32_t) * 2 * (size_t)L.max_tiles);
  L.n_tiles = o; o = up256(o + sizeof(int32_t));
  L.chunks = o; o = up256(o + sizeof(int32_t) * (size_t)route_chunk_ints(T, top_k, E));
  L.rows = o;
  if (out_mode == NVFP4_OUT_COMBINE) o = up256(o + sizeof(float) * R * (size_t)N);
  L.total = o;
  return L;
}

// The no-allocation grouped call's scratch: a fixed device array (one per GPU, held
// until the process ends) in place of the caller's workspace. Host code never passes the
// array's name (a host-side stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = (size_t)NVFP4_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// this thread's current device's scratch address
nvfp4_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVFP4_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int32_t status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: a size is invalid (<= 0, K % 32 != 0, ld too small, or too large)";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: a pointer or leading dimension is misaligned";
    case NVFP4_ERR_ARG: return "NVFP4_ERR_ARG: an enum value or count is out of range";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE: workspace too small";
    case NVFP4_ERR_LAUNCH: return "NVFP4_ERR_LAUNCH: the HIP runtime refused a launch";
    default: return "unknown nvfp4_status";
  }
}

nvfp4_status nvfp4_linear(int32_t act_kind, const void* x, const uint8_t* x_scales,
                          const float* x_ts, int64_t ldx, int64_t M, int64_t N, int64_t K,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_ts,
                          float* y, int64_t ldy, uint32_t flags, uint32_t* faults,
                          void* stream) {
  nvfp4_status st;
  if ((st = check_flags(flags, faults)) != NVFP4_OK) return st;
  if ((st = check_k(K)) != NVFP4_OK) return st;
  if (M <= 0 || N <= 0 || M > kMaxDim || N > kMaxDim) return NVFP4_ERR_SHAPE;
  if ((st = check_act(act_kind, x, x_scales, x_ts, ldx, K)) != NVFP4_OK) return st;
  if (act_kind == NVFP4_ACT_BF16_QUANTIZE && (M != 1 || K > 8192)) return NVFP4_ERR_SHAPE;
  if ((st = check_weight(w_codes, w_scales, w_ts)) != NVFP4_OK) return st;
  if (!y) return NVFP4_ERR_NULL;
  if (ldy < N || ldy > kMaxDim) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 4)) return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the kernels address activation rows with 32-bit buffer offsets
  if (act_kind != NVFP4_ACT_NVFP4 &&
      (M <= kStreamMaxRows ? M * ldx * 2 > kMaxBufferBytes : ldx > gemm_max_ldx()))
    return NVFP4_ERR_SHAPE;
  if (act_kind == NVFP4_ACT_NVFP4 && M * (K / 2) > kMaxBufferBytes) return NVFP4_ERR_SHAPE;
  if (flags & NVFP4_F_CHECK) {
    hipError_t e = launch_check_scales(w_scales, N * (K / 16), w_ts, 1, faults, s);
    if (e == hipSuccess)
      e = check_act_data(act_kind, x, x_scales, x_ts, ldx, M, K, faults, s);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  }
  if (M <= kStreamMaxRows) {
    StreamArgs a{};
    a.x = x; a.x_scales = x_scales; a.x_ts = x_ts; a.ldx = ldx;
    a.w_codes = w_codes; a.w_scales = w_scales; a.w_ts = w_ts;
    a.N = N; a.K = K; a.y = y; a.ldy = ldy; a.M = (int32_t)M; a.apply_ts = 1; a.x_rows = M;
    return launch_status(launch_stream(a, act_kind, false, 1, s));
  }
  GemmArgs g{};
  g.x = x; g.x_scales = x_scales; g.x_ts = x_ts; g.ldx = ldx;
  g.w_codes = w_codes; g.w_scales = w_scales; g.w_ts = w_ts;
  g.M = M; g.N = N; g.K = K; g.y = y; g.ldy = ldy;
  return launch_status(launch_gemm(g, act_kind, s));
}

nvfp4_status nvfp4_quantize_act(int32_t in_type, const void* x, int64_t ldx, int64_t M,
                                int64_t K, int32_t ts_mode, uint8_t* codes, uint8_t* scales,
                                float* ts, uint32_t* faults, void* stream) {
  nvfp4_status st;
  if ((st = check_k(K)) != NVFP4_OK) return st;
  if (in_type != NVFP4_IN_BF16 && in_type != NVFP4_IN_F32) return NVFP4_ERR_ARG;
  if (ts_mode != NVFP4_TS_PER_ROW && ts_mode != NVFP4_TS_PER_TENSOR) return NVFP4_ERR_ARG;
  if (M <= 0 || M > kMaxDim || ldx < K || ldx > kMaxDim) return NVFP4_ERR_SHAPE;
  if (M * (K / 16) > ((int64_t)1 << 40)) return NVFP4_ERR_SHAPE;
  if (!x || !codes || !scales || !ts) return NVFP4_ERR_NULL;
  const int64_t elem = in_type == NVFP4_IN_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ldx * elem) % 16 != 0) return NVFP4_ERR_ALIGN;
  if (!aligned(codes, 16) || !aligned(ts, 4) || (faults && !aligned(faults, 4)))
    return NVFP4_ERR_ALIGN;
  if (ts_mode == NVFP4_TS_PER_ROW && M > (int64_t)UINT32_MAX / 2) return NVFP4_ERR_SHAPE;
  return launch_status(launch_quantize(in_type == NVFP4_IN_BF16 ? 0 : 1, x, ldx, M, K,
                                       ts_mode == NVFP4_TS_PER_ROW ? 0 : 1, codes, scales, ts,
                                       faults, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_grouped_linear(int32_t act_kind, const void* x, const uint8_t* x_scales,
                                  const float* x_ts, int64_t ldx, int32_t rows_mode,
                                  int64_t T, int32_t top_k, int64_t N, int64_t K,
                                  int32_t num_experts, const uint8_t* w_codes,
                                  const uint8_t* w_scales, const float* w_ts,
                                  const int32_t* topk_ids, const float* topk_w,
                                  int32_t out_mode, void* y, void* workspace,
                                  size_t* workspace_bytes, uint32_t flags, uint32_t* faults,
                                  void* stream) {
  nvfp4_status st;
  if (!workspace_bytes) return NVFP4_ERR_NULL;
  if ((st = check_flags(flags, faults)) != NVFP4_OK) return st;
  // the in-call quantization is a dense decode-batch form only
  if (act_kind == NVFP4_ACT_BF16_QUANTIZE) return NVFP4_ERR_ARG;
  // the grouping left in the workspace by the layer's earlier call (combine only)
  const bool reuse = (out_mode & NVFP4_OUT_REUSE_GROUPING) != 0;
  out_mode &= ~(int32_t)NVFP4_OUT_REUSE_GROUPING;
  if (reuse && out_mode != NVFP4_OUT_COMBINE) return NVFP4_ERR_ARG;
  if ((st = check_k(K)) != NVFP4_OK) return st;
  if (num_experts <= 0 || num_experts > kMaxExperts) return NVFP4_ERR_ARG;
  if (top_k <= 0 || top_k > num_experts || top_k > 64) return NVFP4_ERR_ARG;
  if (rows_mode != NVFP4_ROWS_PER_TOKEN && rows_mode != NVFP4_ROWS_PER_ROUTE) return NVFP4_ERR_ARG;
  if (out_mode != NVFP4_OUT_ROUTES && out_mode != NVFP4_OUT_SWIGLU_BF16 &&
      out_mode != NVFP4_OUT_COMBINE)
    return NVFP4_ERR_ARG;
  if (T <= 0 || N <= 0 || T > kMaxDim || N > kMaxDim || T * top_k > kMaxDim) return NVFP4_ERR_SHAPE;
  if (out_mode == NVFP4_OUT_SWIGLU_BF16 && N % 2 != 0) return NVFP4_ERR_SHAPE;
  if ((int64_t)num_experts * N * (K / 2) > ((int64_t)1 << 46)) return NVFP4_ERR_SHAPE;
  if (N * (K / 2) > kMaxBufferBytes) return NVFP4_ERR_SHAPE;  // one expert, 32-bit offsets
  const Layout L = grouped_layout(T, top_k, num_experts, N, out_mode);
  if (!workspace) {
    *workspace_bytes = L.total;
    return NVFP4_OK;
  }
  if (*workspace_bytes < L.total) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  if ((st = check_act(act_kind, x, x_scales, x_ts, ldx, K)) != NVFP4_OK) return st;
  if ((st = check_weight(w_codes, w_scales, w_ts)) != NVFP4_OK) return st;
  {
    const int64_t xrows = rows_mode == NVFP4_ROWS_PER_TOKEN ? T : T * top_k;
    const int64_t xbytes = act_kind == NVFP4_ACT_BF16 ? ((xrows - 1) * ldx + K) * 2 : xrows * (K / 2);
    if (xbytes > kMaxBufferBytes) return NVFP4_ERR_SHAPE;
  }
  if (!topk_ids || !y) return NVFP4_ERR_NULL;
  if (out_mode == NVFP4_OUT_COMBINE && !topk_w) return NVFP4_ERR_NULL;
  if (!aligned(topk_ids, 4) || (topk_w && !aligned(topk_w, 4)) || !aligned(y, 4))
    return NVFP4_ERR_ALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (flags & NVFP4_F_CHECK) {
    const int64_t xrows = rows_mode == NVFP4_ROWS_PER_TOKEN ? T : T * top_k;
    hipError_t e = launch_check_scales(w_scales, (int64_t)num_experts * N * (K / 16), w_ts,
                                       num_experts, faults, s);
    if (e == hipSuccess) e = check_act_data(act_kind, x, x_scales, x_ts, ldx, xrows, K, faults, s);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  }
  char* base = static_cast<char*>(workspace);
  RouteWorkspace ws;
  ws.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  ws.active = reinterpret_cast<int32_t*>(base + L.active);
  ws.n_active = reinterpret_cast<int32_t*>(base + L.n_active);
  ws.route_expert = reinterpret_cast<int32_t*>(base + L.route_expert);
  ws.sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  ws.slots = reinterpret_cast<int32_t*>(base + L.slots);
  ws.max_slots = (int32_t)(T * top_k < num_experts ? T * top_k : num_experts);
  ws.rows = reinterpret_cast<float*>(base + L.rows);
  ws.tiles = reinterpret_cast<int32_t*>(base + L.tiles);
  ws.n_tiles = reinterpret_cast<int32_t*>(base + L.n_tiles);
  ws.chunk_counts = reinterpret_cast<int32_t*>(base + L.chunks);
  const bool gemm = L.max_tiles > 0;
  const bool wide = grouped_uses_wide(T, top_k, num_experts);
  ws.tile_rows = gemm ? gemm_grouped_tile_rows(wide) : 0;
  ws.main_rows = wide ? kWideGroupedRows : 0;

  // dropped routes read as zero rows in the per-route output forms; the grouping kernel
  // clears them
  void* zero_out = out_mode == NVFP4_OUT_COMBINE ? nullptr : y;
  const int64_t zero_row_bytes = out_mode == NVFP4_OUT_ROUTES ? N * 4 : N;  // fp32 / BF16 N/2
  hipError_t e = hipSuccess;
  if (!reuse) {
    e = launch_route_sort(topk_ids, T, top_k, num_experts, ws, faults, zero_out, zero_row_bytes, s);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  }

  const int64_t R = T * top_k;
  if (gemm) {
    // prompt-sized: MFMA tiles of one expert's routes
    GemmArgs g{};
    g.x = x; g.x_scales = x_scales; g.x_ts = x_ts; g.ldx = ldx;
    g.w_codes = w_codes; g.w_scales = w_scales; g.w_ts = w_ts;
    g.N = N; g.K = K;
    g.tiles = ws.tiles; g.n_tiles = ws.n_tiles; g.offsets = ws.offsets; g.sorted = ws.sorted;
    g.x_rows = rows_mode == NVFP4_ROWS_PER_TOKEN ? T : T * top_k;
    g.rows_per_token = rows_mode == NVFP4_ROWS_PER_TOKEN ? 1 : 0;
    g.top_k = top_k;
    if (out_mode == NVFP4_OUT_ROUTES) {
      g.y = static_cast<float*>(y); g.ldy = N; g.apply_ts = 1;
    } else if (out_mode == NVFP4_OUT_SWIGLU_BF16) {
      g.a_out = static_cast<uint16_t*>(y); g.apply_ts = 1;  // the GEMM's epilogue
    } else {
      g.y = ws.rows; g.ldy = N; g.apply_ts = 0;
    }
    if (wide) {
      g.active = ws.active; g.n_active = ws.n_active;
      e = launch_gemm_grouped_wide(g, act_kind, R < num_experts ? R : num_experts, L.max_tiles, s);
    } else {
      e = launch_gemm_grouped(g, act_kind, L.max_tiles, s);
    }
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
    if (out_mode == NVFP4_OUT_COMBINE) {
      e = launch_combine(ws.rows, ws.route_expert, topk_w, w_ts, T, top_k, N,
                         static_cast<float*>(y), s);
    }
    return launch_status(e);
  }
  StreamArgs a{};
  a.x = x; a.x_scales = x_scales; a.x_ts = x_ts; a.ldx = ldx;
  a.w_codes = w_codes; a.w_scales = w_scales; a.w_ts = w_ts;
  a.N = N; a.K = K;
  a.slots = ws.slots; a.sorted = ws.sorted;
  a.rows_per_token = rows_mode == NVFP4_ROWS_PER_TOKEN ? 1 : 0;
  a.x_rows = rows_mode == NVFP4_ROWS_PER_TOKEN ? T : T * top_k;
  a.top_k = top_k;
  // rows per expert pass (sets of four): sized from the mean routes per active expert
  {
    const int64_t active = R < num_experts ? R : num_experts;
    a.M = (int32_t)((R + active - 1) / active);
  }
  if (out_mode == NVFP4_OUT_ROUTES) {
    a.y = static_cast<float*>(y); a.ldy = N; a.apply_ts = 1;
  } else if (out_mode == NVFP4_OUT_SWIGLU_BF16) {
    // the streaming kernel's epilogue applies SwiGLU and writes the BF16 rows
    a.a_out = static_cast<uint16_t*>(y); a.apply_ts = 1;
  } else {
    a.y = ws.rows; a.ldy = N; a.apply_ts = 0;
  }
  const int max_active = (int)(R < num_experts ? R : num_experts);
  e = launch_stream(a, act_kind, true, max_active, s);
  if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  if (out_mode == NVFP4_OUT_COMBINE) {
    e = launch_combine(ws.rows, ws.route_expert, topk_w, w_ts, T, top_k, N,
                       static_cast<float*>(y), s);
  }
  return launch_status(e);
}

nvfp4_status nvfp4_grouped_linear_noalloc(int32_t act_kind, const void* x,
                                          const uint8_t* x_scales, const float* x_ts,
                                          int64_t ldx, int32_t rows_mode, int64_t T,
                                          int32_t top_k, int64_t N, int64_t K,
                                          int32_t num_experts, const uint8_t* w_codes,
                                          const uint8_t* w_scales, const float* w_ts,
                                          const int32_t* topk_ids, const float* topk_w,
                                          int32_t out_mode, void* y, uint32_t flags,
                                          uint32_t* faults, void* stream) {
  // the size this call needs, from the host-side checks alone (nothing is enqueued)
  size_t need = 0;
  nvfp4_status st = nvfp4_grouped_linear(act_kind, x, x_scales, x_ts, ldx, rows_mode, T, top_k,
                                         N, K, num_experts, w_codes, w_scales, w_ts, topk_ids,
                                         topk_w, out_mode, y, nullptr, &need, flags, faults,
                                         stream);
  if (st != NVFP4_OK) return st;
  if (need > kScratchBytes) return NVFP4_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = device_scratch(&ws)) != NVFP4_OK) return st;
  size_t have = kScratchBytes;
  return nvfp4_grouped_linear(act_kind, x, x_scales, x_ts, ldx, rows_mode, T, top_k, N, K,
                              num_experts, w_codes, w_scales, w_ts, topk_ids, topk_w, out_mode,
                              y, ws, &have, flags, faults, stream);
}

nvfp4_status nvfp4_prefetch(const void* buf, int64_t bytes, int32_t workgroups, void* stream) {
  if (!buf) return NVFP4_ERR_NULL;
  if (bytes < 16 || bytes > ((int64_t)1 << 31) - 16 || bytes % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(buf, 16)) return NVFP4_ERR_ALIGN;
  if (workgroups < 0 || workgroups > 8192) return NVFP4_ERR_ARG;
  return launch_status(launch_prefetch(buf, bytes, workgroups ? workgroups : 512,
                                       static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_read_probe(const void* buf, int64_t bytes, int32_t loads_per_thread,
                              uint32_t* sink, void* stream) {
  if (!buf || !sink) return NVFP4_ERR_NULL;
  if (bytes < 16 || bytes > ((int64_t)1 << 31) - 16 || bytes % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return NVFP4_ERR_ALIGN;
  if (loads_per_thread != 1 && loads_per_thread != 2 && loads_per_thread != 4 &&
      loads_per_thread != 8 && loads_per_thread != 16)
    return NVFP4_ERR_ARG;
  return launch_status(launch_read_probe(buf, bytes, loads_per_thread, sink,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
