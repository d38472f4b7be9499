// C ABI of the MoE layer: shape checks, the workspace carve and the fixed
// launch chain route -> sort (count, scan, scatter) -> GEMM2 gate -> GEMM1 ->
// GEMM2 split -> GEMM2 dense -> finalize on one stream.
//
// The workspace carve follows the Shape-template page, section 3 (one byte
// buffer, 256-byte aligned pieces, padding rows after the last chunk); the
// shape limits are this library's own (the page's static_asserts fix
// H % 512 and I % 128, which are kept).
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr uint64_t kAlign = 256;
constexpr int64_t kMaxSlots = int64_t(1) << 23;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_shape(const moe_mxfp4_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID;
  if (s->T < 0 || s->E < 1 || s->E_global < 1 || s->topk < 1 || s->S < 0 || s->H < 1 ||
      s->I < 1 || s->expert_offset < 0)
    return MOE_ERR_INVALID;
  if (static_cast<int64_t>(s->expert_offset) + s->E > s->E_global) return MOE_ERR_INVALID;
  if (!std::isfinite(s->swiglu_limit) || !std::isfinite(s->shared_scale)) return MOE_ERR_INVALID;
  if (s->force_gemm2_path < -1 || s->force_gemm2_path > 1) return MOE_ERR_INVALID;
  if (s->weight_layout != MOE_WEIGHTS_ROW_MAJOR && s->weight_layout != MOE_WEIGHTS_PACKED)
    return MOE_ERR_INVALID;
  if (s->topk > kMaxTopK || s->topk > s->E_global || s->S > kMaxShared) return MOE_ERR_UNSUPPORTED;
  if (s->E + s->S > kMaxExperts || s->E_global > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (s->H % 512 != 0 || s->I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  // the tiled GEMMs keep a tile's scale rows (8 bytes per K element) in LDS
  if (s->H > kMaxTiledK || s->I > kMaxTiledK) return MOE_ERR_UNSUPPORTED;
  if (s->block_n != 16 && s->block_n != 32 && s->block_n != 64 && s->block_n != 128 &&
      s->block_n != 256)
    return MOE_ERR_UNSUPPORTED;
  if (s->activation != MOE_ACT_SWIGLU && s->activation != MOE_ACT_SITU) return MOE_ERR_UNSUPPORTED;
  if (s->activation == MOE_ACT_SITU &&
      !(std::isfinite(s->act_beta) && s->act_beta > 0.0f && std::isfinite(s->act_linear_beta) &&
        s->act_linear_beta > 0.0f))
    return MOE_ERR_INVALID;
  if (s->a_dtype != MOE_ADTYPE_BF16 && s->a_dtype != MOE_ADTYPE_MXFP8 &&
      s->a_dtype != MOE_ADTYPE_MXFP4)
    return MOE_ERR_UNSUPPORTED;
  // the MX-activation split GEMM2 keeps a row's whole K in registers: I <= 512
  if (s->a_dtype != MOE_ADTYPE_BF16 && s->I > 512) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(s->T) * (s->topk + s->S) > kMaxSlots) return MOE_ERR_UNSUPPORTED;
  // the kernels address x and act with 32-bit buffer offsets
  const int64_t rows = static_cast<int64_t>(s->T) * (s->topk + s->S) + 256;
  if (static_cast<int64_t>(s->T) * s->H * 2 >= (int64_t(1) << 31) ||
      rows * s->I * 2 >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

void carve(const moe_mxfp4_shape* s, moe_mxfp4_ws_layout* L) {
  const uint64_t T = s->T, Kp = s->topk + s->S, Ep = s->E + s->S, H = s->H, I = s->I;
  const uint64_t slots = T * Kp;
  const bool mx = s->a_dtype != MOE_ADTYPE_BF16;
  // bytes per activation element times 2: bf16 4, E4M3 2, E2M1 1
  const uint64_t el2 = s->a_dtype == MOE_ADTYPE_MXFP4 ? 1 : (mx ? 2 : 4);
  L->kmax_v = static_cast<int32_t>(Ep + slots / s->block_n);
  L->max_dense_tiles = static_cast<int32_t>(Ep + slots / kDenseMT);
  L->max_units16 = static_cast<int32_t>(Ep + slots / 16);
  L->n_ranges = static_cast<int32_t>(slots == 0 ? 1 : (slots + kRangeSlots - 1) / kRangeSlots);
  const uint64_t pad = s->block_n > kDenseMT ? s->block_n : kDenseMT;
  L->rows_pad = static_cast<int32_t>(slots + pad);
  const uint64_t rp = static_cast<uint64_t>(L->rows_pad);
  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L->counters = take(kCounterWords * 4);
  L->route_ids = take(T * s->topk * 4);
  L->slot_expert = take(slots * 4);
  L->slot_w = take(slots * 4);
  L->range_counts = take(static_cast<uint64_t>(L->n_ranges) * Ep * 4);
  L->counts = take(Ep * 4);
  L->offsets = take((Ep + 1) * 4);
  L->sorted_slot = take(slots * 4);
  L->expanded_idx = take(slots * 4);
  L->vinfo = take(static_cast<uint64_t>(L->kmax_v) * 16);
  L->dense_tiles = take(static_cast<uint64_t>(L->max_dense_tiles) * 16);
  L->units16 = take(static_cast<uint64_t>(L->max_units16) * 16);
  L->act = take(rp * I * el2 / 2);
  L->act_scales = take(mx ? rp * I / 32 : 0);
  L->y = take(rp * H * 2);
  L->xq = take(mx ? T * H * el2 / 2 : 0);
  L->xs = take(mx ? T * H / 32 : 0);
  L->total_bytes = o;
}

}  // namespace

extern "C" {

int moe_mxfp4_query(const moe_mxfp4_shape* shape, uint64_t* workspace_bytes) {
  if (workspace_bytes == nullptr) return MOE_ERR_INVALID;
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  moe_mxfp4_ws_layout L;
  carve(shape, &L);
  *workspace_bytes = L.total_bytes;
  return MOE_OK;
}

int moe_mxfp4_workspace_layout(const moe_mxfp4_shape* shape, moe_mxfp4_ws_layout* layout) {
  if (layout == nullptr) return MOE_ERR_INVALID;
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  carve(shape, layout);
  return MOE_OK;
}

int moe_mxfp4_prepack(const uint8_t* w_dev, uint8_t* w_packed_dev, int64_t rows,
                      int64_t row_bytes, void* stream) {
  if (w_dev == nullptr || w_packed_dev == nullptr || rows <= 0 || row_bytes <= 0)
    return MOE_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(w_dev) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(w_packed_dev) & 15) != 0)
    return MOE_ERR_INVALID;
  if (rows % 16 != 0 || row_bytes % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows > (int64_t{1} << 40) / row_bytes) return MOE_ERR_UNSUPPORTED;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w_dev);
  const uintptr_t b = reinterpret_cast<uintptr_t>(w_packed_dev);
  const uintptr_t n = static_cast<uintptr_t>(rows * row_bytes);
  if (a < b + n && b < a + n) return MOE_ERR_INVALID;
  return moe::launch_prepack(w_dev, w_packed_dev, rows, row_bytes,
                             static_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

const char* moe_mxfp4_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH:
      return "shape needs more scratch than the allocation-free entry point holds";
    default: return "unknown error";
  }
}

}  // extern "C"

namespace {

int forward_impl(const void* x_dev, const float* router_logits_dev, const int32_t* topk_ids_dev,
                 const float* topk_w_dev, const void* shared_logits_dev, const uint8_t* w13_dev,
                 const uint8_t* s13_dev, const uint8_t* w2_dev, const uint8_t* s2_dev,
                 const moe_mxfp4_shape* shape, void* out_dev, void* workspace_dev,
                 uint64_t workspace_bytes, void* stream, void* const* stage_events) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  const moe_mxfp4_shape& s = *shape;
  // the GEMMs read w13 and w2 only in the packed layout
  if (s.weight_layout != MOE_WEIGHTS_PACKED) return MOE_ERR_UNSUPPORTED;
  const bool ids_mode = topk_ids_dev != nullptr || topk_w_dev != nullptr;
  if (ids_mode == (router_logits_dev != nullptr)) return MOE_ERR_INVALID;
  if (ids_mode && (topk_ids_dev == nullptr || topk_w_dev == nullptr)) return MOE_ERR_INVALID;
  if (s.T == 0) return MOE_OK;
  if (x_dev == nullptr || w13_dev == nullptr || s13_dev == nullptr || w2_dev == nullptr ||
      s2_dev == nullptr || out_dev == nullptr || workspace_dev == nullptr)
    return MOE_ERR_INVALID;
  if (s.S > 0 && shared_logits_dev == nullptr) return MOE_ERR_INVALID;
  // x, out, the weights and their scales are accessed with 16-byte vector
  // loads and stores at multiples of 16 bytes from these pointers; the
  // routing inputs with 4-byte loads, the shared logits with 2-byte loads.
  auto aligned = [](const void* p, uintptr_t a) {
    return reinterpret_cast<uintptr_t>(p) % a == 0;  // NULL passes
  };
  if (!aligned(x_dev, 16) || !aligned(out_dev, 16) || !aligned(w13_dev, 16) ||
      !aligned(s13_dev, 16) || !aligned(w2_dev, 16) || !aligned(s2_dev, 16) ||
      !aligned(router_logits_dev, 4) || !aligned(topk_ids_dev, 4) || !aligned(topk_w_dev, 4) ||
      !aligned(shared_logits_dev, 2))
    return MOE_ERR_INVALID;
  moe_mxfp4_ws_layout L;
  carve(&s, &L);
  if (workspace_bytes < L.total_bytes || reinterpret_cast<uintptr_t>(workspace_dev) % kAlign != 0)
    return MOE_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  int stage = 0;
  auto mark = [&]() {
    if (stage_events == nullptr) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(stage_events[stage++]), st);
  };
  uint8_t* ws = static_cast<uint8_t*>(workspace_dev);
  auto at = [&](uint64_t off) { return ws + off; };
  const int Kp = s.topk + s.S, Ep = s.E + s.S;
  const int nslots = s.T * Kp;

  RouteArgs ra;
  ra.logits = router_logits_dev;
  ra.topk_ids = topk_ids_dev;
  ra.topk_w = topk_w_dev;
  ra.shared_logits = static_cast<const uint16_t*>(shared_logits_dev);
  ra.T = s.T;
  ra.Eg = s.E_global;
  ra.topk = s.topk;
  ra.S = s.S;
  ra.E = s.E;
  ra.expert_offset = s.expert_offset;
  ra.shared_scale = s.shared_scale;
  ra.route_ids = reinterpret_cast<int32_t*>(at(L.route_ids));
  ra.slot_expert = reinterpret_cast<int32_t*>(at(L.slot_expert));
  ra.slot_w = reinterpret_cast<float*>(at(L.slot_w));
  if (mark() != hipSuccess || launch_route(ra, st) != hipSuccess) return MOE_ERR_HIP;

  SortArgs sa;
  sa.slot_expert = ra.slot_expert;
  sa.nslots = nslots;
  sa.Ep = Ep;
  sa.B = s.block_n;
  sa.n_ranges = L.n_ranges;
  sa.force_path = s.force_gemm2_path;
  sa.range_counts = reinterpret_cast<int32_t*>(at(L.range_counts));
  sa.counts = reinterpret_cast<int32_t*>(at(L.counts));
  sa.offsets = reinterpret_cast<int32_t*>(at(L.offsets));
  sa.sorted_slot = reinterpret_cast<int32_t*>(at(L.sorted_slot));
  sa.expanded_idx = reinterpret_cast<int32_t*>(at(L.expanded_idx));
  sa.vinfo = reinterpret_cast<int32_t*>(at(L.vinfo));
  sa.units16 = reinterpret_cast<int32_t*>(at(L.units16));
  sa.dense_tiles = reinterpret_cast<int32_t*>(at(L.dense_tiles));
  sa.counters = reinterpret_cast<int32_t*>(at(L.counters));
  if (mark() != hipSuccess || launch_sort_and_gate(sa, st) != hipSuccess) return MOE_ERR_HIP;

  GemmArgs ga;
  ga.x = static_cast<const uint16_t*>(x_dev);
  ga.w13 = w13_dev;
  ga.s13 = s13_dev;
  ga.w2 = w2_dev;
  ga.s2 = s2_dev;
  ga.vinfo = sa.vinfo;
  ga.units16 = sa.units16;
  ga.dense_tiles = sa.dense_tiles;
  ga.counters = sa.counters;
  ga.counts = sa.counts;
  ga.sorted_slot = sa.sorted_slot;
  ga.T = s.T;
  ga.rows_pad = L.rows_pad;
  ga.H = s.H;
  ga.I = s.I;
  ga.Kp = Kp;
  ga.Ep = Ep;
  ga.B = s.block_n;
  ga.kmax_v = L.kmax_v;
  ga.max_dense_tiles = L.max_dense_tiles;
  {
    // The gate picks the dense path only when R >= 64 U, so it then has at
    // most R / 128 + U <= R_max / 128 + R_max / 64 tiles: a decode shape
    // launches a small dense grid that exits at once. A forced dense path
    // can have up to max_dense_tiles.
    const int64_t rmax = static_cast<int64_t>(s.T) * (s.topk + s.S);
    const int64_t bound = rmax / 128 + rmax / 64 + 1;
    ga.dense_grid_tiles = s.force_gemm2_path == MOE_GEMM2_AUTO
                              ? static_cast<int>(std::min<int64_t>(L.max_dense_tiles, bound))
                              : L.max_dense_tiles;
  }
  ga.max_units16 = L.max_units16;
  ga.act_fn.kind = s.activation;
  ga.act_fn.limit = s.swiglu_limit;
  ga.act_fn.beta = s.act_beta;
  ga.act_fn.inv_beta = s.activation == MOE_ACT_SITU ? 1.0f / s.act_beta : 0.0f;
  ga.act_fn.lb = s.act_linear_beta;
  ga.act_fn.inv_lb = s.activation == MOE_ACT_SITU ? 1.0f / s.act_linear_beta : 0.0f;
  ga.act = reinterpret_cast<uint16_t*>(at(L.act));
  ga.y = reinterpret_cast<uint16_t*>(at(L.y));
  ga.a8 = s.a_dtype != MOE_ADTYPE_BF16;  // MX activations (W4A8 or W4A4)
  ga.a4 = s.a_dtype == MOE_ADTYPE_MXFP4;
  ga.xq = at(L.xq);
  ga.xs = at(L.xs);
  ga.act_scales = at(L.act_scales);
  if (mark() != hipSuccess) return MOE_ERR_HIP;
  if (ga.a8 && launch_quant_x(ga.x, s.T, s.H, at(L.xq), at(L.xs), ga.a4 != 0, st) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_gemm1(ga, st) != hipSuccess) return MOE_ERR_HIP;
  if (mark() != hipSuccess || launch_gemm2(ga, st) != hipSuccess) return MOE_ERR_HIP;

  FinalizeArgs fa;
  fa.y = ga.y;
  fa.expanded_idx = sa.expanded_idx;
  fa.slot_w = ra.slot_w;
  fa.T = s.T;
  fa.Kp = Kp;
  fa.H = s.H;
  fa.out = static_cast<uint16_t*>(out_dev);
  if (mark() != hipSuccess || launch_finalize(fa, st) != hipSuccess) return MOE_ERR_HIP;
  if (mark() != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_mxfp4_forward(const void* x_dev, const float* router_logits_dev,
                      const int32_t* topk_ids_dev, const float* topk_w_dev,
                      const void* shared_logits_dev, const uint8_t* w13_dev,
                      const uint8_t* s13_dev, const uint8_t* w2_dev, const uint8_t* s2_dev,
                      const moe_mxfp4_shape* shape, void* out_dev, void* workspace_dev,
                      uint64_t workspace_bytes, void* stream) {
  return forward_impl(x_dev, router_logits_dev, topk_ids_dev, topk_w_dev, shared_logits_dev,
                      w13_dev, s13_dev, w2_dev, s2_dev, shape, out_dev, workspace_dev,
                      workspace_bytes, stream, nullptr);
}

int moe_mxfp4_forward_timed(const void* x_dev, const float* router_logits_dev,
                            const int32_t* topk_ids_dev, const float* topk_w_dev,
                            const void* shared_logits_dev, const uint8_t* w13_dev,
                            const uint8_t* s13_dev, const uint8_t* w2_dev, const uint8_t* s2_dev,
                            const moe_mxfp4_shape* shape, void* out_dev, void* workspace_dev,
                            uint64_t workspace_bytes, void* stream, void* const* stage_events) {
  if (stage_events == nullptr) return MOE_ERR_INVALID;
  for (int i = 0; i <= MOE_NUM_STAGES; ++i)
    if (stage_events[i] == nullptr) return MOE_ERR_INVALID;
  return forward_impl(x_dev, router_logits_dev, topk_ids_dev, topk_w_dev, shared_logits_dev,
                      w13_dev, s13_dev, w2_dev, s2_dev, shape, out_dev, workspace_dev,
                      workspace_bytes, stream, stage_events);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free entry point. The workspace lives in a file-scope device
// array: one copy per GPU the library runs on, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and that
// pointer is what the launch chain receives. Every call on a GPU shares that
// GPU's copy; the chain writes every map it later reads in the same call, so
// nothing has to start at zero, and calls that overlap on one GPU race.
namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int current_device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_mxfp4_forward_noalloc(const void* x_dev, const float* router_logits_dev,
                              const int32_t* topk_ids_dev, const float* topk_w_dev,
                              const void* shared_logits_dev, const uint8_t* w13_dev,
                              const uint8_t* s13_dev, const uint8_t* w2_dev,
                              const uint8_t* s2_dev, const moe_mxfp4_shape* shape,
                              void* out_dev, void* stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  moe_mxfp4_ws_layout L;
  carve(shape, &L);
  if (L.total_bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  const int rs = current_device_scratch(&ws);
  if (rs != MOE_OK) return rs;
  return forward_impl(x_dev, router_logits_dev, topk_ids_dev, topk_w_dev, shared_logits_dev,
                      w13_dev, s13_dev, w2_dev, s2_dev, shape, out_dev, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // extern "C"
