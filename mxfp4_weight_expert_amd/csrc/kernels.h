// Host-side launchers of the layer's kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouteArgs {
  const float* logits;       // [T, Eg] or null (ids mode)
  const int32_t* topk_ids;   // [T, topk] (ids mode)
  const float* topk_w;       // [T, topk] (ids mode)
  const uint16_t* shared_logits;  // [T, S] bf16
  int T, Eg, topk, S, E, expert_offset;
  float shared_scale;
  int32_t* route_ids;    // [T, topk]
  int32_t* slot_expert;  // [T, K']
  float* slot_w;         // [T, K']
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

struct SortArgs {
  const int32_t* slot_expert;
  int nslots, Ep, B, n_ranges, force_path;
  int32_t* range_counts;  // [n_ranges, Ep]
  int32_t* counts;        // [Ep]
  int32_t* offsets;       // [Ep + 1]
  int32_t* sorted_slot;   // [nslots]
  int32_t* expanded_idx;  // [nslots]
  int32_t* vinfo;         // [kmax_v, 4]
  int32_t* units16;       // [max_units16, 4]: 16-row units
  int32_t* dense_tiles;   // [max_dense_tiles, 4]
  int32_t* counters;      // [kCounterWords]
};
// Histogram -> scan (+ chunk table) -> scatter -> GEMM2 gate.
hipError_t launch_sort_and_gate(const SortArgs& a, hipStream_t st);

struct GemmArgs {
  const uint16_t* x;         // [T, H] bf16
  const uint8_t* w13;        // [Ep, 2I, H/2]
  const uint8_t* s13;        // [Ep, 2I, H/32]
  const uint8_t* w2;         // [Ep, H, I/2]
  const uint8_t* s2;         // [Ep, H, I/32]
  const int32_t* vinfo;
  const int32_t* units16;
  const int32_t* dense_tiles;
  const int32_t* counters;
  const int32_t* counts;  // [Ep] rows per local expert
  const int32_t* sorted_slot;
  int T, H, I, Kp, B, kmax_v, max_dense_tiles, max_units16, rows_pad;
  int Ep;  // local experts including the shared ones
  int dense_grid_tiles;  // tiles the dense GEMM2 grid is sized for (the kernels loop past it)
  ActArgs act_fn;  // GEMM1 epilogue activation
  uint16_t* act;  // [rows_pad, I] bf16 (W4A16), E4M3 codes (W4A8) or E2M1 code pairs [rows_pad, I/2] (W4A4)
  uint16_t* y;    // [rows_pad, H] bf16
  // MX activations (a8 != 0: W4A8 MXFP8, or W4A4 MXFP4 when a4 is also set):
  // quantised x and act scales
  int a8;
  int a4;
  const uint8_t* xq;    // [T, H] E4M3 (W4A8) or [T, H/2] E2M1 pairs (W4A4)
  const uint8_t* xs;    // [T, H/32] E8M0
  uint8_t* act_scales;  // [rows_pad, I/32] E8M0
};
hipError_t launch_gemm1(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm2(const GemmArgs& a, hipStream_t st);  // split + dense, gated on device
// LDS-tiled kernels for many rows per expert (gemm_tiled.hip): GEMM1 over the
// chunk table (B >= 64); GEMM2 of both paths in one gated launch (bf16 act
// with I <= kResidentMaxI, or MX act); the generic dense GEMM2 over the dense
// tiles for bf16 act with larger I.
hipError_t launch_gemm1_tiled(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm2_gated(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm2_gated_mx(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm2_dense_tiled(const GemmArgs& a, hipStream_t st);

// x -> MXFP8 (W4A8 path: xq [T, H] E4M3 codes) or MXFP4 (a4, W4A4 path:
// xq [T, H/2] E2M1 code pairs), xs [T, H/32] E8M0 scales.
hipError_t launch_quant_x(const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* xs, bool a4,
                          hipStream_t st);
// MX-activation GEMM1 kernels, W4A8 or W4A4 by a4 (launch_gemm1 dispatches to
// them when a8 is set).
hipError_t launch_gemm1_a8(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm1_tiled_a8(const GemmArgs& a, hipStream_t st);

struct FinalizeArgs {
  const uint16_t* y;
  const int32_t* expanded_idx;
  const float* slot_w;
  int T, Kp, H;
  uint16_t* out;
};
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t st);
hipError_t launch_prepack(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t row_bytes,
                          hipStream_t st);

}  // namespace moe
