// Split-path GEMM2 for short K (I <= 512: K = I in at most four 128-element
// steps), the balanced weight stream. Included by gemm.hip (GEMM1 shares the
// token-step helpers) and gemm_tiled.hip, where the stream and the resident
// dense GEMM2 run in one gated launch.
//
// Source: "Device-side gating of the MoE GEMM2 path", sections 1-2 (Split
// path: one expert block per work item, weights streamed; the other path
// finds zero items). GEMM2: y = act W2[e]^T over K = I, stored bf16 in row
// order ("SGLang CUTLASS MoE", section 4).
#pragma once

#include "common.h"

namespace moe {

// XCD-aware wave id for wave-owned contiguous ranges: the hardware deals
// consecutive block ids round-robin over the 8 XCDs, so consecutive ids here
// are waves of one XCD and neighbouring ranges share its L2.
__device__ __forceinline__ int64_t xcd_wave_id() {
  const int64_t lb = static_cast<int64_t>(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  return lb * 4 + wave_index();
}

// Persistent grid of the streaming GEMM2 kernels: waves split the tile list
// evenly. One block per CU (one wave per SIMD): on MI355X, 768 blocks (three
// per CU, the register limit) kept more loads in flight but streamed slower
// (T64 decode 83.8 -> 80.5 us, Zipf-routed T256 EP decode 31.2 -> 27.6 us
// with one block per CU). Timestamps taken per wave showed why: of the three
// blocks sharing a CU the first-dispatched one finished in about 35 us, the
// second in 57 and the third in 72 (the oldest wave issues first), while
// the chip's read rate rose from about 6 to 7.3-7.9 TB/s as the number of
// waves streaming at once fell. 128 or 192 blocks, or a ring of 2, lose.
#ifndef MOE_STREAM_GRID
#define MOE_STREAM_GRID 256
#endif
constexpr int kStreamGrid = MOE_STREAM_GRID;

// Token code bytes of one 128-element K step: E2M1 pairs or E4M3.
template <bool A4>
constexpr uint32_t tok_step_bytes() {
  return A4 ? 64u : 128u;
}

// bf16 act. The work unit is a 16-row tile of one 16-row unit's output over
// the full K. Waves own equal contiguous ranges of the unit-major tile list
// in whole batches of kStreamAhead tiles, so ranges differ by at most one
// batch. A batch's outputs are regrouped across lanes and leave as two
// 16-byte stores a lane, aligned 64-byte pieces of 16 Y rows (four 8-byte
// stores of 32-byte pieces were 1-3 us slower a call). Within the part of
// its range that falls in one unit, a wave keeps the unit's activation
// fragments in registers and streams tiles through a ring kStreamAhead tiles
// deep; each tile's scales come in with one load of exactly the row's I/32
// bytes. The ring is unrolled by kStreamAhead; iterations past the range
// recompute the last tile and their stores fall outside the unit's output
// buffer, so the hardware drops them (no branches in the stream). The caller
// checks the gate word: this runs only on the Split path.
constexpr int kStreamAhead = 4;  // also the Y store regroup's batch (below)

// A batch's four bf16 output pieces, regrouped for whole 64-byte row stores.
// Before: lane r + 16 g holds, in piece a, features 16 a + 4 g .. + 3 of row r
// (the 16x16 MFMA output layout, one tile per piece). After: lane r + 16 h
// holds features 32 k + 8 h .. + 7 of row r in pieces 2 k and 2 k + 1. As a
// 4 x 4 array over (lane group bits g1 g0, piece bits a1 a0) that moves a0 to
// g1, g1 to g0 and g0 to a0: an exchange of g1 with a0 (lanes 32 apart) and
// then one of g0 with a0 (lanes 16 apart).
__device__ __forceinline__ void y_regroup(uint2 (&p)[4]) {
#pragma unroll
  for (int a = 0; a < 4; a += 2) {
    auto x = __builtin_amdgcn_permlane32_swap(p[a].x, p[a + 1].x, false, false);
    auto y = __builtin_amdgcn_permlane32_swap(p[a].y, p[a + 1].y, false, false);
    p[a].x = x[0]; p[a + 1].x = x[1];
    p[a].y = y[0]; p[a + 1].y = y[1];
  }
#pragma unroll
  for (int a = 0; a < 4; a += 2) {
    auto x = __builtin_amdgcn_permlane16_swap(p[a].x, p[a + 1].x, false, false);
    auto y = __builtin_amdgcn_permlane16_swap(p[a].y, p[a + 1].y, false, false);
    p[a].x = x[0]; p[a + 1].x = x[1];
    p[a].y = y[0]; p[a + 1].y = y[1];
  }
}

template <int NKB>
__device__ __forceinline__ void gemm2_stream_body(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int32_t* __restrict__ units,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ counts, int H, int I,
    uint16_t* __restrict__ y) {
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int tpu = H >> 4;  // tiles per unit
  const int64_t total = static_cast<int64_t>(counters[kCtrNumU]) * tpu;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t wid = xcd_wave_id();
  // ranges start on whole batches (H % 512 == 0 makes a unit's tile count a
  // multiple of the batch), so a batch's four tiles are 128 aligned bytes of
  // each Y row
  int64_t t = total / kStreamAhead * wid / nwaves * kStreamAhead;
  const int64_t t_end = total / kStreamAhead * (wid + 1) / nwaves * kStreamAhead;
  const size_t wrow = static_cast<size_t>(I) >> 1, srow = static_cast<size_t>(I) >> 5;
  const uint32_t tstride = static_cast<uint32_t>(16 * wrow);
  const uint32_t sstride = static_cast<uint32_t>(16 * srow);
  while (t < t_end) {
    const int u = static_cast<int>(t / tpu);
    const int h0 = static_cast<int>(t - static_cast<int64_t>(u) * tpu);  // first tile
    const int nt = static_cast<int>(min(t_end, static_cast<int64_t>(u + 1) * tpu) - t);
    const int4 ui = reinterpret_cast<const int4*>(units)[u];
    const int e = ui.x, r0 = ui.y, nrows = ui.z;
    const size_t row0 = static_cast<size_t>(e) * H + h0 * 16 + r;
    const uint8_t* wp = w2 + (row0 - r) * wrow + r * 64 + g * 16;  // packed layout
    const uint8_t* sp = s2 + row0 * srow;
    const __amdgpu_buffer_rsrc_t ars =
        make_rsrc(act + static_cast<size_t>(r0) * I, static_cast<uint32_t>(nrows) * I * 2);
    const __amdgpu_buffer_rsrc_t yrs =
        make_rsrc(y + static_cast<size_t>(r0) * H, static_cast<uint32_t>(nrows) * H * 2);
    const uint32_t boff = static_cast<uint32_t>(r) * I * 2 + g * 64;
    const uint32_t yrow = static_cast<uint32_t>(r) * H * 2 + (h0 * 16 + g * 4) * 2;
    uint4 xa[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[kb][j] = bld16(ars, boff + kb * 256 + j * 16);
    __builtin_amdgcn_sched_barrier(0);
    // weights read once in this call (the expert's only unit): non-temporal
    auto seg = [&](auto ntw) {
      constexpr bool NTW = decltype(ntw)::value;
      uint4 w[kStreamAhead][NKB];
      uint32_t sc[kStreamAhead][NKB];  // the lane row's I/32 scale bytes
      // prologue in slot order (pinned): the loop head then sees the same
      // pending-load order on entry as on every later iteration
  #pragma unroll
      for (int a = 0; a < kStreamAhead; ++a) {
        const uint32_t ti = static_cast<uint32_t>(min(a, nt - 1));
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb) w[a][kb] = ldw16<NTW>(wp + ti * tstride + kb * kPkBlock);
        ld_dwords(sp + ti * sstride, sc[a]);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int i0 = 0; i0 < nt; i0 += kStreamAhead) {
        uint2 res[kStreamAhead];
  #pragma unroll
        for (int a = 0; a < kStreamAhead; ++a) {
          const int i = i0 + a;
          f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const float s = e8m0_scale_operand((sc[a][kb] >> (8 * g)) & 0xffu);
            const uint32_t ww[4] = {w[a][kb].x, w[a][kb].y, w[a][kb].z, w[a][kb].w};
  #pragma unroll
            for (int j = 0; j < 4; ++j)
              acc = mfma16x16x32(decode_fp4x8(ww[j], s), as_bf16x8(xa[kb][j]), acc);
          }
          __builtin_amdgcn_sched_barrier(0);
          const uint32_t ti = static_cast<uint32_t>(min(i + kStreamAhead, nt - 1));
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb) w[a][kb] = ldw16<NTW>(wp + ti * tstride + kb * kPkBlock);
          ld_dwords(sp + ti * sstride, sc[a]);
          res[a].x = pack_bf16x2(acc[0], acc[1]);
          res[a].y = pack_bf16x2(acc[2], acc[3]);
          __builtin_amdgcn_sched_barrier(0);
        }
        y_regroup(res);
  #pragma unroll
        for (int k = 0; k < 2; ++k)
          bst16(yrs, i0 + 2 * k + (g >> 1) < nt ? yrow + 8 * g + i0 * 32 + 64 * k : 0xfffffff0u,
                uint4{res[2 * k].x, res[2 * k].y, res[2 * k + 1].x, res[2 * k + 1].y});
      }
    };
    if (counts[e] <= 16) seg(BoolC<true>{}); else seg(BoolC<false>{});
    t += nt;
  }
}

// MX act, W4A8 (or W4A4 with A4): the same balanced stream with the MX act
// fragments (and their scale bytes) in registers and one scaled MFMA per tile
// and K step. Split path only, as above.
template <int NKB, bool A4>
__device__ __forceinline__ void gemm2_stream_mx_body(
    const uint8_t* __restrict__ actq, const uint8_t* __restrict__ acts,
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const int32_t* __restrict__ units, const int32_t* __restrict__ counters,
    const int32_t* __restrict__ counts, int H, int I, uint16_t* __restrict__ y) {
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int tpu = H >> 4;
  const int64_t total = static_cast<int64_t>(counters[kCtrNumU]) * tpu;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t wid = xcd_wave_id();
  // ranges start on whole batches (H % 512 == 0 makes a unit's tile count a
  // multiple of the batch), so a batch's four tiles are 128 aligned bytes of
  // each Y row
  int64_t t = total / kStreamAhead * wid / nwaves * kStreamAhead;
  const int64_t t_end = total / kStreamAhead * (wid + 1) / nwaves * kStreamAhead;
  const size_t wrow = static_cast<size_t>(I) >> 1, srow = static_cast<size_t>(I) >> 5;
  const uint32_t tstride = static_cast<uint32_t>(16 * wrow);
  const uint32_t sstride = static_cast<uint32_t>(16 * srow);
  while (t < t_end) {
    const int u = static_cast<int>(t / tpu);
    const int h0 = static_cast<int>(t - static_cast<int64_t>(u) * tpu);
    const int nt = static_cast<int>(min(t_end, static_cast<int64_t>(u + 1) * tpu) - t);
    const int4 ui = reinterpret_cast<const int4*>(units)[u];
    const int e = ui.x, r0 = ui.y, nrows = ui.z;
    const size_t row0 = static_cast<size_t>(e) * H + h0 * 16 + r;
    const uint8_t* wp = w2 + (row0 - r) * wrow + r * 64 + g * 16;  // packed layout
    const uint8_t* sp = s2 + row0 * srow;
    constexpr uint32_t XS = tok_step_bytes<A4>();
    const uint32_t IB = A4 ? static_cast<uint32_t>(I) / 2 : static_cast<uint32_t>(I);
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(actq + static_cast<size_t>(r0) * IB, static_cast<uint32_t>(nrows) * IB);
    const __amdgpu_buffer_rsrc_t ars =
        make_rsrc(acts + static_cast<size_t>(r0) * srow, static_cast<uint32_t>(nrows * srow));
    const __amdgpu_buffer_rsrc_t yrs =
        make_rsrc(y + static_cast<size_t>(r0) * H, static_cast<uint32_t>(nrows) * H * 2);
    const uint32_t qoff = static_cast<uint32_t>(r) * IB + g * 16;
    const uint32_t aoff = static_cast<uint32_t>(r * srow) + g;
    const uint32_t yrow = static_cast<uint32_t>(r) * H * 2 + (h0 * 16 + g * 4) * 2;
    uint4 xa[NKB][2];
    uint32_t xsa[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      xa[kb][0] = bld16(qrs, qoff + kb * XS);
      if (!A4) xa[kb][1] = bld16(qrs, qoff + kb * XS + 64);
      xsa[kb] = bld1(ars, aoff + kb * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
    // weights read once in this call (the expert's only unit): non-temporal
    auto seg = [&](auto ntw) {
      constexpr bool NTW = decltype(ntw)::value;
      uint4 w[kStreamAhead][NKB];
      uint32_t sc[kStreamAhead][NKB];  // the lane row's I/32 scale bytes
  #pragma unroll
      for (int a = 0; a < kStreamAhead; ++a) {
        const uint32_t ti = static_cast<uint32_t>(min(a, nt - 1));
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb) w[a][kb] = ldw16<NTW>(wp + ti * tstride + kb * kPkBlock);
        ld_dwords(sp + ti * sstride, sc[a]);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int i0 = 0; i0 < nt; i0 += kStreamAhead) {
        uint2 res[kStreamAhead];
  #pragma unroll
        for (int a = 0; a < kStreamAhead; ++a) {
          const int i = i0 + a;
          f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            acc = mfma_f4xa<A4>(w[a][kb], (sc[a][kb] >> (8 * g)) & 0xffu, xa[kb][0], xa[kb][1], xsa[kb],
                                acc);
          __builtin_amdgcn_sched_barrier(0);
          const uint32_t ti = static_cast<uint32_t>(min(i + kStreamAhead, nt - 1));
  #pragma unroll
          for (int kb = 0; kb < NKB; ++kb) w[a][kb] = ldw16<NTW>(wp + ti * tstride + kb * kPkBlock);
          ld_dwords(sp + ti * sstride, sc[a]);
          res[a].x = pack_bf16x2(acc[0], acc[1]);
          res[a].y = pack_bf16x2(acc[2], acc[3]);
          __builtin_amdgcn_sched_barrier(0);
        }
        y_regroup(res);
  #pragma unroll
        for (int k = 0; k < 2; ++k)
          bst16(yrs, i0 + 2 * k + (g >> 1) < nt ? yrow + 8 * g + i0 * 32 + 64 * k : 0xfffffff0u,
                uint4{res[2 * k].x, res[2 * k].y, res[2 * k + 1].x, res[2 * k + 1].y});
      }
    };
    if (counts[e] <= 16) seg(BoolC<true>{}); else seg(BoolC<false>{});
    t += nt;
  }
}

}  // namespace moe
