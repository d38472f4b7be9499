// Grouped GEMMs for many rows per expert (the prefill shape), LDS-tiled on
// 32x32x16 bf16 MFMA.
//
// GEMM1 ("SGLang CUTLASS MoE", structure diagram and section 4): per chunk
// of one expert's rows, h = x[token] W13[e]^T with SwiGLU (clamp of the
// Shape-template page, section 4) fused in the epilogue; act stored bf16.
// GEMM2 dense path ("Device-side gating of the MoE GEMM2 path"): per
// 128-row dense tile, y = act W2[e]^T, stored bf16; it runs only when the
// device gate chose the dense path, else its blocks find zero items.
//
// Block tile: 128 token rows x 256 weight rows, 4 waves. The token rows are
// the MFMA N side and are shared by all waves through LDS (a K stage of 128
// is 32 KB, double-buffered); every wave owns 64 weight rows (two 32-row
// MFMA tiles: for GEMM1 the 32 gate rows and the 32 up rows of the same
// features, so SwiGLU pairs meet in one lane) and reads them straight from
// global memory, 16 bytes per lane = 32 E2M1 codes = one scale group,
// decoding them exactly with the scaled convert. No weight byte is read by
// two waves, so weights bypass LDS.
//
// K order inside a 128-step: lane half h and MFMA (q, j) use K = 64q + 32h
// + 8j + [0, 8) on both operands, which keeps each weight load a contiguous
// 16 bytes and leaves the dot products unchanged.
//
// Blocks are mapped XCD-aware: the hardware deals consecutive block ids
// round-robin over the 8 XCDs, so block b works on item
// (b mod 8) * ceil(items / 8) + b / 8, and the blocks that share a token tile
// (consecutive items) and an expert's weights run together on one XCD and
// meet in its L2.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 128;                     // token rows per tile
constexpr int kStageBytes = kTileRows * 128 * 2;   // one K stage of the token tile
constexpr int kTiledThreads = 256;

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Byte offset of 16-byte chunk c (0..15) of tile row r inside a stage. The
// XOR swizzle puts 16 consecutive rows read at one chunk on 16 distinct
// 16-byte bank groups, and 16 consecutive chunks of one row written by 16
// lanes likewise.
__device__ __forceinline__ uint32_t tile_off(int r, int c) {
  return static_cast<uint32_t>(r * 256 + ((c ^ (r & 15)) << 4));
}

}  // namespace

template <bool G1>
__global__ __launch_bounds__(kTiledThreads, 1) void gemm_tiled_kernel(
    const uint16_t* __restrict__ src, uint32_t src_bytes, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ s, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ sorted_slot, int I, int H,
    int Kp, int sub, float limit, uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];
  const int K = G1 ? H : I;
  int ntiles;
  if (G1) {
    ntiles = counters[kCtrNumV];
  } else {
    ntiles = counters[kCtrGate] == 1 ? counters[kCtrGate + 3] : 0;
  }
  const int nspan = G1 ? (I >> 7) : (H >> 8);  // 256-weight-row spans per tile
  const int nitems = ntiles * sub * nspan;
  const int xcd = blockIdx.x & 7;
  const int per = (nitems + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int item = xcd * per + slot;
  if (slot >= per || item >= nitems) return;
  const int span = item % nspan;
  const int ts = item / nspan;
  const int tile = ts / sub;
  const int st = ts - tile * sub;
  const int4 ti = reinterpret_cast<const int4*>(tiles)[tile];
  const int e = ti.x;
  const int row0 = ti.y + st * kTileRows;
  const int nrows = min(kTileRows, ti.z - st * kTileRows);
  if (nrows <= 0) return;

  // ---- token tile loads: thread t moves chunk t%16 of rows 16i + t/16
  const int t = threadIdx.x;
  const int lc = t & 15, lr = t >> 4;
  // Rows past the tile's end get an out-of-range offset (their loads return
  // zero). The row -> slot reads are buffer loads too, so that none of them
  // sits behind a branch.
  uint32_t toff[8];
  if (G1) {
    const __amdgpu_buffer_rsrc_t ssr =
        make_rsrc(sorted_slot + row0, static_cast<uint32_t>(nrows) * 4u);
    uint32_t slotv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      slotv[i] = __builtin_amdgcn_raw_buffer_load_b32(ssr, (i * 16 + lr) * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 16 + lr;
      const uint32_t tok = slotv[i] / static_cast<uint32_t>(Kp);
      toff[i] = tok * static_cast<uint32_t>(K) * 2u + lc * 16 + (r < nrows ? 0u : kNoRow);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 16 + lr;
      toff[i] = static_cast<uint32_t>(row0 + r) * static_cast<uint32_t>(K) * 2u + lc * 16 +
                (r < nrows ? 0u : kNoRow);
    }
  }
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(src, src_bytes);

  // ---- this wave's weight rows
  const int wv = wave_index();
  const int lane = lane_id();
  const int r = lane & 31, h = lane >> 5;
  size_t grow[2];
  int fbase;  // first output column of this wave
  if (G1) {
    fbase = span * 128 + wv * 32;
    grow[0] = static_cast<size_t>(e) * 2 * I + fbase + r;      // gate rows
    grow[1] = grow[0] + I;                                     // up rows
  } else {
    fbase = span * 256 + wv * 64;
    grow[0] = static_cast<size_t>(e) * H + fbase + r;
    grow[1] = grow[0] + 32;
  }
  const size_t wrow = static_cast<size_t>(K) >> 1, srow = static_cast<size_t>(K) >> 5;
  const uint8_t* wp0 = w + grow[0] * wrow + h * 16;
  const uint8_t* wp1 = w + grow[1] * wrow + h * 16;
  const uint8_t* sp0 = s + grow[0] * srow;
  const uint8_t* sp1 = s + grow[1] * srow;

  const int nkb = K >> 7;
  const int last = nkb - 1;
  uint4 tv[8];
  // Weight ring of two stages: stage kb lives in slot kb & 1. The K loop is
  // unrolled by two so that every slot index is a compile-time constant (no
  // register copies between iterations, which would wait on fresh loads).
  uint4 wr[2][2][2];   // [slot][m][q]
  uint32_t sr[2][2];   // [slot][m]: the row's 4 scale bytes of the stage
  auto load_tokens = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) tv[i] = bld16(srs, toff[i] + kb * 256);
  };
  auto store_tokens = [&](int b) {
    uint8_t* base = lds + b * kStageBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(base + tile_off(i * 16 + lr, lc)) = tv[i];
  };
  auto load_weights = [&](int kb, int sl) {
    wr[sl][0][0] = ld16(wp0 + kb * 64);
    wr[sl][0][1] = ld16(wp0 + kb * 64 + 32);
    wr[sl][1][0] = ld16(wp1 + kb * 64);
    wr[sl][1][1] = ld16(wp1 + kb * 64 + 32);
    sr[sl][0] = *reinterpret_cast<const uint32_t*>(sp0 + kb * 4);
    sr[sl][1] = *reinterpret_cast<const uint32_t*>(sp1 + kb * 4);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.0f;

  // One K stage: multiply the stage in LDS buffer / weight slot sl, then
  // move stage kb+1's tokens into the other buffer (read last in stage kb-1,
  // finished by every wave before the previous barrier) and start the loads
  // of stage kb+2 (near the end the last stage again: loaded, never used).
  // Loads retire in issue order, so the issue order (tokens, then weights)
  // is pinned and each wait covers only what it needs.
  auto stage = [&](int kb, int sl) {
    const uint8_t* base = lds + sl * kStageBytes;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      bf16x8_t a[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float scale = e8m0_scale_operand((sr[sl][m] >> (8 * (2 * q + h))) & 0xffu);
        const uint32_t dw[4] = {wr[sl][m][q].x, wr[sl][m][q].y, wr[sl][m][q].z, wr[sl][m][q].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) a[m][j] = decode_fp4x8(dw[j], scale);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t b[4];
#pragma unroll
        for (int n = 0; n < 4; ++n)
          b[n] = as_bf16x8(*reinterpret_cast<const uint4*>(base + tile_off(n * 32 + r, 8 * q + 4 * h + j)));
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 4; ++n) acc[m][n] = mfma32x32x16(a[m][j], b[n], acc[m][n]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    store_tokens(sl ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    const int k2 = min(kb + 2, last);
    load_tokens(k2);
    __builtin_amdgcn_sched_barrier(0);
    load_weights(k2, sl);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };

  // Prologue: stage 0 in LDS, stage 1 in flight.
  load_tokens(0);
  __builtin_amdgcn_sched_barrier(0);
  load_weights(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  store_tokens(0);
  __builtin_amdgcn_sched_barrier(0);
  load_tokens(min(1, last));
  __builtin_amdgcn_sched_barrier(0);
  load_weights(min(1, last), 1);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    stage(kb, 0);
    stage(kb + 1, 1);
  }
  if (kb < nkb) stage(kb, 0);  // odd stage count

  // ---- epilogue. Lane (r, h), accumulator register 4*b4 + i holds weight
  // row 8*b4 + 4*h + i of the 32-row tile against token row 32*n + r.
  if (G1) {
    const __amdgpu_buffer_rsrc_t ors =
        make_rsrc(dst + static_cast<size_t>(row0) * I, static_cast<uint32_t>(nrows) * I * 2);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const f32x16_t& g = acc[0][n];
        const f32x16_t& u = acc[1][n];
        uint2 pk;
        pk.x = pack_bf16x2(swiglu(g[4 * b4 + 0], u[4 * b4 + 0], limit),
                           swiglu(g[4 * b4 + 1], u[4 * b4 + 1], limit));
        pk.y = pack_bf16x2(swiglu(g[4 * b4 + 2], u[4 * b4 + 2], limit),
                           swiglu(g[4 * b4 + 3], u[4 * b4 + 3], limit));
        const uint32_t off =
            static_cast<uint32_t>(n * 32 + r) * I * 2 + (fbase + 8 * b4 + 4 * h) * 2;
        bst8(ors, off, pk);
      }
    }
  } else {
    const __amdgpu_buffer_rsrc_t ors =
        make_rsrc(dst + static_cast<size_t>(row0) * H, static_cast<uint32_t>(nrows) * H * 2);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[m][n][4 * b4 + 0], acc[m][n][4 * b4 + 1]);
          pk.y = pack_bf16x2(acc[m][n][4 * b4 + 2], acc[m][n][4 * b4 + 3]);
          const uint32_t off = static_cast<uint32_t>(n * 32 + r) * H * 2 +
                               (fbase + 32 * m + 8 * b4 + 4 * h) * 2;
          bst8(ors, off, pk);
        }
  }
}

static int tiled_grid(long items) {
  const long per = (items + 7) / 8;
  return static_cast<int>(8 * (per < 1 ? 1 : per));
}

hipError_t launch_gemm1_tiled(const GemmArgs& a, hipStream_t st) {
  const int sub = a.B > kTileRows ? a.B / kTileRows : 1;
  const int grid = tiled_grid(static_cast<long>(a.kmax_v) * sub * (a.I / 128));
  hipLaunchKernelGGL(gemm_tiled_kernel<true>, dim3(grid), dim3(kTiledThreads), 0, st, a.x,
                     static_cast<uint32_t>(static_cast<size_t>(a.T) * a.H * 2), a.w13, a.s13,
                     a.vinfo, a.counters, a.sorted_slot, a.I, a.H, a.Kp, sub, a.limit, a.act);
  return hipGetLastError();
}

hipError_t launch_gemm2_dense_tiled(const GemmArgs& a, hipStream_t st) {
  const int grid = tiled_grid(static_cast<long>(a.max_dense_tiles) * (a.H / 256));
  hipLaunchKernelGGL(gemm_tiled_kernel<false>, dim3(grid), dim3(kTiledThreads), 0, st, a.act,
                     static_cast<uint32_t>(static_cast<size_t>(a.rows_pad) * a.I * 2), a.w2, a.s2,
                     a.dense_tiles, a.counters, a.sorted_slot, a.I, a.H, a.Kp, 1, a.limit, a.y);
  return hipGetLastError();
}

}  // namespace moe
