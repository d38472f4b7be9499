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
// Block tile: 128 token rows (MFMA N side) x 256 weight rows (M side), 8
// waves, two per SIMD so that one wave's converts and LDS reads overlap the
// other's MFMAs. Wave (wm, wn) computes 64 weight rows x 64 tokens: for
// GEMM1 the 32 gate rows and the 32 up rows of the same features, so SwiGLU
// pairs meet in one lane. Each K stage of 128 moves the token tile (32 KB,
// gathered rows) and the packed weight tile (16 KB, 64 bytes per row, four
// lanes per row) from global memory through registers into a double-buffered
// LDS stage; the block's scale rows are copied to LDS once. A wave reads its
// weight fragments from LDS as 16 bytes per lane = 32 E2M1 codes = one scale
// group and decodes them exactly with the scaled convert.
//
// K order inside a 128-step: lane half h and MFMA (q, j) use K = 64q + 32h
// + 8j + [0, 8) on both operands, which keeps each weight fragment a
// contiguous 16 bytes and leaves the dot products unchanged.
//
// Blocks are persistent and mapped XCD-aware: the hardware deals
// consecutive block ids round-robin over the 8 XCDs, so the items are cut
// into 8 contiguous ranges, one per XCD, and the blocks of an XCD walk its
// range in order: blocks that share a token tile (consecutive items) and an
// expert's weights run together on one XCD and meet in its L2.
#include "common.h"
#include "kernels.h"
#include "gemm2_stream.h"

namespace moe {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 128;                     // token rows per tile
constexpr int kTileWRows = 256;                    // weight rows per tile
constexpr int kTiledThreads = 512;
constexpr int kTokStage = kTileRows * 128 * 2;     // bf16 token bytes of one K stage (32 KB)
constexpr int kTok8Stage = kTileRows * 128;        // E4M3 token bytes of one K stage (16 KB)
constexpr int kWStage = kTileWRows * 64;           // packed weight bytes of one K stage (16 KB)

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS bank swizzle of row r: an XOR over 16 chunk slots that is a bijection
// on every 16 aligned rows and, within each row parity, on every 32 aligned
// rows. gfx950 serves a 16-byte LDS access 32 lanes at a time over 128
// banks (16 lanes over 64 banks on earlier parts), so 32 consecutive rows
// read at one logical chunk fall on 32 distinct 16-byte bank groups. It
// depends on r mod 32 only, so rows 32 apart share their lane addresses.
__device__ __forceinline__ int row_swz(int r) { return (r ^ ((r >> 4) & 1)) & 15; }

// Byte offset of 16-byte chunk c (0..15) of bf16 token row r (256-byte rows)
// inside a stage. 32 consecutive rows read at one chunk, and the 16 chunks
// of each of two consecutive rows written by 32 lanes, hit distinct bank
// groups.
__device__ __forceinline__ uint32_t tok_off(int r, int c) {
  return static_cast<uint32_t>(r * 256 + ((c ^ row_swz(r)) << 4));
}
// Byte offset of 16-byte chunk c (0..7) of E4M3 token row r (128-byte rows):
// 16 consecutive rows read at one chunk differ in row parity or in
// (row >> 1) & 7, so they hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t tok8_off(int r, int c) {
  return static_cast<uint32_t>(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
}
// Byte offset of 16-byte chunk c (0..3) of E2M1 token row r (64-byte rows):
// the 32 lanes reading rows r0..r0+15 at chunks g, g' (g, g' < 2, or >= 2)
// hit 32 distinct 16-byte bank groups of a 512-byte bank line, since rows
// r and r + 8 (the same 64-byte unit of the line) swap chunk halves.
__device__ __forceinline__ uint32_t tok4_off(int r, int c) {
  return static_cast<uint32_t>(r * 64 + ((c ^ (((r >> 3) & 1) << 1)) << 4));
}
// MX token row layout of one K stage: E4M3 (128 bytes) or E2M1 (64 bytes).
template <bool A4>
__device__ __forceinline__ uint32_t tokmx_off(int r, int c) {
  if constexpr (A4)
    return tok4_off(r, c);
  else
    return tok8_off(r, c);
}
// Byte offset of 16-byte chunk c (0..3) of weight row rho in a stage of
// ROWS rows (a multiple of 32): chunk-major, so the 32 rows of one MFMA
// fragment are a permutation of 32 consecutive 16-byte slots (conflict-free
// reads); the XOR with 4c ^ 8c (0, 12, 24, 20 for c = 0..3) spreads the four
// chunks of 8 rows, written by 32 neighbouring lanes, over distinct bank
// groups under both the 64- and the 128-bank organisation.
template <int ROWS>
__device__ __forceinline__ uint32_t c_off(int rho, int c) {
  return static_cast<uint32_t>(c * (ROWS * 16) + ((rho ^ (c << 2) ^ (c << 3)) << 4));
}
__device__ __forceinline__ uint32_t w_off(int rho, int c) { return c_off<kTileWRows>(rho, c); }

}  // namespace

// LDS: two stages of tokens, packed weights and weight scales (104 KB for
// MB = 2, 121 KB for MB = 3). The stage copy goes global -> registers -> LDS
// with RING stages of loads in flight.
//
// MB is the number of 32-row weight blocks per wave: the block tile has
// 128 * MB weight rows. For GEMM1 each 32-row block holds the gate rows
// (rows 0..15) and the up rows (16..31) of 16 consecutive features, so that
// a SwiGLU pair meets in one lane (accumulator registers 4b + i and
// 4(b + 2) + i); a tile spans 64 * MB features. For GEMM2 the block's rows
// are 128 * MB consecutive output features.
template <bool G1, int MB>
__global__ __launch_bounds__(kTiledThreads, 2) void gemm_tiled_kernel(
    const uint16_t* __restrict__ src, uint32_t src_bytes, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ s, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ sorted_slot, int I, int H,
    int Kp, int sub, ActArgs actf, uint16_t* __restrict__ dst) {
  constexpr int kWR = 128 * MB;               // weight rows per tile
  constexpr int kRingN = MB == 2 ? 4 : 2;     // stages of loads in flight = stages per scale group
  constexpr int kWSt = kWR * 64;              // packed weight bytes of one K stage
  constexpr int kScG = kWR * 4 * kRingN;      // scale words of one group, stage-major
  constexpr int kWPer = kWR * 4 / kTiledThreads;  // weight chunks per thread and stage
  constexpr int kScPer = (kWR + kTiledThreads - 1) / kTiledThreads;
  static_assert(kWR * 4 % kTiledThreads == 0, "weight chunks must split evenly");
  __shared__ __attribute__((aligned(16))) uint8_t tok_lds[2 * kTokStage];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[2 * kWSt];
  __shared__ __attribute__((aligned(16))) uint8_t sc_lds[2 * kScG];
  const int K = G1 ? H : I;
  int ntiles;
  if (G1) {
    ntiles = counters[kCtrNumV];
  } else {
    ntiles = counters[kCtrGate] == 1 ? counters[kCtrGate + 3] : 0;
  }
  const int nspan = G1 ? I / (64 * MB) : H / kWR;  // weight-row spans per token tile
  const int nitems = ntiles * sub * nspan;
  const int xcd = blockIdx.x & 7;
  const int per = (nitems + 7) >> 3;
  const int nblk_x = static_cast<int>(gridDim.x) >> 3;  // blocks per XCD
  const int t = threadIdx.x;
  const size_t wrow = static_cast<size_t>(K) >> 1, srow = static_cast<size_t>(K) >> 5;
  const int wave = wave_index();
  const int wm = wave & 1, wn = wave >> 1;
  const int lane = lane_id();
  const int r = lane & 31, h = lane >> 5;
  // thread roles in the stage copy: token chunk t%16 of rows 32i + t/16;
  // weight chunk t%4 of tile rows 128i + t/4; the scale words of tile rows
  // (t + 512i) mod kWR (threads that meet a row twice store the same bytes)
  const int lc = t & 15, lr = t >> 4, wc = t & 3, wr = t >> 2;
  for (int slot = blockIdx.x >> 3; slot < per; slot += nblk_x) {
    const int item = xcd * per + slot;
    if (item >= nitems) break;
    const int span = item % nspan;
    const int ts = item / nspan;
    const int tile = ts / sub;
    const int st = ts - tile * sub;
    const int4 ti = reinterpret_cast<const int4*>(tiles)[tile];
    const int e = ti.x;
    const int row0 = ti.y + st * kTileRows;
    const int nrows = min(kTileRows, ti.z - st * kTileRows);
    if (nrows <= 0) continue;
    const int f0 = G1 ? span * 64 * MB : span * kWR;
    // Row of expert e's weight block that tile row rho stands for.
    auto erow_of = [&](int rho) -> uint32_t {
      if (G1) {
        const int rr = rho & 31;
        const int feat = f0 + 16 * (rho >> 5) + (rr & 15);
        return static_cast<uint32_t>(rr < 16 ? feat : I + feat);
      }
      return static_cast<uint32_t>(f0 + rho);
    };

    // Token rows past the tile's end get an out-of-range offset (their loads
    // return zero). The row -> slot reads are buffer loads too, so that none
    // of them sits behind a branch.
    uint32_t toff[4];
    if (G1) {
      const __amdgpu_buffer_rsrc_t ssr =
          make_rsrc(sorted_slot + row0, static_cast<uint32_t>(nrows) * 4u);
      uint32_t slotv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) slotv[i] = bld4(ssr, (i * 32 + lr) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = i * 32 + lr;
        const uint32_t tok = slotv[i] / static_cast<uint32_t>(Kp);
        toff[i] = tok * static_cast<uint32_t>(K) * 2u + lc * 16 + (rr < nrows ? 0u : kNoRow);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = i * 32 + lr;
        toff[i] = static_cast<uint32_t>(row0 + rr) * static_cast<uint32_t>(K) * 2u + lc * 16 +
                  (rr < nrows ? 0u : kNoRow);
      }
    }
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(src, src_bytes);
    // The expert's weight and scale rows through buffers, so that per-lane
    // offsets are 32-bit.
    const size_t erows = G1 ? static_cast<size_t>(2) * I : static_cast<size_t>(H);
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(w + static_cast<size_t>(e) * erows * wrow, static_cast<uint32_t>(erows * wrow));
    const __amdgpu_buffer_rsrc_t scs =
        make_rsrc(s + static_cast<size_t>(e) * erows * srow, static_cast<uint32_t>(erows * srow));
    // tile rows 128i + wr stand for expert rows erow_of(wr) + wstep * i
    // packed layout: 16-row groups of wrow * 16 bytes, 1 KB per 64-byte K step
    const uint32_t er = erow_of(wr);
    const uint32_t woff = (er & ~15u) * static_cast<uint32_t>(wrow) + (er & 15u) * 64 + wc * 16;
    const uint32_t wstep = (G1 ? 64u : 128u) * static_cast<uint32_t>(wrow);
    uint32_t soff[kScPer];
    int srho[kScPer];
#pragma unroll
    for (int i = 0; i < kScPer; ++i) {
      srho[i] = (i * kTiledThreads + t) % kWR;
      soff[i] = erow_of(srho[i]) * static_cast<uint32_t>(srow);
    }

    const int nkb = K >> 7;
    const int last = nkb - 1;
    const int lastg = last / kRingN;
    uint4 tv[kRingN][4], wv[kRingN][kWPer];
    uint4 sg[kScPer];  // scale bytes of the next group of kRingN stages
    auto load_stage = [&](int kb, int sl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tv[sl][i] = bld16s(srs, toff[i], kb * 256);
#pragma unroll
      for (int i = 0; i < kWPer; ++i) wv[sl][i] = bld16s(wrs, woff, kb * kPkBlock + i * wstep);
    };
    auto load_group = [&](int g) {
#pragma unroll
      for (int i = 0; i < kScPer; ++i) {
        if (kRingN == 4) {
          sg[i] = bld16(scs, soff[i] + g * 16);
        } else if (kRingN == 3) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b96(scs, soff[i] + g * 12, 0, 0);
          sg[i] = make_uint4(v[0], v[1], v[2], 0u);
        } else {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(scs, soff[i] + g * 8, 0, 0);
          sg[i] = make_uint4(v[0], v[1], 0u, 0u);
        }
      }
    };
    auto store_group = [&](int g) {
      uint32_t* sb = reinterpret_cast<uint32_t*>(sc_lds + (g & 1) * kScG);
#pragma unroll
      for (int i = 0; i < kScPer; ++i) {
        const uint32_t v[4] = {sg[i].x, sg[i].y, sg[i].z, sg[i].w};
#pragma unroll
        for (int q = 0; q < kRingN; ++q) sb[q * kWR + srho[i]] = v[q];
      }
    };
    // one 16-byte load p of load_stage (same order as the stores below)
    auto load_piece = [&](int kb, int sl, int p) {
      if (p < 4) tv[sl][p] = bld16s(srs, toff[p], kb * 256);
      else if (p - 4 < kWPer) wv[sl][p - 4] = bld16s(wrs, woff, kb * kPkBlock + (p - 4) * wstep);
    };
    // one 16-byte piece p of store_stage: token chunks p < 4, then weight chunks
    auto store_piece = [&](int b, int sl, int p) {
      if (p < 4) {
        *reinterpret_cast<uint4*>(tok_lds + b * kTokStage + tok_off(p * 32 + lr, lc)) = tv[sl][p];
      } else if (p - 4 < kWPer) {
        *reinterpret_cast<uint4*>(w_lds + b * kWSt + c_off<kWR>((p - 4) * 128 + wr, wc)) = wv[sl][p - 4];
      }
    };
    auto store_stage = [&](int b, int sl) {
      uint8_t* tb = tok_lds + b * kTokStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(tb + tok_off(i * 32 + lr, lc)) = tv[sl][i];
      uint8_t* wb = w_lds + b * kWSt;
#pragma unroll
      for (int i = 0; i < kWPer; ++i)
        *reinterpret_cast<uint4*>(wb + c_off<kWR>(i * 128 + wr, wc)) = wv[sl][i];
    };

    int rho[MB];  // tile weight rows of the wave's 32-row MFMA blocks (lane r)
#pragma unroll
    for (int m = 0; m < MB; ++m) rho[m] = (wn * MB + m) * 32 + r;

    f32x16_t acc[MB][2];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.0f;

    // operands of the sub-step deferred to the next stage (zero before the
    // first stage: its group 0 then adds nothing)
    bf16x8_t ac[MB], bc[2];
#pragma unroll
    for (int m = 0; m < MB; ++m) ac[m] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
    for (int n = 0; n < 2; ++n) bc[n] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));

    // One K stage with register slot sl = kb % kRingN: multiply the stage in
    // LDS buffer kb & 1, move stage kb+1 (slot (sl+1) % kRingN, loaded
    // kRingN - 1 stages ago) into the other buffer (read last in stage kb-1,
    // which every wave finished before the previous barrier) one 16-byte
    // piece per sub-step group, so the writes overlap the MFMAs instead of
    // bunching up before the barrier (2.71 -> 2.58 ms at 32k tokens on
    // MI355X; 7 pieces per thread for 384-row tiles, 6 for 256), and refill
    // slot sl (free since its stage went to LDS) with stage kb + kRingN one
    // piece per group too, a further 2.8% (near the end the last stage again:
    // loaded, never used). Scales move in groups of kRingN stages: the first stage of
    // group g loads group g + 1, its last stage stores it to the other scale
    // buffer (last read in group g - 1). Loads retire in issue order; the
    // pinned order keeps each wait to what it needs.
    auto stage = [&](int kb, int sl) {
      const int b = kb & 1;
      const uint8_t* tb = tok_lds + b * kTokStage;
      const uint8_t* wb = w_lds + b * kWSt;
      const uint32_t* sb =
          reinterpret_cast<const uint32_t*>(sc_lds + ((kb / kRingN) & 1) * kScG) + sl * kWR;
      // Eight K sub-steps (q, j) of 16, software-pipelined: the operands of
      // a sub-step are read and decoded one group of MFMAs ahead. Group 0
      // multiplies the previous stage's last sub-step (its operands are in
      // registers, so it needs no barrier) while this stage's scales, packed
      // weights and first tokens arrive; group g = 1..7 multiplies sub-step
      // g - 1 and prepares sub-step g; sub-step 7 waits in (ac, bc) for the
      // next stage's group 0. Each group is a scheduling region of its own,
      // with the LDS reads first and the MFMAs alternating with converts.
      uint32_t sdw[MB];
      uint4 wq[2][MB];
      float scale[2][MB];
      bf16x8_t an[MB], bn[2];
      auto read_tok = [&](int t8, bf16x8_t (&dst)[2]) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
          dst[n] = as_bf16x8(*reinterpret_cast<const uint4*>(
              tb + tok_off(wm * 64 + n * 32 + r, 8 * (t8 >> 2) + 4 * h + (t8 & 3))));
      };
      auto dec = [&](int t8, bf16x8_t (&dst)[MB]) {
        const int q = t8 >> 2, j = t8 & 3;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const uint4 v = wq[q][m];
          const uint32_t dw = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
          dst[m] = decode_fp4x8(dw, scale[q][m]);
        }
      };
      auto mfmas = [&]() {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n) acc[m][n] = mfma32x32x16(ac[m], bc[n], acc[m][n]);
      };
      auto rotate = [&]() {
#pragma unroll
        for (int m = 0; m < MB; ++m) ac[m] = an[m];
#pragma unroll
        for (int n = 0; n < 2; ++n) bc[n] = bn[n];
      };
      // group 0
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < MB; ++m) sdw[m] = sb[rho[m]];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int m = 0; m < MB; ++m)
          wq[q][m] = *reinterpret_cast<const uint4*>(wb + c_off<kWR>(rho[m], 2 * q + h));
      read_tok(0, bn);
      mfmas();
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int m = 0; m < MB; ++m)
          scale[q][m] = e8m0_scale_operand((sdw[m] >> (8 * (2 * q + h))) & 0xffu);
      dec(0, an);
      __builtin_amdgcn_sched_group_barrier(0x100, 3 * MB + 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * MB, 0);      // MFMAs
      __builtin_amdgcn_sched_barrier(0);
      rotate();
#pragma unroll
      for (int t8 = 0; t8 < 7; ++t8) {
        __builtin_amdgcn_sched_barrier(0);
        read_tok(t8 + 1, bn);
        dec(t8 + 1, an);
        store_piece(b ^ 1, (sl + 1) % kRingN, t8);  // next stage, one piece per group
        load_piece(min(kb + kRingN, last), sl, t8);  // slot sl is free: in LDS since stage kb-1
        mfmas();
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
        if (t8 < 4 + kWPer) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        if (t8 < 4 + kWPer) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
#pragma unroll
        for (int k = 0; k < 2 * MB; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU ops
        }
        __builtin_amdgcn_sched_barrier(0);
        rotate();
      }
      __builtin_amdgcn_sched_barrier(0);
      if (4 + kWPer > 7) store_piece(b ^ 1, (sl + 1) % kRingN, 7);
      if (sl == kRingN - 1) store_group(kb / kRingN + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (4 + kWPer > 7) load_piece(min(kb + kRingN, last), sl, 7);
      if (sl == 0) load_group(min(kb / kRingN + 1, lastg));
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };

    // Prologue: scale group 0 and stages 0 .. kRingN-1 in flight, then group
    // 0 and stage 0 in LDS.
    load_group(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < kRingN; ++sl) {
      load_stage(min(sl, last), sl);
      __builtin_amdgcn_sched_barrier(0);
    }
    store_group(0);
    store_stage(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    int kb = 0;
    for (; kb + kRingN - 1 < nkb; kb += kRingN) {
#pragma unroll
      for (int sl = 0; sl < kRingN; ++sl) stage(kb + sl, sl);
    }
#pragma unroll
    for (int sl = 0; sl < kRingN - 1; ++sl)
      if (kb + sl < nkb) stage(kb + sl, sl);
    // the last stage's deferred sub-step
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[m][n] = mfma32x32x16(ac[m], bc[n], acc[m][n]);

    // ---- epilogue. Lane (r, h), accumulator register 4*b4 + i holds row
    // 8*b4 + 4*h + i of the 32-row weight block against token row 32*n + r
    // of the wave's 64 tokens.
    if (G1) {
      const __amdgpu_buffer_rsrc_t ors =
          make_rsrc(dst + static_cast<size_t>(row0) * I, static_cast<uint32_t>(nrows) * I * 2);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int fbase = f0 + 16 * (wn * MB + m);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const f32x16_t& c = acc[m][n];
          uint2 pk[2];
#pragma unroll
          for (int b4 = 0; b4 < 2; ++b4) {
            pk[b4].x = pack_bf16x2(act_apply(c[4 * b4 + 0], c[4 * b4 + 8], actf),
                                   act_apply(c[4 * b4 + 1], c[4 * b4 + 9], actf));
            pk[b4].y = pack_bf16x2(act_apply(c[4 * b4 + 2], c[4 * b4 + 10], actf),
                                   act_apply(c[4 * b4 + 3], c[4 * b4 + 11], actf));
          }
          // lane (r, h) holds features 8 b4 + 4 h .. + 3 in piece b4; one
          // exchange of h with b4 leaves it features 8 h .. + 7 (16 bytes)
          auto x = __builtin_amdgcn_permlane32_swap(pk[0].x, pk[1].x, false, false);
          auto y = __builtin_amdgcn_permlane32_swap(pk[0].y, pk[1].y, false, false);
          const uint32_t off = static_cast<uint32_t>(wm * 64 + n * 32 + r) * I * 2 + (fbase + 8 * h) * 2;
          bst16(ors, off, uint4{x[0], y[0], x[1], y[1]});
        }
      }
    } else {
      const int fbase = f0 + wn * 32 * MB;
      const __amdgpu_buffer_rsrc_t ors =
          make_rsrc(dst + static_cast<size_t>(row0) * H, static_cast<uint32_t>(nrows) * H * 2);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[m][n][4 * b4 + 0], acc[m][n][4 * b4 + 1]);
            pk.y = pack_bf16x2(acc[m][n][4 * b4 + 2], acc[m][n][4 * b4 + 3]);
            const uint32_t off = static_cast<uint32_t>(wm * 64 + n * 32 + r) * H * 2 +
                                 (fbase + 32 * m + 8 * b4 + 4 * h) * 2;
            bst8(ors, off, pk);
          }
    }
  }  // items
}

// ---------------------------------------------------------------------------
// Dense GEMM2, act tile resident in LDS (I <= 384). A block (4 waves) owns a
// 128-row dense tile: it copies the tile's act rows (128 x I bf16) into LDS
// once and then walks all H / 256 output spans. Wave wn computes 64 W2 rows
// x all 128 tokens per span, so every weight byte is fetched once; its
// weights come straight from global memory into registers, and K step kb
// of the next span is loaded into the registers of step kb right after they
// are decoded: the loads have about one span of MFMA work to arrive, and no
// barrier is needed between spans. Each span's outputs pass through the
// wave's own 16 KB of LDS so that the stores write whole 128-byte pieces of
// Y rows (16 bytes per lane) instead of 8-byte pieces of 32 rows at a time,
// which kept the texture address queue full. Y is written once and read
// once by the finalize, after far more than the caches hold has passed
// (3.8 GB at 32k tokens), so the stores are non-temporal. LDS: 128 * I * 2
// + 64 KB.
// ---------------------------------------------------------------------------
constexpr int kResThreads = 256;

template <int NKB>
__device__ __forceinline__ void gemm2_resident_body(
    const uint16_t* __restrict__ act, uint32_t act_bytes, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ counters, int H, uint16_t* __restrict__ y) {
  constexpr int I = NKB * 128;
  constexpr int kRowB = I * 2;                 // act row bytes
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[kTileRows * kRowB];
  // per wave: its 128 x 64 output tile of one span, bf16, 128-byte rows
  __shared__ __attribute__((aligned(16))) uint8_t o_lds[4 * kTileRows * 128];
  const int ntiles = counters[kCtrGate] == 1 ? counters[kCtrGate + 3] : 0;
  const int xcd = blockIdx.x & 7;
  const int per = (ntiles + 7) >> 3;
  const int nblk_x = static_cast<int>(gridDim.x) >> 3;
  const int t = threadIdx.x;
  const int wn = wave_index();
  const int lane = lane_id();
  const int r = lane & 31, h = lane >> 5;
  const int nspan = H >> 8;
  constexpr uint32_t wrow = I / 2, srow = I / 32;
  // Tile row rr lives in LDS row slot (rr % 32) * 4 + rr / 32, so that the
  // four 32-row token blocks a lane reads sit kRowB apart (immediate
  // offsets); its 16-byte chunk c sits at chunk (c & ~15) | ((c ^ row_swz(rr))
  // & 15), which spreads the 16 rows read at one chunk over all banks.
  auto a_off = [](int rr, int c) -> uint32_t {
    const int sl = ((rr & 31) << 2) | (rr >> 5);
    return static_cast<uint32_t>(sl * kRowB + (((c & ~15) | ((c ^ row_swz(rr)) & 15)) << 4));
  };
  // lane's read base for K sub-step (q, j) of any kb: row slot 4r, chunk
  // 8q + 4h + j swizzled; block n and step kb add n * kRowB + kb * 256
  const uint8_t* abase[8];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8)
    abase[s8] = a_lds + r * 4 * kRowB + ((((8 * (s8 >> 2) + 4 * h + (s8 & 3)) ^ row_swz(r)) & 15) << 4);
  // packed layout: lane row r of a 32-row block lies in 16-row group r / 16
  const uint32_t wv_off =
      static_cast<uint32_t>(r >> 4) * 16 * wrow + static_cast<uint32_t>(r & 15) * 64 + h * 16;
  const uint32_t sv_off = static_cast<uint32_t>(r) * srow;
  for (int slot = blockIdx.x >> 3; slot < per; slot += nblk_x) {
    const int tile = xcd * per + slot;
    if (tile >= ntiles) break;
    const int4 ti = reinterpret_cast<const int4*>(tiles)[tile];
    const int e = ti.x, row0 = ti.y, nrows = ti.z;
    // ---- act tile -> LDS (rows past nrows read as zero)
    {
      const __amdgpu_buffer_rsrc_t ars = make_rsrc(act, act_bytes);
      constexpr int kChunks = kTileRows * (kRowB / 16);
      constexpr int kPer = kChunks / kResThreads;
      uint4 v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int q = i * kResThreads + t;
        const int rr = q / (kRowB / 16), c = q % (kRowB / 16);
        v[i] = bld16(ars, static_cast<uint32_t>(row0 + rr) * kRowB + c * 16 +
                              (rr < nrows ? 0u : kNoRow));
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int q = i * kResThreads + t;
        const int rr = q / (kRowB / 16), c = q % (kRowB / 16);
        *reinterpret_cast<uint4*>(a_lds + a_off(rr, c)) = v[i];
      }
    }
    // ---- weights of span 0 into registers; wave-uniform offsets in SGPRs
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(w2 + static_cast<size_t>(e) * H * wrow, static_cast<uint32_t>(H) * wrow);
    const __amdgpu_buffer_rsrc_t scs =
        make_rsrc(s2 + static_cast<size_t>(e) * H * srow, static_cast<uint32_t>(H) * srow);
    uint4 wr[NKB][2][2];   // [kb][m][q]
    uint32_t sw[NKB][2];   // [kb][m]: scale bytes of groups 4kb .. 4kb+3
    auto load_w = [&](int sp, int kb) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t rb = static_cast<uint32_t>(sp * 256 + wn * 64 + m * 32);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          wr[kb][m][q] = bld16s(wrs, wv_off, rb * wrow + kb * kPkBlock + q * 32);
        sw[kb][m] = bld4s(scs, sv_off, rb * srow + kb * 4);
      }
    };
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) load_w(0, kb);
    __syncthreads();  // act tile visible to every wave

    for (int sp = 0; sp < nspan; ++sp) {
      f32x16_t acc[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.0f;
      const int spn = min(sp + 1, nspan - 1);  // last span: reload it, unused
      // Software pipeline over the 8 * NKB K sub-steps (kb, q, j): step s
      // multiplies token fragments read during step s - 1 with weight
      // fragments decoded during the previous (kb, q) block, while it reads
      // the fragments of step s + 1 and decodes one quarter of the next
      // block. Each step is its own scheduling region with the reads first
      // and MFMAs alternating with converts.
      constexpr int kBlocks = 2 * NKB;
      auto decode = [&](int blk, int j, bf16x8_t (&dst)[2][4]) {
        const int kb = blk >> 1, q = blk & 1;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float scale = e8m0_scale_operand((sw[kb][m] >> (8 * (2 * q + h))) & 0xffu);
          const uint4 v = wr[kb][m][q];
          const uint32_t dw = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
          dst[m][j] = decode_fp4x8(dw, scale);
        }
      };
      auto read_b = [&](int stp, bf16x8_t (&dst)[4]) {
        const int kb = stp >> 3, s8 = stp & 7;
#pragma unroll
        for (int n = 0; n < 4; ++n)
          dst[n] = as_bf16x8(*reinterpret_cast<const uint4*>(abase[s8] + n * kRowB + kb * 256));
      };
      bf16x8_t acur[2][4], anxt[2][4], bcur[4], bnxt[4];
      __builtin_amdgcn_sched_barrier(0);
      read_b(0, bcur);
#pragma unroll
      for (int j = 0; j < 4; ++j) decode(0, j, acur);
#pragma unroll
      for (int blk = 0; blk < kBlocks; ++blk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int stp = 4 * blk + j;
          __builtin_amdgcn_sched_barrier(0);
          if (stp + 1 < 4 * kBlocks) read_b(stp + 1, bnxt);
          if (blk + 1 < kBlocks) decode(blk + 1, j, anxt);
#pragma unroll
          for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int m = 0; m < 2; ++m) acc[m][n] = mfma32x32x16(acur[m][j], bcur[n], acc[m][n]);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads first
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // one VALU op
          }
          __builtin_amdgcn_sched_barrier(0);
          if (stp + 1 < 4 * kBlocks) {
#pragma unroll
            for (int n = 0; n < 4; ++n) bcur[n] = bnxt[n];
          }
          // block blk + 1 = (kb, 1) is decoded once blk = (kb, 0) ends:
          // step kb's weights are free for the next span
          if (j == 3 && (blk & 1) == 0) {
            __builtin_amdgcn_sched_barrier(0);
            load_w(spn, blk >> 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (blk + 1 < kBlocks) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) acur[m][j] = anxt[m][j];
        }
      }
      // ---- this span's 64 x 128 outputs of the wave go through its LDS
      // staging rows, so that each store writes 128-byte row pieces. Token
      // row t holds 8 chunks of 8 features; chunk c sits in slot
      // c ^ ((t >> 1) & 7) with its two 8-byte halves swapped when bit 4 of t
      // is set, which puts the 32 8-byte writes of each half-wave on
      // distinct banks.
      uint8_t* stg = o_lds + wn * (kTileRows * 128);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[m][n][4 * b4 + 0], acc[m][n][4 * b4 + 1]);
            pk.y = pack_bf16x2(acc[m][n][4 * b4 + 2], acc[m][n][4 * b4 + 3]);
            const int tk = n * 32 + r;
            const int c = 4 * m + b4;
            *reinterpret_cast<uint2*>(stg + tk * 128 + ((c ^ ((tk >> 1) & 7)) << 4) +
                                      ((h ^ ((tk >> 4) & 1)) << 3)) = pk;
          }
      const int fbase = sp * 256 + wn * 64;
      const __amdgpu_buffer_rsrc_t ors =
          make_rsrc(y + static_cast<size_t>(row0) * H, static_cast<uint32_t>(nrows) * H * 2);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tk = 8 * i + (lane >> 3);
        const int c = lane & 7;
        uint4 v = *reinterpret_cast<const uint4*>(stg + tk * 128 + ((c ^ ((tk >> 1) & 7)) << 4));
        if ((tk >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
        bst16nt(ors, static_cast<uint32_t>(tk) * H * 2 + (fbase + 8 * c) * 2, v);
      }
    }
    __syncthreads();  // every wave done with the act tile before the next copy
  }
}

// GEMM2 of either path in one launch, for I <= 384 ("Device-side gating of
// the MoE GEMM2 path": the gate word picks Dense or Split on the device and
// the launch chain stays fixed). The stream kernel and the resident dense
// kernel both run one 4-wave block per CU (the stream by choice, the dense
// kernel by its LDS and registers), so one persistent grid of kStreamGrid
// blocks serves either body, and the path not taken costs no launch of its
// own (about 4 us per layer at decode shapes on MI355X).
template <int NKB>
__global__ __launch_bounds__(kResThreads, 1) void gemm2_gated_kernel(
    const uint16_t* __restrict__ act, uint32_t act_bytes, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int32_t* __restrict__ units,
    const int32_t* __restrict__ dense_tiles, const int32_t* __restrict__ counters,
    const int32_t* __restrict__ counts, int H, uint16_t* __restrict__ y) {
  if (counters[kCtrGate] == 1)
    gemm2_resident_body<NKB>(act, act_bytes, w2, s2, dense_tiles, counters, H, y);
  else
    gemm2_stream_body<NKB>(act, w2, s2, units, counters, counts, H, NKB * 128, y);
}

hipError_t launch_gemm2_gated(const GemmArgs& a, hipStream_t st) {
  const uint32_t act_bytes = static_cast<uint32_t>(static_cast<size_t>(a.rows_pad) * a.I * 2);
#define MOE_G2G(NK)                                                                             \
  hipLaunchKernelGGL(gemm2_gated_kernel<NK>, dim3(kStreamGrid), dim3(kResThreads), 0, st, a.act, \
                     act_bytes, a.w2, a.s2, a.units16, a.dense_tiles, a.counters, a.counts, a.H, a.y)
  switch (a.I / 128) {
    case 1: MOE_G2G(1); break;
    case 2: MOE_G2G(2); break;
    default: MOE_G2G(3); break;
  }
#undef MOE_G2G
  return hipGetLastError();
}

// Persistent grid: `per_cu` blocks per CU, at most one block per item; a
// multiple of 8 so that every XCD gets the same number of blocks.
static int tiled_grid(long items, int per_cu) {
  long per = (items + 7) / 8;
  if (per < 1) per = 1;
  if (per > 32 * per_cu) per = 32 * per_cu;
  return static_cast<int>(8 * per);
}

hipError_t launch_gemm1_tiled(const GemmArgs& a, hipStream_t st) {
  const int sub = a.B > kTileRows ? a.B / kTileRows : 1;
  const uint32_t x_bytes = static_cast<uint32_t>(static_cast<size_t>(a.T) * a.H * 2);
  if (a.I % 192 == 0) {  // 384-row tiles (192 features): less LDS traffic per MFMA
    const int grid = tiled_grid(static_cast<long>(a.kmax_v) * sub * (a.I / 192), 1);
    hipLaunchKernelGGL((gemm_tiled_kernel<true, 3>), dim3(grid), dim3(kTiledThreads), 0, st, a.x,
                       x_bytes, a.w13, a.s13, a.vinfo, a.counters, a.sorted_slot, a.I, a.H, a.Kp,
                       sub, a.act_fn, a.act);
    return hipGetLastError();
  }
  const int grid = tiled_grid(static_cast<long>(a.kmax_v) * sub * (a.I / 128), 1);
  hipLaunchKernelGGL((gemm_tiled_kernel<true, 2>), dim3(grid), dim3(kTiledThreads), 0, st, a.x,
                     x_bytes, a.w13, a.s13, a.vinfo, a.counters, a.sorted_slot, a.I, a.H, a.Kp,
                     sub, a.act_fn, a.act);
  return hipGetLastError();
}

// Dense GEMM2 for I > 384 (the act tile no longer fits in LDS next to the
// output staging): the generic tiled kernel, launched after the split-path
// kernel of the same chain.
hipError_t launch_gemm2_dense_tiled(const GemmArgs& a, hipStream_t st) {
  const int grid = tiled_grid(static_cast<long>(a.dense_grid_tiles) * (a.H / 256), 1);
  hipLaunchKernelGGL((gemm_tiled_kernel<false, 2>), dim3(grid), dim3(kTiledThreads), 0, st, a.act,
                     static_cast<uint32_t>(static_cast<size_t>(a.rows_pad) * a.I * 2), a.w2, a.s2,
                     a.dense_tiles, a.counters, a.sorted_slot, a.I, a.H, a.Kp, 1, a.act_fn, a.y);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MX-activation tiled GEMMs: W4A8 (MXFP8 tokens) or, with A4, W4A4 (MXFP4
// tokens), E2M1 weights fed to the scaled 16x16x128 MFMA as they are (no
// decode). Same block tile, waves and pipeline as above; a token stage is
// 128 rows x 128 E4M3 bytes (16 KB) or 128 rows x 64 bytes of E2M1 pairs
// (8 KB), plus the rows' four scale bytes. Wave (wm, wn) computes four
// 16-row weight tiles (GEMM1: gate features +0 / +16, then the up rows of
// the same features) x four 16-token tiles: 16 MFMAs per K stage.
// ---------------------------------------------------------------------------
namespace {
constexpr int kTokScStage = kTileRows * 4;    // token scale bytes of one K stage
constexpr int kTok4Stage = kTileRows * 64;    // E2M1 token bytes of one K stage (8 KB)

}  // namespace

template <bool G1, bool A4>
__global__ __launch_bounds__(kTiledThreads, 1) void gemm_tiled_a8_kernel(
    const uint8_t* __restrict__ src, uint32_t src_bytes, const uint8_t* __restrict__ srcs,
    uint32_t srcs_bytes, const uint8_t* __restrict__ w, const uint8_t* __restrict__ s,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ counters,
    const int32_t* __restrict__ sorted_slot, int I, int H, int Kp, int sub, ActArgs actf,
    uint8_t* __restrict__ dstq, uint8_t* __restrict__ dsts, uint16_t* __restrict__ dsty) {
  constexpr int kTokSt = A4 ? kTok4Stage : kTok8Stage;
  constexpr uint32_t XS = A4 ? 64u : 128u;  // token code bytes of a row per K stage
  constexpr int NTP = A4 ? 1 : 2;           // 16-byte token pieces per thread and stage
  __shared__ __attribute__((aligned(16))) uint8_t tok_lds[2 * kTokSt];
  __shared__ __attribute__((aligned(16))) uint8_t tsc_lds[2 * kTokScStage];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[2 * kWStage];
  extern __shared__ __attribute__((aligned(16))) uint8_t s_lds[];
  const int K = G1 ? H : I;
  const uint32_t KB = A4 ? static_cast<uint32_t>(K) / 2 : static_cast<uint32_t>(K);  // token row bytes
  int ntiles;
  if (G1) {
    ntiles = counters[kCtrNumV];
  } else {
    ntiles = counters[kCtrGate] == 1 ? counters[kCtrGate + 3] : 0;
  }
  const int nspan = G1 ? (I >> 7) : (H >> 8);
  const int nitems = ntiles * sub * nspan;
  const int xcd = blockIdx.x & 7;
  const int per = (nitems + 7) >> 3;
  const int nblk_x = static_cast<int>(gridDim.x) >> 3;
  const int t = threadIdx.x;
  const size_t wrow = static_cast<size_t>(K) >> 1, srow = static_cast<size_t>(K) >> 5;
  const int wave = wave_index();
  const int wm = wave & 1, wn = wave >> 1;
  const int lane = lane_id();
  const int c = lane & 15, g = lane >> 4;
  for (int slot = blockIdx.x >> 3; slot < per; slot += nblk_x) {
    const int item = xcd * per + slot;
    if (item >= nitems) break;
    const int span = item % nspan;
    const int ts = item / nspan;
    const int tile = ts / sub;
    const int st = ts - tile * sub;
    const int4 ti = reinterpret_cast<const int4*>(tiles)[tile];
    const int e = ti.x;
    const int row0 = ti.y + st * kTileRows;
    const int nrows = min(kTileRows, ti.z - st * kTileRows);
    if (nrows <= 0) continue;
    const int f0 = G1 ? span * 128 : span * 256;
    auto grow_of = [&](int rho) -> size_t {
      if (G1) return static_cast<size_t>(e) * 2 * I + (rho < 128 ? f0 + rho : I + f0 + rho - 128);
      return static_cast<size_t>(e) * H + f0 + rho;
    };

    // ---- weight scale rows of the tile -> LDS
    {
      const int seg = G1 ? 128 * static_cast<int>(srow) : 256 * static_cast<int>(srow);
      const uint8_t* s0 = s + grow_of(0) * srow;
      for (int o = t * 16; o < seg; o += kTiledThreads * 16)
        *reinterpret_cast<uint4*>(s_lds + o) = ld16(s0 + o);
      if (G1) {
        const uint8_t* s1 = s + grow_of(128) * srow;
        for (int o = t * 16; o < seg; o += kTiledThreads * 16)
          *reinterpret_cast<uint4*>(s_lds + seg + o) = ld16(s1 + o);
      }
    }

    // ---- token rows: thread t moves chunk t%8 of rows 64i + t/8 (E4M3) or
    // chunk t%4 of row t/4 (E2M1), and the 4 scale bytes of row t%128 (four
    // threads per row store the same word).
    const int lc = A4 ? (t & 3) : (t & 7), lr = A4 ? (t >> 2) : (t >> 3), sr = t & 127;
    uint32_t toff[2], soff;
    {
      uint32_t base[3];
      const int rr[3] = {lr, A4 ? lr : 64 + lr, sr};
      if (G1) {
        const __amdgpu_buffer_rsrc_t ssr =
            make_rsrc(sorted_slot + row0, static_cast<uint32_t>(nrows) * 4u);
        uint32_t sv[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) sv[i] = bld4(ssr, rr[i] * 4);
#pragma unroll
        for (int i = 0; i < 3; ++i) base[i] = sv[i] / static_cast<uint32_t>(Kp);
      } else {
#pragma unroll
        for (int i = 0; i < 3; ++i) base[i] = static_cast<uint32_t>(row0 + rr[i]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
        toff[i] = base[i] * KB + lc * 16 + (rr[i] < nrows ? 0u : kNoRow);
      soff = base[2] * static_cast<uint32_t>(srow) + (sr < nrows ? 0u : kNoRow);
    }
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(src, src_bytes);
    const __amdgpu_buffer_rsrc_t ssc = make_rsrc(srcs, srcs_bytes);
    const int wc = t & 3, wr = t >> 2;
    const uint8_t* wsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // packed layout
      const size_t gr = grow_of(i * 128 + wr);
      wsrc[i] = w + (gr & ~static_cast<size_t>(15)) * wrow + (gr & 15) * 64 + wc * 16;
    }

    const int nkb = K >> 7;
    const int last = nkb - 1;
    uint4 tv[2], wv[2];
    uint32_t sv;
    auto load_stage = [&](int kb) {
#pragma unroll
      for (int i = 0; i < NTP; ++i) tv[i] = bld16(srs, toff[i] + kb * XS);
      sv = bld4(ssc, soff + kb * 4);
#pragma unroll
      for (int i = 0; i < 2; ++i) wv[i] = ld16(wsrc[i] + kb * kPkBlock);
    };
    // piece p of load_stage (same order as store_piece; E2M1 tokens have no piece 1)
    auto load_piece = [&](int kb, int p) {
      if (p < NTP) tv[p] = bld16(srs, toff[p] + kb * XS);
      else if (p == 2) sv = bld4(ssc, soff + kb * 4);
      else if (p > 2) wv[p - 3] = ld16(wsrc[p - 3] + kb * kPkBlock);
    };
    // piece p of store_stage: token chunks 0, 1, the scale word 2, weight chunks 3, 4
    auto store_piece = [&](int b, int p) {
      if (p < NTP) {
        *reinterpret_cast<uint4*>(tok_lds + b * kTokSt + tokmx_off<A4>(p * 64 + lr, lc)) = tv[p];
      } else if (p == 2) {
        *reinterpret_cast<uint32_t*>(tsc_lds + b * kTokScStage + sr * 4) = sv;
      } else if (p > 2) {
        *reinterpret_cast<uint4*>(w_lds + b * kWStage + w_off((p - 3) * 128 + wr, wc)) = wv[p - 3];
      }
    };
    auto store_stage = [&](int b) {
      uint8_t* tb = tok_lds + b * kTokSt;
#pragma unroll
      for (int i = 0; i < NTP; ++i)
        *reinterpret_cast<uint4*>(tb + tokmx_off<A4>(i * 64 + lr, lc)) = tv[i];
      *reinterpret_cast<uint32_t*>(tsc_lds + b * kTokScStage + sr * 4) = sv;
      uint8_t* wb = w_lds + b * kWStage;
#pragma unroll
      for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(wb + w_off(i * 128 + wr, wc)) = wv[i];
    };

    // weight tile rows of the wave's four 16-row MFMA tiles (lane c)
    int rho[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (G1) rho[mt] = (mt >> 1) * 128 + wn * 32 + (mt & 1) * 16 + c;
      else rho[mt] = wn * 64 + mt * 16 + c;
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_stage(0);
    __builtin_amdgcn_sched_barrier(0);
    store_stage(0);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(min(1, last));
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
      const int b = kb & 1;
      const uint8_t* tb = tok_lds + b * kTokSt;
      const uint8_t* tsb = tsc_lds + b * kTokScStage;
      const uint8_t* wb = w_lds + b * kWStage;
      uint4 af[4];
      uint32_t as[4];
      // token fragments of tile nt + 1 are read while tile nt's MFMAs run
      uint4 x0c, x1c, x0n, x1n;
      uint32_t bsc, bsn;
      auto read_x = [&](int nt, uint4& x0, uint4& x1, uint32_t& bs) {
        const int tr = wm * 64 + nt * 16 + c;
        x0 = *reinterpret_cast<const uint4*>(tb + tokmx_off<A4>(tr, g));
        if (!A4) x1 = *reinterpret_cast<const uint4*>(tb + tokmx_off<A4>(tr, 4 + g));
        bs = tsb[tr * 4 + g];
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        af[mt] = *reinterpret_cast<const uint4*>(wb + w_off(rho[mt], g));
        as[mt] = s_lds[rho[mt] * srow + kb * 4 + g];
      }
      read_x(0, x0c, x1c, bsc);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        __builtin_amdgcn_sched_barrier(0);
        if (nt < 3) read_x(nt + 1, x0n, x1n, bsn);
        store_piece(b ^ 1, nt);  // next stage, one piece per tile group (as in the bf16 kernel)
        load_piece(min(kb + 2, last), nt);  // the piece's register is free once stored
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt][nt] = mfma_f4xa<A4>(af[mt], as[mt], x0c, x1c, bsc, acc[mt][nt]);
        __builtin_amdgcn_sched_group_barrier(0x100, A4 ? 2 : 3, 0);  // LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // one LDS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then the MFMAs
        __builtin_amdgcn_sched_barrier(0);
        if (nt < 3) {
          x0c = x0n;
          if (!A4) x1c = x1n;
          bsc = bsn;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      store_piece(b ^ 1, 4);
      __builtin_amdgcn_sched_barrier(0);
      load_piece(min(kb + 2, last), 4);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }

    // ---- epilogue. Lane (c, g), register v of tile (mt, nt): weight row
    // 4g + v of the 16-row tile, token row wm*64 + nt*16 + c.
    if (G1) {
      const int fbase = f0 + wn * 32;
      const uint32_t srow_a = static_cast<uint32_t>(I) >> 5;
      const uint32_t IB = A4 ? static_cast<uint32_t>(I) / 2 : static_cast<uint32_t>(I);
      const __amdgpu_buffer_rsrc_t qrs =
          make_rsrc(dstq + static_cast<size_t>(row0) * IB, static_cast<uint32_t>(nrows) * IB);
      const __amdgpu_buffer_rsrc_t ars =
          make_rsrc(dsts + static_cast<size_t>(row0) * srow_a, static_cast<uint32_t>(nrows) * srow_a);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t tr = static_cast<uint32_t>(wm * 64 + nt * 16 + c);
        float a[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 4; ++v) a[4 * h + v] = act_apply(acc[h][nt][v], acc[2 + h][nt][v], actf);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(a[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const uint32_t e0 = tr * I + fbase + 4 * g;  // element index of a[0]
        if constexpr (A4) {
          const uint32_t sb = mxfp4_scale_byte(amax);
          const float inv = mx_inv_scale(sb);
          bst2(qrs, e0 / 2, pack_e2m1x4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv));
          bst2(qrs, e0 / 2 + 8, pack_e2m1x4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv));
          bst1(ars, g == 0 ? tr * srow_a + (fbase >> 5) : kNoRow, sb);
        } else {
          const uint32_t sb = mxfp8_scale_byte(amax);
          const float inv = mxfp8_inv_scale(sb);
          bst4(qrs, e0, pack_e4m3x4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv));
          bst4(qrs, e0 + 16, pack_e4m3x4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv));
          bst1(ars, g == 0 ? tr * srow_a + (fbase >> 5) : kNoRow, sb);
        }
      }
    } else {
      const int fbase = f0 + wn * 64;
      const __amdgpu_buffer_rsrc_t ors =
          make_rsrc(dsty + static_cast<size_t>(row0) * H, static_cast<uint32_t>(nrows) * H * 2);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
          pk.y = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
          const uint32_t off = static_cast<uint32_t>(wm * 64 + nt * 16 + c) * H * 2 +
                               (fbase + 16 * mt + 4 * g) * 2;
          bst8(ors, off, pk);
        }
    }
  }  // items
}

hipError_t launch_gemm1_tiled_a8(const GemmArgs& a, hipStream_t st) {
  const int sub = a.B > kTileRows ? a.B / kTileRows : 1;
  const int grid = tiled_grid(static_cast<long>(a.kmax_v) * sub * (a.I / 128), 1);
  const size_t xbytes = static_cast<size_t>(a.T) * a.H / (a.a4 ? 2 : 1);
#define MOE_GT1A(A4)                                                                          \
  hipLaunchKernelGGL((gemm_tiled_a8_kernel<true, A4>), dim3(grid), dim3(kTiledThreads),      \
                     static_cast<size_t>(8) * a.H, st, a.xq, static_cast<uint32_t>(xbytes),  \
                     a.xs, static_cast<uint32_t>(static_cast<size_t>(a.T) * a.H / 32), a.w13, \
                     a.s13, a.vinfo, a.counters, a.sorted_slot, a.I, a.H, a.Kp, sub, a.act_fn, \
                     reinterpret_cast<uint8_t*>(a.act), a.act_scales, nullptr)
  if (a.a4) MOE_GT1A(true); else MOE_GT1A(false);
#undef MOE_GT1A
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense GEMM2 of the W4A8 path, act tile resident in LDS (I <= 512): the
// structure of gemm2_resident_body with the scaled 16x16x128 MFMA. A block
// (4 waves) owns a 128-row dense tile: its MXFP8 act rows (128 x I E4M3
// bytes) and their scales go to LDS once, then it walks all H / 256 output
// spans. Wave wn takes 64 W2 rows per span as four 16-row tiles against the
// eight 16-token tiles; the E2M1 weights and their E8M0 scales feed the MFMA
// as they are, straight from global memory into registers, refilled for the
// next span as soon as a K step is done. Token fragments are read one MFMA
// group ahead; outputs go through the wave's LDS staging rows like the bf16
// kernel's. LDS: 128 * I * 33 / 32 + 64 KB.
// ---------------------------------------------------------------------------
template <int NKB, bool A4>
__device__ __forceinline__ void gemm2_resident_a8_body(
    const uint8_t* __restrict__ actq, uint32_t actq_bytes, const uint8_t* __restrict__ acts,
    uint32_t acts_bytes, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ counters, int H,
    uint16_t* __restrict__ y) {
  constexpr int I = NKB * 128;
  constexpr int kRowB = A4 ? I / 2 : I;  // act code bytes per row: E2M1 pairs or E4M3
  constexpr int XS = A4 ? 64 : 128;      // of which one K step
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[kTileRows * kRowB];
  // act scales, [kb][row][4]: the four 32-K scale bytes of K step kb
  __shared__ __attribute__((aligned(16))) uint8_t as_lds[NKB * kTileRows * 4];
  __shared__ __attribute__((aligned(16))) uint8_t o_lds[4 * kTileRows * 128];
  const int ntiles = counters[kCtrGate] == 1 ? counters[kCtrGate + 3] : 0;
  const int xcd = blockIdx.x & 7;
  const int per = (ntiles + 7) >> 3;
  const int nblk_x = static_cast<int>(gridDim.x) >> 3;
  const int t = threadIdx.x;
  const int wn = wave_index();
  const int lane = lane_id();
  const int c = lane & 15, g = lane >> 4;
  const int nspan = H >> 8;
  constexpr uint32_t wrow = I / 2, srow = I / 32;
  // act chunk q (16 bytes; 8 per K step for E4M3) of tile row rr: within
  // each K step's 8 chunks the index is XORed with (rr >> 1) & 7, which puts
  // the 16 rows of one MFMA fragment on 16 distinct 16-byte bank groups.
  // E2M1: 4 chunks per K step, XORed with ((rr >> 3) & 1) << 1 (rows r and
  // r + 8 swap chunk halves).
  auto swz = [](int rr) -> int { return A4 ? (((rr >> 3) & 1) << 1) : ((rr >> 1) & 7); };
  auto a_off = [&](int rr, int q) -> uint32_t {
    constexpr int m = A4 ? 3 : 7;
    return static_cast<uint32_t>(rr * kRowB + (((q & ~m) | ((q ^ swz(rr)) & m)) << 4));
  };
  // lane's fragment bases (token c of a 16-token tile, chunks g and 4 + g of
  // a K step, or chunk g for E2M1); tile nt and step kb add
  // nt * 16 * kRowB + kb * XS (nt * 16 leaves the swizzle unchanged)
  const uint8_t* xb0 = a_lds + c * kRowB + (((g ^ swz(c)) & (A4 ? 3 : 7)) << 4);
  const uint8_t* xb1 = a_lds + c * kRowB + ((((4 + g) ^ swz(c)) & 7) << 4);
  const uint8_t* sbase = as_lds + c * 4 + g;  // + (kb * 128 + nt * 16) * 4
  const uint32_t wv_off = static_cast<uint32_t>(c) * 64 + g * 16;  // packed layout
  const uint32_t sv_off = static_cast<uint32_t>(c) * srow + g;
  for (int slot = blockIdx.x >> 3; slot < per; slot += nblk_x) {
    const int tile = xcd * per + slot;
    if (tile >= ntiles) break;
    const int4 ti = reinterpret_cast<const int4*>(tiles)[tile];
    const int e = ti.x, row0 = ti.y, nrows = ti.z;
    // ---- act tile and its scales -> LDS (rows past nrows read as zero)
    {
      const __amdgpu_buffer_rsrc_t ars = make_rsrc(actq, actq_bytes);
      constexpr int kCh = kRowB / 16;
      constexpr int kPer = kTileRows * kCh / 256;
      uint4 v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int q = i * 256 + t;
        const int rr = q / kCh, cq = q % kCh;
        v[i] = bld16(ars, static_cast<uint32_t>(row0 + rr) * kRowB + cq * 16 +
                              (rr < nrows ? 0u : kNoRow));
      }
      const __amdgpu_buffer_rsrc_t srs = make_rsrc(acts, acts_bytes);
      for (int q = t; q < kTileRows * NKB; q += 256) {
        const int rr = q / NKB, kb = q % NKB;
        const uint32_t wv = bld4(srs, static_cast<uint32_t>(row0 + rr) * srow + kb * 4 +
                                          (rr < nrows ? 0u : kNoRow));
        *reinterpret_cast<uint32_t*>(as_lds + (kb * kTileRows + rr) * 4) = wv;
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int q = i * 256 + t;
        const int rr = q / kCh, cq = q % kCh;
        *reinterpret_cast<uint4*>(a_lds + a_off(rr, cq)) = v[i];
      }
    }
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(w2 + static_cast<size_t>(e) * H * wrow, static_cast<uint32_t>(H) * wrow);
    const __amdgpu_buffer_rsrc_t scs =
        make_rsrc(s2 + static_cast<size_t>(e) * H * srow, static_cast<uint32_t>(H) * srow);
    uint4 wf[NKB][4];      // [kb][mt]: 32 E2M1 codes of row c, K block g
    uint32_t ws[NKB][4];   // [kb][mt]: their E8M0 scale
    auto load_w = [&](int sp, int kb) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint32_t rb = static_cast<uint32_t>(sp * 256 + wn * 64 + mt * 16);
        wf[kb][mt] = bld16s(wrs, wv_off, rb * wrow + kb * kPkBlock);
        ws[kb][mt] = bld1s(scs, sv_off, rb * srow + kb * 4);
      }
    };
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) load_w(0, kb);
    __syncthreads();  // act tile visible to every wave

    for (int sp = 0; sp < nspan; ++sp) {
      f32x4_t acc[4][8];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int spn = min(sp + 1, nspan - 1);  // last span: reload it, unused
      // step st = (kb, nt): token fragments read one step ahead
      uint4 x0c, x1c, x0n, x1n;
      uint32_t bsc, bsn;
      auto read_x = [&](int st, uint4& x0, uint4& x1, uint32_t& bs) {
        const int kb = st >> 3, nt = st & 7;
        x0 = *reinterpret_cast<const uint4*>(xb0 + nt * 16 * kRowB + kb * XS);
        if (!A4) x1 = *reinterpret_cast<const uint4*>(xb1 + nt * 16 * kRowB + kb * XS);
        bs = sbase[(kb * kTileRows + nt * 16) * 4];
      };
      __builtin_amdgcn_sched_barrier(0);
      read_x(0, x0c, x1c, bsc);
#pragma unroll
      for (int st = 0; st < 8 * NKB; ++st) {
        const int kb = st >> 3, nt = st & 7;
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < 8 * NKB) read_x(st + 1, x0n, x1n, bsn);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt][nt] = mfma_f4xa<A4>(wf[kb][mt], ws[kb][mt], x0c, x1c, bsc, acc[mt][nt]);
        __builtin_amdgcn_sched_group_barrier(0x100, A4 ? 2 : 3, 0);  // LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then the MFMAs
        __builtin_amdgcn_sched_barrier(0);
        if (nt == 7) {  // step kb done: refill it with the next span
          load_w(spn, kb);
          __builtin_amdgcn_sched_barrier(0);
        }
        x0c = x0n;
        if (!A4) x1c = x1n;
        bsc = bsn;
      }
      // ---- this span's 64 x 128 outputs through the wave's LDS staging rows
      // (token row t: 8 chunks of 8 features; chunk c8 in slot
      // c8 ^ ((t >> 1) & 7), halves swapped when bit 4 of t is set)
      uint8_t* stg = o_lds + wn * (kTileRows * 128);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
          pk.y = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
          const int tk = nt * 16 + c;
          const int c8 = 2 * mt + (g >> 1);
          *reinterpret_cast<uint2*>(stg + tk * 128 + ((c8 ^ ((tk >> 1) & 7)) << 4) +
                                    (((g & 1) ^ ((tk >> 4) & 1)) << 3)) = pk;
        }
      const int fbase = sp * 256 + wn * 64;
      const __amdgpu_buffer_rsrc_t ors =
          make_rsrc(y + static_cast<size_t>(row0) * H, static_cast<uint32_t>(nrows) * H * 2);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tk = 8 * i + (lane >> 3);
        const int c8 = lane & 7;
        uint4 v = *reinterpret_cast<const uint4*>(stg + tk * 128 + ((c8 ^ ((tk >> 1) & 7)) << 4));
        if ((tk >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
        bst16nt(ors, static_cast<uint32_t>(tk) * H * 2 + (fbase + 8 * c8) * 2, v);
      }
    }
    __syncthreads();  // every wave done with the act tile before the next copy
  }
}

// GEMM2 of either path in one launch for MX act (I <= 512), as
// gemm2_gated_kernel does for bf16.
template <int NKB, bool A4>
__global__ __launch_bounds__(256, 1) void gemm2_gated_mx_kernel(
    const uint8_t* __restrict__ actq, uint32_t actq_bytes, const uint8_t* __restrict__ acts,
    uint32_t acts_bytes, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const int32_t* __restrict__ units, const int32_t* __restrict__ dense_tiles,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ counts, int H,
    uint16_t* __restrict__ y) {
  if (counters[kCtrGate] == 1)
    gemm2_resident_a8_body<NKB, A4>(actq, actq_bytes, acts, acts_bytes, w2, s2, dense_tiles, counters,
                                    H, y);
  else
    gemm2_stream_mx_body<NKB, A4>(actq, acts, w2, s2, units, counters, counts, H, NKB * 128, y);
}

template <bool A4>
static hipError_t launch_gemm2_gated_mx_t(const GemmArgs& a, hipStream_t st) {
  // the MX paths admit I <= 512 only, so the act tile always fits in LDS
  const uint8_t* actq = reinterpret_cast<const uint8_t*>(a.act);
  const uint32_t qb = static_cast<uint32_t>(static_cast<size_t>(a.rows_pad) * a.I / (A4 ? 2 : 1));
  const uint32_t sb = static_cast<uint32_t>(static_cast<size_t>(a.rows_pad) * a.I / 32);
#define MOE_G2GA(NK)                                                                              \
  hipLaunchKernelGGL((gemm2_gated_mx_kernel<NK, A4>), dim3(kStreamGrid), dim3(256), 0, st, actq, qb, \
                     a.act_scales, sb, a.w2, a.s2, a.units16, a.dense_tiles, a.counters, a.counts,  \
                     a.H, a.y)
  switch (a.I / 128) {
    case 1: MOE_G2GA(1); break;
    case 2: MOE_G2GA(2); break;
    case 3: MOE_G2GA(3); break;
    default: MOE_G2GA(4); break;
  }
#undef MOE_G2GA
  return hipGetLastError();
}

hipError_t launch_gemm2_gated_mx(const GemmArgs& a, hipStream_t st) {
  return a.a4 ? launch_gemm2_gated_mx_t<true>(a, st) : launch_gemm2_gated_mx_t<false>(a, st);
}

}  // namespace moe
