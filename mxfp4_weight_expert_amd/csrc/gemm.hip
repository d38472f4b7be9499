// Grouped GEMMs of the MoE layer on MXFP4 weights, bf16 MFMA on gfx950.
//
// GEMM1 ("SGLang CUTLASS MoE", structure diagram and section 4): for each
// row of an expert, h = x[token] W13[e]^T over K = H with 2I outputs, gate
// rows [0, I) and up rows [I, 2I); act = silu(g) * u, with the clamp of the
// Shape-template page, section 4, when a limit is set. act is stored bf16.
// GEMM2: y = act W2[e]^T over K = I, H outputs, stored bf16 in row order.
// Split and Dense GEMM2 follow "Device-side gating of the MoE GEMM2 path":
// both kernels always launch; the one the gate did not pick sees 0 items.
//
// This file holds the decode-shape kernels (few rows per expert: weights on
// the MFMA M side, the chunk's tokens on N); the LDS-tiled kernels for many
// rows per expert are in gemm_tiled.hip. K is walked in steps of 128: lane
// (r = lane%16, g = lane/16) loads 16 bytes of weight row r = 32 E2M1 codes
// = exactly one E8M0 scale group, decodes them to bf16 with the hardware
// scaled convert (exact), and feeds four 16x16x32 MFMAs. The K order inside
// a step is permuted identically for both operands (lane group g, MFMA j <->
// K = 128*kb + 32*g + 8*j + [0, 8)), which leaves the dot products unchanged
// and keeps every weight load a contiguous 16 bytes.
#include "common.h"
#include "kernels.h"
#include "gemm2_stream.h"

#include <map>
#include <mutex>
#include <tuple>

namespace moe {

namespace {
constexpr int kGemmBlock = 256;  // 4 waves, one item each at a time
// A compile-time int carried as a value (for generic lambdas).
template <int N>
struct IntC {
  static constexpr int value = N;
};
// Grid cap of the item-strided decode kernels: one block per four items up
// to 16 blocks per CU, more than can be resident, so blocks start as others
// finish and waves end within about one item of each other. Against a cap
// of 8 per CU (2 to 3 items per wave) it took the T512 E256 H7168 I2048
// split GEMMs from 693 / 416 to 675 / 403 us on MI355X; the T64 and T256
// decode shapes did not change.
constexpr int kMaxGrid = 256 * 16;

// XCD-aware item ranges. The hardware deals consecutive block ids round-robin
// over the 8 XCDs, each with its own L2. The item list (unit-major: all
// feature groups of a unit, then the next unit) is cut into 8 contiguous
// ranges, one per XCD, and the blocks of an XCD walk their range. The units
// of one expert are consecutive items, so an expert whose rows span several
// units is read by waves of one XCD at about the same time and its weights
// are re-read from that L2 instead of crossing XCDs. The range length is a
// multiple of 4, so the four waves of a block always take four consecutive
// items of one unit (the grid is a multiple of 8).
struct XcdItems {
  int first, step, end;  // this wave's first item, its stride, the range end
};
__device__ __forceinline__ XcdItems xcd_items(int nitems) {
  const int xcd = static_cast<int>(blockIdx.x) & 7;
  const int per = (((nitems + 7) >> 3) + 3) & ~3;
  const int lo = xcd * per;
  XcdItems r;
  r.first = lo + (static_cast<int>(blockIdx.x) >> 3) * 4 + wave_index();
  r.step = (static_cast<int>(gridDim.x) >> 3) * 4;
  r.end = min(lo + per, nitems);
  return r;
}
}  // namespace

// ---------------------------------------------------------------------------
// Decode GEMMs: a wave streams a 64-row weight block (four 16-row MFMA tiles)
// against one 16-row sub-tile of a chunk. K advances in 128-element steps; a
// ring of D steps of weight and activation loads stays in flight ahead of the
// MFMAs. The chunk's token rows are the N side; each 8-bf16 activation
// fragment feeds the four weight tiles.
//
// Load mix, as measured on MI355X: per-step byte loads of scales and
// activation loads from up to 16 distinct rows each touch 16 cache lines per
// instruction and cut the weight stream's bandwidth nearly in half. So the
// block's 64 scale rows are copied once per item into a per-wave LDS block
// with coalesced 16-byte loads and read from LDS each step, and activations
// use buffer loads whose out-of-range offset (lanes past the chunk's last
// row) returns zero without touching memory.
// ---------------------------------------------------------------------------
// Copy N blocks of `bytes` each (a multiple of 16, at most MAXB * 4 KB) from
// global memory to this wave's LDS. The loads of a batch (four 1 KB pieces
// per block) all go out before its first store, so a batch costs one memory
// round trip; a load-then-store loop waited for every piece in turn, about
// eight dependent round trips for the two 3.5 KB scale blocks of a decode
// GEMM1 item at H = 3584. Straight-line code (batches behind wave-uniform
// guards, no per-lane branch): lanes past the end load and store the
// block's last 16 bytes again, the same data at the same place.
// LDS bytes reserved for a copied block: a direct-to-LDS load instruction
// writes a whole 1 KB (16 bytes per lane, lane order).
__host__ __device__ constexpr int lds_block_bytes(int bytes) { return (bytes + 1023) & ~1023; }

// Copy N blocks of `bytes` each (a multiple of 16, at most MAXP KB) from
// global memory straight into this wave's LDS with 16-byte direct-to-LDS
// buffer loads: no data registers, every piece in flight at once, so the copy
// costs one memory round trip and is waited for like any other load. A
// load-then-store loop waited for every 1 KB piece in turn, about eight
// dependent round trips for the two 3.5 KB scale blocks of a decode GEMM1
// item at H = 3584. Piece i of block b comes through a buffer of its own
// (base + 1024 i, the bytes left), so a lane past the block's end is out of
// range and reads nothing; it lands in the padding of the block's LDS
// region, lds_block_bytes(bytes) long. Lane l's 16 bytes go to
// lds[b] + 1024 i + 16 l.
template <int N, int MAXP>
__device__ __forceinline__ void wave_copy_to_lds(uint8_t* const (&lds)[N],
                                                 const uint8_t* const (&src)[N], int bytes) {
  typedef __attribute__((address_space(3))) void lds_void;
  const uint32_t l16 = static_cast<uint32_t>(lane_id()) * 16;
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    if (i == 0 || i * 1024 < bytes) {  // wave-uniform
#pragma unroll
      for (int b = 0; b < N; ++b) {
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(src[b] + i * 1024, static_cast<uint32_t>(bytes - i * 1024));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds[b] + i * 1024), 16, l16, 0, 0, 0);
      }
    }
  }
}
// Wait until every load this wave issued has completed, direct-to-LDS loads
// included (s_waitcnt vmcnt(0); the other counters are left alone). The
// compiler does not order reads of LDS after direct-to-LDS buffer loads, so
// the streams below call this after their first ring loads, before their
// first read of the scale rows wave_copy_to_lds brought in: on MI355X,
// reads issued ahead of the copy returned the previous item's scales now
// and then (run-to-run differences at H = 512, I = 640).
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Pieces the callers allow for (the shape check caps H and I at kMaxTiledK):
// GEMM1 scale blocks of 16 * TP rows x H / 32 bytes (TP <= 2) and the MX
// GEMM1's 32 rows, at most 8 KB; the split GEMM2's 64 rows x I / 32 bytes,
// at most 16 KB.
static_assert(16 * 2 * (kMaxTiledK / 32) <= 8 * 1024, "GEMM1 scale blocks exceed 8 pieces");
static_assert(64 * (kMaxTiledK / 32) <= 16 * 1024, "split GEMM2 scale blocks exceed 16 pieces");

// acc[s][t] += W_tile_t (16 x K) * B_s^T for NS sub-tiles of 16 token rows.
// wp: lane's weight-row pointer of tile 0, offset by g*16 bytes; tile t is
// wofs[t] bytes further (wave-uniform). ls: lane's scale row in LDS, offset by
// g; tile t is lofs[t] bytes further. brs/boff[s]: buffer and byte offset of
// the lane's row of sub-tile s plus g*64 bytes (kNoRow for lanes past the
// chunk's end). Each decoded weight fragment feeds all NS sub-tiles. NTW:
// the weights are read once in this call (non-temporal loads).
// D divides nkb, so the unrolled body has no tail branches: the
// vector-memory counter retires loads in issue order, and straight-line code
// lets every wait cover only the step it needs.
template <bool NTW, int D, int NS, int NT = 4>
__device__ __forceinline__ void stream_block(const uint8_t* wp, const uint32_t (&wofs)[NT],
                                             const uint8_t* ls, const uint32_t (&lofs)[NT], int nkb,
                                             __amdgpu_buffer_rsrc_t brs, const uint32_t (&boff)[NS],
                                             f32x4_t (&acc)[NS][NT]) {
  uint4 w[D][NT], xb[D][NS][4];
  // Prologue in slot order (pinned), matching the steady-state issue order.
#pragma unroll
  for (int d = 0; d < D; ++d) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) xb[d][s][j] = bld16(brs, boff[s] + d * 256 + j * 16);
#pragma unroll
    for (int t = 0; t < NT; ++t) w[d][t] = ldw16<NTW>(wp + wofs[t] + d * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_all_loads();  // the item's scale rows are in LDS
  __builtin_amdgcn_sched_barrier(0);
  const int last = nkb - 1;
  // One ring step: multiply slot d (step kb), then refill it with step
  // kb + D (near the end the last step again; those loads are never used).
  auto step = [&](int kb, int d) {
    float sc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) sc[t] = e8m0_scale_operand(ls[lofs[t] + kb * 4]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t ww[4] = {w[d][t].x, w[d][t].y, w[d][t].z, w[d][t].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t a = decode_fp4x8(ww[j], sc[t]);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[s][t] = mfma16x16x32(a, as_bf16x8(xb[d][s][j]), acc[s][t]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const int nk = min(kb + D, last);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) xb[d][s][j] = bld16(brs, boff[s] + nk * 256 + j * 16);
#pragma unroll
    for (int t = 0; t < NT; ++t) w[d][t] = ldw16<NTW>(wp + wofs[t] + nk * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
  };
  // The first ring cycle is peeled: the loop is then entered with loads
  // pending in the same order as on every later iteration, so its waits
  // cover only the slot being consumed.
#pragma unroll
  for (int d = 0; d < D; ++d) step(d, d);
  for (int kb0 = D; kb0 < nkb; kb0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(kb0 + d, d);
  }
}

// Token tile of one K step in LDS, shared by the four waves of a block
// (they work on the same chunk): 16 * NS rows x 256 bytes, tok_lds_step<NS>()
// bytes per buffer. 16-byte chunk c of tile row rr sits at
// rr * 256 + 16 * (c ^ tswz(rr)): the 32 lanes that read one fragment (rows
// r = 0..15, chunks 4g + j, g = 0..1) and the 32 lanes that write two rows
// fall on distinct 16-byte bank groups of a 512-byte bank line. The stream
// needs an even step count (D = 2, no tail): H / 128 always is, and the
// split GEMM2 takes this path only when I / 128 is.
template <int NS>
constexpr int tok_lds_step() {
  return 16 * NS * 256;
}
__device__ __forceinline__ uint32_t tswz(int rr) {
  const uint32_t m = static_cast<uint32_t>(rr >> 1) & 7u;
  return (m & 3u) | ((m & 4u) << 1);
}
__device__ __forceinline__ uint32_t tlds_off(int rr, int c) {
  return static_cast<uint32_t>(rr * 256) + ((static_cast<uint32_t>(c) ^ tswz(rr)) << 4);
}

// stream_block with the token fragments read from a block-shared LDS tile
// (two buffers of tok_lds_step<NS>() at tl) instead of per-wave loads, so a token
// row is fetched once per block and K step instead of once per wave. Every
// wave of the block must call it with the same nkb and NS: one barrier per
// K step. Thread t loads 16-byte chunk t % 16 of tile rows t / 16 + 16 i
// (i < NS) from trs at toff[i] (out of range past the chunk's end, which
// reads zero), D = 2 steps ahead like the weights, and stores it to the
// other LDS buffer one step before it is read.
// NL >= NS: the tile holds NL 16-row sub-tiles (NL = 2, NS = 1 for the
// K-halves items, whose second sub-tile is the same rows half the K range
// further on) and the wave reads sub-tiles sub0 .. sub0 + NS - 1.
template <bool NTW, int NS, int NT = 4, int NL = NS>
__device__ __forceinline__ void stream_block_lds(const uint8_t* wp, const uint32_t (&wofs)[NT],
                                                 const uint8_t* ls, const uint32_t (&lofs)[NT],
                                                 int nkb, __amdgpu_buffer_rsrc_t trs,
                                                 const uint32_t (&toff)[NL], uint8_t* tl,
                                                 f32x4_t (&acc)[NS][NT], int sub0 = 0) {
  constexpr int D = 2;
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int lr = static_cast<int>(threadIdx.x) >> 4, lc = static_cast<int>(threadIdx.x) & 15;
  uint4 w[D][NT], tv[D][NL];
#pragma unroll
  for (int d = 0; d < D; ++d) {
#pragma unroll
    for (int i = 0; i < NL; ++i) tv[d][i] = bld16(trs, toff[i] + d * 256);
#pragma unroll
    for (int t = 0; t < NT; ++t) w[d][t] = ldw16<NTW>(wp + wofs[t] + d * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_all_loads();  // the item's scale rows are in LDS
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NL; ++i) *reinterpret_cast<uint4*>(tl + tlds_off(lr + 16 * i, lc)) = tv[0][i];
  __syncthreads();
  const int last = nkb - 1;
  auto step = [&](int kb, int d) {
    // step kb + 2's token rows, issued first: tv[d] held step kb's rows,
    // which went to LDS in step kb - 1
    const int nk = min(kb + D, last);
#pragma unroll
    for (int i = 0; i < NL; ++i) tv[d][i] = bld16(trs, toff[i] + nk * 256);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* tb = tl + (kb & 1) * tok_lds_step<NL>();
    uint4 xb[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xb[s][j] = *reinterpret_cast<const uint4*>(tb + tlds_off(16 * (s + sub0) + r, 4 * g + j));
    float sc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) sc[t] = e8m0_scale_operand(ls[lofs[t] + kb * 4]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t ww[4] = {w[d][t].x, w[d][t].y, w[d][t].z, w[d][t].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t a = decode_fp4x8(ww[j], sc[t]);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[s][t] = mfma16x16x32(a, as_bf16x8(xb[s][j]), acc[s][t]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // step kb + 1's tile (loaded one step ago) into the buffer read in step
    // kb - 1, which every wave left before the last barrier
    uint8_t* nb = tl + ((kb + 1) & 1) * tok_lds_step<NL>();
#pragma unroll
    for (int i = 0; i < NL; ++i) *reinterpret_cast<uint4*>(nb + tlds_off(lr + 16 * i, lc)) = tv[(d + 1) % D][i];
#pragma unroll
    for (int t = 0; t < NT; ++t) w[d][t] = ldw16<NTW>(wp + wofs[t] + nk * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
#pragma unroll
  for (int d = 0; d < D; ++d) step(d, d);
  for (int kb0 = D; kb0 < nkb; kb0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(kb0 + d, d);
  }
}

#ifndef MOE_MAX_RING_DEPTH
#define MOE_MAX_RING_DEPTH 2
#endif
// Largest ring depth <= MOE_MAX_RING_DEPTH that divides the step count.
inline int ring_depth(int nkb) {
  for (int d = MOE_MAX_RING_DEPTH; d > 1; --d)
    if (nkb % d == 0) return d;
  return 1;
}

// GEMM1 + SwiGLU, decode shape. Item = (chunk of at most 16 * NSMAX rows,
// group of 16 * TP features): tile 2p holds gate rows f0 + 16p + [0, 16),
// tile 2p + 1 the up rows I + f0 + 16p + [0, 16). A chunk of more than 16
// rows runs both 16-row sub-tiles against each weight load, so an expert's
// weights are streamed once per chunk; a wider feature group cuts how often
// the chunk's token rows are re-read (once per group). Dynamic LDS: 4 waves
// x TP * H bytes (the group's gate and up scale rows). `units`/`ctr`: the
// chunk table and the counter word holding its length; `counts`: rows per
// expert (an expert of at most 16 * NSMAX rows has its weights read once).
// TL: token tiles shared through LDS (stream_block_lds, D = 2); the dynamic
// LDS then starts with the two token buffers. The four waves of a block
// always hold items of the same chunk (groups is a multiple of 4).
// KH (K halves; H a multiple of 512, and with TL one 16-row sub-tile):
// every (chunk, feature group) pair is two items, the first and the second
// half of K, taken by neighbouring waves of one block (item 2 * pair +
// half). With TL both halves' token rows share the block's LDS tile (two
// sub-tiles). After the stream the second-half wave hands its fp32 sums to
// the first through LDS, and the first adds them (first half + second half,
// always in that order) and stores act. `xi` gives the items each wave
// takes.
template <int D, int NSMAX, int TP, bool TL, bool KH = false>
__device__ __forceinline__ void gemm1_decode_items(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ s13, const int32_t* __restrict__ units, int ctr,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ sorted_slot, int T, int H,
    int I, int Kp, ActArgs actf, uint16_t* __restrict__ act, uint8_t* lds_scales, XcdItems xi) {
  static_assert(!KH || !TL || NSMAX == 1, "K halves share a one-sub-tile LDS token tile");
  constexpr int NT = 2 * TP;
  constexpr int TNS = (KH && TL) ? 2 : NSMAX;  // 16-row sub-tiles of the block's token tile
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int groups = I / (16 * TP);
  const int ipc = KH ? 2 * groups : groups;  // items per chunk
  const size_t wrow = static_cast<size_t>(H) >> 1, srow = static_cast<size_t>(H) >> 5;
  const int nkb = KH ? H >> 8 : H >> 7;  // K steps per item
  const int blk = 16 * TP * static_cast<int>(srow);  // the group's gate (or up) scale rows
  const int blkp = lds_block_bytes(blk);
  uint8_t* tl = lds_scales;
  uint8_t* my = lds_scales + (TL ? 2 * tok_lds_step<TNS>() : 0) + wave_index() * 2 * blkp;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, static_cast<uint32_t>(static_cast<size_t>(T) * H * 2));
  const int lr = static_cast<int>(threadIdx.x) >> 4, lc = static_cast<int>(threadIdx.x) & 15;
  uint32_t wofs[NT], lofs[NT];
#pragma unroll
  for (int p = 0; p < TP; ++p) {
    wofs[2 * p] = static_cast<uint32_t>(16 * p * wrow);
    wofs[2 * p + 1] = static_cast<uint32_t>((I + 16 * p) * wrow);
    lofs[2 * p] = static_cast<uint32_t>(16 * p * srow);
    lofs[2 * p + 1] = static_cast<uint32_t>(blkp + 16 * p * srow);
  }
  for (int item = xi.first; item < xi.end; item += xi.step) {
    const int u = item / ipc;
    const int ig = item - u * ipc;
    const int kh = KH ? ig & 1 : 0;  // which half of K
    const int f0 = (KH ? ig >> 1 : ig) * 16 * TP;
    const int4 ui = reinterpret_cast<const int4*>(units)[u];
    const int e = ui.x, r0 = ui.y, nrows = ui.z;
    const size_t row0 = static_cast<size_t>(e) * 2 * I + f0;
    const uint8_t* sg = s13 + row0 * srow;
    // the chunk's slot numbers (clamped, unconditional loads) go out with the
    // scale-row loads: the item setup waits one round trip for both
    int slot_w[NSMAX], slot_t[NSMAX];
#pragma unroll
    for (int s = 0; s < NSMAX; ++s) slot_w[s] = sorted_slot[r0 + min(16 * s + r, nrows - 1)];
    if (TL) {
#pragma unroll
      for (int i = 0; i < NSMAX; ++i) slot_t[i] = sorted_slot[r0 + min(lr + 16 * i, nrows - 1)];
    }
    {
      uint8_t* const dst[2] = {my, my + blkp};
      const uint8_t* const src[2] = {sg, sg + static_cast<size_t>(I) * srow};
      wave_copy_to_lds<2, 8>(dst, src, blk);
    }
    const uint8_t* wp = w13 + row0 * wrow + r * 64 + g * 16;  // packed layout
    const bool once = counts[e] <= 16 * NSMAX;  // the expert's only chunk
    uint32_t boff[NSMAX];
#pragma unroll
    for (int s = 0; s < NSMAX; ++s) {
      const int rr = 16 * s + r;
      boff[s] = rr < nrows ? static_cast<uint32_t>(slot_w[s] / Kp) * H * 2 + g * 64 : kNoRow;
    }
    uint32_t toff[NSMAX];  // this thread's rows of the block's token tile
    if (TL) {
#pragma unroll
      for (int i = 0; i < NSMAX; ++i) {
        const int rr = lr + 16 * i;
        toff[i] = rr < nrows ? static_cast<uint32_t>(slot_t[i] / Kp) * H * 2 + lc * 16 : kNoRow;
      }
    }
    // rows past the chunk's end fall outside the buffer: stores dropped
    const __amdgpu_buffer_rsrc_t ars =
        make_rsrc(act + static_cast<size_t>(r0) * I, static_cast<uint32_t>(nrows) * I * 2);
    auto store = [&](const f32x4_t (&acc)[NT], int s) {
      const uint32_t aoff = static_cast<uint32_t>(16 * s + r) * I * 2 + (f0 + g * 4) * 2;
#pragma unroll
      for (int p = 0; p < TP; ++p) {
        const f32x4_t& ag = acc[2 * p];
        const f32x4_t& au = acc[2 * p + 1];
        uint2 pk;
        pk.x = pack_bf16x2(act_apply(ag[0], au[0], actf), act_apply(ag[1], au[1], actf));
        pk.y = pack_bf16x2(act_apply(ag[2], au[2], actf), act_apply(ag[3], au[3], actf));
        bst8(ars, aoff + p * 32, pk);
      }
    };
    // K halves: the second-half wave's fp32 sums go to the first-half wave
    // through LDS (with TL the token buffers, else the second wave's own
    // scale block, both free after the stream), then the first adds them
    // (first half + second half) and stores act.
    auto join_store = [&](auto& acc, auto ns) {
      constexpr int NS = decltype(ns)::value;
      float* part = TL ? reinterpret_cast<float*>(tl) + (wave_index() >> 1) * NS * NT * 4 * kWave
                       : reinterpret_cast<float*>(lds_scales + (wave_index() | 1) * 2 * blkp);
      if (kh) {
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[((s2 * NT + t) * 4 + i) * kWave + lane] = acc[s2][t][i];
      }
      __syncthreads();
      if (!kh) {
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[s2][t][i] += part[((s2 * NT + t) * 4 + i) * kWave + lane];
          store(acc[s2], s2);
        }
      }
      __syncthreads();  // the next item overwrites the sums
    };
    const size_t kwo = KH ? static_cast<size_t>(kh) * nkb * kPkBlock : 0;  // this half's K offsets
    const int kso = KH ? kh * nkb * 4 : 0;
    const uint32_t kto = KH ? static_cast<uint32_t>(kh * nkb) * 256u : 0u;
    if (NSMAX == 1 || nrows <= 16) {
      f32x4_t acc[1][NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[0][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint32_t b1[1] = {boff[0] + kto};
      const uint32_t t1[1] = {toff[0]};
      auto run = [&](auto ntw) {
        if constexpr (KH && TL) {
          // sub-tile 1: the same rows, the second half of K
          const uint32_t t2[2] = {toff[0], toff[0] + static_cast<uint32_t>(nkb) * 256u};
          stream_block_lds<decltype(ntw)::value, 1, NT, 2>(
              wp + static_cast<size_t>(kh) * nkb * kPkBlock, wofs, my + r * srow + g + kh * nkb * 4,
              lofs, nkb, xrs, t2, tl, acc, kh);
        } else if constexpr (TL) {
          stream_block_lds<decltype(ntw)::value, 1, NT>(wp, wofs, my + r * srow + g, lofs, nkb, xrs, t1,
                                                        tl, acc);
        } else {
          stream_block<decltype(ntw)::value, D, 1, NT>(wp + kwo, wofs, my + r * srow + g + kso, lofs, nkb,
                                                       xrs, b1, acc);
        }
      };
      if (once) run(BoolC<true>{}); else run(BoolC<false>{});
      if constexpr (KH && !TL) {
        join_store(acc, IntC<1>{});
      } else if constexpr (KH) {
        // the second half's sums go to the first half's wave through the
        // token buffers, free after the stream's last barrier
        float* part = reinterpret_cast<float*>(tl) + (wave_index() >> 1) * NT * 4 * kWave;
        if (kh) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[(t * 4 + i) * kWave + lane] = acc[0][t][i];
        }
        __syncthreads();
        if (!kh) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[0][t][i] += part[(t * 4 + i) * kWave + lane];
          store(acc[0], 0);
        }
        __syncthreads();  // the next item's first token tile overwrites the sums
      } else {
        store(acc[0], 0);
      }
    } else {
      f32x4_t acc[NSMAX][NT];
#pragma unroll
      for (int s = 0; s < NSMAX; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto run = [&](auto ntw) {
        if constexpr (TL)
          stream_block_lds<decltype(ntw)::value, NSMAX, NT>(wp, wofs, my + r * srow + g, lofs, nkb, xrs,
                                                            toff, tl, acc);
        else {
          uint32_t bk[NSMAX];
#pragma unroll
          for (int s2 = 0; s2 < NSMAX; ++s2) bk[s2] = boff[s2] + kto;
          stream_block<decltype(ntw)::value, D, NSMAX, NT>(wp + kwo, wofs, my + r * srow + g + kso, lofs,
                                                           nkb, xrs, bk, acc);
        }
      };
      if (once) run(BoolC<true>{}); else run(BoolC<false>{});
      if constexpr (KH && !TL) {
        join_store(acc, IntC<NSMAX>{});
      } else {
#pragma unroll
        for (int s = 0; s < NSMAX; ++s) store(acc[s], s);
      }
    }
  }
}

// Items of 32 features (TP = 2) re-read the chunk's tokens half as often as
// items of 16; items of 16 give twice the parallelism. With fewer 32-feature
// items than the waves the chip holds at once (a few touched experts with
// many rows, as in the Zipf-routed T256 EP decode: 42 against 51 us on
// MI355X), the kernel takes 16-feature items; otherwise 32 (T64 decode 146
// against 161 us, T512 shared-expert layer 690 against 744 us). The choice
// is read on the device from the chunk count and is the same for every
// block. Dynamic LDS is sized for TP = 2.
constexpr int kNarrowItemsBelow = 4096;
template <int D, int NSMAX, bool TL>
__global__ __launch_bounds__(kGemmBlock) void gemm1_decode_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ s13, const int32_t* __restrict__ units, int ctr,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ sorted_slot, int T, int H, int I, int Kp, ActArgs actf,
    uint16_t* __restrict__ act, int res_xcd) {
  extern __shared__ uint8_t lds_scales[];
  const int nch = counters[ctr];
  const bool narrow = nch * (I / 32) < kNarrowItemsBelow;
  const int P = nch * (narrow ? I / 16 : I / 32);  // (chunk, feature group) pairs
  // A partial last round (res_xcd: the blocks one XCD holds at once, from
  // the host; 0 turns this off): the blocks of whole rounds take four pairs
  // each, and the pairs left over go two to a block as K halves (half as
  // many steps each), so the last items end closer together. Each pair is
  // computed once either way. Zipf-routed T256 EP decode: 4,632 pairs on
  // 4,096 wave slots, GEMM1 43 -> 40 us; T64 decode: 7,284 pairs on 2,048
  // slots, GEMM1 142 -> 138 us (MI355X).
  if ((H & 511) == 0 && res_xcd > 0) {
    const int per = (((P + 7) >> 3) + 3) & ~3;  // pairs per XCD, as xcd_items
    const int nfull = ((per >> 2) / res_xcd) * res_xcd;  // blocks of whole rounds
    const int left = per - 4 * nfull;
    const int gx = static_cast<int>(gridDim.x) >> 3;
    const int srow = H >> 5;
    // without TL the sums pass through the second wave's scale block
    const bool fits = TL ? (NSMAX == 1 && narrow)
                         : 2 * lds_block_bytes(16 * (narrow ? 1 : 2) * srow) >=
                               NSMAX * 2 * (narrow ? 1 : 2) * 4 * kWave * 4;
    if (fits && nfull > 0 && left > 0 && left / 2 <= gx - nfull) {
      const int xcd = static_cast<int>(blockIdx.x) & 7, lb = static_cast<int>(blockIdx.x) >> 3;
      const int lo = xcd * per, endp = min(lo + per, P);
      XcdItems xi;
      xi.step = 1 << 30;  // one item per wave
      const bool whole = lb < nfull;
      if (whole) {
        xi.first = lo + 4 * lb + wave_index();
        xi.end = endp;
      } else {  // K-half items are numbered 2 * pair + half
        xi.first = 2 * (lo + 4 * nfull + 2 * (lb - nfull)) + wave_index();
        xi.end = 2 * endp;
      }
      if (narrow) {
        if (whole)
          gemm1_decode_items<D, NSMAX, 1, TL>(x, w13, s13, units, ctr, counters, counts, sorted_slot,
                                              T, H, I, Kp, actf, act, lds_scales, xi);
        else if constexpr (!TL || NSMAX == 1)
          gemm1_decode_items<D, NSMAX, 1, TL, true>(x, w13, s13, units, ctr, counters, counts,
                                                    sorted_slot, T, H, I, Kp, actf, act, lds_scales, xi);
      } else if constexpr (!TL) {
        if (whole)
          gemm1_decode_items<D, NSMAX, 2, TL>(x, w13, s13, units, ctr, counters, counts, sorted_slot,
                                              T, H, I, Kp, actf, act, lds_scales, xi);
        else
          gemm1_decode_items<D, NSMAX, 2, TL, true>(x, w13, s13, units, ctr, counters, counts,
                                                    sorted_slot, T, H, I, Kp, actf, act, lds_scales, xi);
      }
      return;
    }
  }
  if (narrow)
    gemm1_decode_items<D, NSMAX, 1, TL>(x, w13, s13, units, ctr, counters, counts, sorted_slot, T, H,
                                        I, Kp, actf, act, lds_scales, xcd_items(P));
  else
    gemm1_decode_items<D, NSMAX, 2, TL>(x, w13, s13, units, ctr, counters, counts, sorted_slot, T, H,
                                        I, Kp, actf, act, lds_scales, xcd_items(P));
}

// GEMM2 split path, decode shape, long K. Item = (chunk of at most
// 16 * NSMAX rows, 64 output rows of H). Dynamic LDS: 4 waves x 2I bytes
// (the 64 rows' scales), after the two token buffers when TL (as in
// gemm1_decode_kernel; H / 64 items per chunk, a multiple of 4).
template <int D, int NSMAX, bool TL>
__global__ __launch_bounds__(kGemmBlock) void gemm2_split_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int32_t* __restrict__ units, int ctr,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ counts, int H, int I,
    uint16_t* __restrict__ y) {
  if (counters[kCtrGate] != 0) return;  // dense path chosen: zero items here
  extern __shared__ uint8_t lds_scales[];
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int quads = H >> 6;
  const int nitems = counters[ctr] * quads;
  const size_t wrow = static_cast<size_t>(I) >> 1, srow = static_cast<size_t>(I) >> 5;
  const int nkb = I >> 7;
  const int blk = 64 * static_cast<int>(srow);  // = 2I bytes
  uint8_t* tl = lds_scales;
  uint8_t* my = lds_scales + (TL ? 2 * tok_lds_step<NSMAX>() : 0) + wave_index() * lds_block_bytes(blk);
  const int lr = static_cast<int>(threadIdx.x) >> 4, lc = static_cast<int>(threadIdx.x) & 15;
  const uint32_t wofs[4] = {0u, static_cast<uint32_t>(16 * wrow), static_cast<uint32_t>(32 * wrow),
                            static_cast<uint32_t>(48 * wrow)};
  const uint32_t lofs[4] = {0u, static_cast<uint32_t>(16 * srow), static_cast<uint32_t>(32 * srow),
                            static_cast<uint32_t>(48 * srow)};
  const XcdItems xi = xcd_items(nitems);
  for (int item = xi.first; item < xi.end; item += xi.step) {
    const int u = item / quads;
    const int h0 = (item - u * quads) * 64;
    const int4 ui = reinterpret_cast<const int4*>(units)[u];
    const int e = ui.x, r0 = ui.y, nrows = ui.z;
    const size_t row0 = static_cast<size_t>(e) * H + h0;
    {
      uint8_t* const dst[1] = {my};
      const uint8_t* const src[1] = {s2 + row0 * srow};
      wave_copy_to_lds<1, 16>(dst, src, blk);
    }
    const uint8_t* wp = w2 + row0 * wrow + r * 64 + g * 16;  // packed layout
    const bool once = counts[e] <= 16 * NSMAX;  // the expert's only chunk
    // chunk-relative buffers: rows past the chunk's end read 0 / drop stores
    const __amdgpu_buffer_rsrc_t ars =
        make_rsrc(act + static_cast<size_t>(r0) * I, static_cast<uint32_t>(nrows) * I * 2);
    const __amdgpu_buffer_rsrc_t yrs =
        make_rsrc(y + static_cast<size_t>(r0) * H, static_cast<uint32_t>(nrows) * H * 2);
    uint32_t boff[NSMAX];
#pragma unroll
    for (int s = 0; s < NSMAX; ++s) boff[s] = static_cast<uint32_t>(16 * s + r) * I * 2 + g * 64;
    uint32_t toff[NSMAX];  // this thread's rows of the block's act tile (zero past nrows)
#pragma unroll
    for (int i = 0; i < NSMAX; ++i) toff[i] = static_cast<uint32_t>(lr + 16 * i) * I * 2 + lc * 16;
    // the four 16-feature tiles regrouped across lanes: two 16-byte stores a
    // lane, aligned 64-byte pieces of 16 Y rows (h0 is a multiple of 64)
    auto store = [&](const f32x4_t (&acc)[4], int s) {
      uint2 pk[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        pk[t].x = pack_bf16x2(acc[t][0], acc[t][1]);
        pk[t].y = pack_bf16x2(acc[t][2], acc[t][3]);
      }
      y_regroup(pk);
      const uint32_t yoff = static_cast<uint32_t>(16 * s + r) * H * 2 + h0 * 2 + 16 * g;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        bst16(yrs, yoff + 64 * k, uint4{pk[2 * k].x, pk[2 * k].y, pk[2 * k + 1].x, pk[2 * k + 1].y});
    };
    if (NSMAX == 1 || nrows <= 16) {
      f32x4_t acc[1][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[0][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint32_t b1[1] = {boff[0]};
      const uint32_t t1[1] = {toff[0]};
      auto run = [&](auto ntw) {
        if constexpr (TL)
          stream_block_lds<decltype(ntw)::value, 1>(wp, wofs, my + r * srow + g, lofs, nkb, ars, t1, tl,
                                                    acc);
        else
          stream_block<decltype(ntw)::value, D, 1>(wp, wofs, my + r * srow + g, lofs, nkb, ars, b1, acc);
      };
      if (once) run(BoolC<true>{}); else run(BoolC<false>{});
      store(acc[0], 0);
    } else {
      f32x4_t acc[NSMAX][4];
#pragma unroll
      for (int s = 0; s < NSMAX; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto run = [&](auto ntw) {
        if constexpr (TL)
          stream_block_lds<decltype(ntw)::value, NSMAX>(wp, wofs, my + r * srow + g, lofs, nkb, ars, toff,
                                                        tl, acc);
        else
          stream_block<decltype(ntw)::value, D, NSMAX>(wp, wofs, my + r * srow + g, lofs, nkb, ars, boff,
                                                       acc);
      };
      if (once) run(BoolC<true>{}); else run(BoolC<false>{});
#pragma unroll
      for (int s = 0; s < NSMAX; ++s) store(acc[s], s);
    }
  }
}

// GEMM2 split path for short K with bf16 act where no resident dense kernel
// exists (384 < I <= 512): the stream of gemm2_stream.h in a launch of its
// own, next to the generic tiled dense kernel. For I <= 384 both paths run
// in one gated launch (gemm_tiled.hip).
template <int NKB>
__global__ __launch_bounds__(kGemmBlock) void gemm2_stream_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int32_t* __restrict__ units,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ counts, int H, int I,
    uint16_t* __restrict__ y) {
  if (counters[kCtrGate] != 0) return;  // dense path chosen: zero items here
  gemm2_stream_body<NKB>(act, w2, s2, units, counters, counts, H, I, y);
}

// ---------------------------------------------------------------------------
// MX-activation decode GEMMs: W4A8 (MXFP8 activations) and, with A4, W4A4
// (MXFP4 activations). The E2M1 weights go into the scaled MFMA as they are,
// with their E8M0 scales; no decode. One 16x16x128 MFMA per weight tile and
// K step: lane (r, g) supplies weight row r's codes K [32g, 32g + 32) (the
// same 16-byte load as the bf16 path) and that group's scale byte, and
// token r's codes with its scale byte for block g: E4M3 codes K [16g,
// 16g + 16) and [64 + 16g, 64 + 16g + 16) (a K step is 128 bytes of a token
// row), or E2M1 codes K [32g, 32g + 32), the same 16 bytes as the weight's
// (a K step is 64 bytes).
// ---------------------------------------------------------------------------


// acc[t] += W_tile_t * Xq^T over nkb steps. xrs/xoff: buffer and byte offset
// of the lane's token code row plus 16g (kNoRow past the unit's end);
// srs/soff: the row's scale bytes plus g (kNoRow likewise).
template <bool NTW, int D, bool A4>
__device__ __forceinline__ void stream_block_a8(const uint8_t* wp, const uint32_t (&wofs)[4],
                                                const uint8_t* ls, const uint32_t (&lofs)[4],
                                                int nkb, __amdgpu_buffer_rsrc_t xrs, uint32_t xoff,
                                                __amdgpu_buffer_rsrc_t srs, uint32_t soff,
                                                f32x4_t (&acc)[4]) {
  constexpr uint32_t XS = tok_step_bytes<A4>();
  uint4 w[D][4], xb[D][2];
  uint32_t xsb[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    xb[d][0] = bld16(xrs, xoff + d * XS);
    if (!A4) xb[d][1] = bld16(xrs, xoff + d * XS + 64);
    xsb[d] = bld1(srs, soff + d * 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) w[d][t] = ldw16<NTW>(wp + wofs[t] + d * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_all_loads();  // the item's scale rows are in LDS
  __builtin_amdgcn_sched_barrier(0);
  const int last = nkb - 1;
  auto step = [&](int kb, int d) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc[t] = mfma_f4xa<A4>(w[d][t], ls[lofs[t] + kb * 4], xb[d][0], xb[d][1], xsb[d], acc[t]);
    __builtin_amdgcn_sched_barrier(0);
    const int nk = min(kb + D, last);
    xb[d][0] = bld16(xrs, xoff + nk * XS);
    if (!A4) xb[d][1] = bld16(xrs, xoff + nk * XS + 64);
    xsb[d] = bld1(srs, soff + nk * 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) w[d][t] = ldw16<NTW>(wp + wofs[t] + nk * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) step(d, d);
  for (int kb0 = D; kb0 < nkb; kb0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(kb0 + d, d);
  }
}

// Block-shared token tile of one K step in LDS for the MX stream: 16 rows x
// tok_step_bytes codes, then the rows' four scale bytes.
// E4M3 (128-byte rows): chunk c (0..7) of row rr sits at rr * 128 +
// 16 * (c ^ (((rr >> 2) & 3) << 1)). E2M1 (64-byte rows): chunk c (0..3) at
// rr * 64 + 16 * (c ^ (((rr >> 3) & 1) << 1)). Either way the 32 lanes of a
// fragment read (rows r, the lane group's chunks) and of a write fall on
// distinct 16-byte bank groups.
template <bool A4>
constexpr int tok_mx_lds_step() {
  return 16 * static_cast<int>(tok_step_bytes<A4>()) + 16 * 4;
}
template <bool A4>
__device__ __forceinline__ uint32_t tmx_lds_off(int rr, int c) {
  if constexpr (A4)
    return static_cast<uint32_t>(rr * 64) + ((static_cast<uint32_t>(c) ^ ((static_cast<uint32_t>(rr >> 3) & 1u) << 1)) << 4);
  else
    return static_cast<uint32_t>(rr * 128) + ((static_cast<uint32_t>(c) ^ ((static_cast<uint32_t>(rr >> 2) & 3u) << 1)) << 4);
}
// Threads of a block that copy token codes (16 rows x chunks per row), and
// the first thread of the 16 that copy the rows' scale dwords.
template <bool A4>
constexpr int tok_mx_code_threads() {
  return A4 ? 64 : 128;
}

// stream_block_a8 with the token codes and scales read from a block-shared
// LDS tile (two buffers of tok_mx_lds_step at tl), as stream_block_lds does
// for bf16 tokens: one barrier per K step, every wave of the block calls it
// with the same nkb. Threads t < NC = tok_mx_code_threads load one 16-byte
// code chunk of a tile row (xrs at toff, zero past the unit's end: chunk
// t % 8 of row t / 8 for E4M3, t % 4 of row t / 4 for E2M1), threads
// NC..NC+15 the scale dword of tile row t - NC (srs at tsoff); the rest load
// nothing (out-of-range offsets) and store nothing.
template <bool NTW, bool A4>
__device__ __forceinline__ void stream_block_a8_lds(const uint8_t* wp, const uint32_t (&wofs)[4],
                                                    const uint8_t* ls, const uint32_t (&lofs)[4],
                                                    int nkb, __amdgpu_buffer_rsrc_t xrs, uint32_t toff,
                                                    __amdgpu_buffer_rsrc_t srs, uint32_t tsoff,
                                                    uint8_t* tl, f32x4_t (&acc)[4]) {
  constexpr int D = 2;
  constexpr uint32_t XS = tok_step_bytes<A4>();
  constexpr int NC = tok_mx_code_threads<A4>();
  constexpr int STEP = tok_mx_lds_step<A4>();
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int t = static_cast<int>(threadIdx.x);
  const bool code_role = t < NC, scale_role = t >= NC && t < NC + 16;
  const uint32_t st_off = code_role ? (A4 ? tmx_lds_off<A4>(t >> 2, t & 3) : tmx_lds_off<A4>(t >> 3, t & 7))
                                    : 16 * XS + (t - NC) * 4;
  uint4 w[D][4], tv[D];
  uint32_t ts[D];
  auto put = [&](uint8_t* buf, int d) {
    if (code_role) *reinterpret_cast<uint4*>(buf + st_off) = tv[d];
    if (scale_role) *reinterpret_cast<uint32_t*>(buf + st_off) = ts[d];
  };
#pragma unroll
  for (int d = 0; d < D; ++d) {
    tv[d] = bld16(xrs, toff + d * XS);
    ts[d] = bld4(srs, tsoff + d * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[d][q] = ldw16<NTW>(wp + wofs[q] + d * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_all_loads();  // the item's scale rows are in LDS
  __builtin_amdgcn_sched_barrier(0);
  put(tl, 0);
  __syncthreads();
  const int last = nkb - 1;
  auto step = [&](int kb, int d) {
    // step kb + 2's token codes and scales, issued first: slot d held step
    // kb's, which went to LDS in step kb - 1
    const int nk = min(kb + D, last);
    tv[d] = bld16(xrs, toff + nk * XS);
    ts[d] = bld4(srs, tsoff + nk * 4);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* tb = tl + (kb & 1) * STEP;
    uint4 x0, x1;
    x0 = *reinterpret_cast<const uint4*>(tb + tmx_lds_off<A4>(r, g));
    if (!A4) x1 = *reinterpret_cast<const uint4*>(tb + tmx_lds_off<A4>(r, 4 + g));
    const uint32_t xsb = tb[16 * XS + r * 4 + g];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = mfma_f4xa<A4>(w[d][q], ls[lofs[q] + kb * 4], x0, x1, xsb, acc[q]);
    __builtin_amdgcn_sched_barrier(0);
    put(tl + ((kb + 1) & 1) * STEP, (d + 1) % D);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[d][q] = ldw16<NTW>(wp + wofs[q] + nk * kPkBlock);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
#pragma unroll
  for (int d = 0; d < D; ++d) step(d, d);
  for (int kb0 = D; kb0 < nkb; kb0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(kb0 + d, d);
  }
}

// The 32 act values of one token row and one 32-feature group, spread as 8
// values over the four lanes r, r + 16, r + 32, r + 48 (features 4g + v and
// 16 + 4g + v): MX-quantise them (block amax over the four lanes) and store
// the lane's two runs of four codes at byte offsets o0 and o1 of `qrs` (4
// E4M3 bytes each, or with A4 2 bytes of E2M1 pairs), and the block's scale
// byte at `soff` of `srs` (lanes with g != 0 pass an out-of-range offset).
template <bool A4>
__device__ __forceinline__ void quant_store_act(const float (&a)[8], __amdgpu_buffer_rsrc_t qrs,
                                                uint32_t o0, uint32_t o1,
                                                __amdgpu_buffer_rsrc_t srs, uint32_t soff) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(a[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  if constexpr (A4) {
    const uint32_t b = mxfp4_scale_byte(amax);
    const float inv = mx_inv_scale(b);
    bst2(qrs, o0, pack_e2m1x4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv));
    bst2(qrs, o1, pack_e2m1x4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv));
    bst1(srs, soff, b);
  } else {
    const uint32_t b = mxfp8_scale_byte(amax);
    const float inv = mxfp8_inv_scale(b);
    bst4(qrs, o0, pack_e4m3x4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv));
    bst4(qrs, o1, pack_e4m3x4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv));
    bst1(srs, soff, b);
  }
}

// GEMM1 + SwiGLU + act quantisation, W4A8 (or W4A4 with A4), decode shape.
// Items and LDS as in gemm1_decode_kernel; the 32-feature group of an item
// is exactly one MX block of act. TL: token tiles through LDS
// (stream_block_a8_lds, D = 2), after the scale blocks in the dynamic LDS.
// KH (per-wave token loads only): K halves as in gemm1_decode_items; the
// second-half wave's sums reach the first through its own scale block.
template <int D, bool TL, bool A4, bool KH = false>
__device__ __forceinline__ void gemm1_decode_a8_items(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const int32_t* __restrict__ units, const int32_t* __restrict__ counters,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ sorted_slot, int T, int H,
    int I, int Kp, ActArgs actf, uint8_t* __restrict__ actq, uint8_t* __restrict__ acts,
    uint8_t* lds_scales, XcdItems xi) {
  static_assert(!KH || !TL, "K halves of the MX stream use per-wave token loads");
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int groups = I >> 5;
  const int ipc = KH ? 2 * groups : groups;  // items per unit
  const size_t wrow = static_cast<size_t>(H) >> 1, srow = static_cast<size_t>(H) >> 5;
  const int nkb = KH ? H >> 8 : H >> 7;  // K steps per item
  const int blk = 32 * static_cast<int>(srow);
  const int blkp = lds_block_bytes(blk);
  uint8_t* my = lds_scales + wave_index() * 2 * blkp;
  const uint32_t HB = A4 ? static_cast<uint32_t>(H) / 2 : static_cast<uint32_t>(H);  // x row bytes
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xq, static_cast<uint32_t>(static_cast<size_t>(T) * HB));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(xs, static_cast<uint32_t>(static_cast<size_t>(T) * srow));
  const uint32_t wofs[4] = {0u, static_cast<uint32_t>(I * wrow), static_cast<uint32_t>(16 * wrow),
                            static_cast<uint32_t>((I + 16) * wrow)};
  const uint32_t lofs[4] = {0u, static_cast<uint32_t>(blkp), static_cast<uint32_t>(16 * srow),
                            static_cast<uint32_t>(blkp + 16 * srow)};
  const uint32_t srow_a = static_cast<uint32_t>(I) >> 5;
  uint8_t* tl = lds_scales + 4 * 2 * blkp;
  const int tt = static_cast<int>(threadIdx.x);
  for (int item = xi.first; item < xi.end; item += xi.step) {
    const int u = item / ipc;
    const int ig = item - u * ipc;
    const int kh = KH ? ig & 1 : 0;  // which half of K
    const int f0 = (KH ? ig >> 1 : ig) * 32;
    const int4 ui = reinterpret_cast<const int4*>(units)[u];
    const int e = ui.x, r0 = ui.y, nrows = ui.z;
    const size_t row0 = static_cast<size_t>(e) * 2 * I + f0;
    const uint8_t* sg = s13 + row0 * srow;
    // the slot numbers go out with the scale-row loads (one round trip): the
    // lane's row, and the thread's row of the block's token tile (TL: codes
    // for t < NC, scales for the next 16 threads)
    const int slot = sorted_slot[r0 + min(r, nrows - 1)];
    constexpr int NC = tok_mx_code_threads<A4>();
    const int rr_t = tt < NC ? (A4 ? tt >> 2 : tt >> 3) : tt - NC;
    const int slot_t = TL ? sorted_slot[r0 + min(rr_t, nrows - 1)] : 0;
    {
      uint8_t* const dst[2] = {my, my + blkp};
      const uint8_t* const src[2] = {sg, sg + static_cast<size_t>(I) * srow};
      wave_copy_to_lds<2, 8>(dst, src, blk);
    }
    const uint8_t* wp = w13 + row0 * wrow + r * 64 + g * 16;  // packed layout
    const bool valid = r < nrows;
    const uint32_t tok = static_cast<uint32_t>(slot / Kp);
    const uint32_t xoff = valid ? tok * HB + g * 16 : kNoRow;
    const uint32_t soff = valid ? tok * static_cast<uint32_t>(srow) + g : kNoRow;
    f32x4_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto run = [&](auto ntw) {
      if constexpr (TL) {
        // this thread's row of the block's token tile: codes (t < NC) or scales
        const uint32_t ttok = static_cast<uint32_t>(slot_t / Kp);
        const bool tv_ok = rr_t < nrows;
        const uint32_t toff =
            tt < NC && tv_ok ? ttok * HB + (A4 ? (tt & 3) : (tt & 7)) * 16 : kNoRow;
        const uint32_t tsoff =
            tt >= NC && tt < NC + 16 && tv_ok ? ttok * static_cast<uint32_t>(srow) : kNoRow;
        stream_block_a8_lds<decltype(ntw)::value, A4>(wp, wofs, my + r * srow + g, lofs, nkb, xrs, toff,
                                                      srs, tsoff, tl, acc);
      } else {
        const int kk = kh * nkb;  // this half's first K step
        stream_block_a8<decltype(ntw)::value, D, A4>(
            wp + static_cast<size_t>(kk) * kPkBlock, wofs, my + r * srow + g + kk * 4, lofs, nkb, xrs,
            xoff + static_cast<uint32_t>(kk) * tok_step_bytes<A4>(), srs,
            soff + static_cast<uint32_t>(kk) * 4u, acc);
      }
    };
    // weights read once in this call (the expert's only unit): non-temporal
    if (counts[e] <= 16) run(BoolC<true>{}); else run(BoolC<false>{});
    if constexpr (KH) {
      // the second half's sums to the first-half wave, through the second
      // wave's scale block (free after its stream); first half + second half
      float* part = reinterpret_cast<float*>(lds_scales + (wave_index() | 1) * 2 * blkp);
      if (kh) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) part[(t * 4 + i) * kWave + lane] = acc[t][i];
      }
      __syncthreads();
      if (!kh) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] += part[(t * 4 + i) * kWave + lane];
      }
      __syncthreads();  // the next item's scale copy overwrites the sums
      if (kh) continue;
    }
    // lane (r, g): features f0 + 16h + 4g + v of token row r0 + r
    float a[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) a[4 * h + v] = act_apply(acc[2 * h][v], acc[2 * h + 1][v], actf);
    // act codes: I bytes per row (E4M3) or I / 2 (E2M1 pairs)
    const uint32_t IB = A4 ? static_cast<uint32_t>(I) / 2 : static_cast<uint32_t>(I);
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(actq + static_cast<size_t>(r0) * IB, static_cast<uint32_t>(nrows) * IB);
    const __amdgpu_buffer_rsrc_t ars =
        make_rsrc(acts + static_cast<size_t>(r0) * srow_a, static_cast<uint32_t>(nrows) * srow_a);
    const uint32_t e0 = static_cast<uint32_t>(r) * I + f0 + 4 * g;  // element index of a[0]
    const uint32_t o0 = A4 ? e0 / 2 : e0;
    quant_store_act<A4>(a, qrs, o0, o0 + (A4 ? 8 : 16), ars,
                        g == 0 ? static_cast<uint32_t>(r) * srow_a + (f0 >> 5) : kNoRow);
  }
}

// Four blocks per CU (four waves per SIMD) for the per-wave token path at
// ring depth <= 2: its K-half instance would otherwise take the kernel to
// 133 registers a lane, one wave per SIMD fewer.
template <int D, bool TL, bool A4>
__global__ __launch_bounds__(kGemmBlock, (TL || D > 2) ? 1 : 4) void gemm1_decode_a8_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const int32_t* __restrict__ units, const int32_t* __restrict__ counters,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ sorted_slot, int T, int H,
    int I, int Kp, ActArgs actf, uint8_t* __restrict__ actq, uint8_t* __restrict__ acts,
    int res_xcd) {
  extern __shared__ uint8_t lds_scales[];
  const int P = counters[kCtrNumU] * (I >> 5);  // (unit, 32-feature group) pairs
  if constexpr (!TL) {
    // a partial last round as K halves, as in gemm1_decode_kernel (the sums
    // of 16 floats a lane fit the second wave's two scale blocks)
    if ((H & 511) == 0 && (H >> 8) % D == 0 && res_xcd > 0 &&
        2 * lds_block_bytes(H) >= 16 * kWave * 4) {
      const int per = (((P + 7) >> 3) + 3) & ~3;  // pairs per XCD, as xcd_items
      const int nfull = ((per >> 2) / res_xcd) * res_xcd;  // blocks of whole rounds
      const int left = per - 4 * nfull;
      const int gx = static_cast<int>(gridDim.x) >> 3;
      if (nfull > 0 && left > 0 && left / 2 <= gx - nfull) {
        const int xcd = static_cast<int>(blockIdx.x) & 7, lb = static_cast<int>(blockIdx.x) >> 3;
        const int lo = xcd * per, endp = min(lo + per, P);
        XcdItems xi;
        xi.step = 1 << 30;  // one item per wave
        if (lb < nfull) {
          xi.first = lo + 4 * lb + wave_index();
          xi.end = endp;
          gemm1_decode_a8_items<D, TL, A4>(xq, xs, w13, s13, units, counters, counts, sorted_slot, T,
                                           H, I, Kp, actf, actq, acts, lds_scales, xi);
        } else {  // K-half items are numbered 2 * pair + half
          xi.first = 2 * (lo + 4 * nfull + 2 * (lb - nfull)) + wave_index();
          xi.end = 2 * endp;
          gemm1_decode_a8_items<D, TL, A4, true>(xq, xs, w13, s13, units, counters, counts,
                                                 sorted_slot, T, H, I, Kp, actf, actq, acts,
                                                 lds_scales, xi);
        }
        return;
      }
    }
  }
  gemm1_decode_a8_items<D, TL, A4>(xq, xs, w13, s13, units, counters, counts, sorted_slot, T, H, I,
                                   Kp, actf, actq, acts, lds_scales, xcd_items(P));
}

// Token tiles through LDS (stream_block_lds) pay off once chunks carry
// several rows: on MI355X they took the T512 E256 H7168 GEMMs from 925 / 518
// to 692 / 414 us and the Zipf-routed T256 EP decode GEMM1 from 68 to 50 us,
// but cost 1% at the T64 E896 decode (about one row per expert), where the
// per-step barrier buys nothing. Chosen by the average rows per local expert
// (T K' / E', known on the host), and only with a two-step ring.
static bool token_tiles_in_lds(const GemmArgs& a, int ring) {
  return ring == 2 && static_cast<long>(a.T) * a.Kp >= 2L * a.Ep;
}

// Blocks of a kernel that one XCD holds at once (an eighth of the chip),
// from the occupancy the runtime reports for its registers and LDS; 0 if
// a query fails. Cached per (device, kernel, LDS bytes).
static int resident_blocks_per_xcd(const void* kernel, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, kernel, lds);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  int res = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kGemmBlock, lds) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    res = per_cu * cus / 8;
  cache.emplace(key, res);
  return res;
}

// One block per four items, at most kMaxGrid, a multiple of 8 (xcd_items).
static int grid_for(long items) {
  long blocks = (items + 3) / 4;
  if (blocks < 8) blocks = 8;
  if (blocks > kMaxGrid) blocks = kMaxGrid;
  return static_cast<int>((blocks + 7) / 8 * 8);
}

hipError_t launch_gemm1(const GemmArgs& a, hipStream_t st) {
  if (a.a8) return a.B <= 32 ? launch_gemm1_a8(a, st) : launch_gemm1_tiled_a8(a, st);
  if (a.B <= 32) {
    // B = 32: the 32-row chunk table (chunks of more than 16 rows run both
    // sub-tiles per weight load); B = 16: the 16-row units
    const bool c32 = a.B == 32;
    const int32_t* units = c32 ? a.vinfo : a.units16;
    const int ctr = c32 ? kCtrNumV : kCtrNumU;
    const int d = ring_depth(a.H / 128);
    const bool tl = token_tiles_in_lds(a, d);
    const bool kh = a.H % 512 == 0;  // K-half items possible
    // grid for the 16-feature items (the larger count)
    const int grid = grid_for(static_cast<long>(c32 ? a.kmax_v : a.max_units16) * (a.I / 16));
    // per wave: the gate and up scale blocks of a 32-feature item (H bytes
    // each; a 16-feature item's half-size blocks fit in the same space)
    size_t lds = static_cast<size_t>(4) * 2 * lds_block_bytes(a.H) +
                 (tl ? 2 * (c32 ? tok_lds_step<2>() : tok_lds_step<1>()) : 0);
    if (kh && tl && !c32) {  // two token sub-tiles and 16-feature scale blocks
      const size_t lds_kh = static_cast<size_t>(4) * 2 * lds_block_bytes(a.H / 2) + 2 * tok_lds_step<2>();
      if (lds_kh > lds) lds = lds_kh;
    }
#define MOE_G1D(DD, NS, TL)                                                                       \
  hipLaunchKernelGGL((gemm1_decode_kernel<DD, NS, TL>), dim3(grid), dim3(kGemmBlock), lds, st,      \
                     a.x, a.w13, a.s13, units, ctr, a.counters, a.counts, a.sorted_slot, a.T, a.H,   \
                     a.I, a.Kp, a.act_fn, a.act,                                                   \
                     kh ? resident_blocks_per_xcd(reinterpret_cast<const void*>(                     \
                              gemm1_decode_kernel<DD, NS, TL>), lds) : 0)
    if (c32) {
      if (tl) MOE_G1D(2, 2, true); else if (d == 2) MOE_G1D(2, 2, false); else MOE_G1D(1, 2, false);
    } else {
      if (tl) MOE_G1D(2, 1, true); else if (d == 2) MOE_G1D(2, 1, false); else MOE_G1D(1, 1, false);
    }
#undef MOE_G1D
    return hipGetLastError();
  }
  return launch_gemm1_tiled(a, st);
}

hipError_t launch_gemm2(const GemmArgs& a, hipStream_t st) {
  if (a.a8) return launch_gemm2_gated_mx(a, st);
  if (a.I <= kResidentMaxI) return launch_gemm2_gated(a, st);
  const int nkb2 = a.I / 128;
  if (nkb2 == 4) {  // I = 512: the stream, then the generic tiled dense kernel
    hipLaunchKernelGGL(gemm2_stream_kernel<4>, dim3(kStreamGrid), dim3(kGemmBlock), 0, st, a.act,
                       a.w2, a.s2, a.units16, a.counters, a.counts, a.H, a.I, a.y);
  } else {
    const bool c32 = a.B == 32;
    const int32_t* units = c32 ? a.vinfo : a.units16;
    const int ctr = c32 ? kCtrNumV : kCtrNumU;
    const int gsplit = grid_for(static_cast<long>(c32 ? a.kmax_v : a.max_units16) * (a.H / 64));
    const int d = ring_depth(a.I / 128);
    const bool tl = token_tiles_in_lds(a, d);
    const size_t lds2 = static_cast<size_t>(4) * lds_block_bytes(2 * a.I) +
                        (tl ? 2 * (c32 ? tok_lds_step<2>() : tok_lds_step<1>()) : 0);
#define MOE_G2D(DD, NS, TL)                                                                     \
  hipLaunchKernelGGL((gemm2_split_kernel<DD, NS, TL>), dim3(gsplit), dim3(kGemmBlock), lds2, st, \
                     a.act, a.w2, a.s2, units, ctr, a.counters, a.counts, a.H, a.I, a.y)
    if (c32) {
      if (tl) MOE_G2D(2, 2, true); else if (d == 2) MOE_G2D(2, 2, false); else MOE_G2D(1, 2, false);
    } else {
      if (tl) MOE_G2D(2, 1, true); else if (d == 2) MOE_G2D(2, 1, false); else MOE_G2D(1, 1, false);
    }
#undef MOE_G2D
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_gemm2_dense_tiled(a, st);
}

template <bool A4>
static hipError_t launch_gemm1_mx(const GemmArgs& a, hipStream_t st) {
  const int grid = grid_for(static_cast<long>(a.max_units16) * (a.I / 32));
  const int ring = ring_depth(a.H / 128) >= 2 ? 2 : 1;
  const bool tl = token_tiles_in_lds(a, ring);
  const size_t lds =
      static_cast<size_t>(4) * 2 * lds_block_bytes(a.H) + (tl ? 2 * tok_mx_lds_step<A4>() : 0);
  uint8_t* actq = reinterpret_cast<uint8_t*>(a.act);
#define MOE_G1A(DD, TL)                                                                          \
  hipLaunchKernelGGL((gemm1_decode_a8_kernel<DD, TL, A4>), dim3(grid), dim3(kGemmBlock), lds, st, \
                     a.xq, a.xs, a.w13, a.s13, a.units16, a.counters, a.counts, a.sorted_slot, a.T,  \
                     a.H, a.I, a.Kp, a.act_fn, actq, a.act_scales,                                \
                     (!(TL) && a.H % 512 == 0)                                                    \
                         ? resident_blocks_per_xcd(                                                \
                               reinterpret_cast<const void*>(gemm1_decode_a8_kernel<DD, TL, A4>), lds) \
                         : 0)
  if (tl) {
    MOE_G1A(2, true);
  } else {
    switch (ring_depth(a.H / 128)) {
      case 4: MOE_G1A(4, false); break;
      case 3: MOE_G1A(3, false); break;
      case 2: MOE_G1A(2, false); break;
      default: MOE_G1A(1, false); break;
    }
  }
#undef MOE_G1A
  return hipGetLastError();
}

hipError_t launch_gemm1_a8(const GemmArgs& a, hipStream_t st) {
  return a.a4 ? launch_gemm1_mx<true>(a, st) : launch_gemm1_mx<false>(a, st);
}

}  // namespace moe
