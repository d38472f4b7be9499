// Internal device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mxfp4.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kMaxTopK = 32;
constexpr int kMaxShared = 8;
constexpr int kMaxExperts = 2048;  // E + S
// Slots per sort range (one wave each) above kSmallSlots. Smaller ranges
// give the count and scatter kernels more waves and the range scan more
// per-range counts: at 524k slots, with the multi-block range scan, 2048 /
// 1024 / 512 took 78 / 67 / 70 us for the whole sort on MI355X.
constexpr int kRangeSlots = 1024;
constexpr int kSmallSlots = 8192;  // up to this many slots the sort runs in one block
constexpr int kGateTau = 64;       // dense GEMM2 when rows >= kGateTau * touched experts
constexpr int kDenseMT = 128;      // dense-path row tile
constexpr int kResidentMaxI = 384;  // largest I whose bf16 dense-path act tile stays in LDS
constexpr int kMaxTiledK = 8192;   // largest H and I (LDS budget of the tiled GEMMs)
constexpr int kCounterWords = 64;
constexpr int kCtrNumV = 0;
constexpr int kCtrNumU = 1;        // 16-row units (decode GEMM work list)
constexpr int kCtrGate = 4;        // 4 words: path, U, R, dense tiles

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
// Two floats -> packed bf16 (lo in bits 0..15), round to nearest even, with
// the gfx950 packed convert (one instruction, no branches).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// -------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }
// Wave index in the block, as a value the compiler knows is wave-uniform
// (kept in scalar registers; buffer descriptors built from it stay scalar).
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Lanes below this one set in mask.
__device__ __forceinline__ int popc_below(uint64_t mask) {
  uint32_t lo = static_cast<uint32_t>(mask), hi = static_cast<uint32_t>(mask >> 32);
  return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
    uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}
// Wave-wide max of 64-bit values by DPP row shifts and row broadcasts (no
// LDS traffic); every lane receives the result.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int lo = static_cast<int>(static_cast<uint32_t>(v));
  const int hi = static_cast<int>(static_cast<uint32_t>(v >> 32));
  const uint32_t nlo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false));
  const uint32_t nhi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false));
  const uint64_t n = (static_cast<uint64_t>(nhi) << 32) | nlo;
  return n > v ? n : v;
}
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8  -> lane 15 of each row: row max
  v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 -> rows 1, 3
  v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 -> rows 2, 3: lane 63 = wave max
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 63);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Inclusive prefix sum across the wave on DPP lane moves (no LDS round
// trips; the sort's expert scan pass went 3.5 -> 2.5 us at the T64 decode
// on MI355X against cross-lane shuffles): shifts by 1, 2, 4 and 8 lanes
// within each row of 16 (lanes whose source falls before the row start add
// 0), then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into rows
// 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// ------------------------------------------------------------- MX decoding
// E8M0 byte as the float scale operand of the gfx950 scaled converts.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t e) {
  return __uint_as_float(e << 23);
}

// Eight E2M1 codes (one dword, low nibble first) times 2^(e-127) -> 8 bf16.
// The products are bf16 numbers for e in [0, 252], so the conversion is exact;
// the convert takes the scale from the exponent field of its float operand.
// The packed pairs are moved as whole dwords: extracting single bf16 lanes of
// the convert's result has been seen to duplicate the low half.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_sel(uint32_t packed, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, SEL));
}
__device__ __forceinline__ bf16x8_t decode_fp4x8(uint32_t packed, float scale) {
  uint4 r;
  r.x = cvt_fp4x2_sel<0>(packed, scale);
  r.y = cvt_fp4x2_sel<1>(packed, scale);
  r.z = cvt_fp4x2_sel<2>(packed, scale);
  r.w = cvt_fp4x2_sel<3>(packed, scale);
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ MXFP8
// MXFP8 block scale of a 32-element block with maximum magnitude amax (a
// finite float): the shared exponent floor(log2(amax)) - 8 (8 = the largest
// E4M3 exponent), biased by 127 and clamped to [0, 254]; amax = 0 gives 0.
// With the exponent field e of amax this is max(e - 8, 0): subnormal and
// zero amax (e = 0) clamp to 0, and e <= 254 keeps the result <= 246.
__device__ __forceinline__ uint32_t mxfp8_scale_byte(float amax) {
  const uint32_t e = (__float_as_uint(amax) >> 23) & 0xffu;
  return e >= 8u ? e - 8u : 0u;
}
// 2^(127 - b) for a scale byte b <= 246: a normal float, so v * factor is
// exact for every element of the block (|v * factor| < 512).
__device__ __forceinline__ float mxfp8_inv_scale(uint32_t b) {
  return __uint_as_float((254u - b) << 23);
}
// Four scaled values -> four E4M3 codes (byte i = value i), round to nearest
// even, saturating at +-448 (the hardware convert itself does not saturate).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const float m = 448.0f;
  a = fminf(fmaxf(a, -m), m);
  b = fminf(fmaxf(b, -m), m);
  c = fminf(fmaxf(c, -m), m);
  d = fminf(fmaxf(d, -m), m);
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return static_cast<uint32_t>(p);
}

// Scaled MFMA, 16x16 output, K = 128: A = 16 rows of E2M1 codes (lane group
// g holds K [32g, 32g + 32) of its row, 16 bytes, low nibble first), B = 16
// columns of E4M3 codes (lane group g holds K [16g, 16g + 16) in x0 and
// K [64 + 16g, 64 + 16g + 16) in x1). Scales are E8M0 bytes in the low byte
// of sa / sb: lane (i, g) gives the scale of row / column i for the K block
// [32g, 32g + 32). D lane (i, g), register v = row 4g + v, column i.
__device__ __forceinline__ f32x4_t mfma_f4xf8(const uint4& w, uint32_t sa, const uint4& x0,
                                              const uint4& x1, uint32_t sb, f32x4_t c) {
  const i32x8_t a = {static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                     static_cast<int>(w.w), 0, 0, 0, 0};
  const i32x8_t b = {static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                     static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                     static_cast<int>(x1.z), static_cast<int>(x1.w)};
  // format codes: 4 = E2M1 (A), 0 = E4M3 (B)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, static_cast<int>(sa), 0,
                                                          static_cast<int>(sb));
}

// Scaled MFMA, 16x16 output, K = 128, both operands E2M1 (W4A4): A as in
// mfma_f4xf8; B = 16 columns of E2M1 codes in the same layout as A (lane
// group g holds K [32g, 32g + 32) of its column, 16 bytes, low nibble
// first), with its E8M0 scale byte for K block g in sb.
__device__ __forceinline__ f32x4_t mfma_f4xf4(const uint4& w, uint32_t sa, const uint4& x,
                                              uint32_t sb, f32x4_t c) {
  const i32x8_t a = {static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                     static_cast<int>(w.w), 0, 0, 0, 0};
  const i32x8_t b = {static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
                     static_cast<int>(x.w), 0, 0, 0, 0};
  // format codes: 4 = E2M1 for both operands
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, static_cast<int>(sa), 0,
                                                          static_cast<int>(sb));
}

// The scaled MFMA of the MX-activation paths: W4A8 (E4M3 tokens in x0, x1)
// or, with A4, W4A4 (E2M1 tokens in x0; x1 unused).
template <bool A4>
__device__ __forceinline__ f32x4_t mfma_f4xa(const uint4& w, uint32_t sa, const uint4& x0,
                                             const uint4& x1, uint32_t sb, f32x4_t c) {
  if constexpr (A4)
    return mfma_f4xf4(w, sa, x0, sb, c);
  else
    return mfma_f4xf8(w, sa, x0, x1, sb, c);
}

// ------------------------------------------------------------------ MXFP4
// MXFP4 block scale of a 32-element block with maximum magnitude amax: the
// shared exponent floor(log2(amax)) - 2 (2 = the largest E2M1 exponent,
// 6 = 1.5 * 2^2), biased by 127 and clamped to [0, 254]: max(e - 2, 0) with
// e the exponent field of amax (<= 252 for finite amax).
__device__ __forceinline__ uint32_t mxfp4_scale_byte(float amax) {
  const uint32_t e = (__float_as_uint(amax) >> 23) & 0xffu;
  return e >= 2u ? e - 2u : 0u;
}
// E2M1 code of v (already divided by the block scale): the nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6}, a tie to the even code, |v| > 6 saturating to
// 6; the sign bit is v's, so a negative value rounding to zero gives 8 (-0).
// Each comparison threshold is a midpoint between neighbours: strict where
// the lower neighbour's code is even, non-strict where the upper one's is.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float m = fabsf(v);
  const uint32_t c = static_cast<uint32_t>(m > 0.25f) + static_cast<uint32_t>(m >= 0.75f) +
                     static_cast<uint32_t>(m > 1.25f) + static_cast<uint32_t>(m >= 1.75f) +
                     static_cast<uint32_t>(m > 2.5f) + static_cast<uint32_t>(m >= 3.5f) +
                     static_cast<uint32_t>(m > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}
// Four scaled values -> four E2M1 codes in 16 bits, value i in nibble i.
__device__ __forceinline__ uint32_t pack_e2m1x4(float a, float b, float c, float d) {
  return e2m1_code(a) | (e2m1_code(b) << 4) | (e2m1_code(c) << 8) | (e2m1_code(d) << 12);
}
// 2^(127 - b) for an MX scale byte b <= 253: a normal float, so v * factor is
// exact wherever the result matters (an underflow there rounds to a zero code
// either way).
__device__ __forceinline__ float mx_inv_scale(uint32_t b) {
  return __uint_as_float((254u - b) << 23);
}

// ---------------------------------------------------------------- activation
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Activation of the GEMM1 epilogue on the gate half g and the up half u.
//   kind MOE_ACT_SWIGLU: silu(g) * u, with the clamp when limit > 0 (the
//     Shape-template page, section 4; the Marlin page's swiglu limit);
//   kind MOE_ACT_SITU: beta tanh(g / beta) sigmoid(g) * lb tanh(u / lb), the
//     SiTU activation of the same section (printed there for beta = 4,
//     lb = 25 as 2 tanh(g/4)(1 + tanh(g/2)) * 25 tanh(u/25)).
// The reciprocals come from the host.
struct ActArgs {
  int kind;
  float limit;
  float beta, inv_beta, lb, inv_lb;
};
__device__ __forceinline__ float swiglu(float g, float u, float limit);
__device__ __forceinline__ float act_apply(float g, float u, const ActArgs& a) {
  if (a.kind == MOE_ACT_SITU) {
    const float sg = 1.0f / (1.0f + __expf(-g));
    return (a.beta * tanhf(g * a.inv_beta) * sg) * (a.lb * tanhf(u * a.inv_lb));
  }
  return swiglu(g, u, a.limit);
}

__device__ __forceinline__ float swiglu(float g, float u, float limit) {
  if (limit > 0.0f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  return silu_f(g) * u;
}

// Plain 16-byte global load through the vector path.
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// N consecutive dwords (1 <= N <= 4) at a 4-byte aligned address: exactly 4N
// bytes, e.g. one weight row's I/32 scale bytes. The array's last row ends
// the caller's buffer, so a wider load there would read past its end.
template <int N>
__device__ __forceinline__ void ld_dwords(const void* p, uint32_t (&d)[N]) {
  static_assert(N >= 1 && N <= 4, "1 to 4 dwords");
  const uint32_t* q = static_cast<const uint32_t*>(p);
#pragma unroll
  for (int i = 0; i < N; ++i) d[i] = q[i];
}

// 16-byte weight load. NT = true marks it non-temporal: for weights that
// this layer call reads exactly once (their expert's rows fit one work
// unit), so the streamed bytes do not displace reusable lines in L2 and the
// Infinity Cache. On MI355X that took the decode GEMMs from 5.5 to 6.1 TB/s;
// where an expert spans several units its weights are re-read and the plain
// (cached) load is kept.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ldw16(const void* p) {
  if constexpr (NT)
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  else
    return *reinterpret_cast<const uint4*>(p);
}
// A compile-time bool carried as a value (selects a template instance from
// a run-time test in a generic lambda).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// ------------------------------------------------------------ buffer access
// Raw buffer loads and stores return zero / are dropped for offsets at or
// beyond the descriptor's size, without touching memory.
// Packed weight layout (moe_mxfp4_prepack): 1 KB blocks of 16 rows x 64
// bytes, the blocks of a 16-row group in K order. A lane's 16-byte piece at
// byte b of row r (r % 16 = rr, 16-aligned row r0 = r - rr) sits at
// (r0 / 16) * nks * 1024 + (b / 64) * 1024 + rr * 64 + b % 64, nks = row
// bytes / 64: a 16-row group is nks KB, a 64-byte K step 1 KB.
constexpr uint32_t kPkBlock = 1024;

constexpr uint32_t kNoRow = 0x80000000u;  // buffer offset beyond any operand (< 2 GiB)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Wave-uniform part of the offset in an SGPR (soff).
__device__ __forceinline__ uint4 bld16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), r,
                                         off, 0, 0);
}
__device__ __forceinline__ void bst16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), r,
                                         off, soff, 0);
}
// Non-temporal 16-byte buffer store (cache-policy operand 2), for data
// written once and read once much later, past what the caches hold.
__device__ __forceinline__ void bst16nt(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), r,
                                         off, 0, 2);
}
__device__ __forceinline__ void bst8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) uint32_t, v), r,
                                        off, 0, 0);
}
__device__ __forceinline__ void bst4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void bst2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v), r, off, 0, 0);
}
__device__ __forceinline__ void bst1(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(v), r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bld1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bld1s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bld4s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}

}  // namespace moe
