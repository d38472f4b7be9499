// MX quantisation of the layer input x for the W4A8 and W4A4 paths:
// bf16 [T, H] -> element codes and one E8M0 scale per 32 consecutive
// elements [T, H/32]. MXFP8: E4M3 codes [T, H] (one byte each); MXFP4: E2M1
// codes [T, H/2] (two per byte, the even element in the low nibble).
//
// Sources: "Generalizing the Kimi-K3.1 MXFP4 decode MoE kernel with a Shape
// template", section 2 (token activations in MXFP8: 8-bit elements with one
// 8-bit power-of-two scale per 32 along K); "SGLang CUTLASS MoE", section 6
// (FP4 activations). The scale rule follows the OCP microscaling format:
// shared exponent floor(log2(amax)) - emax (8 for E4M3, 2 for E2M1),
// elements rounded to nearest even with saturation; every step is exact in
// fp32, so the codes are the correctly rounded ones.
#include "common.h"
#include "kernels.h"

namespace moe {

// One thread per 32-element block; block i covers x[32i, 32i + 32) of the
// flattened [T, H] array, whose scale is xs[i]. A4: MXFP4, else MXFP8.
template <bool A4>
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* __restrict__ x, int nblk,
                                                      uint8_t* __restrict__ xq,
                                                      uint8_t* __restrict__ xs) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  const uint16_t* src = x + static_cast<size_t>(i) * 32;
  uint4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = ld16(src + k * 8);
  float f[32];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t d[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[8 * k + 2 * j] = __uint_as_float(d[j] << 16);
      f[8 * k + 2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(f[k]));
  if constexpr (A4) {
    const uint32_t b = mxfp4_scale_byte(amax);
    const float inv = mx_inv_scale(b);
    uint32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      q[k] = pack_e2m1x4(f[8 * k] * inv, f[8 * k + 1] * inv, f[8 * k + 2] * inv,
                         f[8 * k + 3] * inv) |
             (pack_e2m1x4(f[8 * k + 4] * inv, f[8 * k + 5] * inv, f[8 * k + 6] * inv,
                          f[8 * k + 7] * inv)
              << 16);
    *reinterpret_cast<uint4*>(xq + static_cast<size_t>(i) * 16) = make_uint4(q[0], q[1], q[2], q[3]);
    xs[i] = static_cast<uint8_t>(b);
  } else {
    const uint32_t b = mxfp8_scale_byte(amax);
    const float inv = mxfp8_inv_scale(b);
    uint32_t q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      q[k] = pack_e4m3x4(f[4 * k] * inv, f[4 * k + 1] * inv, f[4 * k + 2] * inv, f[4 * k + 3] * inv);
    uint4* dst = reinterpret_cast<uint4*>(xq + static_cast<size_t>(i) * 32);
    dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
    dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
    xs[i] = static_cast<uint8_t>(b);
  }
}

hipError_t launch_quant_x(const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* xs, bool a4,
                          hipStream_t st) {
  const int nblk = T * (H / 32);
  if (nblk == 0) return hipSuccess;
  if (a4)
    hipLaunchKernelGGL(quant_x_kernel<true>, dim3((nblk + 255) / 256), dim3(256), 0, st, x, nblk, xq, xs);
  else
    hipLaunchKernelGGL(quant_x_kernel<false>, dim3((nblk + 255) / 256), dim3(256), 0, st, x, nblk, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
