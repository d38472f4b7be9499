// MXFP8 quantisation of the layer input x for the W4A8 path: bf16 [T, H] ->
// E4M3 codes [T, H] and one E8M0 scale per 32 consecutive elements [T, H/32].
//
// Source: "Generalizing the Kimi-K3.1 MXFP4 decode MoE kernel with a Shape
// template", section 2 (token activations in MXFP8: 8-bit elements with one
// 8-bit power-of-two scale per 32 along K). The scale rule follows the OCP
// microscaling format: shared exponent floor(log2(amax)) - 8, elements
// rounded to nearest even in E4M3 with saturation; every step is exact in
// fp32, so the codes are the correctly rounded ones.
#include "common.h"
#include "kernels.h"

namespace moe {

// One thread per 32-element block; block i covers x[32i, 32i + 32) of the
// flattened [T, H] array, whose scale is xs[i].
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

hipError_t launch_quant_x(const uint16_t* x, int T, int H, uint8_t* xq, uint8_t* xs,
                          hipStream_t st) {
  const int nblk = T * (H / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_x_kernel, dim3((nblk + 255) / 256), dim3(256), 0, st, x, nblk, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
