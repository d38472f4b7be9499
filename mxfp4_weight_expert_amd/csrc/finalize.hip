// Weighted per-token finalize: out[t] = sum over columns k of w[t,k] *
// y[row(t,k)], skipping columns whose row is -1, in ascending k with fp32
// accumulation, then rounded to bf16. One block per token, no atomics.
//
// Sources: "SGLang CUTLASS MoE", section 5 (apply_shuffle_mul_sum restores
// token order, multiplies by the routing weight and sums, in one kernel);
// "Generalizing the Kimi-K3.1 MXFP4 decode MoE kernel with a Shape template",
// section 5 (the deferred finalize skips slots whose expanded index is -1).
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void finalize_kernel(const uint16_t* __restrict__ y,
                                                       const int32_t* __restrict__ expanded_idx,
                                                       const float* __restrict__ slot_w, int Kp,
                                                       int H, uint16_t* __restrict__ out) {
  __shared__ int32_t s_row[kMaxTopK + kMaxShared];
  __shared__ float s_w[kMaxTopK + kMaxShared];
  const int t = blockIdx.x;
  if (threadIdx.x < Kp) {
    s_row[threadIdx.x] = expanded_idx[static_cast<size_t>(t) * Kp + threadIdx.x];
    s_w[threadIdx.x] = slot_w[static_cast<size_t>(t) * Kp + threadIdx.x];
  }
  __syncthreads();
  const int nvec = H >> 3;  // 8 bf16 per 16-byte vector
  for (int c = threadIdx.x; c < nvec; c += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < Kp; ++k) {
      const int row = s_row[k];
      if (row < 0) continue;
      const float w = s_w[k];
      const uint4 v = ld16(y + static_cast<size_t>(row) * H + c * 8);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w * __uint_as_float(d[q] << 16);
        acc[2 * q + 1] += w * __uint_as_float(d[q] & 0xffff0000u);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * H + c * 8) = o;
  }
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(a.T), dim3(256), 0, st, a.y, a.expanded_idx, a.slot_w,
                     a.Kp, a.H, a.out);
  return hipGetLastError();
}

}  // namespace moe
