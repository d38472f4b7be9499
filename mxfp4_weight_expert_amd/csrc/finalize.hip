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
// One wave per block: a block covers 64 16-byte vectors (1 KB) of a token's
// output row, so H / 512 blocks per token leave no lane idle (256-thread
// blocks left a quarter of every second block idle at H = 3584: 730 against
// 690 us at 32k tokens on MI355X).
constexpr int kFinBlock = 64;

// Grid: T x nblk blocks; block (t, b) covers 16-byte vectors [64b, 64b + 64)
// of token t's output row. The wave first compacts the token's valid columns
// (row >= 0) into LDS, keeping their order, so the accumulation loop has no
// branches and issues its row loads back to back. Every row of y is read
// exactly once per call, so the loads are non-temporal (at 32k tokens y is
// 3.8 GB, far past what the caches hold: 836 -> 768 us on MI355X).
__global__ __launch_bounds__(kFinBlock) void finalize_kernel(const uint16_t* __restrict__ y,
                                                       const int32_t* __restrict__ expanded_idx,
                                                       const float* __restrict__ slot_w, int Kp,
                                                       int H, int nblk, uint16_t* __restrict__ out) {
  __shared__ int32_t s_row[kMaxTopK + kMaxShared];
  __shared__ float s_w[kMaxTopK + kMaxShared];
  __shared__ int s_n;
  const int t = blockIdx.x / nblk;
  const int b = blockIdx.x - t * nblk;
  if (threadIdx.x < kWave) {
    const int k = threadIdx.x;
    const int row = k < Kp ? expanded_idx[static_cast<size_t>(t) * Kp + k] : -1;
    const bool valid = row >= 0;
    const uint64_t m = ballot(valid);
    if (valid) {
      const int pos = popc_below(m);
      s_row[pos] = row;
      s_w[pos] = slot_w[static_cast<size_t>(t) * Kp + k];
    }
    if (k == 0) s_n = __popcll(m);
  }
  __syncthreads();
  const int c = b * kFinBlock + threadIdx.x;  // 16-byte vector index in the row
  if (c >= (H >> 3)) return;
  const int n = s_n;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4& v, float w) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += w * __uint_as_float(d[q] << 16);
      acc[2 * q + 1] += w * __uint_as_float(d[q] & 0xffff0000u);
    }
  };
  const uint16_t* yc = y + static_cast<size_t>(c) * 8;
  int k = 0;
  for (; k + 8 <= n; k += 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ldw16<true>(yc + static_cast<size_t>(s_row[k + u]) * H);
#pragma unroll
    for (int u = 0; u < 8; ++u) add(v[u], s_w[k + u]);
  }
  // the last 1..7 columns: all loads issued before the first add (one load
  // at a time, each waiting for the one before, had cost the Zipf-routed
  // EP decode, whose tokens keep 0..16 local columns, about 1 us)
  if (k < n) {
    uint4 v[7];
#pragma unroll
    for (int u = 0; u < 7; ++u)
      if (k + u < n) v[u] = ldw16<true>(yc + static_cast<size_t>(s_row[k + u]) * H);
#pragma unroll
    for (int u = 0; u < 7; ++u)
      if (k + u < n) add(v[u], s_w[k + u]);
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * H + c * 8) = o;
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t st) {
  const int nblk = ((a.H >> 3) + kFinBlock - 1) / kFinBlock;
  hipLaunchKernelGGL(finalize_kernel, dim3(a.T * nblk), dim3(kFinBlock), 0, st, a.y, a.expanded_idx,
                     a.slot_w, a.Kp, a.H, nblk, a.out);
  return hipGetLastError();
}

}  // namespace moe
