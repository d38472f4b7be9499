// Routing: top-k with softmax weights (or given ids/weights), the local
// expert map with expert offset, and the fused sigmoid shared-expert append.
//
// Sources: "Generalizing the Kimi-K3.1 MXFP4 decode MoE kernel with a Shape
// template", section 5 (ids outside [expert_offset, expert_offset + E) and
// the masked id -1 get no row); "SGLang MoE shared-expert optimisation",
// the append kernel after the change (shared column s: expert N_BASE + s,
// weight sigmoid(float(bf16 logit)) * scale, computed in registers).
#include "common.h"
#include "kernels.h"

namespace moe {

// Total order on float logits, larger first: map the bits so that unsigned
// comparison follows the float order. -0.0 is folded into +0.0 first so the
// two compare equal (the tie then goes to the lower id). Every NaN maps to
// 0, below -inf (0x007FFFFF): a NaN logit ranks last, NaNs by lower id.
__device__ __forceinline__ uint32_t order_bits(float f) {
  if (__builtin_isnan(f)) return 0u;
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorder_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ void write_shared_columns(const uint16_t* shared_logits, int t, int topk,
                                                     int S, int E, float shared_scale,
                                                     int32_t* slot_expert, float* slot_w) {
  const int lane = lane_id();
  const int Kp = topk + S;
  if (lane >= topk && lane < Kp) {
    const int s = lane - topk;
    const float lg = bf16_to_f32(shared_logits[static_cast<size_t>(t) * S + s]);
    const float sig = 1.0f / (1.0f + expf(-lg));
    slot_expert[static_cast<size_t>(t) * Kp + lane] = E + s;
    slot_w[static_cast<size_t>(t) * Kp + lane] = sig * shared_scale;
  }
}

// Wave-wide maximum of a 32-bit value (DPP row shifts and row broadcasts;
// lane 63 ends with the maximum, which every lane receives).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// One wave per token. The token's logits become 64-bit keys (ordered logit
// << 32 | ~id), NPL per lane (E_global <= 64 * NPL); larger key = larger
// logit, equal logits: lower id. A NaN's key is ~id alone: above the empty
// key 0 and below every number's. The top-k keys are found in three passes
// over registers and a little LDS:
//  1. thr: the largest 32-bit ordered logit that at least topk lane maxima
//     reach (radix select, most significant bit first, one ballot per bit).
//     At least topk keys have a logit >= thr, so every top-k key does;
//  2. the candidates (non-empty keys with logit >= thr; typically topk plus
//     a few) are packed into the wave's LDS row in ballot order;
//  3. each candidate's rank is the number of larger candidates (all 64 bits:
//     ties of equal logits rank by id), and the key of rank r goes to lane r.
// About 400 instructions per token against about 1,300 for topk rounds of a
// wave-wide maximum. More than 64 candidates (many logits equal at the
// threshold, or mostly NaN rows) take the round-based selection: every lane
// keeps its four largest keys below a ceiling, sorted; each of topk rounds
// finds the wave's largest head key (a 32-bit DPP maximum over the ordered
// logits, and over the ids only when several lanes tie) and pops it from its
// lane; a lane whose list runs empty rebuilds it from its keys below the key
// it gave last. Either way lane r ends with the r-th largest key.
template <int NPL>
__global__ __launch_bounds__(256) void route_logits_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ shared_logits, int T, int Eg,
    int topk, int S, int E, int expert_offset, float shared_scale, int32_t* __restrict__ route_ids,
    int32_t* __restrict__ slot_expert, float* __restrict__ slot_w) {
  __shared__ uint64_t s_key[4][kWave];  // per wave: the candidates, then the selection
  const int lane = lane_id();
  const int wv = static_cast<int>(threadIdx.x) >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * Eg;
  // Unconditional loads (clamped index) so all of them are in flight at once.
  float lv[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) lv[j] = row[min(lane + kWave * j, Eg - 1)];
  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int idx = lane + kWave * j;
    const uint64_t k = (static_cast<uint64_t>(order_bits(lv[j])) << 32) | static_cast<uint32_t>(~idx);
    key[j] = idx < Eg ? k : 0ull;  // 0 is below every real key
  }
  // 1. the threshold logit
  uint64_t lmax = 0ull;
#pragma unroll
  for (int j = 0; j < NPL; ++j) lmax = max_u64(lmax, key[j]);
  const uint32_t lhi = static_cast<uint32_t>(lmax >> 32);
  uint32_t thr = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = thr | (1u << b);
    if (__popcll(ballot(lhi >= c)) >= topk) thr = c;
  }
  // 2. the candidates
  uint64_t bal[NPL];
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    bal[j] = ballot(key[j] != 0ull && static_cast<uint32_t>(key[j] >> 32) >= thr);
    ncand += __popcll(bal[j]);
  }
  uint64_t mine = 0;  // lane r keeps the r-th selected key
  if (ncand <= kWave) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint64_t* row_lds = s_key[wv];
    int base = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      if ((bal[j] >> lane) & 1ull) row_lds[base + __popcll(bal[j] & lt)] = key[j];
      base += __popcll(bal[j]);
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t ck = lane < ncand ? row_lds[lane] : 0ull;
    // 3. ranks (candidate keys are distinct: the ids differ)
    int rank = 0;
    for (int i = 0; i < ncand; ++i) {
      const uint64_t ki =
          (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ck >> 32), i))) << 32) |
          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ck), i));
      rank += ki > ck ? 1 : 0;
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < ncand && rank < topk) row_lds[rank] = ck;
    __builtin_amdgcn_wave_barrier();
    mine = lane < topk ? row_lds[lane] : 0ull;
  } else {
    // the lane's four largest keys below `ceil`, descending (0 = none)
    uint64_t L[4];
    auto build = [&](uint64_t ceil) {
#pragma unroll
      for (int i = 0; i < 4; ++i) L[i] = 0ull;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        uint64_t x = key[j] < ceil ? key[j] : 0ull;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t hi = max_u64(L[i], x);
          x = min_u64(L[i], x);
          L[i] = hi;
        }
      }
    };
    build(~0ull);
    for (int r = 0; r < topk; ++r) {
      const uint32_t h0 = static_cast<uint32_t>(L[0] >> 32), l0 = static_cast<uint32_t>(L[0]);
      const uint32_t mh = wave_max_u32(h0);
      const bool cand = h0 == mh;
      const uint64_t bl = ballot(cand);
      uint32_t ml;
      if (__popcll(bl) == 1) {
        ml = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(l0), __builtin_ctzll(bl)));
      } else {
        ml = wave_max_u32(cand ? l0 : 0u);
      }
      const uint64_t m = (static_cast<uint64_t>(mh) << 32) | ml;
      if (lane == r) mine = m;
      if (L[0] == m) {  // the one lane holding the winner (keys are distinct)
        L[0] = L[1];
        L[1] = L[2];
        L[2] = L[3];
        L[3] = 0ull;
        if (L[0] == 0ull) build(m);
      }
    }
  }
  const bool sel = lane < topk;
  const float lg = unorder_bits(static_cast<uint32_t>(mine >> 32));
  const int id = static_cast<int>(~static_cast<uint32_t>(mine));
  // A selected NaN (only when fewer than topk logits are numbers) gets
  // weight 0; infinities follow IEEE arithmetic.
  const float lmax_f = __shfl(lg, 0, kWave);
  const float ex = (sel && !__builtin_isnan(lg)) ? expf(lg - lmax_f) : 0.0f;
  const float sum = wave_sum_f(ex);
  const int Kp = topk + S;
  if (sel) {
    route_ids[static_cast<size_t>(t) * topk + lane] = id;
    const int loc = id - expert_offset;
    slot_expert[static_cast<size_t>(t) * Kp + lane] = (loc >= 0 && loc < E) ? loc : -1;
    slot_w[static_cast<size_t>(t) * Kp + lane] = ex / sum;
  }
  write_shared_columns(shared_logits, t, topk, S, E, shared_scale, slot_expert, slot_w);
}

// Ids mode: one wave per token, lanes over the K' columns.
__global__ __launch_bounds__(256) void route_ids_kernel(
    const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
    const uint16_t* __restrict__ shared_logits, int T, int topk, int S, int E, int expert_offset,
    float shared_scale, int32_t* __restrict__ route_ids, int32_t* __restrict__ slot_expert,
    float* __restrict__ slot_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int Kp = topk + S;
  if (lane < topk) {
    const size_t i = static_cast<size_t>(t) * topk + lane;
    const int id = topk_ids[i];
    route_ids[i] = id;
    const int loc = id - expert_offset;
    slot_expert[static_cast<size_t>(t) * Kp + lane] = (id >= 0 && loc >= 0 && loc < E) ? loc : -1;
    slot_w[static_cast<size_t>(t) * Kp + lane] = topk_w[i];
  }
  write_shared_columns(shared_logits, t, topk, S, E, shared_scale, slot_expert, slot_w);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const dim3 grid((a.T + 3) / 4), block(256);
  if (a.logits == nullptr) {
    hipLaunchKernelGGL(route_ids_kernel, grid, block, 0, st, a.topk_ids, a.topk_w, a.shared_logits,
                       a.T, a.topk, a.S, a.E, a.expert_offset, a.shared_scale, a.route_ids,
                       a.slot_expert, a.slot_w);
    return hipGetLastError();
  }
#define MOE_ROUTE(N)                                                                        \
  hipLaunchKernelGGL(route_logits_kernel<N>, grid, block, 0, st, a.logits, a.shared_logits, a.T, \
                     a.Eg, a.topk, a.S, a.E, a.expert_offset, a.shared_scale, a.route_ids,       \
                     a.slot_expert, a.slot_w)
  const int npl = (a.Eg + kWave - 1) / kWave;
  if (npl <= 1) MOE_ROUTE(1);
  else if (npl <= 2) MOE_ROUTE(2);
  else if (npl <= 4) MOE_ROUTE(4);
  else if (npl <= 8) MOE_ROUTE(8);
  else if (npl <= 14) MOE_ROUTE(14);
  else if (npl <= 16) MOE_ROUTE(16);
  else MOE_ROUTE(32);
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
