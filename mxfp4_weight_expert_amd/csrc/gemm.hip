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
// Tile: one wave computes 16 weight rows (16 gate + 16 up rows for GEMM1)
// against up to NT*16 rows of one chunk, weights on the MFMA M side and
// tokens on N (the decode shape: few tokens per expert). K is walked in
// steps of 128: lane (r = lane%16, g = lane/16) loads 16 bytes of weight row
// r = 32 E2M1 codes = exactly one E8M0 scale group, decodes them to bf16 with
// the hardware scaled convert (exact), and feeds four 16x16x32 MFMAs. The
// K order inside a step is permuted identically for both operands (lane
// group g, MFMA j <-> K = 128*kb + 32*g + 8*j + [0, 8)), which leaves the dot
// products unchanged and keeps every weight load a contiguous 16 bytes.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kGemmBlock = 256;  // 4 waves, one item each
constexpr int kMaxGrid = 256 * 8;
}  // namespace

template <int NT>
__global__ __launch_bounds__(kGemmBlock) void gemm1_tn_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ s13, const int32_t* __restrict__ vinfo,
    const int32_t* __restrict__ counters, const int32_t* __restrict__ sorted_slot, int H, int I,
    int Kp, float limit, uint16_t* __restrict__ act) {
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int ftiles = I >> 4;
  const int nitems = counters[kCtrNumV] * ftiles;
  const size_t wrow = static_cast<size_t>(H) >> 1, srow = static_cast<size_t>(H) >> 5;
  const int nkb = H >> 7;
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < nitems; item += gridDim.x * 4) {
    const int v = item / ftiles;
    const int ft = item - v * ftiles;
    const int4 vi = reinterpret_cast<const int4*>(vinfo)[v];
    const int e = vi.x, r0 = vi.y, nrows = vi.z;
    const int nsub = (nrows + 15) >> 4;
    const size_t grow = static_cast<size_t>(e) * 2 * I + ft * 16 + r;
    const uint8_t* wg = w13 + grow * wrow + g * 16;
    const uint8_t* wu = wg + static_cast<size_t>(I) * wrow;
    const uint8_t* sg = s13 + grow * srow + g;
    const uint8_t* su = sg + static_cast<size_t>(I) * srow;
    const uint16_t* xr[NT];
    bool tv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int ri = n * 16 + r;
      tv[n] = ri < nrows;
      const int tok = tv[n] ? sorted_slot[r0 + ri] / Kp : 0;
      xr[n] = x + static_cast<size_t>(tok) * H + g * 32;
    }
    f32x4_t accg[NT], accu[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      accg[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accu[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int kb = 0; kb < nkb; ++kb) {
      const uint4 wgv = ld16(wg + kb * 64);
      const uint4 wuv = ld16(wu + kb * 64);
      const float scg = e8m0_scale_operand(sg[kb * 4]);
      const float scu = e8m0_scale_operand(su[kb * 4]);
      const uint32_t gw[4] = {wgv.x, wgv.y, wgv.z, wgv.w};
      const uint32_t uw[4] = {wuv.x, wuv.y, wuv.z, wuv.w};
      bf16x8_t a_g[4], a_u[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a_g[j] = decode_fp4x8(gw[j], scg);
        a_u[j] = decode_fp4x8(uw[j], scu);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n < nsub) {
          uint4 xv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xv[j] = tv[n] ? ld16(xr[n] + kb * 128 + j * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            accg[n] = mfma16x16x32(a_g[j], as_bf16x8(xv[j]), accg[n]);
            accu[n] = mfma16x16x32(a_u[j], as_bf16x8(xv[j]), accu[n]);
          }
        }
      }
    }
    // Lane (r, g) holds features 4g..4g+3 of this tile for chunk row n*16 + r.
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int ri = n * 16 + r;
      if (n < nsub && ri < nrows) {
        const float o0 = swiglu(accg[n][0], accu[n][0], limit);
        const float o1 = swiglu(accg[n][1], accu[n][1], limit);
        const float o2 = swiglu(accg[n][2], accu[n][2], limit);
        const float o3 = swiglu(accg[n][3], accu[n][3], limit);
        uint2 pk;
        pk.x = pack_bf16x2(o0, o1);
        pk.y = pack_bf16x2(o2, o3);
        *reinterpret_cast<uint2*>(act + static_cast<size_t>(r0 + ri) * I + ft * 16 + g * 4) = pk;
      }
    }
  }
}

// GEMM2, tokens on N. DENSE selects the item list (gate tiles vs chunks) and
// the gate value this kernel runs on.
template <int NT, bool DENSE>
__global__ __launch_bounds__(kGemmBlock) void gemm2_tn_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int32_t* __restrict__ items,
    const int32_t* __restrict__ counters, int H, int I, uint16_t* __restrict__ y) {
  const int path = counters[kCtrGate];
  if (path != (DENSE ? 1 : 0)) return;  // the unselected path: zero items
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int htiles = H >> 4;
  const int nitems = (DENSE ? counters[kCtrGate + 3] : counters[kCtrNumV]) * htiles;
  const size_t wrow = static_cast<size_t>(I) >> 1, srow = static_cast<size_t>(I) >> 5;
  const int nkb = I >> 7;
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < nitems; item += gridDim.x * 4) {
    const int v = item / htiles;
    const int ht = item - v * htiles;
    const int4 vi = reinterpret_cast<const int4*>(items)[v];
    const int e = vi.x, r0 = vi.y, nrows = vi.z;
    const int nsub = (nrows + 15) >> 4;
    const size_t grow = static_cast<size_t>(e) * H + ht * 16 + r;
    const uint8_t* wp = w2 + grow * wrow + g * 16;
    const uint8_t* sp = s2 + grow * srow + g;
    const uint16_t* ar[NT];
    bool tv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int ri = n * 16 + r;
      tv[n] = ri < nrows;
      ar[n] = act + static_cast<size_t>(r0 + (tv[n] ? ri : 0)) * I + g * 32;
    }
    f32x4_t acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < nkb; ++kb) {
      const uint4 wv = ld16(wp + kb * 64);
      const float sc = e8m0_scale_operand(sp[kb * 4]);
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
      bf16x8_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = decode_fp4x8(ww[j], sc);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n < nsub) {
          uint4 av[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            av[j] = tv[n] ? ld16(ar[n] + kb * 128 + j * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[n] = mfma16x16x32(a[j], as_bf16x8(av[j]), acc[n]);
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int ri = n * 16 + r;
      if (n < nsub && ri < nrows) {
        uint2 pk;
        pk.x = pack_bf16x2(acc[n][0], acc[n][1]);
        pk.y = pack_bf16x2(acc[n][2], acc[n][3]);
        *reinterpret_cast<uint2*>(y + static_cast<size_t>(r0 + ri) * H + ht * 16 + g * 4) = pk;
      }
    }
  }
}

static int grid_for(long items) {
  long blocks = (items + 3) / 4;
  if (blocks < 1) blocks = 1;
  return static_cast<int>(blocks < kMaxGrid ? blocks : kMaxGrid);
}

hipError_t launch_gemm1(const GemmArgs& a, hipStream_t st) {
  const int grid = grid_for(static_cast<long>(a.kmax_v) * (a.I / 16));
#define MOE_G1(N)                                                                              \
  hipLaunchKernelGGL(gemm1_tn_kernel<N>, dim3(grid), dim3(kGemmBlock), 0, st, a.x, a.w13, a.s13, \
                     a.vinfo, a.counters, a.sorted_slot, a.H, a.I, a.Kp, a.limit, a.act)
  switch (a.B) {
    case 16: MOE_G1(1); break;
    case 32: MOE_G1(2); break;
    case 64: MOE_G1(4); break;
    case 128: MOE_G1(8); break;
    default: MOE_G1(16); break;
  }
#undef MOE_G1
  return hipGetLastError();
}

hipError_t launch_gemm2(const GemmArgs& a, hipStream_t st) {
  const int gsplit = grid_for(static_cast<long>(a.kmax_v) * (a.H / 16));
  const int gdense = grid_for(static_cast<long>(a.max_dense_tiles) * (a.H / 16));
  switch (a.B) {
    case 16:
      hipLaunchKernelGGL((gemm2_tn_kernel<1, false>), dim3(gsplit), dim3(kGemmBlock), 0, st, a.act,
                         a.w2, a.s2, a.vinfo, a.counters, a.H, a.I, a.y);
      break;
    case 32:
      hipLaunchKernelGGL((gemm2_tn_kernel<2, false>), dim3(gsplit), dim3(kGemmBlock), 0, st, a.act,
                         a.w2, a.s2, a.vinfo, a.counters, a.H, a.I, a.y);
      break;
    case 64:
      hipLaunchKernelGGL((gemm2_tn_kernel<4, false>), dim3(gsplit), dim3(kGemmBlock), 0, st, a.act,
                         a.w2, a.s2, a.vinfo, a.counters, a.H, a.I, a.y);
      break;
    case 128:
      hipLaunchKernelGGL((gemm2_tn_kernel<8, false>), dim3(gsplit), dim3(kGemmBlock), 0, st, a.act,
                         a.w2, a.s2, a.vinfo, a.counters, a.H, a.I, a.y);
      break;
    default:
      hipLaunchKernelGGL((gemm2_tn_kernel<16, false>), dim3(gsplit), dim3(kGemmBlock), 0, st,
                         a.act, a.w2, a.s2, a.vinfo, a.counters, a.H, a.I, a.y);
      break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((gemm2_tn_kernel<kDenseMT / 16, true>), dim3(gdense), dim3(kGemmBlock), 0, st,
                     a.act, a.w2, a.s2, a.dense_tiles, a.counters, a.H, a.I, a.y);
  return hipGetLastError();
}

}  // namespace moe
