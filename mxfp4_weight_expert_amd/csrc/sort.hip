// Deterministic device sort of token slots into per-expert rows, the B-row
// chunk table, and the device-side GEMM2 path gate.
//
// Sources: "SGLang CUTLASS MoE", section 1 (prepare_moe_input: per-expert
// offsets, the row permutation and its inverse); "Generalizing the Kimi-K3.1
// MXFP4 decode MoE kernel with a Shape template", sections 1 and 5 (chunks
// of at most BlockN rows -- "virtual experts" -- bounded by
// E + T*top-k/BlockN; rows of an expert ranked in token order so the result
// does not depend on atomic order); "Device-side gating of the MoE GEMM2
// path", sections 1-2 (one wave reads the sorted table and picks Dense or
// Split; the other path's kernels launch and find zero items).
//
// Up to kSmallSlots slots: one block does everything (histogram, scan,
// chunk table, placement, gate). Beyond that the slots t*K' + k are cut into
// ranges of kRangeSlots, one wave each:
//   count:   per-range expert histograms (LDS atomics: order-free counts);
//   scan:    per-expert exclusive scan over ranges, expert offsets, chunks,
//            and the gate (one block);
//   scatter: each wave walks its range in slot order, 64 slots at a time.
// Placement ranks equal experts inside a wave by ballot/popcount (a wave
// multisplit), so rows follow slot order exactly.
#include "common.h"
#include "kernels.h"

namespace moe {

// Block of 1024 threads: from per-expert row counts (LDS), write counts,
// offsets (exclusive scan, offsets[Ep] = R), the chunk table in expert-major
// order and the chunk count, the same table for 16-row units (the decode
// GEMMs' work list), and the GEMM2 gate: rows R and touched experts U, Dense
// iff R >= kGateTau * U (or forced); on Dense the per-expert 128-row tile
// list, experts in order. Gate word: {path, U, R, dense tiles (0 on Split)}.
// One pass over the experts and one barrier for all of it. If next_row is
// given, it receives offsets[e]. Every thread of the block must call it.
__device__ void block_scan_and_gate(const int32_t* s_cnt, int Ep, int B, int force_path,
                                    int32_t* counts, int32_t* offsets, int32_t* vinfo,
                                    int32_t* units16, int32_t* counters, int32_t* dense_tiles,
                                    int32_t* next_row) {
  __shared__ int32_t s_w[5][16];  // per wave: rows, chunks, units, dense tiles, touched experts
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int per = (Ep + 1023) / 1024;
  const int e0 = tid * per;
  int rows = 0, chunks = 0, units = 0, tiles = 0, touched = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < Ep) {
      const int n = s_cnt[e];
      rows += n;
      chunks += (n + B - 1) / B;
      units += (n + 15) / 16;
      tiles += (n + kDenseMT - 1) / kDenseMT;
      touched += n > 0;
    }
  }
  const int rin = wave_incl_scan(rows), cin = wave_incl_scan(chunks), uin = wave_incl_scan(units);
  const int tin = wave_incl_scan(tiles), gin = wave_incl_scan(touched);
  if (lane == kWave - 1) {
    s_w[0][w] = rin;
    s_w[1][w] = cin;
    s_w[2][w] = uin;
    s_w[3][w] = tin;
    s_w[4][w] = gin;
  }
  __syncthreads();
  int rbase = 0, cbase = 0, ubase = 0, tbase = 0, Rt = 0, Ut = 0, ttot = 0;
  for (int j = 0; j < 16; ++j) {
    const bool before = j < w;
    rbase += before ? s_w[0][j] : 0;
    cbase += before ? s_w[1][j] : 0;
    ubase += before ? s_w[2][j] : 0;
    tbase += before ? s_w[3][j] : 0;
    Rt += s_w[0][j];
    ttot += s_w[3][j];
    Ut += s_w[4][j];
  }
  int path = (Ut > 0 && Rt >= kGateTau * Ut) ? 1 : 0;
  if (force_path == 0 || force_path == 1) path = force_path;
  int row = rbase + rin - rows, chunk = cbase + cin - chunks, unit = ubase + uin - units;
  int tile = tbase + tin - tiles;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= Ep) break;
    const int n = s_cnt[e];
    counts[e] = n;
    offsets[e] = row;
    if (next_row != nullptr) next_row[e] = row;
    for (int c = 0; c * B < n; ++c) {
      int4 v;
      v.x = e;
      v.y = row + c * B;
      v.z = min(B, n - c * B);
      v.w = c;
      reinterpret_cast<int4*>(vinfo)[chunk + c] = v;
    }
    for (int c = 0; c * 16 < n; ++c) {
      int4 v;
      v.x = e;
      v.y = row + c * 16;
      v.z = min(16, n - c * 16);
      v.w = c;
      reinterpret_cast<int4*>(units16)[unit + c] = v;
    }
    if (path == 1) {
      for (int m = 0; m * kDenseMT < n; ++m) {
        int4 v;
        v.x = e;
        v.y = row + m * kDenseMT;
        v.z = min(kDenseMT, n - m * kDenseMT);
        v.w = m;
        reinterpret_cast<int4*>(dense_tiles)[tile + m] = v;
      }
    }
    row += n;
    chunk += (n + B - 1) / B;
    unit += (n + 15) / 16;
    tile += (n + kDenseMT - 1) / kDenseMT;
  }
  if (tid == 1023) {
    offsets[Ep] = row;  // thread 1023 owns the last experts (or none): row = R
    counters[kCtrNumV] = chunk;
    counters[kCtrNumU] = unit;
  }
  if (tid == 0) {
    int4 g;
    g.x = path;
    g.y = Ut;
    g.z = Rt;
    g.w = path == 1 ? ttot : 0;
    *reinterpret_cast<int4*>(counters + kCtrGate) = g;
  }
}

// Rank 64 slots (one per lane, in slot order) among equal experts and place
// them, so rows follow slot order within each expert. next[e] (LDS) is the
// expert's next free row; the group's first lane advances it by the group
// size after every lane of the group has read it.
__device__ __forceinline__ void place_slots(int s, bool in, int e, int key_bits, int Ep,
                                            int32_t* next, int32_t* sorted_slot,
                                            int32_t* expanded_idx) {
  const int lane = lane_id();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool valid = e >= 0;
  const int key = valid ? e : Ep;  // Ep marks empty lanes
  uint64_t match = ~0ull;
  for (int b = 0; b < key_bits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = ballot(bit);
    match &= bit ? bal : ~bal;
  }
  const int rank = __popcll(match & lt);
  int base = 0;
  if (valid) base = next[e];
  __builtin_amdgcn_wave_barrier();
  if (valid) {
    const int row = base + rank;
    sorted_slot[row] = s;
    expanded_idx[s] = row;
    if (rank == 0) next[e] = base + __popcll(match);
  } else if (in) {
    expanded_idx[s] = -1;
  }
  __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------- small shapes
// Equal-expert groups among 64 slots (one per lane): each lane's match mask.
__device__ __forceinline__ uint64_t match_mask(int key, int key_bits) {
  uint64_t match = ~0ull;
  for (int b = 0; b < key_bits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = ballot(bit);
    match &= bit ? bal : ~bal;
  }
  return match;
}

constexpr int kSmallWaves = 16;
constexpr int kSmallGroups = kSmallSlots / (kSmallWaves * kWave);  // 64-slot groups per wave

// One block of 16 waves. Wave w owns slots [w*rw, (w+1)*rw) (rw a multiple of
// 64): it counts its experts into its own 16-bit histogram (the first lane of
// each equal-expert group adds the group size: no atomics), the block scans
// the histograms per expert (wave bases) and over experts (offsets, chunk
// table), then each wave places its own slots in slot order, and the block
// runs the GEMM2 gate. Dynamic LDS: kSmallWaves * Ep 16-bit counters.
__global__ __launch_bounds__(1024) void sort_small_kernel(
    const int32_t* __restrict__ slot_expert, int nslots, int Ep, int B, int key_bits,
    int force_path, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ expanded_idx,
    int32_t* __restrict__ vinfo, int32_t* __restrict__ units16, int32_t* __restrict__ counters,
    int32_t* __restrict__ dense_tiles) {
  extern __shared__ uint16_t s_wcnt[];  // [kSmallWaves][Ep]
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts];
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = tid; i < kSmallWaves * Ep; i += 1024) s_wcnt[i] = 0;
  const int rw = ((nslots + kSmallWaves * kWave - 1) / (kSmallWaves * kWave)) * kWave;
  const int s0 = w * rw;
  int ex[kSmallGroups];
#pragma unroll
  for (int gi = 0; gi < kSmallGroups; ++gi)  // clamped, unconditional loads
    ex[gi] = slot_expert[min(s0 + gi * kWave + lane, nslots - 1)];
#pragma unroll
  for (int gi = 0; gi < kSmallGroups; ++gi) {
    const int s = s0 + gi * kWave + lane;
    if (!(gi * kWave < rw && s < nslots)) ex[gi] = -1;
  }
  __syncthreads();
  uint16_t* h = s_wcnt + w * Ep;
  uint64_t mm[kSmallGroups];  // each lane's equal-expert mask per group, kept for the placement
#pragma unroll
  for (int gi = 0; gi < kSmallGroups; ++gi) {
    mm[gi] = 0ull;
    if (gi * kWave < rw) {
      const uint64_t match = match_mask(ex[gi] >= 0 ? ex[gi] : Ep, key_bits);
      mm[gi] = match;
      if (ex[gi] >= 0 && __popcll(match & lt) == 0)
        h[ex[gi]] = static_cast<uint16_t>(h[ex[gi]] + __popcll(match));
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  // per expert: exclusive scan over the waves (in place) and the total
  for (int e = tid; e < Ep; e += 1024) {
    int run = 0;
#pragma unroll
    for (int v = 0; v < kSmallWaves; ++v) {
      const int c = s_wcnt[v * Ep + e];
      s_wcnt[v * Ep + e] = static_cast<uint16_t>(run);
      run += c;
    }
    s_cnt[e] = run;
  }
  __syncthreads();
  block_scan_and_gate(s_cnt, Ep, B, force_path, counts, offsets, vinfo, units16, counters,
                      dense_tiles, s_off);
  __syncthreads();
  // placement of this wave's slots
#pragma unroll
  for (int gi = 0; gi < kSmallGroups; ++gi) {
    if (gi * kWave < rw) {
      const int s = s0 + gi * kWave + lane;
      const int e = ex[gi];
      const bool valid = e >= 0;
      const uint64_t match = mm[gi];
      const int rank = __popcll(match & lt);
      int base = 0;
      if (valid) base = h[e];
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        const int row = s_off[e] + base + rank;
        sorted_slot[row] = s;
        expanded_idx[s] = row;
        if (rank == 0) h[e] = static_cast<uint16_t>(base + __popcll(match));
      } else if (s < nslots) {
        expanded_idx[s] = -1;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ------------------------------------------------------------ large shapes
// One wave per block (ranges spread over the CUs): range r's expert
// histogram in LDS, written range-major to range_counts[r][Ep].
__global__ __launch_bounds__(64) void sort_count_kernel(const int32_t* __restrict__ slot_expert,
                                                        int nslots, int Ep, int n_ranges,
                                                        int32_t* __restrict__ range_counts) {
  extern __shared__ int32_t lds[];
  const int lane = lane_id();
  const int r = blockIdx.x;
  int32_t* h = lds;
  for (int i = lane; i < Ep; i += kWave) h[i] = 0;
  __builtin_amdgcn_wave_barrier();
  const int s0 = r * kRangeSlots;
  const int s1 = min(nslots, s0 + kRangeSlots);
  for (int s = s0 + lane; s < s1; s += kWave) {
    const int e = slot_expert[s];
    if (e >= 0) atomicAdd(&h[e], 1);
  }
  __builtin_amdgcn_wave_barrier();
  for (int i = lane; i < Ep; i += kWave) range_counts[static_cast<size_t>(r) * Ep + i] = h[i];
}

// Per expert, the exclusive scan of its per-range counts, in place
// (range_counts [n_ranges][Ep] becomes each range's first row offset within
// the expert), and the expert's total row count into counts[e]. A block
// covers 64 experts (one per lane, so loads are coalesced across the lanes)
// and its four waves cover four quarters of the ranges: each wave sums its
// quarter, the quarters' totals are scanned in LDS, and each wave rewrites
// its quarter starting from its prefix.
__global__ __launch_bounds__(256) void sort_range_scan_kernel(int32_t* __restrict__ range_counts,
                                                              int n_ranges, int Ep,
                                                              int32_t* __restrict__ counts) {
  __shared__ int32_t s_part[4][kWave];
  const int lane = lane_id(), q = wave_index();
  const int e = blockIdx.x * kWave + lane;
  const bool live = e < Ep;
  const int ec = live ? e : Ep - 1;
  const int r_lo = n_ranges * q / 4, r_hi = n_ranges * (q + 1) / 4;
  auto at = [&](int r) -> int32_t* { return range_counts + static_cast<size_t>(r) * Ep + ec; };
  int sum = 0;
  for (int r0 = r_lo; r0 < r_hi; r0 += 32) {
    int c[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = *at(min(r0 + j, r_hi - 1));
#pragma unroll
    for (int j = 0; j < 32; ++j) sum += r0 + j < r_hi ? c[j] : 0;
  }
  s_part[q][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int k = 0; k < q; ++k) run += s_part[k][lane];
  if (q == 3 && live) counts[e] = run + sum;
  if (!live || r_lo >= r_hi) return;  // no barrier follows
  // rewrite the quarter; the next round's loads go out before this round's
  // stores (they never overlap)
  int c[32], n[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) c[j] = *at(min(r_lo + j, r_hi - 1));
  for (int r0 = r_lo; r0 < r_hi; r0 += 32) {
    const int r1 = r0 + 32;
#pragma unroll
    for (int j = 0; j < 32; ++j) n[j] = *at(min(r1 + j, r_hi - 1));
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (r0 + j < r_hi) {
        *at(r0 + j) = run;
        run += c[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = n[j];
  }
}

// One block of 1024 threads. From the per-expert totals (counts, written by
// sort_range_scan_kernel), writes counts, offsets, the chunk table and the
// chunk count, then runs the GEMM2 gate.
__global__ __launch_bounds__(1024) void sort_scan_kernel(int Ep, int B, int force_path,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ vinfo,
                                                         int32_t* __restrict__ units16,
                                                         int32_t* __restrict__ counters,
                                                         int32_t* __restrict__ dense_tiles) {
  __shared__ int32_t s_cnt[kMaxExperts];
  const int tid = threadIdx.x;
  // 1) the per-expert totals
  for (int e = tid; e < Ep; e += 1024) s_cnt[e] = counts[e];
  __syncthreads();
  // 2) expert offsets, the chunk tables and the gate
  block_scan_and_gate(s_cnt, Ep, B, force_path, counts, offsets, vinfo, units16, counters,
                      dense_tiles, nullptr);
}

__global__ __launch_bounds__(64) void sort_scatter_kernel(
    const int32_t* __restrict__ slot_expert, int nslots, int Ep, int n_ranges, int key_bits,
    const int32_t* __restrict__ range_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ expanded_idx) {
  constexpr int kGroups = kRangeSlots / kWave;
  extern __shared__ int32_t lds[];
  const int lane = lane_id();
  const int r = blockIdx.x;
  const int s0 = r * kRangeSlots;
  const int s1 = min(nslots, s0 + kRangeSlots);
  // the range's experts, all loads in flight at once (clamped index)
  int ex[kGroups];
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) ex[gi] = slot_expert[min(s0 + gi * kWave + lane, nslots - 1)];
  int32_t* next = lds;  // next free row per expert for this range
  for (int i = lane; i < Ep; i += kWave)
    next[i] = offsets[i] + range_base[static_cast<size_t>(r) * Ep + i];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int s = s0 + gi * kWave + lane;
    const bool in = s < s1;
    if (s0 + gi * kWave < s1)  // wave-uniform
      place_slots(s, in, in ? ex[gi] : -1, key_bits, Ep, next, sorted_slot, expanded_idx);
  }
}

hipError_t launch_sort_and_gate(const SortArgs& a, hipStream_t st) {
  int key_bits = 1;
  while ((1 << key_bits) <= a.Ep) ++key_bits;  // keys 0..Ep inclusive
  if (a.nslots <= kSmallSlots) {
    const size_t lds = static_cast<size_t>(kSmallWaves) * a.Ep * sizeof(uint16_t);
    hipLaunchKernelGGL(sort_small_kernel, dim3(1), dim3(1024), lds, st, a.slot_expert, a.nslots,
                       a.Ep, a.B, key_bits, a.force_path, a.counts, a.offsets, a.sorted_slot,
                       a.expanded_idx, a.vinfo, a.units16, a.counters, a.dense_tiles);
    return hipGetLastError();
  }
  const size_t lds = static_cast<size_t>(a.Ep) * sizeof(int32_t);
  hipLaunchKernelGGL(sort_count_kernel, dim3(a.n_ranges), dim3(64), lds, st, a.slot_expert, a.nslots,
                     a.Ep, a.n_ranges, a.range_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_range_scan_kernel, dim3((a.Ep + kWave - 1) / kWave), dim3(256), 0, st,
                     a.range_counts, a.n_ranges, a.Ep, a.counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(1024), 0, st, a.Ep, a.B, a.force_path,
                     a.counts, a.offsets, a.vinfo, a.units16, a.counters, a.dense_tiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(a.n_ranges), dim3(64), lds, st, a.slot_expert,
                     a.nslots, a.Ep, a.n_ranges, key_bits, a.range_counts, a.offsets,
                     a.sorted_slot, a.expanded_idx);
  return hipGetLastError();
}

}  // namespace moe
