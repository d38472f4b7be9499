// Weight prepack: row-major nibble-packed matrix -> blocks of 16 rows x 64
// bytes (1 KB), the blocks of one 16-row group in K order. Only moves bytes.
#include "common.h"
#include "kernels.h"

namespace moe {

// One thread per 16-byte piece of the source, read coalesced; piece
// (row, c) with c = byte / 16 goes to the block of (row / 16, c / 4).
__global__ __launch_bounds__(256) void prepack_kernel(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst, int64_t rows,
                                                      int64_t row_pieces) {
  const int64_t n = rows * row_pieces;
  const int64_t nks = row_pieces >> 2;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = i / row_pieces;
    const int64_t c = i - row * row_pieces;
    const int64_t j = ((row >> 4) * nks + (c >> 2)) * 64 + (row & 15) * 4 + (c & 3);
    dst[j] = src[i];
  }
}

hipError_t launch_prepack(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t row_bytes,
                          hipStream_t st) {
  const int64_t pieces = rows * (row_bytes >> 4);
  int64_t blocks = (pieces + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(prepack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), rows,
                     row_bytes >> 4);
  return hipGetLastError();
}

}  // namespace moe
