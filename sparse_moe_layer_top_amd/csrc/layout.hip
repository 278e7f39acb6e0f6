// Row order -> fragment order of expert weight matrices (a byte permutation).
//
// Fragment order: 16-row blocks of the matrix, each cut into 64-byte column
// slices; slice f of block b is 1024 contiguous bytes whose 16-byte chunk
// L = r + 16c holds bytes [64f + 16c, +16) of the block's row r.  A wavefront
// lane L takes exactly that chunk as its share of a 16 x 16 x 32 matrix-core
// operand (row r = L%16, quarter c = L/16 of the slice), so the expert kernels
// read a whole slice with one 16-byte load per lane over consecutive addresses
// (8 full cache lines) instead of 16 rows x 64 bytes (16 half lines).
#include "common.h"

namespace beam {

// One thread per 16-byte chunk of the output (writes consecutive, reads 16-byte pieces of rows).
__global__ __launch_bounds__(256) void pack_weights_kernel(long rows, int row_bytes, const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst) {
  const long nch = row_bytes / 16;             // 16-byte chunks per row
  const long block_ch = 16 * nch;              // chunks per 16-row block
  const long total = rows * nch;
  for (long d = (long)blockIdx.x * 256 + threadIdx.x; d < total; d += (long)gridDim.x * 256) {
    const long b = d / block_ch, in = d % block_ch;
    const long f = in / 64;
    const int L = (int)(in % 64), r = L % 16, c = L / 16;
    dst[d] = src[(b * 16 + r) * nch + 4 * f + c];
  }
}

hipError_t launch_pack_weights(long rows, int row_bytes, const void* src, void* dst, hipStream_t stream) {
  const long total = rows * (row_bytes / 16);
  const int grid = (int)std::min<long>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(grid), dim3(256), 0, stream, rows, row_bytes,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst));
  return hipGetLastError();
}

}  // namespace beam
