// Row order -> fragment order of expert weight matrices and MXFP4 scale
// matrices (a byte permutation).
//
// Fragment order: 16-row blocks of the matrix, each cut into column slices of
// W bytes (64 for weights, 16 for MXFP4 scales); slice f of block b is 16W
// contiguous bytes whose 16-byte chunk L = r + 16c holds bytes [Wf + 16c, +16)
// of the block's row r.  For weights a wavefront lane L takes exactly that
// chunk as its share of a 16 x 16 x 32 matrix-core operand (row r = L%16,
// quarter c = L/16 of the slice), so the expert kernels read a whole slice
// with one 16-byte load per lane over consecutive addresses (8 full cache
// lines) instead of 16 rows x 64 bytes (16 half lines); for scales a slice is
// the 16 rows' scale bytes of four 128-deep windows, two whole lines.
#include "common.h"

namespace beam {

// One thread per 16-byte chunk of the output (writes consecutive, reads 16-byte pieces of rows); cq = W/16
// chunks per row and slice.
__global__ __launch_bounds__(256) void pack_fragments_kernel(long rows, int row_bytes, int cq,
                                                             const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  const long nch = row_bytes / 16;             // 16-byte chunks per row
  const long block_ch = 16 * nch;              // chunks per 16-row block
  const long slice_ch = 16 * cq;               // chunks per slice
  const long total = rows * nch;
  for (long d = (long)blockIdx.x * 256 + threadIdx.x; d < total; d += (long)gridDim.x * 256) {
    const long b = d / block_ch, in = d % block_ch;
    const long f = in / slice_ch;
    const int L = (int)(in % slice_ch), r = L % 16, c = L / 16;
    dst[d] = src[(b * 16 + r) * nch + cq * f + c];
  }
}

hipError_t launch_pack_fragments(long rows, int row_bytes, int slice_bytes, const void* src, void* dst,
                                 hipStream_t stream) {
  const long total = rows * (row_bytes / 16);
  const int grid = (int)std::min<long>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_fragments_kernel, dim3(grid), dim3(256), 0, stream, rows, row_bytes, slice_bytes / 16,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst));
  return hipGetLastError();
}

}  // namespace beam
