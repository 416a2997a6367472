// Operand preparation of the FP8 batched GEMM (MATE FlashInfer-API page, section "GEMM", bmm_fp8):
// its B is (batch, k, n) with n contiguous, while the matrix-core loop reads both operands K-major.
// One HBM-bound pass turns each batch's (k, n) byte matrix into (n, k).
#include "internal.h"

namespace fp8g {
namespace kernels {

constexpr int kTr = 128;  // tile edge in bytes: whole 128-byte lines on both sides

// dst[b][c][r] = src[b][r][c] for a rows x cols byte matrix per batch; rows and cols are multiples
// of 16. A 256-lane workgroup moves one 128x128 tile: 16-byte loads of source rows into LDS (four
// per lane), then each lane gathers 16 bytes of a source column and writes them as 16 bytes of a
// destination row (four times). Tiles cover whole cache lines, so no line is fetched twice.
__global__ void __launch_bounds__(256)
transpose_bytes_kernel(const uint8_t* __restrict__ src, int rows, int cols, uint8_t* __restrict__ dst) {
  __shared__ uint8_t tile[kTr][kTr + 4];
  const int64_t plane = (int64_t)rows * cols;
  const uint8_t* s = src + blockIdx.z * plane;
  uint8_t* d = dst + blockIdx.z * plane;
  const int r0 = blockIdx.y * kTr, c0 = blockIdx.x * kTr;
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * 32 + (t >> 3), c = (t & 7) * 16;
    if (r0 + r < rows && c0 + c < cols) {
      const uint4 v = *reinterpret_cast<const uint4*>(s + (int64_t)(r0 + r) * cols + c0 + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(&tile[r][c + 4 * q]) = w[q];
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = it * 32 + (t >> 3), r = (t & 7) * 16;  // destination row c0 + c, bytes [r0 + r, +16)
    if (c0 + c < cols && r0 + r < rows) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < 16; ++q) w[q >> 2] |= (uint32_t)tile[r + q][c] << (8 * (q & 3));
      *reinterpret_cast<uint4*>(d + (int64_t)(c0 + c) * rows + r0 + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace kernels

hipError_t launch_transpose_bytes(const uint8_t* src, int batch, int rows, int cols, uint8_t* dst,
                                  hipStream_t stream) {
  const dim3 grid((cols + kernels::kTr - 1) / kernels::kTr, (rows + kernels::kTr - 1) / kernels::kTr, batch);
  hipLaunchKernelGGL(kernels::transpose_bytes_kernel, grid, dim3(256), 0, stream, src, rows, cols, dst);
  return hipGetLastError();
}

}  // namespace fp8g
