// Producers of the GEMM's a operand: the 1x128 E4M3 activation quantiser and the fused
// add-RMSNorm with 1x128 quantisation (MATE FlashInfer-API page, section "norm":
// fused_add_rmsnorm_fp8_block_quant; the quantised rows are the a operand of the section "GEMM"
// calls with a 1x128 a_scale).
//
// Both are HBM-bound row kernels: one workgroup per row, 16-lane teams per 128-wide block.
#include "internal.h"
#include "quant_common.h"

namespace fp8g {
namespace kernels {

constexpr int kQuantThreads = 256;  // 16 teams of 16 lanes

// Scale element of (row, block) in the requested layout: K-major (rows, nblk) or MN-major (nblk, rows).
__device__ __forceinline__ int64_t scale_index(int row, int blk, int rows, int nblk, bool mn_major) {
  return mn_major ? (int64_t)blk * rows + row : (int64_t)row * nblk + blk;
}

__global__ void __launch_bounds__(kQuantThreads)
quantize_1x128_kernel(const uint16_t* __restrict__ x, int rows, int cols, uint8_t* __restrict__ out,
                      float* __restrict__ scale_out, bool mn_major) {
  const int row = blockIdx.x;
  const int nblk = cols / 128;
  const int sub = threadIdx.x & 15;
  const uint16_t* xrow = x + (int64_t)row * cols;
  uint8_t* orow = out + (int64_t)row * cols;
  for (int blk = threadIdx.x >> 4; blk < nblk; blk += kQuantThreads / 16) {
    const int col = blk * 128 + sub * 8;
    float v[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(xrow + col), v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = team16_max(amax);
    quant_store_8(v, amax, orow + col, scale_out + scale_index(row, blk, rows, nblk, mn_major), sub == 0);
  }
}

// residual <- bf16(input + residual) (FP32 sum, round-to-nearest-even), in place;
// normed_out <- bf16(r * (1 / sqrt(mean(r^2) + eps)) * weight), r the new residual row, all FP32
// (the mean is an FP32 sum of squares divided by hidden; square root and reciprocal are IEEE);
// out, scale_out <- the 1x128 quantisation of the normed_out values.
// Each lane reads back only the residual elements it wrote itself, and writes normed_out only where
// it read input, so normed_out may be input and the row needs no barrier between the two passes
// beyond the one of the block-wide sum.
__global__ void __launch_bounds__(kQuantThreads)
fused_add_rmsnorm_quant_kernel(const uint16_t* input, uint16_t* __restrict__ residual,
                               const uint16_t* __restrict__ weight, float eps, int rows, int hidden,
                               uint16_t* normed_out, uint8_t* __restrict__ out,
                               float* __restrict__ scale_out, bool mn_major) {
  __shared__ float wave_sum[kQuantThreads / 64];
  const int row = blockIdx.x;
  const int nblk = hidden / 128;
  const int sub = threadIdx.x & 15;
  const int64_t base = (int64_t)row * hidden;
  float ss = 0.0f;
  for (int blk = threadIdx.x >> 4; blk < nblk; blk += kQuantThreads / 16) {
    const int col = blk * 128 + sub * 8;
    float a[8], b[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(input + base + col), a);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(residual + base + col), b);
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      packed[i] = pack_bf16x2(a[2 * i] + b[2 * i], a[2 * i + 1] + b[2 * i + 1]);
      const float r0 = bf16_bits_to_float(packed[i] & 0xFFFFu), r1 = bf16_bits_to_float(packed[i] >> 16);
      ss = __builtin_fmaf(r0, r0, ss);
      ss = __builtin_fmaf(r1, r1, ss);
    }
    *reinterpret_cast<uint4*>(residual + base + col) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = ss;
  __syncthreads();
  float total = 0.0f;
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) total += wave_sum[w];
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(total, (float)hidden) + eps));
  for (int blk = threadIdx.x >> 4; blk < nblk; blk += kQuantThreads / 16) {
    const int col = blk * 128 + sub * 8;
    float r[8], w[8], v[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(residual + base + col), r);  // this lane's own writes
    unpack_bf16x8(*reinterpret_cast<const uint4*>(weight + col), w);
    uint32_t packed[4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      packed[i] = pack_bf16x2(r[2 * i] * inv * w[2 * i], r[2 * i + 1] * inv * w[2 * i + 1]);
      v[2 * i] = bf16_bits_to_float(packed[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_float(packed[i] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
    }
    *reinterpret_cast<uint4*>(normed_out + base + col) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    amax = team16_max(amax);
    quant_store_8(v, amax, out + base + col, scale_out + scale_index(row, blk, rows, nblk, mn_major), sub == 0);
  }
}

}  // namespace kernels

hipError_t launch_quantize_1x128(const uint16_t* x, int rows, int cols, uint8_t* out, float* scale_out,
                                 bool mn_major, hipStream_t stream) {
  hipLaunchKernelGGL(kernels::quantize_1x128_kernel, dim3(rows), dim3(kernels::kQuantThreads), 0, stream, x, rows,
                     cols, out, scale_out, mn_major);
  return hipGetLastError();
}

hipError_t launch_fused_add_rmsnorm_quant(const uint16_t* input, uint16_t* residual, const uint16_t* weight,
                                          float eps, int rows, int hidden, uint16_t* normed_out, uint8_t* out,
                                          float* scale_out, bool mn_major, hipStream_t stream) {
  hipLaunchKernelGGL(kernels::fused_add_rmsnorm_quant_kernel, dim3(rows), dim3(kernels::kQuantThreads), 0, stream,
                     input, residual, weight, eps, rows, hidden, normed_out, out, scale_out, mn_major);
  return hipGetLastError();
}

}  // namespace fp8g
