// Producers of the GEMM's a operand: the 1x128 E4M3 activation quantiser and the fused
// add-RMSNorm with 1x128 quantisation (MATE FlashInfer-API page, section "norm":
// fused_add_rmsnorm_fp8_block_quant; the quantised rows are the a operand of the section "GEMM"
// calls with a 1x128 a_scale).
//
// Both are HBM-bound. A 16-lane team owns a 128-wide block (8 elements per lane, 16-byte loads); the
// quantiser spreads a row over small workgroups, the add-RMSNorm gives a row one workgroup,
// since the row's sum of squares comes before any output.
#include "internal.h"
#include "quant_common.h"

namespace fp8g {
namespace kernels {

constexpr int kQuantThreads = 256;  // 16 teams of 16 lanes

// Scale element of (row, block) in the requested layout: K-major (rows, nblk) or MN-major (nblk, rows).
__device__ __forceinline__ int64_t scale_index(int row, int blk, int rows, int nblk, bool mn_major) {
  return mn_major ? (int64_t)blk * rows + row : (int64_t)row * nblk + blk;
}

// One 16-lane team per 128-wide block, one 16-byte load per lane: a row spreads over wgs_per_row
// workgroups of blockDim.x/16 teams. Output row r reads source row src_row[r] when src_row is given
// (rows whose source is outside [0, num_src) are skipped), else row r. (Four blocks per team, with
// their loads issued together, measured slower: the kernel is bound by the divisions' VALU work
// more than by load latency.)
__global__ void __launch_bounds__(kQuantThreads)
quantize_1x128_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ src_row, int num_src, int rows,
                      int nblk, int wgs_per_row, uint8_t* __restrict__ out, float* __restrict__ scale_out,
                      bool mn_major) {
  const int row = blockIdx.x / wgs_per_row;
  const int blk = (blockIdx.x - row * wgs_per_row) * (blockDim.x >> 4) + (threadIdx.x >> 4);
  if (blk >= nblk) return;  // whole teams leave together
  const int t = src_row != nullptr ? src_row[row] : row;
  if (t < 0 || t >= num_src) return;
  const int64_t cols = (int64_t)nblk * 128;
  const int col = blk * 128 + (threadIdx.x & 15) * 8;
  float v[8];
  unpack_bf16x8(*reinterpret_cast<const uint4*>(x + t * cols + col), v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = team16_max(amax);
  quant_store_8(v, amax, out + row * cols + col, scale_out + scale_index(row, blk, rows, nblk, mn_major),
                (threadIdx.x & 15) == 0);
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


// Row-resident variant for hidden <= 1024 * 8 * PER: one workgroup of up to 1024 lanes per row, each
// 16-lane team owning PER blocks, all held in registers between the two passes (no re-read). The
// arithmetic is that of the kernel above; only the order of the FP32 sum of squares differs.
template <int PER>
__global__ void __launch_bounds__(1024)
fused_add_rmsnorm_quant_rows_kernel(const uint16_t* input, uint16_t* __restrict__ residual,
                                    const uint16_t* __restrict__ weight, float eps, int rows, int hidden,
                                    uint16_t* normed_out, uint8_t* __restrict__ out, float* __restrict__ scale_out,
                                    bool mn_major) {
  __shared__ float wave_sum[16];
  const int row = blockIdx.x;
  const int nblk = hidden / 128;
  const int teams = blockDim.x >> 4;
  const int team = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  const int64_t base = (int64_t)row * hidden;
  uint4 ra[PER], rb[PER], rw[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int blk = team + p * teams;
    if (blk < nblk) {
      const int col = blk * 128 + sub * 8;
      ra[p] = *reinterpret_cast<const uint4*>(input + base + col);
      rb[p] = *reinterpret_cast<const uint4*>(residual + base + col);
      rw[p] = *reinterpret_cast<const uint4*>(weight + col);
    }
  }
  float r[PER][8];
  float ss = 0.0f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int blk = team + p * teams;
    if (blk < nblk) {
      float a[8], b[8];
      unpack_bf16x8(ra[p], a);
      unpack_bf16x8(rb[p], b);
      uint32_t packed[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        packed[i] = pack_bf16x2(a[2 * i] + b[2 * i], a[2 * i + 1] + b[2 * i + 1]);
        r[p][2 * i] = bf16_bits_to_float(packed[i] & 0xFFFFu);
        r[p][2 * i + 1] = bf16_bits_to_float(packed[i] >> 16);
        ss = __builtin_fmaf(r[p][2 * i], r[p][2 * i], ss);
        ss = __builtin_fmaf(r[p][2 * i + 1], r[p][2 * i + 1], ss);
      }
      *reinterpret_cast<uint4*>(residual + base + blk * 128 + sub * 8) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = ss;
  __syncthreads();
  float total = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) total += wave_sum[w];
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(total, (float)hidden) + eps));
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int blk = team + p * teams;
    if (blk < nblk) {
      const int col = blk * 128 + sub * 8;
      float w[8], v[8];
      unpack_bf16x8(rw[p], w);
      uint32_t packed[4];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        packed[i] = pack_bf16x2(r[p][2 * i] * inv * w[2 * i], r[p][2 * i + 1] * inv * w[2 * i + 1]);
        v[2 * i] = bf16_bits_to_float(packed[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_float(packed[i] >> 16);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
      }
      *reinterpret_cast<uint4*>(normed_out + base + col) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      amax = team16_max(amax);
      quant_store_8(v, amax, out + base + col, scale_out + scale_index(row, blk, rows, nblk, mn_major), sub == 0);
    }
  }
}

}  // namespace kernels

// Teams per workgroup: 16 or 8 when they divide the row's block count, else 4 for short rows or 16.
static int quant_teams_per_wg(int nblk) {
  if (nblk % 16 == 0) return 16;
  if (nblk % 8 == 0) return 8;
  return nblk % 4 == 0 || nblk < 16 ? 4 : 16;
}

hipError_t launch_quantize_rows_1x128(const uint16_t* x, const int32_t* src_row, int num_src, int rows, int cols,
                                      uint8_t* out, float* scale_out, bool mn_major, hipStream_t stream) {
  const int nblk = cols / 128;
  const int teams = quant_teams_per_wg(nblk);
  const int wgs_per_row = (nblk + teams - 1) / teams;
  if ((int64_t)rows * wgs_per_row > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernels::quantize_1x128_kernel, dim3(rows * wgs_per_row), dim3(teams * 16), 0, stream, x,
                     src_row, num_src, rows, nblk, wgs_per_row, out, scale_out, mn_major);
  return hipGetLastError();
}

hipError_t launch_quantize_1x128(const uint16_t* x, int rows, int cols, uint8_t* out, float* scale_out,
                                 bool mn_major, hipStream_t stream) {
  return launch_quantize_rows_1x128(x, nullptr, rows, rows, cols, out, scale_out, mn_major, stream);
}

hipError_t launch_fused_add_rmsnorm_quant(const uint16_t* input, uint16_t* residual, const uint16_t* weight,
                                          float eps, int rows, int hidden, uint16_t* normed_out, uint8_t* out,
                                          float* scale_out, bool mn_major, hipStream_t stream) {
  const int nblk = hidden / 128;
  if (nblk <= 256) {
    // up to 64 teams (1024 lanes); a team keeps PER = ceil(nblk / 64) blocks in registers
    const int threads = nblk <= 64 ? (nblk * 16 + 63) / 64 * 64 : 1024;
    const int per = (nblk + threads / 16 - 1) / (threads / 16);
    auto kern = per == 1 ? kernels::fused_add_rmsnorm_quant_rows_kernel<1>
              : per == 2 ? kernels::fused_add_rmsnorm_quant_rows_kernel<2>
                         : kernels::fused_add_rmsnorm_quant_rows_kernel<4>;
    hipLaunchKernelGGL(kern, dim3(rows), dim3(threads), 0, stream, input, residual, weight, eps, rows, hidden,
                       normed_out, out, scale_out, mn_major);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kernels::fused_add_rmsnorm_quant_kernel, dim3(rows), dim3(kernels::kQuantThreads), 0, stream,
                     input, residual, weight, eps, rows, hidden, normed_out, out, scale_out, mn_major);
  return hipGetLastError();
}

}  // namespace fp8g
