// Memory-bound steps of the FP8 block-scale expert FFN around the grouped GEMM (flashinfer-rs
// README, section "API Example: Fused MoE FP8 (cudarc)", DeepSeek FP8 block-scale mode): routing
// entries -> expert-contiguous permutation, BF16 tokens -> 1x128 E4M3 (gathered into the permuted
// order), SiLU(gate)*up -> 1x128 E4M3, and the top-k weighted combine.
//
// The 1x128 quantiser takes scale = amax/448 and code = E4M3_RNE(x / scale) with IEEE FP32
// division, so that its decisions are reproducible; a block of zeros gets scale 1. Each 128-wide
// block is handled by 16 lanes holding 8 consecutive elements (16-byte loads), and its amax is a
// 16-lane butterfly reduction.
#include "internal.h"

namespace fp8g {
namespace kernels {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ void unpack_bf16x8(const uint4 raw, float v[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_float(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};  // round-to-nearest-even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint32_t, v);
}

// Quantise the 8 values a lane holds, given the amax of its 16-lane team; writes 8 codes + scale.
__device__ __forceinline__ void quant_store_8(const float v[8], float amax, uint8_t* codes_out, float* scale_out,
                                              bool write_scale) {
  const float s = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = __fdiv_rn(v[i], s);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  *reinterpret_cast<uint2*>(codes_out) = make_uint2((uint32_t)lo, (uint32_t)hi);
  if (write_scale) *scale_out = s;
}

__device__ __forceinline__ float team16_max(float v) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 16));
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

constexpr int kPermThreads = 256;
constexpr int kPermPerThread = 8;
constexpr int kMaxExperts = 1024;

// One workgroup per expert. Every workgroup histograms all entries (the ids are small and stay in
// L2), takes its region offset as the sum of the 128-padded counts of the experts before it, and
// then compacts its own entries in ascending entry order with a block-wide exclusive scan, so the
// result does not depend on scheduling.
__global__ void __launch_bounds__(kPermThreads)
moe_permutation_kernel(const int32_t* __restrict__ ids, int entries, int top_k, int num_experts,
                       int m_alloc, int32_t* __restrict__ m_indices, int32_t* __restrict__ src_token,
                       int32_t* __restrict__ row_of_entry) {
  __shared__ int hist[kMaxExperts];
  __shared__ int wave_part[kPermThreads / 64];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < num_experts; i += kPermThreads) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < entries; i += kPermThreads) {
    const int v = ids[i];
    if (v >= 0 && v < num_experts) atomicAdd(&hist[v], 1);
  }
  __syncthreads();

  int part = 0;
  for (int i = tid; i < e; i += kPermThreads) part += (hist[i] + 127) & ~127;
  part = wave_sum(part);
  if (lane == 0) wave_part[wave] = part;
  __syncthreads();
  int offset = 0;
#pragma unroll
  for (int w = 0; w < kPermThreads / 64; ++w) offset += wave_part[w];
  const int count = hist[e];
  const int padded = (count + 127) & ~127;
  __syncthreads();  // wave_part is reused below

  int base = 0;
  for (int c0 = 0; c0 < entries; c0 += kPermThreads * kPermPerThread) {
    const int first = c0 + tid * kPermPerThread;
    int flags = 0, mine = 0;
#pragma unroll
    for (int u = 0; u < kPermPerThread; ++u) {
      const int idx = first + u;
      if (idx < entries && ids[idx] == e) {
        flags |= 1 << u;
        ++mine;
      }
    }
    const int incl = wave_inclusive_scan(mine, lane);
    if (lane == 63) wave_part[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPermThreads / 64; ++w) {
      before += w < wave ? wave_part[w] : 0;
      total += wave_part[w];
    }
    int row = offset + base + before + incl - mine;
#pragma unroll
    for (int u = 0; u < kPermPerThread; ++u) {
      if (flags & (1 << u)) {
        const int idx = first + u;
        m_indices[row] = e;
        src_token[row] = idx / top_k;
        row_of_entry[idx] = row;
        ++row;
      }
    }
    base += total;
    __syncthreads();
  }

  for (int r = offset + count + tid; r < offset + padded; r += kPermThreads) {
    m_indices[r] = -1;
    src_token[r] = -1;
  }
  if (e == num_experts - 1) {
    for (int r = offset + padded + tid; r < m_alloc; r += kPermThreads) {
      m_indices[r] = -1;
      src_token[r] = -1;
    }
  }
  if (e == 0) {
    for (int i = tid; i < entries; i += kPermThreads) {
      const int v = ids[i];
      if (v < 0 || v >= num_experts) row_of_entry[i] = -1;
    }
  }
}

constexpr int kRowThreads = 256;  // 16 teams of 16 lanes, one 128-wide block per team and pass

__global__ void __launch_bounds__(kRowThreads)
moe_gather_quant_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ src_token,
                        int num_tokens, int hidden, uint8_t* __restrict__ a_out,
                        float* __restrict__ a_scale_out) {
  const int row = blockIdx.x;
  const int t = src_token[row];
  if (t < 0 || t >= num_tokens) return;
  const int nblk = hidden / 128;
  const int sub = threadIdx.x & 15;
  const uint16_t* xrow = x + (int64_t)t * hidden;
  uint8_t* orow = a_out + (int64_t)row * hidden;
  for (int blk = threadIdx.x >> 4; blk < nblk; blk += kRowThreads / 16) {
    const int col = blk * 128 + sub * 8;
    float v[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(xrow + col), v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = team16_max(amax);
    quant_store_8(v, amax, orow + col, a_scale_out + (int64_t)row * nblk + blk, sub == 0);
  }
}

__global__ void __launch_bounds__(kRowThreads)
moe_silu_mul_quant_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ m_indices,
                          int inter, uint8_t* __restrict__ a_out, float* __restrict__ a_scale_out) {
  const int row = blockIdx.x;
  if (m_indices[row] < 0) return;
  const int nblk = inter / 128;
  const int sub = threadIdx.x & 15;
  const uint16_t* yrow = y + (int64_t)row * 2 * inter;
  uint8_t* orow = a_out + (int64_t)row * inter;
  for (int blk = threadIdx.x >> 4; blk < nblk; blk += kRowThreads / 16) {
    const int col = blk * 128 + sub * 8;
    float gate[8], up[8], h[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(yrow + col), gate);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(yrow + inter + col), up);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = __fdiv_rn(gate[i], 1.0f + expf(-gate[i])) * up[i];
      amax = fmaxf(amax, fabsf(h[i]));
    }
    amax = team16_max(amax);
    quant_store_8(h, amax, orow + col, a_scale_out + (int64_t)row * nblk + blk, sub == 0);
  }
}

__global__ void __launch_bounds__(kRowThreads)
moe_combine_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ row_of_entry,
                   const float* __restrict__ weights, int top_k, int hidden, int m_alloc,
                   uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int32_t* rows = row_of_entry + (int64_t)t * top_k;
  const float* w = weights + (int64_t)t * top_k;
  for (int c = threadIdx.x * 8; c < hidden; c += kRowThreads * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < top_k; ++s) {
      const int r = rows[s];
      if (r < 0 || r >= m_alloc) continue;
      const float ws = w[s];
      float v[8];
      unpack_bf16x8(*reinterpret_cast<const uint4*>(y + (int64_t)r * hidden + c), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(ws, v[i], acc[i]);
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + (int64_t)t * hidden + c) = o;
  }
}

}  // namespace kernels

using namespace kernels;

hipError_t launch_moe_build_permutation(const int32_t* topk_ids, int num_tokens, int top_k,
                                        int num_experts, int m_alloc, int32_t* m_indices,
                                        int32_t* src_token, int32_t* row_of_entry,
                                        hipStream_t stream) {
  hipLaunchKernelGGL(moe_permutation_kernel, dim3(num_experts), dim3(kPermThreads), 0, stream, topk_ids,
                     num_tokens * top_k, top_k, num_experts, m_alloc, m_indices, src_token, row_of_entry);
  return hipGetLastError();
}

hipError_t launch_moe_gather_quant(const uint16_t* x, const int32_t* src_token, int num_tokens,
                                   int hidden, int m_alloc, uint8_t* a_out, float* a_scale_out,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(moe_gather_quant_kernel, dim3(m_alloc), dim3(kRowThreads), 0, stream, x, src_token,
                     num_tokens, hidden, a_out, a_scale_out);
  return hipGetLastError();
}

hipError_t launch_moe_silu_mul_quant(const uint16_t* y, const int32_t* m_indices, int rows,
                                     int inter, uint8_t* a_out, float* a_scale_out,
                                     hipStream_t stream) {
  hipLaunchKernelGGL(moe_silu_mul_quant_kernel, dim3(rows), dim3(kRowThreads), 0, stream, y, m_indices,
                     inter, a_out, a_scale_out);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* y, const int32_t* row_of_entry,
                              const float* topk_weights, int num_tokens, int top_k, int hidden,
                              int m_alloc, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(num_tokens), dim3(kRowThreads), 0, stream, y, row_of_entry,
                     topk_weights, top_k, hidden, m_alloc, out);
  return hipGetLastError();
}

}  // namespace fp8g
