// Memory-bound steps of the FP8 block-scale expert FFN around the grouped GEMM (flashinfer-rs
// README, section "API Example: Fused MoE FP8 (cudarc)", DeepSeek FP8 block-scale mode): routing
// entries -> expert-contiguous permutation, BF16 tokens -> 1x128 E4M3 (gathered into the permuted
// order), SiLU(gate)*up -> 1x128 E4M3, and the top-k weighted combine.
//
// The 1x128 quantiser takes scale = amax/448 and code = E4M3_RNE(x / scale) with IEEE FP32
// division, so that its decisions are reproducible; a block of zeros gets scale 1. Each 128-wide
// block is handled by 16 lanes holding 8 consecutive elements (16-byte loads), and its amax is a
// 16-lane butterfly reduction.
#include <algorithm>
#include <mutex>

#include "internal.h"
#include "quant_common.h"

namespace fp8g {
namespace kernels {

constexpr int kPermThreads = 1024;  // 16 waves; one routing entry per thread and chunk
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kMaxExperts = 1024;

// Lanes of this wave whose (valid) id equals this lane's: one ballot per id bit. Valid ids are
// below num_experts, so bits from `bits` = ceil(log2(num_experts)) up are zero in all of them.
__device__ __forceinline__ uint64_t match_id(int id, bool valid, int bits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const uint64_t ones = __ballot(valid && ((id >> b) & 1));
    m &= ((id >> b) & 1) ? ones : ~ones;
  }
  return m;
}

__device__ __forceinline__ int id_bits_of(int num_experts) { return num_experts > 1 ? 32 - __clz(num_experts - 1) : 0; }

// The permutation is a stable counting sort of the (token, slot) entries by expert, in three passes
// over chunks of kPermThreads entries, with one int per (chunk, expert) in `hist`:
//   1. histogram: chunk c's entry count per expert -> hist[c][e]; every row of m_indices and
//      src_token is set to -1 (the padding value) on the way;
//   2. scan (one workgroup): expert e owns rows [region_e, region_e + ceil(count_e/128)*128), in
//      expert order; hist[c][e] becomes the first row of chunk c's entries of expert e, i.e. region_e
//      plus the entries of e in earlier chunks;
//   3. scatter: an entry's row is hist[c][e] plus the entries of its expert earlier in the chunk
//      (earlier waves, from per-wave counts in LDS; earlier lanes, by matching ids with ballots).
// Every pass is linear in the number of entries, and entries keep their order inside an expert.

__global__ void __launch_bounds__(kPermThreads)
moe_perm_histogram_kernel(const int32_t* __restrict__ ids, int entries, int num_experts, int chunks,
                          int32_t* __restrict__ hist, int m_alloc, int32_t* __restrict__ m_indices,
                          int32_t* __restrict__ src_token) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int r = blockIdx.x * kPermThreads + tid; r < m_alloc; r += gridDim.x * kPermThreads) {
    m_indices[r] = -1;
    src_token[r] = -1;
  }
  if ((int)blockIdx.x >= chunks) return;  // uniform: the grid may be wider than the chunks
  for (int e = tid; e < num_experts; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const int idx = blockIdx.x * kPermThreads + tid;
  const int id = idx < entries ? ids[idx] : -1;
  const bool valid = id >= 0 && id < num_experts;
  const uint64_t same = match_id(id, valid, id_bits_of(num_experts));
  if (valid && (same >> lane) == 1) atomicAdd(&cnt[id], __popcll(same));  // the last lane of each id adds for all
  __syncthreads();
  int32_t* h = hist + (int64_t)blockIdx.x * num_experts;
  for (int e = tid; e < num_experts; e += kPermThreads) h[e] = cnt[e];
}

// One workgroup. Thread t serves expert e = t % E and chunk slice s = t / E (E*S <= 1024 threads,
// S = 1024 / E slices of consecutive chunks), so the reads of one chunk's row of hist are coalesced.
__global__ void __launch_bounds__(kPermThreads)
moe_perm_scan_kernel(int32_t* __restrict__ hist, int num_experts, int chunks) {
  __shared__ int part[kPermThreads];     // [s][e]: entries of e in slice s
  __shared__ int region[kMaxExperts];    // first row of e's region
  __shared__ int scan_part[kPermWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = num_experts;
  const int S = kPermThreads / E;
  const int e = tid % E, s = tid / E;
  const bool active = s < S;
  const int per = (chunks + S - 1) / S;
  const int c0 = min(s * per, chunks), c1 = min(c0 + per, chunks);
  int sum = 0;
  if (active)
    for (int c = c0; c < c1; ++c) sum += hist[(int64_t)c * E + e];
  if (active) part[s * E + e] = sum;
  __syncthreads();
  // 128-padded count of expert tid, and the block-wide exclusive scan of those counts
  int count = 0;
  if (tid < E)
    for (int j = 0; j < S; ++j) count += part[j * E + tid];
  const int padded = (count + 127) & ~127;
  int incl = padded;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) scan_part[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += scan_part[w];
  if (tid < E) region[tid] = before + incl - padded;
  __syncthreads();
  if (!active) return;
  int row = region[e];
  for (int j = 0; j < s; ++j) row += part[j * E + e];
  for (int c = c0; c < c1; ++c) {
    int32_t* p = hist + (int64_t)c * E + e;
    const int v = *p;
    *p = row;
    row += v;
  }
}

__global__ void __launch_bounds__(kPermThreads)
moe_perm_scatter_kernel(const int32_t* __restrict__ ids, int entries, int top_k, int num_experts,
                        const int32_t* __restrict__ first_row, int32_t* __restrict__ m_indices,
                        int32_t* __restrict__ src_token, int32_t* __restrict__ row_of_entry) {
  __shared__ int wave_cnt[kPermWaves][kMaxExperts];  // entries of each expert in each wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = num_experts;
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wave_cnt[i / E][i % E] = 0;
  const int idx = blockIdx.x * kPermThreads + tid;
  const int id = idx < entries ? ids[idx] : -1;
  const bool valid = id >= 0 && id < E;
  const uint64_t same = match_id(id, valid, id_bits_of(E));
  __syncthreads();
  if (valid && (same >> lane) == 1) wave_cnt[wave][id] = __popcll(same);
  __syncthreads();
  if (valid) {
    int row = first_row[(int64_t)blockIdx.x * E + id] + __popcll(same & ((1ull << lane) - 1));
    for (int w = 0; w < wave; ++w) row += wave_cnt[w][id];
    m_indices[row] = id;
    src_token[row] = idx / top_k;
    row_of_entry[idx] = row;
  } else if (idx < entries) {
    row_of_entry[idx] = -1;
  }
}

constexpr int kRowThreads = 256;  // 16 teams of 16 lanes, one 128-wide block per team and pass

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

// One workgroup per token with one lane per 8 columns (up to 1024 lanes; wider rows loop). A lane
// loads its 8 columns of up to 8 routed rows before the first FMA, then sums in slot order. The
// loads are unconditional (a slot with no row reads row 0 and adds nothing), so all of them are
// in flight together rather than each waiting behind its own branch.
constexpr int kCombineBatch = 8;

__global__ void __launch_bounds__(1024)
moe_combine_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ row_of_entry,
                   const float* __restrict__ weights, int top_k, int hidden, int m_alloc,
                   uint16_t* __restrict__ out, bool out_fp16) {
  const int t = blockIdx.x;
  const int32_t* rows = row_of_entry + (int64_t)t * top_k;
  const float* w = weights != nullptr ? weights + (int64_t)t * top_k : nullptr;  // null: weight 1
  for (int c = threadIdx.x * 8; c < hidden; c += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < top_k; s0 += kCombineBatch) {
      uint4 raw[kCombineBatch];
      bool live[kCombineBatch];
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        const int r = s0 + j < top_k ? rows[s0 + j] : -1;
        live[j] = r >= 0 && r < m_alloc;
        raw[j] = *reinterpret_cast<const uint4*>(y + (int64_t)(live[j] ? r : 0) * hidden + c);
      }
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        if (!live[j]) continue;
        const float ws = w != nullptr ? w[s0 + j] : 1.0f;
        float v[8];
        unpack_bf16x8(raw[j], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(ws, v[i], acc[i]);
      }
    }
    uint4 o;
    if (out_fp16) {
      o.x = pack_f16x2(acc[0], acc[1]);
      o.y = pack_f16x2(acc[2], acc[3]);
      o.z = pack_f16x2(acc[4], acc[5]);
      o.w = pack_f16x2(acc[6], acc[7]);
    } else {
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
    }
    *reinterpret_cast<uint4*>(out + (int64_t)t * hidden + c) = o;
  }
}

}  // namespace kernels

using namespace kernels;

// Scratch of the allocation-free permutation (fp8_moe_build_permutation_noalloc): the per-chunk
// expert counts, one int32 per (chunk of 1024 entries, expert), at most kPermScratchInts of them. Each
// device holds its own copy for the life of the process. Host code must not pass `scratch` itself to
// a kernel (the name is a host-side stand-in there); it uses the device address looked up below.
static __device__ __align__(256) int32_t scratch[kPermScratchInts];

namespace {
std::mutex g_scratch_mutex;
int32_t* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t permutation_scratch(int device, int32_t** ptr) {
  if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    // with `device` current (the caller's current device): this device's copy of the array
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = static_cast<int32_t*>(p);
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

int64_t moe_permutation_scratch_ints(int64_t entries, int64_t num_experts) {
  return (entries + kPermThreads - 1) / kPermThreads * num_experts;
}

hipError_t launch_moe_build_permutation(const int32_t* topk_ids, int num_tokens, int top_k,
                                        int num_experts, int m_alloc, int32_t* m_indices,
                                        int32_t* src_token, int32_t* row_of_entry, int32_t* hist,
                                        hipStream_t stream) {
  const int entries = num_tokens * top_k;
  const int chunks = (entries + kPermThreads - 1) / kPermThreads;
  const int fill_blocks = (m_alloc + kPermThreads - 1) / kPermThreads;
  // one workgroup per chunk (every chunk needs its own), and enough for the fill's grid-stride loop
  const int grid1 = std::max(1, std::max(chunks, std::min(fill_blocks, 4096)));
  hipLaunchKernelGGL(moe_perm_histogram_kernel, dim3(grid1), dim3(kPermThreads), 0, stream, topk_ids, entries,
                     num_experts, chunks, hist, m_alloc, m_indices, src_token);
  if (chunks == 0) return hipGetLastError();
  hipLaunchKernelGGL(moe_perm_scan_kernel, dim3(1), dim3(kPermThreads), 0, stream, hist, num_experts, chunks);
  hipLaunchKernelGGL(moe_perm_scatter_kernel, dim3(chunks), dim3(kPermThreads), 0, stream, topk_ids, entries, top_k,
                     num_experts, hist, m_indices, src_token, row_of_entry);
  return hipGetLastError();
}

hipError_t launch_moe_gather_quant(const uint16_t* x, const int32_t* src_token, int num_tokens,
                                   int hidden, int m_alloc, uint8_t* a_out, float* a_scale_out,
                                   hipStream_t stream) {
  return launch_quantize_rows_1x128(x, src_token, num_tokens, m_alloc, hidden, a_out, a_scale_out, false, stream);
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
                              int m_alloc, uint16_t* out, bool out_fp16, hipStream_t stream) {
  const int threads = std::min(1024, (hidden / 8 + 63) / 64 * 64);
  // The kernel reads row 0 of y for slots with no row; with no rows at all no slot can hold one,
  // and the output is zero, so it runs with no slots.
  if (m_alloc == 0) top_k = 0;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(num_tokens), dim3(threads), 0, stream, y, row_of_entry,
                     topk_weights, top_k, hidden, m_alloc, out, out_fp16);
  return hipGetLastError();
}

}  // namespace fp8g
