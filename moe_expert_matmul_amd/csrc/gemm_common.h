// Device helpers shared by the groupwise GEMM kernels: operand fragments, LDS slab loads,
// buffer resources, pipeline waits and the workgroup-to-tile mapping.
#pragma once
#include "internal.h"

namespace fp8g {
namespace kernels {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int KBLK = 128;         // K-block width = bytes of one row per K block
constexpr int SLAB_ROWS = 8;      // rows filled by one wave-wide 16-byte-per-lane LDS load
constexpr int E8M0_ONE = 127;     // 2^0 as an E8M0 block scale
constexpr int FMT_E4M3 = 0;       // f8f6f4 operand format code of FP8 E4M3

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002;
constexpr int SG_MFMA = 0x008;
constexpr int SG_DS_READ = 0x100;
constexpr int SG_VMEM = 0x010;

// A sched_group_barrier of n (0..12) memory instructions; n folds to a constant after unrolling.
__device__ __forceinline__ void sched_vmem_group(int n) {
  switch (n) {
    case 1: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 1, 0); break;
    case 2: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 2, 0); break;
    case 3: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 3, 0); break;
    case 4: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 4, 0); break;
    case 5: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 5, 0); break;
    case 6: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 6, 0); break;
    case 7: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 7, 0); break;
    case 8: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 8, 0); break;
    case 9: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 9, 0); break;
    case 10: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 10, 0); break;
    case 11: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 11, 0); break;
    case 12: __builtin_amdgcn_sched_group_barrier(SG_VMEM, 12, 0); break;
    default: break;
  }
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8). A real S_WAITCNT, so the compiler's own wait insertion sees it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS pipeline. The LDS reads of this wave are retired first
// (lgkmcnt(0)) so a stage can be refilled after it; the slab loads' visibility is handled by the
// caller's vmcnt wait. Unlike __syncthreads() it carries no release fence, which would drain every
// load in flight, including the ones meant to stay in flight across the barrier. The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_pipeline_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maximum
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer resource (base, byte size) for the loads below; word 3 is the gfx9 raw-buffer format.
// Accesses past `bytes` read zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// A pointer that is the same in every lane, moved into scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane l reads
// byte offset voff + soff and writes bytes [16l, 16l+16) of the 1 KB block at the wave-uniform
// address `lds`. soff is a scalar, so the per-lane offset is the only vector register used.
__device__ __forceinline__ void load_lds_16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}

// 4 bytes per lane into LDS: lane l writes bytes [4l, 4l+4) at `lds`.
__device__ __forceinline__ void load_lds_4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// Renumber workgroups so that ids t and t+1 run on the same XCD (dispatch is round-robin).
__device__ __forceinline__ int xcd_local_order(int t, int total) {
  const int full = total & ~7;
  return t < full ? (t & 7) * (full >> 3) + (t >> 3) : t;
}

// Row r of `rows` rows, each with `per_row` consecutive entries, for workgroup id b: XCD x (ids
// with b % 8 == x) receives rows x, x+8, x+16, ... in order, each row's entries one after another;
// the last rows % 8 rows follow in plain order. A bijection of [0, rows * per_row).
__device__ __forceinline__ void xcd_row_interleave(int b, int rows, int per_row, int& row, int& entry) {
  const int rem = rows & 7;
  const int full = (rows - rem) * per_row;
  if (b < full) {
    const int j = b >> 3;
    const int r = j / per_row;
    entry = j - r * per_row;
    row = r * 8 + (b & 7);
  } else {
    const int t = b - full;
    const int r = t / per_row;
    entry = t - r * per_row;
    row = rows - rem + r;
  }
}

__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int gid = t / per_group;
  const int first = gid * group_m;
  const int gm = min(tiles_m - first, group_m);
  const int r = t - gid * per_group;
  tm = first + r % gm;
  tn = r / gm;
}

// Physical 16-byte chunk of logical chunk c in tile row r is c ^ swizzle(r).
__device__ __forceinline__ int swizzle(int row) { return (row >> 1) & 7; }

// One 16x128 FP8 operand fragment: lane l supplies row (l & 15) of the 16-row group and the 16-byte
// chunks g and g+4 of the K block, g = l >> 4. Both operands use the same K assignment, which is
// all the matrix core needs for a dot product over the block. (Lane groups reading chunks g and
// g+4 keep each ds_read_b128 free of bank conflicts; chunks 2g and 2g+1 measured half the rate.)
__device__ __forceinline__ i32x8 load_frag(const uint8_t* slab, int row, int lane) {
  const uint8_t* rp = slab + row * KBLK;
  const int c0 = lane >> 4;
  const int sw = swizzle(row);
  const i32x4 lo = *reinterpret_cast<const i32x4*>(rp + ((c0 ^ sw) << 4));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(rp + (((c0 + 4) ^ sw) << 4));
  return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// ---- operand b stored k-major (n contiguous in memory), as bmm_fp8 takes it ----------------
// In LDS the K block is 128 rows of BN bytes (one row per k, BN consecutive columns); the 16-byte
// chunk c of row k sits at c ^ kn_swizzle(k). The fragment reads below (ds_read_b64_tr_b8) have
// each half-wave read 16 bytes from each of 16 rows {k0 + r, k0 + 16 + r : r < 8} at one logical
// chunk; the swizzle gives those 16 rows 16 distinct bank positions (BN = 256: 16 chunks per
// 64-bank row; BN = 128: two rows per 64 banks, 8 chunks each, rows of one parity distinct).
template <int BN>
__device__ __forceinline__ int kn_swizzle(int k) {
  static_assert(BN == 128 || BN == 256, "k-major b tiles are 128 or 256 columns wide");
  return BN == 256 ? (k & 7) | ((k >> 1) & 8) : ((k >> 1) & 3) | ((k >> 2) & 4);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));

// Eight k of one column per lane: ds_read_b64_tr_b8 takes, in each 16-lane group, 8 bytes from
// every lane (lane 2r + h: bytes 8h .. 8h+7 of row r's 16 columns) and returns to lane c the byte of
// column c from each of the 8 rows, row 0 in the lowest byte.
// The pointer is __restrict__ so that the read carries alias information, as the plain LDS reads
// do: without it the compiler makes the read wait for every slab load in flight (vmcnt(0)), the
// next stage's included. The pipeline's own waits and barriers order the reads after their slabs.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// The fragment load_frag gives for b rows col .. col+15 (lane l: column col + (l & 15), k bytes
// 16g .. 16g+15 and 64+16g .. 64+16g+15 of the block, g = l >> 4), read from a k-major slab with
// four transposing reads of 8 k each.
template <int BN>
__device__ __forceinline__ i32x8 load_frag_kn(const uint8_t* slab, int col, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int c = col >> 4;
  const int r = i >> 1, h8 = (i & 1) * 8;
  auto rd = [&](int k) { return lds_read_tr8(slab + k * BN + ((c ^ kn_swizzle<BN>(k)) << 4) + h8); };
  const i32x2 x0 = rd(16 * g + r), x1 = rd(16 * g + 8 + r), x2 = rd(64 + 16 * g + r), x3 = rd(64 + 16 * g + 8 + r);
  return i32x8{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
}

}  // namespace kernels
}  // namespace fp8g
