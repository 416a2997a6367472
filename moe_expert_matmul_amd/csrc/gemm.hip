// FP8 (E4M3) groupwise-scaled NT GEMM for CDNA4 (gfx950).
//
// Computes, for the three forms of the MATE FlashInfer-API page (section "GEMM":
// gemm_fp8_nt_groupwise, group_deepgemm_fp8_nt_groupwise, batch_deepgemm_fp8_nt_groupwise),
//     out[i][j] = bf16( sum_kb sa(i,kb) * sb(j/128,kb) * P_kb[i][j] ),
//     P_kb[i][j] = sum over the 128 k of K block kb of a[i][k] * b[j][k]
// with a 1x128 scale per row of a and a 128x128 scale per block of b.
//
// Mapping onto the matrix cores: one v_mfma_scale_f32_16x16x128_f8f6f4 covers a 16x16 output
// block over exactly one 128-wide K block (its own E8M0 block scales are left at 2^0), so every
// MFMA yields one P_kb sub-block in FP32 which is promoted into the FP32 accumulator with one
// fused multiply-add by sa*sb. The operands are swapped (the MFMA's row operand is b, its column
// operand is a) so that each lane holds four outputs of one row i and four consecutive columns j:
// the promotion then needs a single scale per lane and 16-row group, and the epilogue stores 8
// contiguous bytes of a row.
//
// Data movement per workgroup and K block: the BMx128 slab of a and the BNx128 slab of b go from
// HBM straight into LDS (global_load_lds_dwordx4, no VGPR staging), in two to four stages so the
// loads of the next blocks overlap the MFMAs of block kb (the masked form: one a buffer and three
// b slots, see SPLIT below). Rows are 128 bytes in LDS with their 16-byte chunks
// XOR-swizzled by ((row >> 1) & 7), which spreads the 16 rows of a fragment over all 64 four-byte
// banks; together with the fragment's chunk assignment (see load_frag) a fragment read runs at the
// LDS's full rate. The swizzle is applied on the global side: lane l of a load writes LDS chunk l of
// its 1 KB slab and fetches the logical chunk that belongs there.
//
// In the plain and masked forms the MFMAs of a K block's last column group (and the promotions of
// its last two groups) are issued after the barrier that opens the next block, while that block's
// first fragment reads are in flight; each output still receives its promotions in K-block order.
//
// Tile scheduling: the 1-D grid is renumbered so that consecutive tiles run on the same XCD (the
// hardware deals workgroups round-robin over the 8 XCDs, each with its own L2) and then rasterised
// in groups of `group_m` row tiles, or, for the contiguous form's 128-row tiles with a read in
// place, in bands of `group_n` column tiles. The masked form maps the grid to (group, row tile,
// col tile) and drops tiles at or beyond masked_m[g]; the contiguous form reads the tile's
// m_indices and drops tiles that hold only padding. With 256-row tiles the contiguous grid has two
// entries per tile, one per 128-row half, dealt to the XCDs by tile row: a tile whose halves hold
// one expert runs as its first entry, one whose halves hold two experts as two. Rows that are not valid are still computed when they share a wave
// with valid rows (each output row depends only on its own a row and scale) but never stored.
//
// Modes (the MODE template argument) on the same loop:
//   PLAIN, CONTIG, MASKED  the three forms above; BF16 or FP16 out, and E4M3 with an output scale in
//                          the plain form;
//   CONTIG_SWIGLU          the expert FFN's fc1: SiLU(gate)*up and its 1x128 requantisation in the
//                          epilogue (flashinfer-rs README, "API Example: Fused MoE FP8 (cudarc)");
//   BMM                    bmm_fp8 of the MATE page: per-tensor or per-row/column scales, so each
//                          MFMA accumulates straight into the sum over all of K and the scales are
//                          applied once in the epilogue; b is read as the caller gives it, (k, n)
//                          with n contiguous, as slabs of k rows (see load_frag_kn);
//   CONTIG_PT(_SWIGLU)     the README's per-tensor FP8 FFN: the BMM loop under the contiguous
//                          scheduler, one dequantisation scale per expert.
#include "gemm_common.h"

namespace fp8g {
namespace kernels {

// The next stage's loads are issued over the first LOAD_GROUPS column groups of a K block (the
// first LOAD_GROUPS_DEFER in the deferred schedule of the plain and masked forms), and each column
// group reads the b fragment of the group BPRE ahead of it.
constexpr int LOAD_GROUPS = 4;
constexpr int LOAD_GROUPS_DEFER = 6;
constexpr int BPRE = 1;  // measured against 2 and 3: the expert FFN 1.5% faster, the plain form level
// a's row scales are fetched a group of K blocks at a time (Tile::SGRP), one group ahead, into a
// ring of SA_SLOTS slots (see the load assignment in the kernel).
constexpr int SA_SLOTS = 3;
#ifndef FP8G_POISON_LDS
#define FP8G_POISON_LDS 0
#endif
#ifndef FP8G_LDS_EPILOGUE
#define FP8G_LDS_EPILOGUE 1
#endif
constexpr bool LDS_EPILOGUE = FP8G_LDS_EPILOGUE;
#ifndef FP8G_SPLIT_PIPELINE
#define FP8G_SPLIT_PIPELINE 1
#endif

// SPLIT: the split pipeline (see the kernel): one a buffer and STAGES + 1 b slots instead of
// STAGES stages of both.
template <int BM, int BN, int WM, int WN, int STAGES, bool SPLIT = false>
struct Tile {
  static constexpr int NWAVES = WM * WN;
  static constexpr int NTHREADS = NWAVES * 64;
  static constexpr int WTM = BM / WM;  // rows of a per wave
  static constexpr int WTN = BN / WN;  // rows of b (output columns) per wave
  static constexpr int IG = WTM / 16;
  static constexpr int JG = WTN / 16;
  static constexpr int A_BYTES = BM * KBLK;
  static constexpr int B_BYTES = BN * KBLK;
  static constexpr int SB_OFF = A_BYTES + B_BYTES;  // 64 floats: b's scales (BN/128 used)
  static constexpr int STAGE_BYTES = SB_OFF + 64 * 4;
  // split pipeline: the a buffer at 0, then B_STAGES slots of b's slabs and scales
  static constexpr int B_STAGES = SPLIT ? STAGES + 1 : STAGES;
  static constexpr int B_SLOT = B_BYTES + 64 * 4;
  // a's row scales: a ring of SA_SLOTS slots after the stages, each the scales of SGRP K blocks
  // for the BM rows. 8 blocks where the ring fits in LDS, else 4.
  static constexpr int SA_RING_OFF = SPLIT ? A_BYTES + B_STAGES * B_SLOT : STAGES * STAGE_BYTES;
  static constexpr int SGRP = SA_RING_OFF + SA_SLOTS * BM * 32 <= 160 * 1024 ? 8 : 4;
  static constexpr int SA_SLOT = BM * SGRP * 4;
  static constexpr int SMEM_BYTES = SA_RING_OFF + SA_SLOTS * SA_SLOT;
  static constexpr int A_LOADS = BM / SLAB_ROWS / NWAVES;  // per wave and K block
  static constexpr int B_LOADS = BN / SLAB_ROWS / NWAVES;
  static constexpr int LOADS = A_LOADS + B_LOADS + 1;      // + one scale load per wave
  // the loads spread over a block's column groups: all of them, or (split) b's and the scales
  static constexpr int SPREAD_LOADS = SPLIT ? B_LOADS + 1 : LOADS;
  static_assert(BM / 64 < NWAVES, "one wave per 64 a-scale rows, and one more for b's scales");
  static_assert(STAGE_BYTES % 256 == 0 && B_SLOT % 256 == 0 && A_BYTES % 256 == 0, "stages keep the slabs' bank alignment");
  static_assert(BM % (SLAB_ROWS * NWAVES) == 0 && BN % (SLAB_ROWS * NWAVES) == 0, "slabs");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "16x16 MFMA blocks");
  static_assert(128 % WTN == 0 || WTN == 128, "a wave's columns sit in one 128-wide b-scale block (two with SWIGLU)");
  static_assert(STAGES >= 2 && STAGES <= 4, "two to four LDS stages");
  static_assert((STAGES - 2) * LOADS < 64 && SPREAD_LOADS < 64, "vmcnt range");
  static_assert(SMEM_BYTES <= 160 * 1024, "LDS");
  static_assert(64 % SGRP == 0, "a group's part covers 64 / SGRP rows");
};

__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }  // RNE

constexpr float kE4M3MaxOut = 448.0f;  // largest finite E4M3FN value

// Epilogue of the expert FFN's fc1 (CONTIG_SWIGLU): the values the unfused path would store in
// BF16 -- gate and up of each output column -- are rounded to BF16 here too, then
// h = silu(gate) * up with silu(g) = g / (1 + exp(-g)) in FP32, and each row's 128 h values of the
// column tile are quantised to E4M3 with scale amax/448 (IEEE division; 1 for an all-zero block).
// This is, operation for operation, what fp8_moe_silu_mul_quant does with the BF16 fc1 output, so
// the codes and scales are identical. A row's 128 columns are spread over the WN waves of its row
// block; their partial amax meet in LDS.
template <typename T, int WN>
__device__ __forceinline__ void swiglu_epilogue(const GemmParams& p, const f32x4 (&acc)[T::IG][T::JG], uint8_t* smem,
                                                int row0, int row_end, int bsel, int tn, int i0, int wave, int lane,
                                                bool wave_live, int wave_ids) {
  constexpr int OUTW = 128 / WN;
  constexpr int HALF = T::JG / 2;  // column groups of gate (then the same number of up)
  const int fr = lane & 15, q = wave % WN;
  float h[T::IG][HALF][4];
  float part[T::IG];
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) {
    float m = 0.0f;
#pragma unroll
    for (int jg = 0; jg < HALF; ++jg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = bf16_round(acc[ig][jg][r]), u = bf16_round(acc[ig][HALF + jg][r]);
        h[ig][jg][r] = __fdiv_rn(g, 1.0f + expf(-g)) * u;
        m = fmaxf(m, fabsf(h[ig][jg][r]));
      }
    m = fmaxf(m, __shfl_xor(m, 16, 64));  // the four lane groups hold the wave's columns of a row
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    part[ig] = m;
  }
  // partial amax per (wave column q, tile row): the main loop's stages are free after this barrier
  float* amax_lds = reinterpret_cast<float*>(smem);
  lds_pipeline_barrier();
  if (lane < 16) {
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) amax_lds[q * 256 + i0 + ig * 16 + fr] = part[ig];
  }
  lds_pipeline_barrier();
  if (!wave_live) return;
  const int nblk = p.inter / 128;
  const int cl = (lane >> 4) * 4;
  int row_id[T::IG];  // m_indices of each lane's rows, from the wave's registers
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) row_id[ig] = __shfl(wave_ids, ig * 16 + fr, 64);
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) {
    const int tr = i0 + ig * 16 + fr;  // tile row
    const int i = row0 + tr;
    if (i >= row_end || row_id[ig] != bsel) continue;
    float amax = 0.0f;
#pragma unroll
    for (int w = 0; w < WN; ++w) amax = fmaxf(amax, amax_lds[w * 256 + tr]);
    const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    uint8_t* orow = p.q_out + (int64_t)i * p.inter + 128 * tn + q * OUTW;
#pragma unroll
    for (int jg = 0; jg < HALF; ++jg) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = __fdiv_rn(h[ig][jg][r], sc);
      int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      w4 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w4, true);
      *reinterpret_cast<int*>(orow + jg * 16 + cl) = w4;
    }
    if (q == 0 && lane < 16) p.q_scale_out[(int64_t)i * nblk + tn] = sc;
  }
}

// Epilogue of the per-tensor expert FFN's fc1 (CONTIG_PT_SWIGLU): gate and up are the FP32 sums
// times the expert's dequantisation scale d, h = silu(gate) * up in FP32 (silu(g) = g / (1 + exp(-g))),
// and the code is E4M3_RNE(saturate(h * act_quant)) -- one per-tensor (or per-expert) scale, so no
// row maximum and no exchange between waves. Column mapping as in swiglu_epilogue.
template <typename T, int WN>
__device__ __forceinline__ void swiglu_pt_epilogue(const GemmParams& p, const f32x4 (&acc)[T::IG][T::JG], int row0,
                                                   int row_end, int bsel, int tn, int i0, int wave, int lane,
                                                   bool wave_live, int wave_ids, float d, float qs) {
  if (!wave_live) return;
  constexpr int OUTW = 128 / WN;
  constexpr int HALF = T::JG / 2;
  const int fr = lane & 15, q = wave % WN;
  const int cl = (lane >> 4) * 4;
  int row_id[T::IG];  // m_indices of each lane's rows, from the wave's registers
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) row_id[ig] = __shfl(wave_ids, ig * 16 + fr, 64);
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) {
    const int i = row0 + i0 + ig * 16 + fr;
    if (i >= row_end || row_id[ig] != bsel) continue;
    uint8_t* orow = p.q_out + (int64_t)i * p.inter + 128 * tn + q * OUTW;
#pragma unroll
    for (int jg = 0; jg < HALF; ++jg) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = acc[ig][jg][r] * d, u = acc[ig][HALF + jg][r] * d;
        v[r] = __fdiv_rn(g, 1.0f + expf(-g)) * u * qs;
        if (!(fabsf(v[r]) <= kE4M3MaxOut) && v[r] == v[r]) v[r] = copysignf(kE4M3MaxOut, v[r]);  // saturate
      }
      int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      w4 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w4, true);
      *reinterpret_cast<int*>(orow + jg * 16 + cl) = w4;
    }
  }
}

// Measurement aid: the shader-clock and wall-clock stamps of the first workgroup of the most recent
// GEMM launch (start cycles, start ticks, end cycles, end ticks); fp8g_gemm_clock_record reads them.
__device__ unsigned long long g_gemm_clock[4];

// Writes the first workgroup's end stamps when it leaves the kernel, on every return path.
struct ClockStamp {
  unsigned long long c0 = 0, w0 = 0;
  bool on = false;
  __device__ ClockStamp() {
    on = blockIdx.x == 0 && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;  // wave 0: uniform
    if (on) {
      c0 = clock64();
      w0 = wall_clock64();
    }
  }
  __device__ ~ClockStamp() {
    if (on && threadIdx.x == 0) {
      const unsigned long long c1 = clock64(), w1 = wall_clock64();
      g_gemm_clock[0] = c0;
      g_gemm_clock[1] = w0;
      g_gemm_clock[2] = c1;
      g_gemm_clock[3] = w1;
    }
  }
};

template <int BM, int BN, int WM, int WN, int STAGES, int MODE>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_fp8_groupwise_kernel(const GemmParams p) {
  const ClockStamp stamp;
  constexpr bool PT = MODE == MODE_CONTIG_PT || MODE == MODE_CONTIG_PT_SWIGLU;
  constexpr bool CONTIG = MODE == MODE_CONTIG || MODE == MODE_CONTIG_SWIGLU || PT;
  constexpr bool SWIGLU = MODE == MODE_CONTIG_SWIGLU || MODE == MODE_CONTIG_PT_SWIGLU;
  constexpr bool NO_PROMOTION = MODE == MODE_BMM || PT;  // scales constant along K: applied at the end
  // bmm_fp8 takes b as (batch, k, n): its slabs are k rows of the tile's columns, read into
  // fragments by transposing LDS reads (load_frag_kn)
  constexpr bool B_KMAJOR = MODE == MODE_BMM;
  // Split pipeline (the masked form's two-stage tiles): one a buffer and three b slots. Iteration
  // kb computes block kb; once every wave has read its a fragments of block kb (a second barrier,
  // mid-block), the a slabs of block kb+1 are loaded into the a buffer, and the b slabs and scales
  // of block kb+2 go into a free b slot over the block's column groups. The b slabs, which stream
  // from HBM, thus have two blocks to arrive instead of one, and a's (mostly L2 hits) one; 96 KB
  // are in flight per workgroup instead of 64. Measured: the masked form 5% faster; the plain form
  // (compute-bound) 11% and the contiguous form's 256-row tiles (fc2) 1-3% slower, so they keep
  // the two stages.
  constexpr bool SPLIT = FP8G_SPLIT_PIPELINE && STAGES == 2 && MODE == MODE_MASKED;
  using T = Tile<BM, BN, WM, WN, STAGES, SPLIT>;
  // SWIGLU: wave column q of the WN holds the gate and the up columns of OUTW output columns; its
  // b rows ("virtual columns" v of the tile) are OUTW gate rows then OUTW up rows.
  constexpr int OUTW = SWIGLU ? 128 / WN : 0;
  static_assert(!SWIGLU || (BN == 256 && T::WTN == 2 * (128 / WN)), "SWIGLU tiles are 256 wide");
  // first of the loads issued during column group jg (the SPREAD_LOADS loads spread over JG groups)
  constexpr int LG = T::JG < LOAD_GROUPS ? T::JG : LOAD_GROUPS;
  constexpr auto load_first = [](int jg) { return ((jg < LG ? jg : LG) * T::SPREAD_LOADS + LG - 1) / LG; };
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::SMEM_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
#if FP8G_POISON_LDS
  // Debug build: LDS starts as 0x7F bytes (E4M3 NaN codes; 3.4e38 as an FP32 scale), so a fragment or
  // scale read that ran ahead of its load would reach the output.
  for (int i = threadIdx.x * 16; i < (int)sizeof(smem); i += T::NTHREADS * 16)
    *reinterpret_cast<uint4*>(smem + i) = uint4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
  __syncthreads();
#endif

  // ---- tile scheduling ---------------------------------------------------------------------
  int t = xcd_local_order(blockIdx.x, gridDim.x);
  int g = 0;
  if (MODE == MODE_MASKED || MODE == MODE_BMM) {
    const int per = p.tiles_m * p.tiles_n;
    g = t / per;
    t -= g * per;
  }
  int tm, tn;
  // Contiguous form with 256-row tiles: the grid holds two entries per tile and column tile (one
  // per 128-row half), so a tile whose halves belong to different experts runs as two workgroups.
  // Its tile rows are dealt round-robin over the XCDs, each with all its entries (so they share
  // the tile's a rows in one L2): the live rows of an expert workspace sized for the worst case
  // are a prefix of it, and this spreads any prefix over every XCD.
  int half = 0;
  if (CONTIG && BM == 256) {
    int k;
    xcd_row_interleave(blockIdx.x, p.tiles_m / 2, 2 * p.tiles_n, tm, k);
    half = k / p.tiles_n;
    tn = k - half * p.tiles_n;
  } else if (p.group_n > 0) {
    raster(t, p.tiles_n, p.tiles_m, p.group_n, tn, tm);
  } else {
    raster(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  }
  const int row0 = tm * BM;
  const int col0 = tn * BN;

  int row_end = p.m;  // rows at or beyond row_end hold no valid output
  // The b group this workgroup multiplies with, and the 128-row halves of the tile it covers
  // (bit h: waves of half h take part). Plain: b, whole tile. Masked: group g, whole tile.
  // Contiguous: each 128-row half holds one expert (plus padding); the first entry of a tile whose
  // halves hold the same expert covers the whole tile and the second exits, otherwise each entry
  // covers its own half (or exits when that half is padding only).
  int bsel = 0;
  int half_mask = 3;
  // Contiguous form: the tile's m_indices, one entry per lane and 64-row quarter, all loaded before
  // any is used so the tile's head costs one memory round trip (m is a multiple of 128, so a half
  // whose first row is in range lies wholly in range).
  constexpr int QUARTERS = CONTIG ? BM / 64 : 1;
  int tile_ids[QUARTERS];
  // Tile row of this lane's a load q (q < A_LOADS) and of its a-scale load (q == A_LOADS), clamped
  // to the valid rows; with gathered rows (a_rows), their indices are loaded with the m_indices.
  auto a_tile_row = [&](int q, int last) {
    return min(q < T::A_LOADS ? row0 + (wave * T::A_LOADS + q) * SLAB_ROWS + (lane >> 3) : row0 + wave * 64 + lane, last);
  };
  int gathered[T::A_LOADS + 1];
  if (MODE == MODE_BMM) {
    bsel = g;
  } else if (MODE == MODE_MASKED) {
    const int mm = max(0, min(p.rowinfo[g], p.m));
    if (row0 >= mm) return;
    row_end = mm;
    bsel = g;
  } else if (CONTIG) {
    constexpr int HALVES = BM / 128;
#pragma unroll
    for (int q = 0; q < QUARTERS; ++q)
      tile_ids[q] = row0 + (q / 2) * 128 < p.m ? p.rowinfo[row0 + q * 64 + lane] : -1;
    // ids outside [0, num_groups) are padding; mapped to -1 before the tile's expert (the largest
    // id) is taken, so that a stray id cannot hide the rows of the half's real expert
#pragma unroll
    for (int q = 0; q < QUARTERS; ++q) tile_ids[q] = (unsigned)tile_ids[q] < (unsigned)p.num_groups ? tile_ids[q] : -1;
    if (p.a_rows != nullptr) {
#pragma unroll
      for (int q = 0; q <= T::A_LOADS; ++q) gathered[q] = p.a_rows[a_tile_row(q, p.m - 1)];
    }
    int ex[HALVES];
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
      // uniform: keeps b's resource scalar; -1: padding only
      ex[h] = __builtin_amdgcn_readfirstlane(wave_max(max(tile_ids[2 * h], tile_ids[2 * h + 1])));
    }
    if (HALVES == 2 && ex[0] >= 0 && ex[0] == ex[HALVES - 1]) {
      if (half == 1) return;
      bsel = ex[0];
    } else {
      if (ex[half] < 0) return;
      bsel = ex[half];
      half_mask = 1 << half;
    }
  }

  const uint8_t* A = p.a + (int64_t)g * p.a_group_stride;
  const float* SA = p.sa + (int64_t)g * p.sa_group_stride;
  // Per-tensor modes: the expert's scales, and the plain form's E4M3 output scale, read now so that
  // the epilogue waits on no load.
  float pt_dequant = 1.0f, pt_act_quant = 1.0f, out_scale = 1.0f;
  if (MODE == MODE_PLAIN && p.out_scale != nullptr) out_scale = *p.out_scale;
  if constexpr (PT) {
    pt_dequant = p.group_dequant[bsel];
    if constexpr (MODE == MODE_CONTIG_PT_SWIGLU) pt_act_quant = p.act_quant[p.act_quant_per_group ? bsel : 0];
  }

  // ---- HBM -> LDS load assignment ----------------------------------------------------------
  // Slab s (1 KB) holds tile rows [8s, 8s+8); lane l fills its chunk l, i.e. tile row
  // 8s + (l >> 3) at physical chunk (l & 7), which holds logical chunk (l & 7) ^ swizzle(row).
  // Every wave issues the same number of loads for every K block (rows past the valid range are
  // clamped to the last valid row), so the pipeline can wait on a fixed count of outstanding loads.
  const int lrow = lane >> 3;
  const int a_last = row_end - 1;
  // SWIGLU: b row of virtual column v of column tile tn (output columns [128 tn, 128 tn + 128))
  auto swiglu_b_row = [&](int v) {
    constexpr int W = OUTW > 0 ? OUTW : 1;  // OUTW is 0 outside SWIGLU, where this is never called
    const int q = v / (2 * W), r = v % (2 * W);
    return (r < W ? 0 : p.inter) + 128 * tn + q * W + (r % W);
  };
  // The rows of a this lane's a loads read (entries 0 .. A_LOADS-1) and the row of a_scale its
  // scale load reads (entry A_LOADS, used by the a-scale waves): the tile rows themselves, or
  // a_rows[tile row] when the contiguous form gathers its rows (indices out of range read row 0;
  // those rows are never stored).
  int a_src[T::A_LOADS + 1];
#pragma unroll
  for (int q = 0; q <= T::A_LOADS; ++q) a_src[q] = a_tile_row(q, q < T::A_LOADS ? a_last : p.m - 1);
  if (CONTIG && p.a_rows != nullptr) {
#pragma unroll
    for (int q = 0; q <= T::A_LOADS; ++q)
      a_src[q] = (gathered[q] >= 0 && gathered[q] < p.a_src_rows) ? gathered[q] : 0;
  }
  uint32_t a_off[T::A_LOADS], b_off[T::B_LOADS];
  // Bit q: a slab q of this wave holds a row whose output the tile keeps. A slab with no such row
  // (rows past the group's valid count, padding rows, rows of the other expert in a split tile)
  // is read out of range: no memory traffic (clamped or gathered rows would otherwise re-read one
  // row many times over), zeros in LDS, rows never stored.
  uint32_t a_live_bits = 0;
#pragma unroll
  for (int q = 0; q < T::A_LOADS; ++q) {
    const int slab_row = (wave * T::A_LOADS + q) * SLAB_ROWS;
    const int lchunk = (lane & 7) ^ swizzle(slab_row + lrow);
    a_off[q] = (uint32_t)a_src[q] * (uint32_t)p.k + lchunk * 16;
    bool live;
    if constexpr (CONTIG) {
      // m_indices entry of the slab row this lane loads: lane (row % 64) of the row's quarter
      const int quarter = slab_row >> 6;
      int ids = tile_ids[0];
#pragma unroll
      for (int r = 1; r < QUARTERS; ++r)
        if (quarter == r) ids = tile_ids[r];
      const int id = __shfl(ids, (slab_row & 63) + lrow, 64);
      live = __ballot(id == bsel && ((half_mask >> (slab_row / 128)) & 1)) != 0;
    } else {
      live = row0 + slab_row < row_end;
    }
    a_live_bits |= (uint32_t)live << q;
  }
  a_live_bits = __builtin_amdgcn_readfirstlane(a_live_bits);
  // A dead slab's offset lies past the operand: out of the resource's range the load touches no
  // memory and writes zeros (or, for an operand of 2 GiB or more, reads bytes of a inside its range).
#pragma unroll
  for (int q = 0; q < T::A_LOADS; ++q)
    if (!((a_live_bits >> q) & 1)) a_off[q] = 0x80000000u;
#pragma unroll
  for (int q = 0; q < T::B_LOADS; ++q) {
    if constexpr (B_KMAJOR) {
      // Slab s of the k-major tile holds k rows [KN_ROWS s, KN_ROWS s + KN_ROWS); lane l fills its
      // chunk l: row KN_ROWS s + l / KN_CHUNKS at physical chunk l % KN_CHUNKS, which holds logical
      // chunk (l % KN_CHUNKS) ^ kn_swizzle(row), columns col0 + 16 * that. Chunks past n (n is a
      // multiple of 16) re-read the last chunk; those columns are never stored.
      constexpr int KN_CHUNKS = BN / 16, KN_ROWS = 64 / KN_CHUNKS;
      const int kr = (wave * T::B_LOADS + q) * KN_ROWS + lane / KN_CHUNKS;
      const int lchunk = (lane % KN_CHUNKS) ^ kn_swizzle<BN>(kr);
      b_off[q] = (uint32_t)kr * (uint32_t)p.n + (uint32_t)min(col0 + lchunk * 16, p.n - 16);
    } else {
      const int slab_row = (wave * T::B_LOADS + q) * SLAB_ROWS;
      const int lchunk = (lane & 7) ^ swizzle(slab_row + lrow);
      int r = min(col0 + slab_row + lrow, p.n - 1);
      if (SWIGLU) r = swiglu_b_row(slab_row + lrow);
      b_off[q] = (uint32_t)r * (uint32_t)p.k + lchunk * 16;
    }
  }
  // byte step of b's slabs from one K block to the next
  const uint32_t b_kb_step = B_KMAJOR ? (uint32_t)KBLK * (uint32_t)p.n : (uint32_t)KBLK;

  // Buffer resources of this tile's operands (per group for the grouped forms).
  const uint8_t* B = p.b + (int64_t)bsel * p.b_group_stride;
  const float* SB = p.sb + (int64_t)bsel * p.sb_group_stride;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A, (uint32_t)p.a_src_rows * (uint32_t)p.k);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(B, (uint32_t)p.n * (uint32_t)p.k);

  // Scales. Every wave issues one 4-byte-per-lane scale load per K block. Waves BM/64 and up fetch
  // b's BN/128 block scales of the block (identical data to the same place) into its stage. Waves
  // 0 .. BM/64-1 own 64 rows each and fetch a's row scales a group of G = SGRP K blocks at a time,
  // in G parts: the load issued with block kb's slabs fetches part kb % G of group kb / G + 1, so a
  // group is complete one group before its first block; group 0 is fetched ahead of the pipeline.
  // A part is the shape that touches the fewest lines: in the K-major layout PR = 64/G rows x G
  // blocks (a row's G blocks are 4G contiguous bytes), so an instruction touches PR lines where a
  // per-block fetch would touch 64; in the MN-major layout, and for gathered rows, one block of all
  // 64 rows. In LDS each part is 256 bytes, block-major with the rows of a block in consecutive
  // words, so the 16 consecutive rows a fragment's lanes read sit in 16 consecutive or (PR = 8)
  // two 8-word runs; with PR = 8 the blocks of odd parts are stored XOR 2 (block b at position
  // b ^ 2), which puts the two runs 64 bytes apart in the bank space instead of on the same banks.
  // So the scale of row r (of the wave's 64) and block b sits at byte
  //   row parts:   256 (r / PR) + 4 (PR (b ^ x) + r % PR), x = 2 ((r / PR) & 1) if PR = 8 else 0
  //   block parts: 256 b + 4 r
  // of the wave's 256G bytes, and lane l of part qq fetches row PR qq + l % PR, block (l / PR) ^ x.
  // Group g sits in slot g % 3: it is written while blocks of groups g-1 and g-2 may still be read,
  // never g-3's. Part qq's offset is part 0's plus qq times a scalar step, plus a per-lane term for
  // odd qq (the swizzle; 0 for the b-scale waves, which have a zero step too: selecting between
  // vector values on a wave-uniform condition would make the compiler split the scheduled loop
  // body). Rows past the end read zeros or unused scales, both within the buffer; such rows are
  // never stored.
  constexpr int SGRP = T::SGRP;
  constexpr int PART_ROWS = 64 / SGRP;
  constexpr bool PART_SWIZZLE = PART_ROWS == 8;
  const bool a_scale_wave = wave < BM / 64;
  const bool sa_block_parts = p.sa_kb_stride != 1 || (CONTIG && p.a_rows != nullptr);
  uint32_t s_voff0;
  uint32_t s_qodd = 0;  // added for odd parts: the block swizzle of row parts
  const uint32_t s_qstep = !a_scale_wave ? 0u
                           : sa_block_parts ? (uint32_t)p.sa_kb_stride * 4u
                                            : (uint32_t)PART_ROWS * (uint32_t)p.sa_row_stride * 4u;
  if (a_scale_wave) {
    // gathered rows: the lane's own row's source row, loaded with the m_indices
    const int src_row = CONTIG && p.a_rows != nullptr ? a_src[T::A_LOADS]
                                                      : row0 + wave * 64 + (sa_block_parts ? lane : lane % PART_ROWS);
    const int blk = lane / PART_ROWS;
    const uint32_t blk_off = sa_block_parts ? 0u : (uint32_t)blk * p.sa_kb_stride * 4;
    s_voff0 = (uint32_t)src_row * p.sa_row_stride * 4 + blk_off;
    if (PART_SWIZZLE && !sa_block_parts)  // block blk ^ 2: two blocks on, or two back
      s_qodd = (blk & 2) ? 0u - 2u * (uint32_t)p.sa_kb_stride * 4u : 2u * (uint32_t)p.sa_kb_stride * 4u;
  } else {
    const int nb = SWIGLU ? min((lane == 0 ? 0 : p.inter / 128) + tn, p.nblocks - 1)
                          : min(col0 / 128 + lane, p.nblocks - 1);
    s_voff0 = (uint32_t)nb * p.sb_nb_stride * 4;
  }
  const uint32_t s_kb_bytes = (uint32_t)(a_scale_wave ? p.sa_kb_stride : p.sb_kb_stride) * 4;
  // (built from values made explicitly wave-uniform: the compiler otherwise keeps the descriptor in
  // vector registers and wraps every scale load in a loop over its distinct values)
  const __amdgpu_buffer_rsrc_t rS =
      make_rsrc(uniform_ptr(a_scale_wave ? (const void*)SA : (const void*)SB),
                __builtin_amdgcn_readfirstlane(a_scale_wave ? (uint32_t)p.a_src_rows * p.kblocks * 4
                                                            : (uint32_t)p.nblocks * p.kblocks * 4));

  // ---- this wave's output block --------------------------------------------------------------
  // Waves are numbered row-major over the WM x WN wave grid. Waves are dealt to the CU's 4 SIMDs
  // round-robin, so the waves of one row block sit on different SIMDs and a tile whose valid rows
  // cover only its first row blocks still spreads its work over all SIMDs.
  const int i0 = (wave / WN) * T::WTM;
  const int j0 = (wave % WN) * T::WTN;
  const int fr = lane & 15;
  bool wave_live = (row0 + i0 < row_end) && (col0 + j0 < p.n) && ((half_mask >> (i0 / 128)) & 1);
  // In the contiguous form a wave none of whose rows belongs to the expert holds padding (or the
  // other half's rows) only: one m_indices entry per lane, WTM == 64.
  // wave_ids: lane l holds the m_indices entry of this wave's row i0 + l (the epilogue reads its
  // rows' entries from here rather than from memory).
  int wave_ids = -1;
  if (CONTIG) {
    static_assert(T::WTM == 64, "one lane per wave row");
    wave_ids = tile_ids[0];
#pragma unroll
    for (int q = 1; q < QUARTERS; ++q)
      if (i0 == q * 64) wave_ids = tile_ids[q];
    wave_live = wave_live && __ballot(wave_ids == bsel) != 0;
  }

  f32x4 acc[T::IG][T::JG];

  // A zero-size resource: loads through it touch no memory and write zeros into LDS. The pipeline
  // uses it for the blocks past the end of K, so that every iteration issues the same loads (and
  // the scale loads of the modes that apply the scales in the epilogue).
  const __amdgpu_buffer_rsrc_t rNone = make_rsrc(A, 0);
  const __amdgpu_buffer_rsrc_t rSc = NO_PROMOTION ? rNone : rS;

  // Stages of K block kb: a's slabs, b's slabs, b's scales (after b's slabs).
  auto a_stage = [&](int kb) -> uint8_t* { return SPLIT ? smem : smem + (kb % STAGES) * T::STAGE_BYTES; };
  auto b_stage = [&](int kb) -> uint8_t* {
    return SPLIT ? smem + T::A_BYTES + (kb % T::B_STAGES) * T::B_SLOT : smem + (kb % STAGES) * T::STAGE_BYTES + T::A_BYTES;
  };

  // The loads of a K block go through the resources of the current iteration: rNone for the
  // blocks past the end of K. They are picked once per iteration (set_load_rsrc), not per load, and
  // by selects, not branches: a branch would split the scheduled block.
  __amdgpu_buffer_rsrc_t rA_it = rA, rB_it = rB, rS_it = rSc;
  auto set_load_rsrc = [&](bool a_live, bool b_live) {
    rA_it = a_live ? rA : rNone;
    rB_it = b_live ? rB : rNone;
    rS_it = b_live ? rSc : rNone;
  };
  auto issue_a = [&](int kb, int q) {
    load_lds_16(rA_it, a_stage(kb) + (wave * T::A_LOADS + q) * 1024, a_off[q], (uint32_t)kb * KBLK);
  };
  auto issue_b = [&](int kb, int q) {
    load_lds_16(rB_it, b_stage(kb) + (wave * T::B_LOADS + q) * 1024, b_off[q], (uint32_t)kb * b_kb_step);
  };
  auto issue_s = [&](int kb) {
    const int qq = kb & (SGRP - 1), grp = kb / SGRP + 1;
    uint8_t* dst = a_scale_wave ? smem + T::SA_RING_OFF + (grp % SA_SLOTS) * T::SA_SLOT + wave * 256 * SGRP + qq * 256
                                : b_stage(kb) + T::B_BYTES;
    const uint32_t soff = (uint32_t)(a_scale_wave ? grp * SGRP : kb) * s_kb_bytes;
    load_lds_4(rS_it, dst, s_voff0 + (uint32_t)qq * s_qstep + (uint32_t)(qq & 1) * s_qodd, soff);
  };
  // Spread load i of K block kb, i < SPREAD_LOADS: the scale load, then a's slabs (not in the split
  // pipeline, which loads them at once), then b's. The scale load goes first: its lines are
  // scattered (a's rows), and issued behind the slabs it finished last (measured: the contiguous
  // form 8% faster, the expert FFN 5%); the deferred schedule keeps it last, as first it makes the
  // compiler shuffle registers in that loop.
  auto issue_load = [&](int kb, int i_) {
    constexpr bool SCALE_LAST = !NO_PROMOTION && (MODE == MODE_PLAIN || MODE == MODE_MASKED);
    const int i = SCALE_LAST ? (i_ + 1) % T::SPREAD_LOADS : i_;
    if (i == 0)
      issue_s(kb);
    else if (!SPLIT && i <= T::A_LOADS)
      issue_a(kb, i - 1);
    else
      issue_b(kb, i - 1 - (SPLIT ? 0 : T::A_LOADS));
  };
  auto issue_a_all = [&](int kb) {
#pragma unroll
    for (int q = 0; q < T::A_LOADS; ++q) issue_a(kb, q);
  };
  // Split pipeline, mid-block: once every wave has read its a fragments of block kb (its LDS reads
  // retired, then the barrier), load block kb+1's. The memory clobber keeps those reads above the
  // barrier; the loads, side effects like the barrier, stay below it. (Unlike lds_pipeline_barrier,
  // no clobber after the barrier: with one, the deferred schedule spills registers.)
  auto split_refill_a = [&](int kb) {
    if constexpr (SPLIT) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      issue_a_all(kb + 1);
    }
  };
  // a's row scales of group 0 (K blocks 0 .. SGRP-1), ahead of the pipeline
  auto issue_scale_group0 = [&]() {
    if (a_scale_wave) {
#pragma unroll
      for (int qq = 0; qq < SGRP; ++qq)
        load_lds_4(rSc, smem + T::SA_RING_OFF + wave * 256 * SGRP + qq * 256,
                   s_voff0 + (uint32_t)qq * s_qstep + (uint32_t)(qq & 1) * s_qodd, 0);
    }
  };
  // a's scale of row i0 + 16 ig + fr (this lane's row of 16-row group ig) for K block kb. A wave's
  // rows lie in one 64-row part of the ring (WTM == 64), so the lane's offset is fixed.
  static_assert(T::WTM == 64, "a wave's rows are one a-scale wave's rows");
  // Row r = 16 ig + fr of the wave's 64: row parts put it in part (16 ig + fr) / PR, the odd parts
  // (fr >= 8 when PR = 8) with the block swizzle (block b at b ^ 2: 8 words on for b & 2 == 0, else
  // back); block parts at word r of block b.
  const int sa_lane_off = T::SA_RING_OFF + (i0 / 64) * 256 * SGRP +
                          (sa_block_parts ? fr * 4 : (fr / PART_ROWS) * 256 + (fr % PART_ROWS) * 4);
  const int sa_ig_step = sa_block_parts ? 64 : 16 / PART_ROWS * 256;
  const int sa_blk_step = sa_block_parts ? 256 : 4 * PART_ROWS;
  const int sa_lane_sw = (PART_SWIZZLE && !sa_block_parts && fr >= 8) ? 2 * 4 * PART_ROWS : 0;
  auto a_scale_at = [&](int kb, int ig) {
    const int b = kb & (SGRP - 1);
    const int sc = ((kb / SGRP) % SA_SLOTS) * T::SA_SLOT + ig * sa_ig_step + b * sa_blk_step;
    return *reinterpret_cast<const float*>(smem + sa_lane_off + sa_lane_sw * (1 - (b & 2)) + sc);
  };
  auto issue_loads = [&](int kb) {
#pragma unroll
    for (int i = 0; i < T::SPREAD_LOADS; ++i) issue_load(kb, i);
  };

  // One K block of this wave's MFMAs and promotions, in explicit issue order. The body is cut into
  // regions by full scheduling barriers: a prologue that reads the block's scales, the a fragments
  // and the first BPRE b fragments, then one region per column group jg that issues its share of
  // the next block's loads, reads the b fragment of group jg+BPRE, and alternates one MFMA of
  // group jg with the four promotion FMAs of group jg-1, so the matrix core never waits on a VALU
  // read of its own result and no LDS read is hoisted far ahead of its use.
  // BMM: the same issue order without scales -- each MFMA accumulates straight into acc, over all
  // of K, and the scales are applied once in the epilogue.
  auto compute_bmm = [&](int kb, int kb_load) {
    const uint8_t* sA = a_stage(kb);
    const uint8_t* sB = b_stage(kb);
    i32x8 af[T::IG];
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) af[ig] = load_frag(sA, i0 + ig * 16 + fr, lane);
    // b's fragment of column group jg (k-major b: four transposing reads instead of two)
    auto b_frag = [&](int jg) {
      if constexpr (B_KMAJOR)
        return load_frag_kn<BN>(sB, j0 + jg * 16, lane);
      else
        return load_frag(sB, j0 + jg * 16 + fr, lane);
    };
    constexpr int B_FRAG_READS = B_KMAJOR ? 4 : 2;
    i32x8 bq[T::JG];
#pragma unroll
    for (int jg = 0; jg < BPRE && jg < T::JG; ++jg) bq[jg] = b_frag(jg);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jg = 0; jg < T::JG; ++jg) {
#pragma unroll
      for (int i = load_first(jg); i < load_first(jg + 1); ++i) issue_load(kb_load, i);
      if (jg + BPRE < T::JG) bq[jg + BPRE] = b_frag(jg + BPRE);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig)
        acc[ig][jg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq[jg], af[ig], acc[ig][jg], FMT_E4M3, FMT_E4M3,
                                                                      0, E8M0_ONE, 0, E8M0_ONE);
      sched_vmem_group(load_first(jg + 1) - load_first(jg));
      if (jg + BPRE < T::JG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, B_FRAG_READS, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, T::IG, 0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto compute = [&](int kb, int kb_load) {
    const uint8_t* sA = a_stage(kb);
    const uint8_t* sB = b_stage(kb);
    const float* sSB = reinterpret_cast<const float*>(sB + T::B_BYTES);
    const float sbv = SWIGLU ? sSB[0] : sSB[(col0 + j0) / 128 - col0 / 128];
    const float sbv_up = SWIGLU ? sSB[1] : sbv;  // SWIGLU: the up columns' block
    float s[T::IG], s_up[T::IG];
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) {
      const float sav = a_scale_at(kb, ig);
      s[ig] = sav * sbv;
      s_up[ig] = SWIGLU ? sav * sbv_up : s[ig];
    }
    i32x8 af[T::IG];
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) af[ig] = load_frag(sA, i0 + ig * 16 + fr, lane);
    i32x8 bq[T::JG];
#pragma unroll
    for (int jg = 0; jg < BPRE && jg < T::JG; ++jg) bq[jg] = load_frag(sB, j0 + jg * 16 + fr, lane);
    __builtin_amdgcn_sched_barrier(0);
    split_refill_a(kb);
    f32x4 prod[T::JG][T::IG];
#pragma unroll
    for (int jg = 0; jg < T::JG; ++jg) {
#pragma unroll
      for (int i = load_first(jg); i < load_first(jg + 1); ++i) issue_load(kb_load, i);
      if (jg + BPRE < T::JG) bq[jg + BPRE] = load_frag(sB, j0 + (jg + BPRE) * 16 + fr, lane);
      __builtin_amdgcn_s_setprio(1);  // favour the wave that is issuing MFMAs
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) {
        prod[jg][ig] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bq[jg], af[ig], f32x4{0.f, 0.f, 0.f, 0.f}, FMT_E4M3, FMT_E4M3, 0, E8M0_ONE, 0, E8M0_ONE);
        if (jg > 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[ig][jg - 1][r] = __builtin_fmaf(prod[jg - 1][ig][r], jg - 1 < T::JG / 2 ? s[ig] : s_up[ig], acc[ig][jg - 1][r]);
        }
      }
      sched_vmem_group(load_first(jg + 1) - load_first(jg));
      if (jg + BPRE < T::JG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if (jg > 0) __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[ig][T::JG - 1][r] = __builtin_fmaf(prod[T::JG - 1][ig][r], s_up[ig], acc[ig][T::JG - 1][r]);
  };

  // Deferred schedule (plain and masked forms): the MFMAs of the last column group of block kb-1,
  // and the promotions of its last two groups, run after the barrier that opens block kb,
  // interleaved with the reads of block kb's a fragments, so the matrix core has work while those
  // reads are in flight. Their operands are already in registers, so the stage they came from may
  // be refilled. The products and every FP32 operation are those of `compute`, in the same order
  // per output: the results are identical. (The contiguous form's 256-row tiles would spill
  // registers with it, so the grouped forms keep `compute`.)
  constexpr bool DEFER = !NO_PROMOTION && (MODE == MODE_PLAIN || MODE == MODE_MASKED);
  constexpr int LGD = (T::JG - 1) < LOAD_GROUPS_DEFER ? (T::JG - 1) : LOAD_GROUPS_DEFER;
  constexpr auto load_first_d = [](int jg) { return ((jg < LGD ? jg : LGD) * T::SPREAD_LOADS + LGD - 1) / LGD; };
  static_assert(!DEFER || (T::JG >= 3 && BPRE < T::JG), "the deferred schedule needs three column groups");
  i32x8 dq_a[T::IG];
  i32x8 dq_b[T::JG];
  f32x4 dq_prod[T::JG][T::IG];
  float dq_s[T::IG];   // sa*sb of the block being computed
  float dq_sp[T::IG];  // sa*sb of the previous block, for its deferred promotions

  auto compute_deferred = [&](int kb, int kb_load, bool first) {
    const uint8_t* sA = a_stage(kb);
    const uint8_t* sB = b_stage(kb);
    const float* sSB = reinterpret_cast<const float*>(sB + T::B_BYTES);
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) dq_sp[ig] = dq_s[ig];
    const float sbv = sSB[(col0 + j0) / 128 - col0 / 128];
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) dq_s[ig] = a_scale_at(kb, ig) * sbv;
    dq_b[0] = load_frag(sB, j0 + fr, lane);
    __builtin_amdgcn_sched_barrier(0);
    if (!first) {
      // block kb-1: last group's MFMAs, the promotions of its second-to-last group, and this
      // block's a fragments read into the registers each MFMA has just consumed
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) {
        dq_prod[T::JG - 1][ig] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            dq_b[T::JG - 1], dq_a[ig], f32x4{0.f, 0.f, 0.f, 0.f}, FMT_E4M3, FMT_E4M3, 0, E8M0_ONE, 0, E8M0_ONE);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[ig][T::JG - 2][r] = __builtin_fmaf(dq_prod[T::JG - 2][ig][r], dq_sp[ig], acc[ig][T::JG - 2][r]);
        dq_a[ig] = load_frag(sA, i0 + ig * 16 + fr, lane);
      }
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) dq_a[ig] = load_frag(sA, i0 + ig * 16 + fr, lane);
    }
#pragma unroll
    for (int jg = 1; jg < BPRE; ++jg) dq_b[jg] = load_frag(sB, j0 + jg * 16 + fr, lane);
    __builtin_amdgcn_sched_barrier(0);
    split_refill_a(kb);
    // groups 0 .. JG-2 of block kb; group 0's MFMAs carry the last promotions of block kb-1
#pragma unroll
    for (int jg = 0; jg < T::JG - 1; ++jg) {
#pragma unroll
      for (int i = load_first_d(jg); i < load_first_d(jg + 1); ++i) issue_load(kb_load, i);
      if (jg + BPRE < T::JG) dq_b[jg + BPRE] = load_frag(sB, j0 + (jg + BPRE) * 16 + fr, lane);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) {
        dq_prod[jg][ig] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            dq_b[jg], dq_a[ig], f32x4{0.f, 0.f, 0.f, 0.f}, FMT_E4M3, FMT_E4M3, 0, E8M0_ONE, 0, E8M0_ONE);
        if (jg > 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[ig][jg - 1][r] = __builtin_fmaf(dq_prod[jg - 1][ig][r], dq_s[ig], acc[ig][jg - 1][r]);
        } else if (!first) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[ig][T::JG - 1][r] = __builtin_fmaf(dq_prod[T::JG - 1][ig][r], dq_sp[ig], acc[ig][T::JG - 1][r]);
        }
      }
      sched_vmem_group(load_first_d(jg + 1) - load_first_d(jg));
      if (jg + BPRE < T::JG) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if (jg > 0 || !first) __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // what the last block left deferred: its last group's MFMAs and its last two promotions
  auto compute_deferred_tail = [&]() {
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) {
      dq_prod[T::JG - 1][ig] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          dq_b[T::JG - 1], dq_a[ig], f32x4{0.f, 0.f, 0.f, 0.f}, FMT_E4M3, FMT_E4M3, 0, E8M0_ONE, 0, E8M0_ONE);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[ig][T::JG - 2][r] = __builtin_fmaf(dq_prod[T::JG - 2][ig][r], dq_s[ig], acc[ig][T::JG - 2][r]);
    }
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[ig][T::JG - 1][r] = __builtin_fmaf(dq_prod[T::JG - 1][ig][r], dq_s[ig], acc[ig][T::JG - 1][r]);
  };

  // Pipeline: K block kb (slabs and scales) lives in stage kb % STAGES. Iteration kb waits until
  // its own loads, issued STAGES-1 iterations earlier, have landed -- with three stages the loads of
  // kb+1 stay in flight -- synchronises the workgroup (which also retires every read of the stage
  // about to be refilled), then computes while issuing the loads of kb+STAGES-1. No load in the
  // loop targets a register, so nothing else makes the wave wait on memory.
  const int KB = p.kblocks;
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig)
#pragma unroll
    for (int jg = 0; jg < T::JG; ++jg) acc[ig][jg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) dq_s[ig] = 0.0f;
  if (KB > 0) {
    if constexpr (SPLIT) {
      // a and b of block 0, a's scale group 0, b of block 1 (block 0's wait covers all but the last)
      set_load_rsrc(true, true);
      issue_a_all(0);
      issue_loads(0);
      issue_scale_group0();
      set_load_rsrc(true, 1 < KB);
      issue_loads(1);
    } else {
#pragma unroll
      for (int b = 0; b < STAGES - 1; ++b) {
        set_load_rsrc(b < KB, b < KB);
        issue_loads(b);
        // group 0 of a's scales after block 0's slabs (which it must not delay) and before block
        // 1's (so that block 0's wait covers it)
        if (b == 0) issue_scale_group0();
      }
    }
  }

  for (int kb = 0; kb < KB; ++kb) {
    // block kb has landed once at most the loads of blocks kb+1 .. kb+STAGES-2 are in flight
    // (split: b's and the scales of block kb+1, issued after a's slabs of block kb)
    if constexpr (SPLIT)
      wait_vmcnt<T::SPREAD_LOADS>();
    else
      wait_vmcnt<(STAGES - 2) * T::LOADS>();
    lds_pipeline_barrier();
    const int kb_load = kb + (SPLIT ? 2 : STAGES - 1);
    set_load_rsrc(kb + (SPLIT ? 1 : STAGES - 1) < KB, kb_load < KB);
    if (wave_live) {
      if constexpr (NO_PROMOTION)
        compute_bmm(kb, kb_load);
      else if constexpr (DEFER) {
        if (kb == 0)
          compute_deferred(kb, kb_load, true);
        else
          compute_deferred(kb, kb_load, false);
      } else
        compute(kb, kb_load);
    } else {
      split_refill_a(kb);  // the same barriers as the computing waves
      issue_loads(kb_load);
    }
  }
  if constexpr (DEFER) {
    if (wave_live && KB > 0) compute_deferred_tail();
  }
  wait_vmcnt<0>();  // the zero-fill loads of the last iterations

  if constexpr (MODE == MODE_CONTIG_PT_SWIGLU) {
    swiglu_pt_epilogue<T, WN>(p, acc, row0, row_end, bsel, tn, i0, wave, lane, wave_live, wave_ids, pt_dequant,
                              pt_act_quant);
    return;
  } else if constexpr (SWIGLU) {
    swiglu_epilogue<T, WN>(p, acc, smem, row0, row_end, bsel, tn, i0, wave, lane, wave_live, wave_ids);
    return;
  }

  // ---- epilogue through LDS (plain, masked and contiguous forms, 16-bit output, all of the tile's
  // columns in range, n a multiple of 8): the waves write their rounded values into the now idle
  // stages as a BMxBN row-major tile, then every wave stores whole rows, 16 bytes per lane, so each
  // store instruction writes two (BN = 256) or four (BN = 128) complete 2*BN-byte row segments
  // instead of 16 rows x 32 bytes. In LDS the 8-byte unit c of tile row r sits at unit
  // c ^ (2 * (r & 15)): the 16 rows a fragment lane group writes land on distinct banks, and a lane's
  // two units of a 16-byte read stay adjacent. The contiguous form's row validity (the row's expert
  // is this tile's, and its half is covered here) travels as one byte per row after the tile.
  constexpr bool LDS_EPI_MODE = MODE == MODE_PLAIN || MODE == MODE_MASKED || MODE == MODE_CONTIG ||
                                MODE == MODE_CONTIG_PT;
  if constexpr (LDS_EPILOGUE && LDS_EPI_MODE) {
    static_assert(BM * BN * 2 + BM <= T::SA_RING_OFF, "the output tile and its row flags fit in the stages");
    if (p.out_scale == nullptr && (p.n & 7) == 0 && col0 + BN <= p.n) {  // uniform
      constexpr int PITCH = BN * 2;  // bytes per tile row
      uint8_t* row_flag = smem + BM * BN * 2;
      lds_pipeline_barrier();        // every wave has finished reading the stages
      if constexpr (CONTIG) {
        // the first wave of each row block: one flag per row of the block (lane l: row i0 + l)
        if (wave % WN == 0)
          row_flag[i0 + lane] = (wave_live && wave_ids == bsel && row0 + i0 + lane < row_end) ? 1 : 0;
      }
      if (wave_live) {
        const int jl = (lane >> 4) * 4;
        const float d = PT ? pt_dequant : 1.0f;
#pragma unroll
        for (int ig = 0; ig < T::IG; ++ig) {
          const int r = i0 + ig * 16 + fr;
#pragma unroll
          for (int jg = 0; jg < T::JG; ++jg) {
            const int c = (j0 + jg * 16 + jl) >> 2;  // 8-byte unit of the row
            f32x4 a = acc[ig][jg];
            if constexpr (PT) a *= d;
            uint2 v;
            if (p.out_fp16) {
              v.x = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[0], (_Float16)a[1]});
              v.y = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[2], (_Float16)a[3]});
            } else {
              v.x = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a[0], (__bf16)a[1]});
              v.y = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a[2], (__bf16)a[3]});
            }
            *reinterpret_cast<uint2*>(smem + r * PITCH + ((c ^ (2 * (r & 15))) << 3)) = v;
          }
        }
      }
      lds_pipeline_barrier();
      constexpr int LANES_PER_ROW = PITCH / 16;
      constexpr int ROWS_PER_STORE = 64 / LANES_PER_ROW;
      constexpr int ROWS_PER_WAVE = BM / T::NWAVES;
      const int u = 2 * (lane % LANES_PER_ROW);  // first 8-byte unit of this lane's 16 bytes
      uint16_t* O = p.out + (int64_t)g * p.out_group_stride;
#pragma unroll
      for (int s0 = 0; s0 < ROWS_PER_WAVE; s0 += ROWS_PER_STORE) {
        const int r = wave * ROWS_PER_WAVE + s0 + lane / LANES_PER_ROW;
        const uint4 v = *reinterpret_cast<const uint4*>(smem + r * PITCH + ((u ^ (2 * (r & 15))) << 3));
        const bool ok = CONTIG ? row_flag[r] != 0 : row0 + r < row_end;
        if (ok) *reinterpret_cast<uint4*>(O + (int64_t)(row0 + r) * p.n + col0 + 4 * u) = v;
      }
      return;
    }
  }

  // ---- epilogue: BF16 or FP16 round-to-nearest-even (8-byte stores), or E4M3 codes (4-byte
  // stores) when the plain form has an output scale; valid rows and columns only. A lane holds 4
  // consecutive columns; when n is not a multiple of 4 the row starts lose that alignment and each
  // column is stored on its own.
  if (wave_live) {
  const int jl = (lane >> 4) * 4;
  const bool vec = (p.n & 3) == 0;
  if constexpr (MODE == MODE_CONTIG_PT) {
    const float d = pt_dequant;
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig)
#pragma unroll
      for (int jg = 0; jg < T::JG; ++jg)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ig][jg][r] *= d;
  }
  if constexpr (MODE == MODE_BMM) {
    // out = sa * sb * acc in FP32 (one rounding per product), before the output rounding
    const float* SAg = p.sa + (p.bmm_sa_rows ? (int64_t)g * p.m : 0);
    const float* SBg = p.sb + (p.bmm_sb_cols ? (int64_t)g * p.n : 0);
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) {
      const int i = min(row0 + i0 + ig * 16 + fr, p.m - 1);
      const float sav = SAg[p.bmm_sa_rows ? i : 0];
#pragma unroll
      for (int jg = 0; jg < T::JG; ++jg) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = min(col0 + j0 + jg * 16 + jl + r, p.n - 1);
          acc[ig][jg][r] = acc[ig][jg][r] * (sav * SBg[p.bmm_sb_cols ? j : 0]);
        }
      }
    }
  }
  if (MODE == MODE_PLAIN && p.out_scale != nullptr) {
    const float so = out_scale;
    uint8_t* O = reinterpret_cast<uint8_t*>(p.out);
    auto codes4 = [&](const f32x4& a) {
      float q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        q[r] = __fdiv_rn(a[r], so);
        if (!(fabsf(q[r]) <= kE4M3MaxOut) && q[r] == q[r]) q[r] = copysignf(kE4M3MaxOut, q[r]);  // saturate; NaN stays
      }
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      return __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
    };
    if (vec && col0 + j0 + T::WTN <= p.n) {
      // all of the wave's columns in range: row addresses formed once, stores at immediate offsets
      int* rowp[T::IG];
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig)
        rowp[ig] = reinterpret_cast<int*>(O + (int64_t)(row0 + i0 + ig * 16 + fr) * p.n + col0 + j0 + jl);
#pragma unroll
      for (int ig = 0; ig < T::IG; ++ig) {
        if (row0 + i0 + ig * 16 + fr >= row_end) continue;
#pragma unroll
        for (int jg = 0; jg < T::JG; ++jg) rowp[ig][jg * 4] = codes4(acc[ig][jg]);  // 16 columns = 4 words
      }
    } else {
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) {
      const int i = row0 + i0 + ig * 16 + fr;
      if (i >= row_end) continue;
      uint8_t* orow = O + (int64_t)i * p.n;
#pragma unroll
      for (int jg = 0; jg < T::JG; ++jg) {
        const int j = col0 + j0 + jg * 16 + jl;
        if (j >= p.n) continue;
        const int w4 = codes4(acc[ig][jg]);
        if (vec) {
          *reinterpret_cast<int*>(orow + j) = w4;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (j + r < p.n) orow[j + r] = (uint8_t)((uint32_t)w4 >> (8 * r));
        }
      }
    }
    }  // columns reaching past n, or n not a multiple of 4
  } else {
  uint16_t* O = p.out + (int64_t)g * p.out_group_stride;
  int row_id[T::IG];  // contiguous form: m_indices of each lane's rows, from the wave's registers
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) row_id[ig] = CONTIG ? __shfl(wave_ids, ig * 16 + fr, 64) : 0;
  auto pack4 = [&](const f32x4& a) {
    uint2 v;
    if (p.out_fp16) {
      v.x = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[0], (_Float16)a[1]});
      v.y = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[2], (_Float16)a[3]});
    } else {
      v.x = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a[0], (__bf16)a[1]});
      v.y = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a[2], (__bf16)a[3]});
    }
    return v;
  };
  if (vec && col0 + j0 + T::WTN <= p.n) {
    // All of the wave's columns are in range: each lane's row addresses are formed once, before
    // the first store, and every store is an immediate offset from one of them. (A store whose
    // address registers are overwritten must first complete, so recomputing one address register
    // per store would make every store wait for the previous one.)
    uint2* rowp[T::IG];
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig)
      rowp[ig] = reinterpret_cast<uint2*>(O + (int64_t)(row0 + i0 + ig * 16 + fr) * p.n + col0 + j0 + jl);
#pragma unroll
    for (int ig = 0; ig < T::IG; ++ig) {
      const int i = row0 + i0 + ig * 16 + fr;
      if (!(i < row_end && (!CONTIG || row_id[ig] == bsel))) continue;
#pragma unroll
      for (int jg = 0; jg < T::JG; ++jg) rowp[ig][jg * 4] = pack4(acc[ig][jg]);  // 16 columns = 4 uint2
    }
  } else {
#pragma unroll
  for (int ig = 0; ig < T::IG; ++ig) {
    const int i = row0 + i0 + ig * 16 + fr;
    bool ok = i < row_end;
    if (CONTIG) ok = ok && row_id[ig] == bsel;
    if (!ok) continue;
    uint16_t* orow = O + (int64_t)i * p.n;
#pragma unroll
    for (int jg = 0; jg < T::JG; ++jg) {
      const int j = col0 + j0 + jg * 16 + jl;
      if (j >= p.n) continue;
      uint2 v;
      if (p.out_fp16) {
        const f16x2 lo = {(_Float16)acc[ig][jg][0], (_Float16)acc[ig][jg][1]};
        const f16x2 hi = {(_Float16)acc[ig][jg][2], (_Float16)acc[ig][jg][3]};
        v.x = __builtin_bit_cast(uint32_t, lo);
        v.y = __builtin_bit_cast(uint32_t, hi);
      } else {
        const bf16x2 lo = {(__bf16)acc[ig][jg][0], (__bf16)acc[ig][jg][1]};
        const bf16x2 hi = {(__bf16)acc[ig][jg][2], (__bf16)acc[ig][jg][3]};
        v.x = __builtin_bit_cast(uint32_t, lo);
        v.y = __builtin_bit_cast(uint32_t, hi);
      }
      if (vec) {
        *reinterpret_cast<uint2*>(orow + j) = v;
      } else {
        const uint16_t e[4] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16)};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j + r < p.n) orow[j + r] = e[r];
      }
    }
  }
  }  // columns reaching past n, or n not a multiple of 4
  }  // 16-bit output
  }  // wave_live
}

template <int BM, int BN, int WM, int WN, int STAGES>
hipError_t launch_cfg(GemmMode mode, const GemmParams& p, int grid, hipStream_t stream) {
  const dim3 block(WM * WN * 64);
  switch (mode) {
    case MODE_PLAIN:
      hipLaunchKernelGGL((gemm_fp8_groupwise_kernel<BM, BN, WM, WN, STAGES, MODE_PLAIN>), dim3(grid), block, 0, stream, p);
      break;
    case MODE_CONTIG:
      hipLaunchKernelGGL((gemm_fp8_groupwise_kernel<BM, BN, WM, WN, STAGES, MODE_CONTIG>), dim3(grid), block, 0, stream, p);
      break;
    case MODE_MASKED:
      hipLaunchKernelGGL((gemm_fp8_groupwise_kernel<BM, BN, WM, WN, STAGES, MODE_MASKED>), dim3(grid), block, 0, stream, p);
      break;
    case MODE_BMM:
      hipLaunchKernelGGL((gemm_fp8_groupwise_kernel<BM, BN, WM, WN, STAGES, MODE_BMM>), dim3(grid), block, 0, stream, p);
      break;
    case MODE_CONTIG_PT:
      hipLaunchKernelGGL((gemm_fp8_groupwise_kernel<BM, BN, WM, WN, STAGES, MODE_CONTIG_PT>), dim3(grid), block, 0, stream, p);
      break;
    case MODE_CONTIG_PT_SWIGLU:
      if constexpr (BN == 256) {
        hipLaunchKernelGGL((gemm_fp8_groupwise_kernel<BM, BN, WM, WN, STAGES, MODE_CONTIG_PT_SWIGLU>), dim3(grid), block,
                           0, stream, p);
        break;
      }
      return hipErrorInvalidValue;
    case MODE_CONTIG_SWIGLU:
      if constexpr (BN == 256) {
        hipLaunchKernelGGL((gemm_fp8_groupwise_kernel<BM, BN, WM, WN, STAGES, MODE_CONTIG_SWIGLU>), dim3(grid), block, 0,
                           stream, p);
        break;
      }
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kernels

using namespace kernels;

int tile_rows(TileConfig cfg) { return (cfg == TILE_128x256 || cfg == TILE_128x128) ? 128 : 256; }
int tile_cols(TileConfig cfg) {
  return (cfg == TILE_256x128 || cfg == TILE_128x128) ? 128 : 256;
}

hipError_t gemm_clock_record(unsigned long long* host4) {
  return hipMemcpyFromSymbol(host4, HIP_SYMBOL(kernels::g_gemm_clock), 4 * sizeof(unsigned long long));
}

hipError_t launch_gemm(GemmMode mode, TileConfig cfg, GemmParams p, int grid, hipStream_t stream) {
  switch (cfg) {
    case TILE_256x256: return launch_cfg<256, 256, 4, 2, 2>(mode, p, grid, stream);
    case TILE_128x256: return launch_cfg<128, 256, 2, 4, 3>(mode, p, grid, stream);
    case TILE_256x128: return launch_cfg<256, 128, 4, 2, 3>(mode, p, grid, stream);
    case TILE_128x128: return launch_cfg<128, 128, 2, 2, 4>(mode, p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fp8g
