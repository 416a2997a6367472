// Internal interface between the C-ABI layer (api.hip) and the kernel files (gemm.hip, moe.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8g {

// Which tile scheduler the GEMM kernel runs.
enum GemmMode : int {
  MODE_PLAIN = 0,   // out = a @ b.T
  MODE_CONTIG = 1,  // per 128-row tile, b chosen by the tile's expert in m_indices
  MODE_MASKED = 2,  // per group g, rows below masked_m[g]
  MODE_CONTIG_SWIGLU = 3,  // contiguous, epilogue silu(gate) * up -> 1x128 E4M3 (expert-FFN fc1)
  MODE_BMM = 4,     // per batch g: out = sa * sb * (a @ b), b (k, n); scales per tensor or per row / column
  MODE_CONTIG_PT = 5,         // contiguous, out = group_dequant[e] * (a @ b[e].T) (per-tensor FP8)
  MODE_CONTIG_PT_SWIGLU = 6,  // contiguous per-tensor, epilogue E4M3(silu(gate) * up * act_quant)
};

// Everything the GEMM kernel needs, passed by value as the kernel argument. Strides in elements.
struct GemmParams {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  uint16_t* out;           // BF16, or FP16 when out_fp16; E4M3 bytes when out_scale is set
  const int32_t* rowinfo;  // m_indices (CONTIG) or masked_m (MASKED)
  const int32_t* a_rows;   // CONTIG only: row r of the product takes row a_rows[r] of a; null: r
  int32_t a_src_rows;      // rows of a (and of a_scale) in memory
  // CONTIG_SWIGLU: b holds gate rows [0, inter) then up rows [inter, 2 inter); column tile t
  // computes gate and up of output columns [128 t, 128 t + 128) and writes
  // q_out[r][c] = E4M3(silu(gate) * up / q_scale_out[r][t]) with a 1x128 scale per row and tile.
  int32_t out_fp16;
  // PLAIN only: E4M3 output, out[i][j] = E4M3_RNE(saturate(acc / out_scale[0])); null: 16-bit output
  const float* out_scale;
  // BMM: a_scale holds one value (0) or one per row of each batch (1); b_scale one value or one per
  // column of each batch; scale groups are m (a) and n (b) values apart.
  int32_t bmm_sa_rows, bmm_sb_cols;
  // CONTIG_PT(_SWIGLU): one dequantisation scale per group (expert) applied to the FP32 sum; the
  // SWIGLU form multiplies h by act_quant[e] (act_quant_per_group) or act_quant[0] and writes E4M3.
  const float* group_dequant;
  const float* act_quant;
  int32_t act_quant_per_group;
  int32_t inter;
  uint8_t* q_out;
  float* q_scale_out;
  int64_t a_group_stride, b_group_stride, sa_group_stride, sb_group_stride, out_group_stride;
  int32_t m;  // PLAIN/CONTIG: rows of a; MASKED: max_m
  int32_t n, k;
  int32_t kblocks, nblocks;
  int32_t sa_row_stride, sa_kb_stride;  // a_scale element of (row, kb)
  int32_t sb_nb_stride, sb_kb_stride;   // b_scale element of (n block, kb)
  int32_t num_groups;
  int32_t tiles_m, tiles_n, group_m;
  // group_n > 0: tiles are rastered in bands of group_n column tiles (consecutive tiles walk the
  // band's column tiles for one row tile, then the next row tile); else in bands of group_m row tiles
  int32_t group_n;
};

// Tile configurations the host may pick. Results are identical for every configuration.
enum TileConfig : int {
  TILE_256x256 = 0,  // 8 waves as 4 (rows) x 2 (cols), 64x128 per wave, 2 LDS stages
  TILE_128x256 = 1,  // 8 waves as 2 x 4, 64x64 per wave, 3 LDS stages
  TILE_256x128 = 2,  // 8 waves as 4 x 2, 64x64 per wave, 3 LDS stages
  TILE_128x128 = 3,  // 4 waves as 2 x 2, 64x64 per wave, 4 LDS stages (weight streaming)
};

// Tile configuration forced through the FP8G_TILE environment variable ("256x256", "128x256",
// "256x128", "128x128"), read at every call; -1 when unset. For tuning and for the tests that check that
// results never depend on the tile. The contiguous form uses 128x256 tiles by default and 256x256
// tiles for short K with large expert regions (k <= 2048 and at least 512 rows per expert on
// average); with 256-row tiles the grid holds one entry per 128-row half, and a tile whose halves
// belong to different experts runs as two workgroups, each covering its own half.
int tile_override();
// Row tiles per raster group, forced through the FP8G_GROUP_M environment variable (a positive
// integer), read at every call; `group_m` when unset. Tile order only: results never change.
int group_m_override(int group_m);
// Column tiles per raster band (GemmParams::group_n), forced through FP8G_GROUP_N (0 turns the
// bands off), read at every call; `group_n` when unset. Tile order only: results never change.
int group_n_override(int group_n);

int tile_rows(TileConfig cfg);
int tile_cols(TileConfig cfg);

hipError_t launch_gemm(GemmMode mode, TileConfig cfg, GemmParams p, int grid, hipStream_t stream);

hipError_t launch_quantize_rows_1x128(const uint16_t* x, const int32_t* src_row, int num_src, int rows, int cols,
                                      uint8_t* out, float* scale_out, bool mn_major, hipStream_t stream);
hipError_t launch_quantize_1x128(const uint16_t* x, int rows, int cols, uint8_t* out, float* scale_out,
                                 bool mn_major, hipStream_t stream);
hipError_t launch_fused_add_rmsnorm_quant(const uint16_t* input, uint16_t* residual, const uint16_t* weight,
                                          float eps, int rows, int hidden, uint16_t* normed_out, uint8_t* out,
                                          float* scale_out, bool mn_major, hipStream_t stream);

// The permutation's scratch: one int32 per (chunk of 1024 routing entries, expert).
int64_t moe_permutation_scratch_ints(int64_t entries, int64_t num_experts);
// The library's own permutation scratch (a device array of kPermScratchInts int32, one copy per
// device, held until the process ends), for callers that cannot allocate; `device` must be current.
constexpr int64_t kPermScratchInts = 1 << 20;  // 4 MiB
constexpr int kMaxScratchDevices = 64;
hipError_t permutation_scratch(int device, int32_t** ptr);
hipError_t launch_moe_build_permutation(const int32_t* topk_ids, int num_tokens, int top_k,
                                        int num_experts, int m_alloc, int32_t* m_indices,
                                        int32_t* src_token, int32_t* row_of_entry, int32_t* hist,
                                        hipStream_t stream);
hipError_t launch_moe_gather_quant(const uint16_t* x, const int32_t* src_token, int num_tokens,
                                   int hidden, int m_alloc, uint8_t* a_out, float* a_scale_out,
                                   hipStream_t stream);
hipError_t launch_moe_silu_mul_quant(const uint16_t* y, const int32_t* m_indices, int rows,
                                     int inter, uint8_t* a_out, float* a_scale_out,
                                     hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t* y, const int32_t* row_of_entry,
                              const float* topk_weights, int num_tokens, int top_k, int hidden,
                              int m_alloc, uint16_t* out, bool out_fp16, hipStream_t stream);

// Stamps of the first workgroup of the most recent GEMM launch on the current device (start cycles,
// start wall ticks, end cycles, end wall ticks), copied to host memory; synchronous.
hipError_t gemm_clock_record(unsigned long long* host4);
// One wave spinning for spin_ticks of the wall clock; out[0] = shader-clock cycles, out[1] = wall ticks.
hipError_t launch_clock_probe(unsigned long long* out, unsigned long long spin_ticks, hipStream_t stream);

}  // namespace fp8g
