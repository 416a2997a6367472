// C ABI of libfp8g.so: argument validation, tile-configuration choice and launch.
//
// Conventions (flashmla-rs README, section "Design Notes"): caller-owned memory, work enqueued on
// the caller's stream without synchronisation, exceptions caught at the boundary and reported as a
// status plus a thread-local message. Validation happens before any launch (flashmla-rs README,
// section "flashmla"), and a device other than gfx950 is an error rather than a fallback
// (flashinfer-rs README, section "Architecture Handling").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <string>

#include "../../include/fp8g.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

struct Failure {
  fp8g_status_t status;
};

[[noreturn]] void fail(fp8g_status_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  throw Failure{status};
}

void require(bool cond, const char* fmt, ...) {
  if (cond) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  throw Failure{FP8G_INVALID_ARGUMENT};
}

void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(FP8G_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device answer to "is this a gfx950?": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

void check_device() {
  int dev = -1;
  check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) fail(FP8G_NOT_SUPPORTED, "device ordinal %d out of range", dev);
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    check_hip(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
    if (state == 2)
      fail(FP8G_NOT_SUPPORTED, "device %d is %s; this library runs on gfx950 (MI355X) only", dev,
           prop.gcnArchName);
  }
  if (state == 2) fail(FP8G_NOT_SUPPORTED, "device %d is not a gfx950 (MI355X)", dev);
}

void check_granularity(int32_t gm, int32_t gn, int32_t gk) {
  if (gm != 1 || gn != 128 || gk != 128)
    fail(FP8G_NOT_SUPPORTED, "scale granularity (%d,%d,%d) not supported; only (1,128,128)", gm, gn, gk);
}

void check_out_dtype(int32_t dt) {
  require(dt == FP8G_OUT_BF16 || dt == FP8G_OUT_FP16, "out_dtype must be 0 (BF16) or 1 (FP16), got %d", dt);
}

void check_scale_major(int32_t sm) {
  require(sm == FP8G_SCALE_K_MAJOR || sm == FP8G_SCALE_MN_MAJOR, "scale_major must be 0 (K) or 1 (MN), got %d", sm);
}

constexpr int64_t kInt32Max = 2147483647;
constexpr int64_t kUint32Max = 4294967295LL;

template <typename F>
fp8g_status_t guarded(F&& body) {
  try {
    g_last_error.clear();
    body();
    return FP8G_OK;
  } catch (const Failure& f) {
    return f.status;
  } catch (const std::exception& e) {
    g_last_error = std::string("internal error: ") + e.what();
    return FP8G_INTERNAL;
  } catch (...) {
    g_last_error = "internal error: unknown exception";
    return FP8G_INTERNAL;
  }
}

// Shapes shared by the three GEMM forms.
// n_tail: the plain form takes any n (the last b-scale block then covers fewer than 128 rows of b);
// the grouped and masked forms need whole 128-row blocks.
void check_gemm_dims(int64_t rows, int64_t n, int64_t k, bool n_tail = false) {
  require(rows >= 0 && n >= 0 && k >= 0, "sizes must be non-negative (rows %lld, n %lld, k %lld)",
          (long long)rows, (long long)n, (long long)k);
  require(k % 128 == 0, "k (%lld) must be a multiple of 128", (long long)k);
  require(n_tail || n % 128 == 0, "n (%lld) must be a multiple of 128", (long long)n);
  require(rows <= kInt32Max && n <= kInt32Max && k <= kInt32Max, "sizes must fit in int32");
  require(rows * k <= kUint32Max && n * k <= kUint32Max, "one operand matrix must stay below 4 GiB");
  require(rows * (k / 128) <= kInt32Max, "a_scale must have fewer than 2^31 elements per group");
}

void check_operands(const void* a, const void* b, const float* sa, const float* sb, const void* out, int64_t k) {
  // with k == 0 the operands and scales are empty and may be null; out is still written
  require(out != nullptr, "out must be non-null");
  require(k == 0 || (a && b && sa && sb), "a, b, a_scale and b_scale must be non-null");
  require(aligned(a, 16) && aligned(b, 16) && aligned(out, 16), "a, b and out must be 16-byte aligned");
  require(aligned(sa, 4) && aligned(sb, 4), "scales must be 4-byte aligned");
}

void set_scale_strides(fp8g::GemmParams& p, int32_t scale_major, int64_t rows) {
  const int32_t kb = p.kblocks, nb = p.nblocks;
  if (scale_major == FP8G_SCALE_K_MAJOR) {
    p.sa_row_stride = kb;
    p.sa_kb_stride = 1;
    p.sb_nb_stride = kb;
    p.sb_kb_stride = 1;
  } else {
    p.sa_row_stride = 1;
    p.sa_kb_stride = (int32_t)rows;
    p.sb_nb_stride = 1;
    p.sb_kb_stride = nb;
  }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// a * b for non-negative sizes, saturated at INT64_MAX instead of overflowing (validation compares
// products of caller-supplied sizes against limits before anything is narrowed).
int64_t mul_sat(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

}  // namespace

int fp8g::group_m_override(int group_m) {
  const char* e = std::getenv("FP8G_GROUP_M");
  if (!e) return group_m;
  const int v = std::atoi(e);
  return v > 0 ? v : group_m;
}

int fp8g::group_n_override(int group_n) {
  const char* e = std::getenv("FP8G_GROUP_N");
  if (!e) return group_n;
  return std::atoi(e);
}

int fp8g::tile_override() {
  const char* e = std::getenv("FP8G_TILE");
  if (!e) return -1;
  if (!std::strcmp(e, "256x256")) return (int)TILE_256x256;
  if (!std::strcmp(e, "128x256")) return (int)TILE_128x256;
  if (!std::strcmp(e, "256x128")) return (int)TILE_256x128;
  if (!std::strcmp(e, "128x128")) return (int)TILE_128x128;
  return -1;
}

namespace {

const char* mode_name(fp8g::GemmMode mode) {
  switch (mode) {
    case fp8g::MODE_PLAIN: return "plain";
    case fp8g::MODE_CONTIG: return "contiguous";
    case fp8g::MODE_MASKED: return "masked";
    case fp8g::MODE_CONTIG_SWIGLU: return "contiguous+silu-quant";
    case fp8g::MODE_BMM: return "bmm";
    case fp8g::MODE_CONTIG_PT: return "contiguous per-tensor";
    case fp8g::MODE_CONTIG_PT_SWIGLU: return "contiguous per-tensor+silu-quant";
  }
  return "?";
}

// Launch a GEMM; with FP8G_LOG set (to anything but "0") the call, its sizes and the tile
// configuration chosen are written to stderr first. Read at every call, like FP8G_TILE.
void launch_logged(const char* what, fp8g::GemmMode mode, fp8g::TileConfig cfg, const fp8g::GemmParams& p,
                   int64_t grid, void* stream) {
  const char* env = std::getenv("FP8G_LOG");
  if (env && *env && std::strcmp(env, "0") != 0)
    std::fprintf(stderr, "fp8g: %s [%s] m=%d n=%d k=%d groups=%d tile=%dx%d grid=%lld tiles=%dx%d stream=%p\n", what,
                 mode_name(mode), p.m, p.n, p.k, p.num_groups, fp8g::tile_rows(cfg), fp8g::tile_cols(cfg),
                 (long long)grid, p.tiles_m, p.tiles_n, stream);
  check_hip(fp8g::launch_gemm(mode, cfg, p, (int)grid, (hipStream_t)stream), what);
}

}  // namespace

extern "C" {

const char* fp8g_last_error(void) { return g_last_error.c_str(); }

fp8g_status_t fp8g_clock_probe(unsigned long long* out, int64_t spin_us, void* stream) {
  return guarded([&] {
    require(out != nullptr && aligned(out, 8), "out must be non-null and 8-byte aligned");
    require(spin_us >= 0 && spin_us <= 100000, "spin_us must be in [0, 100000]");
    check_device();
    int dev = 0, khz = 0;
    check_hip(hipGetDevice(&dev), "hipGetDevice");
    check_hip(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev), "wall clock rate");
    check_hip(fp8g::launch_clock_probe(out, (unsigned long long)spin_us * (unsigned long long)khz / 1000,
                                       (hipStream_t)stream),
              "fp8g_clock_probe launch");
  });
}

fp8g_status_t fp8g_gemm_clock_record(unsigned long long* host_out) {
  return guarded([&] {
    require(host_out != nullptr, "host_out must be non-null");
    check_device();
    check_hip(fp8g::gemm_clock_record(host_out), "fp8g_gemm_clock_record");
  });
}

int64_t fp8g_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}

int32_t fp8g_version(void) { return 100; }  // 0.1.0

}  // extern "C"

namespace {

// The plain form for both output kinds: 16-bit (out_dtype) or E4M3 with out_scale.
void plain_gemm(const void* a, const void* b, const float* a_scale, const float* b_scale, void* out,
                int32_t out_dtype, const float* out_scale, int64_t m, int64_t n, int64_t k, int32_t scale_major,
                int32_t gran_m, int32_t gran_n, int32_t gran_k, void* stream, const char* what) {
  check_gemm_dims(m, n, k, /*n_tail=*/true);
  check_scale_major(scale_major);
  check_granularity(gran_m, gran_n, gran_k);
  if (out_scale == nullptr) check_out_dtype(out_dtype);
  if (m == 0 || n == 0) return;
  check_operands(a, b, a_scale, b_scale, out, k);
  fp8g::GemmParams p{};
  p.a = static_cast<const uint8_t*>(a);
  p.b = static_cast<const uint8_t*>(b);
  p.sa = a_scale;
  p.sb = b_scale;
  p.out = static_cast<uint16_t*>(out);
  p.out_fp16 = out_dtype == FP8G_OUT_FP16;
  p.out_scale = out_scale;
  p.m = (int32_t)m;
  p.n = (int32_t)n;
  p.k = (int32_t)k;
  p.kblocks = (int32_t)(k / 128);
  p.nblocks = (int32_t)ceil_div(n, 128);
  p.num_groups = 1;
  p.a_src_rows = (int32_t)m;
  set_scale_strides(p, scale_major, m);
  fp8g::TileConfig cfg = m > 128 ? fp8g::TILE_256x256 : fp8g::TILE_128x256;
  if (fp8g::tile_override() >= 0) cfg = (fp8g::TileConfig)fp8g::tile_override();
  p.tiles_m = (int32_t)ceil_div(m, fp8g::tile_rows(cfg));
  p.tiles_n = (int32_t)ceil_div(n, fp8g::tile_cols(cfg));
  p.group_m = fp8g::group_m_override(4);
  const int64_t grid = mul_sat(p.tiles_m, p.tiles_n);
  require(grid <= kInt32Max, "too many tiles");
  check_device();
  launch_logged(what, fp8g::MODE_PLAIN, cfg, p, grid, stream);
}

}  // namespace

extern "C" {

fp8g_status_t fp8_gemm_nt_groupwise(const void* a, const void* b, const float* a_scale,
                                    const float* b_scale, void* out, int32_t out_dtype, int64_t m,
                                    int64_t n, int64_t k, int32_t scale_major, int32_t gran_m,
                                    int32_t gran_n, int32_t gran_k, void* stream) {
  return guarded([&] {
    plain_gemm(a, b, a_scale, b_scale, out, out_dtype, nullptr, m, n, k, scale_major, gran_m, gran_n, gran_k, stream,
               "fp8_gemm_nt_groupwise launch");
  });
}

fp8g_status_t fp8_gemm_nt_groupwise_fp8_out(const void* a, const void* b, const float* a_scale,
                                            const float* b_scale, void* out, const float* output_scale,
                                            int64_t m, int64_t n, int64_t k, int32_t scale_major,
                                            int32_t gran_m, int32_t gran_n, int32_t gran_k, void* stream) {
  return guarded([&] {
    require(output_scale != nullptr, "output_scale must be non-null");
    require(aligned(output_scale, 4), "output_scale must be 4-byte aligned");
    plain_gemm(a, b, a_scale, b_scale, out, FP8G_OUT_BF16, output_scale, m, n, k, scale_major, gran_m, gran_n,
               gran_k, stream, "fp8_gemm_nt_groupwise_fp8_out launch");
  });
}

}  // extern "C"

namespace {

// The contiguous form, with a's rows read directly (a_rows null, a_src_rows == m) or gathered.
// With q_out non-null (the expert FFN's fc1), b holds gate then up rows (n = 2 inter) and the
// epilogue writes silu(gate) * up, 1x128-quantised, to q_out / q_scale_out instead of out.
void group_gemm_contiguous(const void* a, const float* a_scale, int64_t a_src_rows, const int32_t* a_rows,
                           const void* b, const float* b_scale, const int32_t* m_indices, void* out, int64_t m,
                           int64_t n, int64_t k, int64_t num_groups, int32_t scale_major, int32_t gran_m,
                           int32_t gran_n, int32_t gran_k, void* stream, const char* what,
                           int32_t out_dtype = FP8G_OUT_BF16, void* q_out = nullptr, float* q_scale_out = nullptr,
                           const float* group_dequant = nullptr, const float* act_quant = nullptr,
                           int32_t act_quant_per_group = 0) {
  const bool swiglu = q_out != nullptr;
  const bool pt = group_dequant != nullptr;  // per-tensor FP8: one dequantisation scale per group
  check_out_dtype(out_dtype);
  check_gemm_dims(m, n, k);
  check_gemm_dims(a_src_rows, n, k);
  require(num_groups >= 0 && num_groups <= kInt32Max, "num_groups must be in [0, 2^31)");
  require(m % 128 == 0, "m (%lld) must be a multiple of 128 (128-row-aligned expert regions)", (long long)m);
  check_scale_major(scale_major);
  check_granularity(gran_m, gran_n, gran_k);
  if (m == 0 || n == 0 || num_groups == 0) return;
  if (pt) {
    require((swiglu ? q_out : out) != nullptr, "the output must be non-null");
    require(k == 0 || (a && b), "a and b must be non-null");
    require(aligned(a, 16) && aligned(b, 16) && aligned(swiglu ? q_out : out, 16),
            "a, b and the output must be 16-byte aligned");
    require(aligned(group_dequant, 4), "the dequantisation scales must be 4-byte aligned");
    if (swiglu) require(act_quant != nullptr && aligned(act_quant, 4), "fc2_quant must be non-null and 4-byte aligned");
  } else {
    check_operands(a, b, a_scale, b_scale, swiglu ? q_out : out, k);
  }
  require(m_indices != nullptr && aligned(m_indices, 4), "m_indices must be non-null and 4-byte aligned");
  require(a_rows == nullptr || aligned(a_rows, 4), "a_rows must be 4-byte aligned");
  if (swiglu && !pt) {
    require(n % 256 == 0, "2*inter (%lld) must be a multiple of 256", (long long)n);
    require(q_scale_out != nullptr && aligned(q_scale_out, 4) && aligned(q_out, 16),
            "q_out must be 16-byte aligned and q_scale_out non-null and 4-byte aligned");
  }
  if (swiglu) require(n % 256 == 0, "2*inter (%lld) must be a multiple of 256", (long long)n);
  require(k == 0 || a_src_rows > 0, "a must have at least one row");
  check_device();
  fp8g::GemmParams p{};
  p.a = static_cast<const uint8_t*>(a);
  p.b = static_cast<const uint8_t*>(b);
  p.sa = a_scale;
  p.sb = b_scale;
  p.out = static_cast<uint16_t*>(out);
  p.out_fp16 = out_dtype == FP8G_OUT_FP16;
  p.rowinfo = m_indices;
  p.a_rows = a_rows;
  p.inter = (int32_t)(n / 2);
  p.q_out = static_cast<uint8_t*>(q_out);
  p.q_scale_out = q_scale_out;
  p.group_dequant = group_dequant;
  p.act_quant = act_quant;
  p.act_quant_per_group = act_quant_per_group;
  p.a_src_rows = (int32_t)a_src_rows;
  p.m = (int32_t)m;
  p.n = (int32_t)n;
  p.k = (int32_t)k;
  p.kblocks = (int32_t)(k / 128);
  p.nblocks = (int32_t)(n / 128);
  p.num_groups = (int32_t)num_groups;
  p.b_group_stride = n * k;
  p.sb_group_stride = (n / 128) * (k / 128);
  set_scale_strides(p, scale_major, a_src_rows);
  // 128x256 tiles: the weights stream from HBM here, and the three-stage pipeline of that tile
  // hides the latency better than the two stages of the 256x256 tile. With 256-row tiles a tile
  // whose two 128-row halves hold different experts is split into two workgroups, so the grid
  // counts two entries per 256-row tile.
  // Short K with large expert regions (the expert FFN's fc2: k = 2048, about 600 rows per expert):
  // a K loop of 16 blocks pays a tile's prologue and epilogue often, and 256x256 tiles halve their
  // number (measured at the 4096-token FFN workload: 796 against 854 us with block scales, 723
  // against 789 us with per-tensor scales; fc1 gains nothing from them).
  fp8g::TileConfig cfg = (!swiglu && k <= 2048 && m >= 512 * num_groups) ? fp8g::TILE_256x256
                                                                         : fp8g::TILE_128x256;
  if (fp8g::tile_override() >= 0) cfg = (fp8g::TileConfig)fp8g::tile_override();
  if (swiglu && fp8g::tile_cols(cfg) != 256) cfg = fp8g::TILE_128x256;  // gate and up share a 256-wide tile
  p.tiles_m = (int32_t)(ceil_div(m, fp8g::tile_rows(cfg)) * (fp8g::tile_rows(cfg) / 128));
  p.tiles_n = swiglu ? (int32_t)(n / 256) : (int32_t)ceil_div(n, fp8g::tile_cols(cfg));
  // 128-row tiles with a gathered a (the expert FFN's fc1): the row tiles of one column tile run
  // together and share b's slab in L2; a's rows come from the much smaller token matrix, whose
  // re-reads hit in cache. 128-row tiles with a read in place: bands of 8 column tiles, so an
  // XCD's 32 workgroups are 4 row tiles x 8 column tiles that share both a's rows and b's slabs
  // in L2 (a is otherwise re-read once per column tile). Measured against the column order: 32
  // Zipf experts x 8192 rows (n 4096, k 7168) 343 against 363 us, 64 x 512 rows 1045 against
  // 1115, 64 Zipf x 16384 660 against 733, k 2048 / n 7168 199 against 208, and 2-4% on experts
  // whose row tiles straddle the bands (64 x 576 or 520 rows, 32 x 300, 8 x 2000); the gathered
  // fc1 1393-1402 against 1304 us, so it keeps the column order. (The expert FFN's fc2, k 2048,
  // takes 256-row tiles; on 128-row tiles it measured 735 with bands against 686 us.)
  // 256-row tiles: the column tiles of one row tile run together and share a's rows in L2 (each
  // expert's weights are streamed once either way); measured 1.8x faster for them.
  p.group_m = fp8g::group_m_override(fp8g::tile_rows(cfg) == 256 ? 1 : p.tiles_m);
  p.group_n = fp8g::group_n_override(a_rows == nullptr && fp8g::tile_rows(cfg) == 128 ? 8 : 0);
  const int64_t grid = mul_sat(p.tiles_m, p.tiles_n);
  require(grid <= kInt32Max, "too many tiles");
  const fp8g::GemmMode mode = pt ? (swiglu ? fp8g::MODE_CONTIG_PT_SWIGLU : fp8g::MODE_CONTIG_PT)
                                 : (swiglu ? fp8g::MODE_CONTIG_SWIGLU : fp8g::MODE_CONTIG);
  launch_logged(what, mode, cfg, p, grid, stream);
}

}  // namespace

extern "C" {

fp8g_status_t fp8_group_gemm_contiguous(const void* a, const void* b, const float* a_scale,
                                        const float* b_scale, const int32_t* m_indices, void* out,
                                        int32_t out_dtype, int64_t m, int64_t n, int64_t k,
                                        int64_t num_groups, int32_t scale_major, int32_t gran_m,
                                        int32_t gran_n, int32_t gran_k, void* stream) {
  return guarded([&] {
    group_gemm_contiguous(a, a_scale, m, nullptr, b, b_scale, m_indices, out, m, n, k, num_groups, scale_major,
                          gran_m, gran_n, gran_k, stream, "fp8_group_gemm_contiguous launch", out_dtype);
  });
}

fp8g_status_t fp8_group_gemm_contiguous_gather(const void* a, const float* a_scale, int64_t a_rows_total,
                                               const int32_t* a_rows, const void* b, const float* b_scale,
                                               const int32_t* m_indices, void* out, int32_t out_dtype,
                                               int64_t m, int64_t n, int64_t k, int64_t num_groups,
                                               int32_t scale_major, int32_t gran_m, int32_t gran_n,
                                               int32_t gran_k, void* stream) {
  return guarded([&] {
    require(m == 0 || a_rows != nullptr, "a_rows must be non-null");
    group_gemm_contiguous(a, a_scale, a_rows_total, a_rows, b, b_scale, m_indices, out, m, n, k, num_groups,
                          scale_major, gran_m, gran_n, gran_k, stream, "fp8_group_gemm_contiguous_gather launch",
                          out_dtype);
  });
}

fp8g_status_t fp8_moe_fc1_silu_quant(const void* a, const float* a_scale, int64_t a_rows_total,
                                     const int32_t* a_rows, const void* w1, const float* w1_scale,
                                     const int32_t* m_indices, void* q_out, float* q_scale_out, int64_t m,
                                     int64_t inter, int64_t hidden, int64_t num_experts, int32_t scale_major,
                                     int32_t gran_m, int32_t gran_n, int32_t gran_k, void* stream) {
  return guarded([&] {
    require(inter >= 0 && inter <= kInt32Max / 2, "inter must be in [0, 2^30)");
    require(inter % 128 == 0, "inter (%lld) must be a multiple of 128", (long long)inter);
    if (m == 0 || inter == 0 || num_experts == 0) {
      check_gemm_dims(m, 2 * inter, hidden);
      return;
    }
    require(q_out != nullptr, "q_out must be non-null");
    group_gemm_contiguous(a, a_scale, a_rows == nullptr ? m : a_rows_total, a_rows, w1, w1_scale, m_indices, nullptr,
                          m, 2 * inter, hidden, num_experts, scale_major, gran_m, gran_n, gran_k, stream,
                          "fp8_moe_fc1_silu_quant launch", FP8G_OUT_BF16, q_out, q_scale_out);
  });
}

fp8g_status_t fp8_group_gemm_contiguous_per_tensor(const void* a, int64_t a_rows_total, const int32_t* a_rows,
                                                  const void* b, const float* b_dequant, const int32_t* m_indices,
                                                  void* out, int32_t out_dtype, int64_t m, int64_t n, int64_t k,
                                                  int64_t num_groups, void* stream) {
  return guarded([&] {
    if (m > 0 && n > 0 && num_groups > 0) require(b_dequant != nullptr, "b_dequant must be non-null");
    group_gemm_contiguous(a, nullptr, a_rows == nullptr ? m : a_rows_total, a_rows, b, nullptr, m_indices, out, m, n,
                          k, num_groups, FP8G_SCALE_K_MAJOR, 1, 128, 128, stream,
                          "fp8_group_gemm_contiguous_per_tensor launch", out_dtype, nullptr, nullptr, b_dequant);
  });
}

fp8g_status_t fp8_moe_fc1_silu_quant_per_tensor(const void* a, int64_t a_rows_total, const int32_t* a_rows,
                                                const void* w1, const float* fc1_dequant, const float* fc2_quant,
                                                int32_t fc2_quant_per_expert, const int32_t* m_indices, void* q_out,
                                                int64_t m, int64_t inter, int64_t hidden, int64_t num_experts,
                                                void* stream) {
  return guarded([&] {
    require(inter >= 0 && inter <= kInt32Max / 2, "inter must be in [0, 2^30)");
    require(inter % 128 == 0, "inter (%lld) must be a multiple of 128", (long long)inter);
    require(fc2_quant_per_expert == 0 || fc2_quant_per_expert == 1, "fc2_quant_per_expert must be 0 or 1");
    if (m == 0 || inter == 0 || num_experts == 0) {
      check_gemm_dims(m, 2 * inter, hidden);
      return;
    }
    require(q_out != nullptr, "q_out must be non-null");
    require(fc1_dequant != nullptr, "fc1_dequant must be non-null");
    group_gemm_contiguous(a, nullptr, a_rows == nullptr ? m : a_rows_total, a_rows, w1, nullptr, m_indices, nullptr, m,
                          2 * inter, hidden, num_experts, FP8G_SCALE_K_MAJOR, 1, 128, 128, stream,
                          "fp8_moe_fc1_silu_quant_per_tensor launch", FP8G_OUT_BF16, q_out, nullptr, fc1_dequant,
                          fc2_quant, fc2_quant_per_expert);
  });
}

fp8g_status_t fp8_batch_gemm_masked(const void* a, const void* b, const float* a_scale,
                                    const float* b_scale, const int32_t* masked_m,
                                    int64_t expected_m, void* out, int32_t out_dtype,
                                    int64_t num_groups, int64_t max_m, int64_t n, int64_t k,
                                    int32_t scale_major, int32_t gran_m, int32_t gran_n,
                                    int32_t gran_k, void* stream) {
  return guarded([&] {
    check_gemm_dims(max_m, n, k);
    require(num_groups >= 0 && num_groups <= 65535, "num_groups must be in [0, 65535]");
    require(expected_m >= 0, "expected_m must be non-negative");
    check_scale_major(scale_major);
    check_granularity(gran_m, gran_n, gran_k);
    check_out_dtype(out_dtype);
    if (max_m == 0 || n == 0 || num_groups == 0) return;
    check_operands(a, b, a_scale, b_scale, out, k);
    require(masked_m != nullptr && aligned(masked_m, 4), "masked_m must be non-null and 4-byte aligned");
    check_device();
    fp8g::GemmParams p{};
    p.a = static_cast<const uint8_t*>(a);
    p.b = static_cast<const uint8_t*>(b);
    p.sa = a_scale;
    p.sb = b_scale;
    p.out = static_cast<uint16_t*>(out);
    p.out_fp16 = out_dtype == FP8G_OUT_FP16;
    p.rowinfo = masked_m;
    p.m = (int32_t)max_m;
    p.n = (int32_t)n;
    p.k = (int32_t)k;
    p.kblocks = (int32_t)(k / 128);
    p.nblocks = (int32_t)(n / 128);
    p.num_groups = (int32_t)num_groups;
    p.a_group_stride = max_m * k;
    p.b_group_stride = n * k;
    p.sa_group_stride = max_m * (k / 128);
    p.a_src_rows = (int32_t)max_m;
    p.sb_group_stride = (n / 128) * (k / 128);
    p.out_group_stride = max_m * n;
    set_scale_strides(p, scale_major, max_m);
    // expected_m picks the row tile: one 256-row tile per group reads each b tile once; smaller
    // expected groups use 128-row tiles so that the second row tile is usually skipped.
    fp8g::TileConfig cfg = (max_m > 128 && expected_m > 64) ? fp8g::TILE_256x256 : fp8g::TILE_128x256;
    if (fp8g::tile_override() >= 0) cfg = (fp8g::TileConfig)fp8g::tile_override();
    p.tiles_m = (int32_t)ceil_div(max_m, fp8g::tile_rows(cfg));
    p.tiles_n = (int32_t)ceil_div(n, fp8g::tile_cols(cfg));
    p.group_m = fp8g::group_m_override(p.tiles_m);
    const int64_t grid = mul_sat(num_groups, mul_sat(p.tiles_m, p.tiles_n));
    require(grid <= kInt32Max, "too many tiles");
    launch_logged("fp8_batch_gemm_masked launch", fp8g::MODE_MASKED, cfg, p, grid, stream);
  });
}

int64_t fp8_moe_permutation_workspace_size(int64_t num_tokens, int64_t top_k, int64_t num_experts) {
  if (num_tokens < 0 || top_k < 0 || num_experts < 1 || num_experts > 1024 || mul_sat(num_tokens, top_k) > kInt32Max)
    return -1;
  return 4 * fp8g::moe_permutation_scratch_ints(num_tokens * top_k, num_experts);
}

}  // extern "C"

namespace {

// Validation shared by the permutation entry points; returns false when there is nothing to do.
bool check_permutation(const int32_t* topk_ids, int64_t num_tokens, int64_t top_k, int64_t num_experts,
                       int64_t m_alloc, const int32_t* m_indices, const int32_t* src_token,
                       const int32_t* row_of_entry) {
  require(num_tokens >= 0 && top_k >= 0 && num_experts >= 1 && m_alloc >= 0, "sizes must be non-negative, num_experts >= 1");
  require(num_experts <= 1024, "num_experts must be at most 1024");
  require(mul_sat(num_tokens, top_k) <= kInt32Max && m_alloc <= kInt32Max, "sizes must fit in int32");
  require(m_alloc % 128 == 0, "m_alloc must be a multiple of 128");
  const int64_t need = ceil_div(num_tokens * top_k + num_experts * 127, 128) * 128;
  require(m_alloc >= need, "m_alloc (%lld) must be at least %lld for this many entries and experts",
          (long long)m_alloc, (long long)need);
  if (m_alloc == 0) return false;
  require(m_indices && src_token && (num_tokens * top_k == 0 || (topk_ids && row_of_entry)),
          "pointers must be non-null");
  require(aligned(topk_ids, 4) && aligned(m_indices, 4) && aligned(src_token, 4) && aligned(row_of_entry, 4),
          "pointers must be 4-byte aligned");
  return true;
}

}  // namespace

extern "C" {

fp8g_status_t fp8_moe_build_permutation(const int32_t* topk_ids, int64_t num_tokens,
                                        int64_t top_k, int64_t num_experts, int64_t m_alloc,
                                        int32_t* m_indices, int32_t* src_token,
                                        int32_t* row_of_entry, void* workspace, int64_t workspace_bytes,
                                        void* stream) {
  return guarded([&] {
    if (!check_permutation(topk_ids, num_tokens, top_k, num_experts, m_alloc, m_indices, src_token, row_of_entry))
      return;
    const int64_t need = 4 * fp8g::moe_permutation_scratch_ints(num_tokens * top_k, num_experts);
    require(workspace_bytes >= need, "workspace (%lld bytes) must hold %lld bytes", (long long)workspace_bytes,
            (long long)need);
    require(need == 0 || (workspace != nullptr && aligned(workspace, 4)),
            "workspace must be non-null and 4-byte aligned");
    check_device();
    check_hip(fp8g::launch_moe_build_permutation(topk_ids, (int)num_tokens, (int)top_k, (int)num_experts,
                                                 (int)m_alloc, m_indices, src_token, row_of_entry,
                                                 static_cast<int32_t*>(workspace), (hipStream_t)stream),
              "fp8_moe_build_permutation launch");
  });
}

fp8g_status_t fp8_moe_build_permutation_noalloc(const int32_t* topk_ids, int64_t num_tokens, int64_t top_k,
                                                int64_t num_experts, int64_t m_alloc, int32_t* m_indices,
                                                int32_t* src_token, int32_t* row_of_entry, void* stream) {
  return guarded([&] {
    if (!check_permutation(topk_ids, num_tokens, top_k, num_experts, m_alloc, m_indices, src_token, row_of_entry))
      return;
    const int64_t need = fp8g::moe_permutation_scratch_ints(num_tokens * top_k, num_experts);
    require(need <= fp8g::kPermScratchInts,
            "num_tokens*top_k (%lld) over num_experts (%lld) needs %lld scratch ints; the library's own scratch "
            "holds %lld (ceil(num_tokens*top_k/1024)*num_experts must not exceed it)",
            (long long)(num_tokens * top_k), (long long)num_experts, (long long)need,
            (long long)fp8g::kPermScratchInts);
    check_device();
    int dev = 0;
    check_hip(hipGetDevice(&dev), "hipGetDevice");
    int32_t* hist = nullptr;
    check_hip(fp8g::permutation_scratch(dev, &hist), "looking up the permutation scratch");
    check_hip(fp8g::launch_moe_build_permutation(topk_ids, (int)num_tokens, (int)top_k, (int)num_experts,
                                                 (int)m_alloc, m_indices, src_token, row_of_entry, hist,
                                                 (hipStream_t)stream),
              "fp8_moe_build_permutation_noalloc launch");
  });
}

fp8g_status_t fp8_moe_gather_quant(const void* x, const int32_t* src_token, int64_t num_tokens,
                                   int64_t hidden, int64_t m_alloc, void* a_out,
                                   float* a_scale_out, void* stream) {
  return guarded([&] {
    require(num_tokens >= 0 && hidden >= 0 && m_alloc >= 0, "sizes must be non-negative");
    require(hidden % 128 == 0, "hidden (%lld) must be a multiple of 128", (long long)hidden);
    require(m_alloc <= kInt32Max && hidden <= kInt32Max && num_tokens <= kInt32Max, "sizes must fit in int32");
    require(src_token != nullptr || m_alloc <= num_tokens, "without src_token, m_alloc must not exceed num_tokens");
    require(m_alloc * (hidden / 128) < (int64_t)1 << 31, "m_alloc * hidden / 128 must be below 2^31");
    if (m_alloc == 0 || hidden == 0) return;
    require(x && a_out && a_scale_out, "pointers must be non-null");
    require(aligned(x, 16) && aligned(a_out, 16) && aligned(a_scale_out, 4) && aligned(src_token, 4),
            "x and a_out must be 16-byte aligned, src_token and a_scale_out 4-byte aligned");
    check_device();
    check_hip(fp8g::launch_moe_gather_quant(static_cast<const uint16_t*>(x), src_token, (int)num_tokens,
                                            (int)hidden, (int)m_alloc, static_cast<uint8_t*>(a_out), a_scale_out,
                                            (hipStream_t)stream),
              "fp8_moe_gather_quant launch");
  });
}

fp8g_status_t fp8_bmm(const void* a, const void* b, const float* a_scale, int32_t a_scale_per_row,
                      const float* b_scale, int32_t b_scale_per_col, void* out, int32_t out_dtype, int64_t batch,
                      int64_t m, int64_t n, int64_t k, void* stream) {
  return guarded([&] {
    require(batch >= 0 && batch <= 65535, "batch (%lld) must be in [0, 65535]", (long long)batch);
    check_gemm_dims(m, n, k, /*n_tail=*/true);
    require(n % 16 == 0, "n (%lld) must be a multiple of 16", (long long)n);
    check_out_dtype(out_dtype);
    require(a_scale_per_row == 0 || a_scale_per_row == 1, "a_scale_per_row must be 0 or 1");
    require(b_scale_per_col == 0 || b_scale_per_col == 1, "b_scale_per_col must be 0 or 1");
    if (batch == 0 || m == 0 || n == 0) return;
    require(mul_sat(batch, mul_sat(m, n)) <= ((int64_t)1 << 40) && mul_sat(batch, mul_sat(n, k)) <= ((int64_t)1 << 40),
            "sizes too large");
    require(out && a_scale && b_scale, "out and the scales must be non-null");
    require(k == 0 || (a && b), "a and b must be non-null");
    require(aligned(a, 16) && aligned(b, 16) && aligned(out, 16), "a, b and out must be 16-byte aligned");
    require(aligned(a_scale, 4) && aligned(b_scale, 4), "scales must be 4-byte aligned");
    check_device();
    fp8g::GemmParams p{};
    p.a = static_cast<const uint8_t*>(a);
    p.b = static_cast<const uint8_t*>(b);
    p.sa = a_scale;
    p.sb = b_scale;
    p.out = static_cast<uint16_t*>(out);
    p.out_fp16 = out_dtype == FP8G_OUT_FP16;
    p.bmm_sa_rows = a_scale_per_row;
    p.bmm_sb_cols = b_scale_per_col;
    p.m = (int32_t)m;
    p.n = (int32_t)n;
    p.k = (int32_t)k;
    p.kblocks = (int32_t)(k / 128);
    p.nblocks = (int32_t)ceil_div(n, 128);
    p.num_groups = (int32_t)batch;
    p.a_src_rows = (int32_t)m;
    p.a_group_stride = m * k;
    p.b_group_stride = n * k;
    p.out_group_stride = m * n;
    fp8g::TileConfig cfg = m > 128 ? fp8g::TILE_256x256 : fp8g::TILE_128x256;
    if (fp8g::tile_override() >= 0) cfg = (fp8g::TileConfig)fp8g::tile_override();
    p.tiles_m = (int32_t)ceil_div(m, fp8g::tile_rows(cfg));
    p.tiles_n = (int32_t)ceil_div(n, fp8g::tile_cols(cfg));
    p.group_m = 4;
    const int64_t grid = mul_sat(batch, mul_sat(p.tiles_m, p.tiles_n));
    require(grid <= kInt32Max, "too many tiles");
    launch_logged("fp8_bmm launch", fp8g::MODE_BMM, cfg, p, grid, stream);
  });
}

fp8g_status_t fp8_quantize_1x128(const void* x, int64_t rows, int64_t cols, void* out, float* scale_out,
                                 int32_t scale_major, void* stream) {
  return guarded([&] {
    require(rows >= 0 && cols >= 0, "sizes must be non-negative");
    require(cols % 128 == 0, "cols (%lld) must be a multiple of 128", (long long)cols);
    require(rows <= kInt32Max && cols <= kInt32Max && rows * (cols / 128) < (int64_t)1 << 31, "sizes too large");
    check_scale_major(scale_major);
    if (rows == 0 || cols == 0) return;
    require(x && out && scale_out, "pointers must be non-null");
    require(aligned(x, 16) && aligned(out, 16) && aligned(scale_out, 4),
            "x and out must be 16-byte aligned, scale_out 4-byte aligned");
    check_device();
    check_hip(fp8g::launch_quantize_1x128(static_cast<const uint16_t*>(x), (int)rows, (int)cols,
                                          static_cast<uint8_t*>(out), scale_out, scale_major == FP8G_SCALE_MN_MAJOR,
                                          (hipStream_t)stream),
              "fp8_quantize_1x128 launch");
  });
}

fp8g_status_t fp8_fused_add_rmsnorm_quant(void* out, float* block_scale, void* normed_out, const void* input,
                                          void* residual, const void* weight, float eps, int64_t rows,
                                          int64_t hidden, int32_t scale_major, void* stream) {
  return guarded([&] {
    require(rows >= 0 && hidden >= 0, "sizes must be non-negative");
    require(hidden % 128 == 0, "hidden (%lld) must be a multiple of 128", (long long)hidden);
    require(rows <= kInt32Max && hidden <= kInt32Max && rows * hidden <= (int64_t)1 << 40, "sizes too large");
    require(eps >= 0.0f && eps < INFINITY, "eps must be finite and non-negative");
    check_scale_major(scale_major);
    if (rows == 0 || hidden == 0) return;
    require(out && block_scale && normed_out && input && residual && weight, "pointers must be non-null");
    require(aligned(out, 16) && aligned(normed_out, 16) && aligned(input, 16) && aligned(residual, 16) &&
                aligned(weight, 16) && aligned(block_scale, 4),
            "tensors must be 16-byte aligned, block_scale 4-byte aligned");
    require(residual != input && residual != normed_out && residual != weight,
            "residual must not alias input, normed_out or weight");
    check_device();
    check_hip(fp8g::launch_fused_add_rmsnorm_quant(
                  static_cast<const uint16_t*>(input), static_cast<uint16_t*>(residual),
                  static_cast<const uint16_t*>(weight), eps, (int)rows, (int)hidden,
                  static_cast<uint16_t*>(normed_out), static_cast<uint8_t*>(out), block_scale,
                  scale_major == FP8G_SCALE_MN_MAJOR, (hipStream_t)stream),
              "fp8_fused_add_rmsnorm_quant launch");
  });
}

fp8g_status_t fp8_moe_silu_mul_quant(const void* y, const int32_t* m_indices, int64_t rows,
                                     int64_t inter, void* a_out, float* a_scale_out,
                                     void* stream) {
  return guarded([&] {
    require(rows >= 0 && inter >= 0, "sizes must be non-negative");
    require(inter % 128 == 0, "inter (%lld) must be a multiple of 128", (long long)inter);
    require(rows <= kInt32Max && inter <= kInt32Max / 2, "sizes must fit in int32");
    if (rows == 0 || inter == 0) return;
    require(y && m_indices && a_out && a_scale_out, "pointers must be non-null");
    require(aligned(y, 16) && aligned(a_out, 16) && aligned(a_scale_out, 4) && aligned(m_indices, 4),
            "y and a_out must be 16-byte aligned, m_indices and a_scale_out 4-byte aligned");
    check_device();
    check_hip(fp8g::launch_moe_silu_mul_quant(static_cast<const uint16_t*>(y), m_indices, (int)rows,
                                              (int)inter, static_cast<uint8_t*>(a_out), a_scale_out,
                                              (hipStream_t)stream),
              "fp8_moe_silu_mul_quant launch");
  });
}

fp8g_status_t fp8_moe_combine(const void* y, const int32_t* row_of_entry,
                              const float* topk_weights, int64_t num_tokens, int64_t top_k,
                              int64_t hidden, int64_t m_alloc, void* out, int32_t out_dtype, void* stream) {
  return guarded([&] {
    require(num_tokens >= 0 && top_k >= 0 && hidden >= 0 && m_alloc >= 0, "sizes must be non-negative");
    require(hidden % 128 == 0, "hidden (%lld) must be a multiple of 128", (long long)hidden);
    require(num_tokens <= kInt32Max && top_k <= 64 && hidden <= kInt32Max && m_alloc <= kInt32Max,
            "sizes out of range (top_k must be at most 64)");
    check_out_dtype(out_dtype);
    if (num_tokens == 0 || hidden == 0) return;
    require(out && (top_k == 0 || (y && row_of_entry)), "pointers must be non-null");
    require(aligned(y, 16) && aligned(out, 16) && aligned(row_of_entry, 4) && aligned(topk_weights, 4),
            "y and out must be 16-byte aligned, row_of_entry and topk_weights 4-byte aligned");
    check_device();
    check_hip(fp8g::launch_moe_combine(static_cast<const uint16_t*>(y), row_of_entry, topk_weights,
                                       (int)num_tokens, (int)top_k, (int)hidden, (int)m_alloc,
                                       static_cast<uint16_t*>(out), out_dtype == FP8G_OUT_FP16, (hipStream_t)stream),
              "fp8_moe_combine launch");
  });
}

}  // extern "C"
