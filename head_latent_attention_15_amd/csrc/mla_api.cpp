// C ABI of libmla: host-side validation, split planning and dispatch to the kernels.
// Every check runs before any HIP call, so a rejected call touches no device state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launchers.h"
#include "mla.h"

namespace {

thread_local char g_detail[512] = "";

mla_status_t fail(mla_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return st;
}

mla_status_t ok() {
  g_detail[0] = '\0';
  return MLA_OK;
}

mla_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

bool is_dtype(mla_dtype_t d) { return d == MLA_F32 || d == MLA_BF16; }

constexpr int kMaxSplits = 4096;

int32_t pages_per_split(int32_t max_pages, int32_t num_splits) {
  return (max_pages + num_splits - 1) / num_splits;
}

mla_status_t check_paged_shape(const mla_paged_shape_t* shp) {
  if (shp == nullptr) return fail(MLA_ERR_NULL, "shape is NULL");
  if (shp->batch < 1 || shp->num_heads < 1 || shp->d_latent < 1 || shp->d_rope < 1 ||
      shp->page_size < 1 || shp->max_pages_per_seq < 1 || shp->num_pages < 1)
    return fail(MLA_ERR_SHAPE,
                "shape fields must be >= 1 (B=%d H=%d d_c=%d d_R=%d P=%d max_pages=%d pages=%d)",
                shp->batch, shp->num_heads, shp->d_latent, shp->d_rope, shp->page_size,
                shp->max_pages_per_seq, shp->num_pages);
  if (shp->page_size % 16 != 0)
    return fail(MLA_ERR_SHAPE, "page_size %d is not a multiple of 16", shp->page_size);
  if (shp->d_rope % 2 != 0) return fail(MLA_ERR_SHAPE, "d_rope %d is odd", shp->d_rope);
  if (static_cast<int64_t>(shp->max_pages_per_seq) * shp->page_size > INT32_MAX)
    return fail(MLA_ERR_SHAPE, "max_pages_per_seq * page_size overflows int32");
  return MLA_OK;
}

// Projections: bf16 MFMA weight streaming where it applies, the fp32 tile GEMM otherwise
// (fp32 weights, bf16 output, k not a multiple of 128, weights stored [in, out]).  Large
// single products (8 MB of weights and up, 1024 output columns and up) take one of the
// one-workgroup-per-CU kernels, which measured faster there: the activation-stationary
// one for short k (up to 4096, 4096 columns and up: W^UQ, W^QR at the DeepSeek-V2 sizes),
// the persistent one otherwise (W^DQ, W^O).  Smaller and batched products take the
// tile-grid kernel.
hipError_t gemm(const mla::GemmArgs& g, hipStream_t s) {
  const bool large = g.batch == 1 && g.N >= 1024 &&
                     static_cast<int64_t>(g.N) * g.K * 2 >= (int64_t{8} << 20);
  int tn, sl, grid;
  if (large && g.K <= 4096 && g.N >= 4096 && mla::gemm_xs_supported(g) &&
      mla::gemm_xs_plan(g, &tn, &sl, &grid))
    return mla::launch_gemm_xs_with(g, tn, sl, grid, s);
  if (large && mla::gemm_stream_supported(g)) return mla::launch_gemm_stream(g, s);
  return mla::gemm_rows_supported(g) ? mla::launch_gemm_rows(g, s) : mla::launch_gemm_small(g, s);
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t st) {
  switch (st) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH";
    case MLA_ERR_INDEX: return "MLA_ERR_INDEX";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error_detail(void) { return g_detail; }

size_t mla_cache_bytes(int64_t B, int64_t T, int64_t layers, int32_t d_c, int32_t d_R,
                       int32_t elem_bytes) {
  if (B < 0 || T < 0 || layers < 0 || d_c < 0 || d_R < 0 || elem_bytes < 0) return 0;
  return static_cast<size_t>(B) * static_cast<size_t>(T) * static_cast<size_t>(layers) *
         static_cast<size_t>(d_c + d_R) * static_cast<size_t>(elem_bytes);
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t d_c, int32_t num_splits) {
  if (B < 1 || H < 1 || d_c < 1 || num_splits < 1) return 0;
  const size_t rows = static_cast<size_t>(B) * H * num_splits;
  return align256(rows * d_c * sizeof(float)) + align256(rows * sizeof(float));
}

int32_t mla_suggest_num_splits(int32_t B, int32_t max_seq_len, int64_t total_tokens,
                               int32_t page_size, int32_t num_cus) {
  if (B < 1 || max_seq_len < 1 || page_size < 1) return 1;
  if (num_cus < 1) num_cus = 256;
  const int64_t max_pages = (static_cast<int64_t>(max_seq_len) + page_size - 1) / page_size;
  int64_t S;
  if (total_tokens <= 0 || total_tokens >= static_cast<int64_t>(B) * max_seq_len) {
    // uniform lengths: one (sequence, split) item per compute unit
    S = (num_cus + B - 1) / B;
  } else {
    // ragged: split size from the mean load per compute unit, at most a quarter of it so
    // that uneven sequence ends still balance
    const int64_t total_pages = (total_tokens + page_size - 1) / page_size;
    int64_t cps = total_pages / (4 * static_cast<int64_t>(num_cus));
    if (cps < 1) cps = 1;
    S = (max_pages + cps - 1) / cps;
  }
  if (S > max_pages) S = max_pages;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return static_cast<int32_t>(S);
}

// Where the combined result of a decode that also merges its splits goes.
struct MergeReq {
  int32_t* counters;  // 2 per query row + 1 error word, zero on entry, left zero
  float* out;
  float* lse_out;
};

// Decode attention for n_q query tokens per sequence (1 for plain decode).  With `merge`
// (num_splits > 1) the split partials are also combined into merge->out: inside the
// attention launch when the head-partitioned kernel runs with its whole grid resident,
// else by the combine kernel right after it.
static mla_status_t decode_attn(const void* q_lat, const void* q_pe, const void* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const mla_paged_shape_t* shape, float softmax_scale,
                             int32_t num_splits, void* o_part, mla_dtype_t part_dtype,
                             float* lse_part, mla_dtype_t dtype, int32_t n_q, int32_t kernel,
                             void* stream, const MergeReq* merge = nullptr) {
  if (!q_lat || !q_pe || !kv_cache || !block_table || !seq_lens || !o_part)
    return fail(MLA_ERR_NULL, "mla_decode_attn: a required pointer is NULL");
  mla_status_t st = check_paged_shape(shape);
  if (st != MLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_SHAPE, "num_splits %d outside [1, %d]", num_splits, kMaxSplits);
  if (num_splits > 1 && lse_part == nullptr)
    return fail(MLA_ERR_NULL, "lse_part is NULL with num_splits %d > 1", num_splits);
  if (!std::isfinite(softmax_scale))
    return fail(MLA_ERR_SHAPE, "softmax_scale is not finite");
  if (!is_dtype(dtype) && dtype != MLA_FP8)
    return fail(MLA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (!is_dtype(part_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "unknown partial dtype %d", part_dtype);
  if (n_q < 1 || static_cast<int64_t>(shape->batch) * n_q > 65535)
    return fail(MLA_ERR_SHAPE, "n_q %d outside [1, 65535 / batch]", n_q);

  mla::PagedArgs a;
  a.q_lat = q_lat;
  a.q_pe = q_pe;
  a.cache = kv_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.B = shape->batch;
  a.H = shape->num_heads;
  a.d_c = shape->d_latent;
  a.d_R = shape->d_rope;
  a.page_size = shape->page_size;
  a.max_pages = shape->max_pages_per_seq;
  a.num_pages = shape->num_pages;
  a.scale = softmax_scale;
  a.num_splits = num_splits;
  a.pages_per_split = pages_per_split(shape->max_pages_per_seq, num_splits);
  a.o_part = o_part;
  a.part_bf16 = part_dtype == MLA_BF16;
  a.lse_part = lse_part;
  a.n_q = n_q;
  hipStream_t s = as_stream(stream);

  if (kernel < 0 || kernel > 4) return fail(MLA_ERR_UNSUPPORTED, "attention kernel %d unknown", kernel);
  if (dtype == MLA_FP8) {
    if (a.d_c != 512 || a.d_R != 64 || !mla::attn_mfma_fp8_supported(a) ||
        (kernel != 0 && kernel != 1 && kernel != 4) || (kernel == 4 && !mla::attn_wide_supported(a)))
      return fail(MLA_ERR_UNSUPPORTED, "fp8 cache: d_latent 512, d_rope 64, H = 128, pages of "
                  ">= 32 tokens (a power of two), <= 1024 pages per split, aligned tensors, "
                  "kernel 0, 1 or 4");
    // the library's choice is the kernel with 32 heads per wavefront
    if (kernel == 0) kernel = mla::attn_wide_supported(a) ? 4 : 1;
    const mla_status_t st2 =
        kernel == 4 ? launched(mla::launch_attn_wide_fp8(a, s), "attention (fp8 cache, 32 heads per wavefront)")
                    : launched(mla::launch_attn_mfma_fp8(a, s), "attention (fp8 cache)");
    if (st2 != MLA_OK || merge == nullptr || num_splits == 1) return st2;
    return launched(mla::launch_splitk_combine(o_part, part_dtype == MLA_BF16, lse_part,
                                               a.B * n_q, a.H, num_splits, a.d_c, merge->out,
                                               merge->lse_out, s),
                    "split-K combine");
  }
  if (dtype == MLA_BF16 && a.d_c == 512 && a.d_R == 64 && a.H <= 128) {
    const bool cols = mla::attn_cols_supported(a), heads = mla::attn_mfma_supported(a);
    const bool merging = merge != nullptr && num_splits > 1;
    if (kernel == 0) {
      // A fused call runs on the head-partitioned kernel (whose in-launch merge it takes
      // when the grid fits, and whose two launches it runs otherwise, with the same bits);
      // otherwise 128 heads take the 32-heads-per-wavefront kernel (fewer LDS reads and
      // MFMA issues per tile).
      if (merging && heads) kernel = 1;
      else kernel = mla::attn_wide_supported(a) ? 4 : heads ? 1 : cols ? 2 : 3;
    }
    if (kernel == 2 && !cols)
      return fail(MLA_ERR_UNSUPPORTED, "attention kernel 2 needs H = 128, pages of >= 32 tokens "
                  "(a power of two), <= 1024 pages per split and 16-byte aligned tensors");
    if (kernel == 1 && !heads)
      return fail(MLA_ERR_UNSUPPORTED, "attention kernel 1 needs H in {16, 32, 64, 128}, pages of "
                  ">= 32 tokens (a power of two), <= 1024 pages per split, aligned tensors");
    if (kernel == 4 && !mla::attn_wide_supported(a))
      return fail(MLA_ERR_UNSUPPORTED, "attention kernel 4 needs H = 128, pages of >= 32 tokens "
                  "(a power of two), <= 1024 pages per split and 16-byte aligned tensors");
    if (merging && kernel == 1 && num_splits <= 64 && mla::attn_mfma_grid_resident(a)) {
      a.merge_cnt = merge->counters;
      a.out = merge->out;
      a.lse_out = merge->lse_out;
      return launched(mla::launch_attn_mfma_bf16_512_64(a, s), "attention (bf16 MFMA, merged splits)");
    }
    mla_status_t st2;
    if (kernel == 4) st2 = launched(mla::launch_attn_wide_bf16_512_64(a, s), "attention (bf16 MFMA, 32 heads per wavefront)");
    else if (kernel == 2) st2 = launched(mla::launch_attn_cols_bf16_512_64(a, s), "attention (bf16 MFMA, column-partitioned)");
    else if (kernel == 1) st2 = launched(mla::launch_attn_mfma_bf16_512_64(a, s), "attention (bf16 MFMA)");
    else st2 = launched(mla::launch_attn_generic_bf16_512_64(a, s), "attention (bf16 generic)");
    if (st2 != MLA_OK || !merging) return st2;
    return launched(mla::launch_splitk_combine(o_part, part_dtype == MLA_BF16, lse_part,
                                               a.B * n_q, a.H, num_splits, a.d_c, merge->out,
                                               merge->lse_out, s),
                    "split-K combine");
  }
  if (merge != nullptr)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_fused: d_latent 512, d_rope 64, BF16 only");
  if (kernel == 1 || kernel == 2 || kernel == 4)
    return fail(MLA_ERR_UNSUPPORTED, "attention kernels 1, 2 and 4 need d_latent 512, d_rope 64, BF16");
  if (dtype == MLA_F32 && a.d_c == 64 && a.d_R == 16 && a.H <= 64)
    return launched(mla::launch_attn_generic_f32_64_16(a, s), "attention (fp32)");
  return fail(MLA_ERR_UNSUPPORTED,
              "mla_decode_attn: (d_latent=%d, d_rope=%d, H=%d, dtype=%d) is not compiled; "
              "supported: (512, 64, H<=128, BF16) and (64, 16, H<=64, F32)",
              a.d_c, a.d_R, a.H, dtype);
}

mla_status_t mla_decode_attn(const void* q_lat, const void* q_pe, const void* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const mla_paged_shape_t* shape, float softmax_scale,
                             int32_t num_splits, void* o_part, mla_dtype_t part_dtype,
                             float* lse_part, mla_dtype_t dtype, void* stream) {
  return decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale,
                     num_splits, o_part, part_dtype, lse_part, dtype, 1, 0, stream);
}

mla_status_t mla_decode_attn_planned(const void* q_lat, const void* q_pe, const void* kv_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const mla_paged_shape_t* shape, int32_t n_q,
                                     float softmax_scale, int32_t num_splits, void* o_part,
                                     mla_dtype_t part_dtype, float* lse_part, mla_dtype_t dtype,
                                     int32_t kernel, void* stream) {
  return decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale,
                     num_splits, o_part, part_dtype, lse_part, dtype, n_q, kernel, stream);
}

mla_status_t mla_decode_attn_multi(const void* q_lat, const void* q_pe, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const mla_paged_shape_t* shape, int32_t n_q,
                                   float softmax_scale, int32_t num_splits, void* o_part,
                                   mla_dtype_t part_dtype, float* lse_part, mla_dtype_t dtype,
                                   void* stream) {
  return decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale,
                     num_splits, o_part, part_dtype, lse_part, dtype, n_q, 0, stream);
}

mla_status_t mla_decode_fused(const void* q_lat, const void* q_pe, const void* kv_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const mla_paged_shape_t* shape, int32_t n_q, float softmax_scale,
                              int32_t num_splits, void* o_part, mla_dtype_t part_dtype,
                              float* lse_part, int32_t* counters, float* out, float* lse_out,
                              mla_dtype_t dtype, void* stream) {
  if (!out) return fail(MLA_ERR_NULL, "mla_decode_fused: out is NULL");
  if (num_splits == 1)  // nothing to merge: the attention writes out directly
    return decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale, 1,
                       out, MLA_F32, lse_out, dtype, n_q, 0, stream);
  if (!counters) return fail(MLA_ERR_NULL, "mla_decode_fused: counters is NULL");
  if (((reinterpret_cast<uintptr_t>(o_part) | reinterpret_cast<uintptr_t>(out)) & 15) != 0)
    return fail(MLA_ERR_SHAPE, "mla_decode_fused: o_part and out must be 16-byte aligned");
  if (num_splits > 64)
    return fail(MLA_ERR_SHAPE, "mla_decode_fused: num_splits %d > 64", num_splits);
  const MergeReq m{counters, out, lse_out};
  return decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale,
                     num_splits, o_part, part_dtype, lse_part, dtype, n_q, 0, stream, &m);
}

int32_t mla_decode_fused_single_launch(const mla_paged_shape_t* shape, int32_t n_q,
                                       int32_t num_splits) {
  if (shape == nullptr || check_paged_shape(shape) != MLA_OK) return 0;
  if (num_splits < 2 || num_splits > 64 || n_q < 1) return 0;
  mla::PagedArgs a{};
  a.B = shape->batch;
  a.H = shape->num_heads;
  a.d_c = shape->d_latent;
  a.d_R = shape->d_rope;
  a.page_size = shape->page_size;
  a.max_pages = shape->max_pages_per_seq;
  a.num_pages = shape->num_pages;
  a.num_splits = num_splits;
  a.pages_per_split = pages_per_split(shape->max_pages_per_seq, num_splits);
  a.n_q = n_q;
  // stand-in aligned pointers: the alignment rule is stated for the caller's tensors
  a.q_lat = a.q_pe = a.cache = reinterpret_cast<const void*>(static_cast<uintptr_t>(256));
  return mla::attn_mfma_supported(a) && mla::attn_mfma_grid_resident(a) ? 1 : 0;
}

// Workgroups of the flattened ragged launch: one per compute unit of the current device,
// or more when the pool holds over 1024 pages per compute unit (a workgroup's range of
// pages must fit its LDS block table).
static int ragged_grid(int32_t num_pages) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  const int per = mla::attn_mfma_ragged_max_range_pages();
  return std::max(cus, (num_pages + per - 1) / per);
}

struct RaggedLayout {
  size_t slots_off, lse_off, part_off, total;
};

static RaggedLayout ragged_layout(int32_t B, int32_t H, int32_t d_c, int grid) {
  RaggedLayout l;
  const size_t slots = static_cast<size_t>(grid) + B;
  l.slots_off = 0;
  l.lse_off = align256((2 * static_cast<size_t>(B) + 1) * sizeof(int32_t));
  l.part_off = l.lse_off + align256(slots * H * sizeof(float));
  l.total = l.part_off + align256(slots * H * d_c * sizeof(uint16_t));
  return l;
}

size_t mla_decode_ragged_workspace_bytes(const mla_paged_shape_t* shape) {
  if (shape == nullptr || shape->batch < 1 || shape->num_heads < 1 || shape->d_latent < 1 ||
      shape->num_pages < 1)
    return 0;
  return ragged_layout(shape->batch, shape->num_heads, shape->d_latent,
                       ragged_grid(shape->num_pages)).total;
}

mla_status_t mla_decode_ragged(const void* q_lat, const void* q_pe, const void* kv_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const mla_paged_shape_t* shape, float softmax_scale,
                               void* workspace, size_t workspace_bytes, float* out,
                               float* lse_out, mla_dtype_t dtype, void* stream) {
  if (!q_lat || !q_pe || !kv_cache || !block_table || !seq_lens || !out)
    return fail(MLA_ERR_NULL, "mla_decode_ragged: a required pointer is NULL");
  mla_status_t st = check_paged_shape(shape);
  if (st != MLA_OK) return st;
  if (!std::isfinite(softmax_scale))
    return fail(MLA_ERR_SHAPE, "mla_decode_ragged: softmax_scale is not finite");
  mla::PagedArgs a{};
  a.q_lat = q_lat;
  a.q_pe = q_pe;
  a.cache = kv_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.B = shape->batch;
  a.H = shape->num_heads;
  a.d_c = shape->d_latent;
  a.d_R = shape->d_rope;
  a.page_size = shape->page_size;
  a.max_pages = shape->max_pages_per_seq;
  a.num_pages = shape->num_pages;
  a.scale = softmax_scale;
  a.num_splits = 1;
  a.pages_per_split = 1;
  a.n_q = 1;
  const bool fp8 = dtype == MLA_FP8;
  if ((dtype != MLA_BF16 && !fp8) || !mla::attn_mfma_supported(a))
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_ragged: needs BF16 or FP8 rows, d_latent 512, "
                "d_rope 64, H in {16, 32, 64, 128} (128 for FP8), pages of >= 32 tokens (a power "
                "of two) and 16-byte aligned tensors");
  if ((reinterpret_cast<uintptr_t>(out) & 15) != 0)
    return fail(MLA_ERR_SHAPE, "mla_decode_ragged: out is not 16-byte aligned");
  const int grid = ragged_grid(a.num_pages);
  const RaggedLayout l = ragged_layout(a.B, a.H, a.d_c, grid);
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(MLA_ERR_WORKSPACE, "mla_decode_ragged: workspace %zu bytes, need %zu",
                workspace ? workspace_bytes : static_cast<size_t>(0), l.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(MLA_ERR_WORKSPACE, "mla_decode_ragged: workspace is not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  int32_t* seq_slots = reinterpret_cast<int32_t*>(ws + l.slots_off);
  a.lse_part = reinterpret_cast<float*>(ws + l.lse_off);
  a.o_part = ws + l.part_off;
  a.part_bf16 = 1;
  if (fp8 && !mla::attn_wide_supported(a))
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_ragged: FP8 rows need H = 128 and 16-byte "
                "aligned tensors");
  hipStream_t s = as_stream(stream);
  st = mla::attn_wide_supported(a)
           ? launched(mla::launch_attn_wide_ragged(a, grid, seq_slots, seq_slots + 2 * a.B, s, fp8),
                      "attention (flattened ragged work list, 32 heads per wavefront)")
           : launched(mla::launch_attn_mfma_ragged(a, grid, seq_slots, seq_slots + 2 * a.B, s),
                      "attention (flattened ragged work list)");
  if (st != MLA_OK) return st;
  return launched(mla::launch_combine_slots(a.o_part, 1, a.lse_part, seq_slots, a.B, a.H, out,
                                            lse_out, s),
                  "ragged combine");
}

mla_status_t mla_splitk_combine(const void* o_part, mla_dtype_t part_dtype,
                                const float* lse_part, int32_t B, int32_t H, int32_t num_splits,
                                int32_t d_c, float* out, float* lse_out, void* stream) {
  if (!o_part || !lse_part || !out)
    return fail(MLA_ERR_NULL, "mla_splitk_combine: a required pointer is NULL");
  if (B < 1 || H < 1 || d_c < 1 || num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_SHAPE, "mla_splitk_combine: bad sizes B=%d H=%d S=%d d_c=%d", B, H,
                num_splits, d_c);
  if (d_c % 4 != 0) return fail(MLA_ERR_SHAPE, "mla_splitk_combine: d_c %d %% 4 != 0", d_c);
  // the kernels load partials and store out with 8- and 16-byte accesses
  if ((reinterpret_cast<uintptr_t>(o_part) & 15) != 0 || (reinterpret_cast<uintptr_t>(out) & 15) != 0)
    return fail(MLA_ERR_SHAPE, "mla_splitk_combine: o_part and out must be 16-byte aligned");
  if (!is_dtype(part_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "mla_splitk_combine: unknown partial dtype %d", part_dtype);
  return launched(mla::launch_splitk_combine(o_part, part_dtype == MLA_BF16, lse_part, B, H,
                                             num_splits, d_c, out, lse_out, as_stream(stream)),
                  "split-K combine");
}

mla_status_t mla_combine_out_proj(const void* o_part, mla_dtype_t part_dtype,
                                  const float* lse_part, int32_t B, int32_t H, int32_t num_splits,
                                  int32_t d_c, const void* w_uv, mla_dtype_t w_dtype, int32_t d_h,
                                  float* o_heads, void* stream) {
  if (!o_part || !lse_part || !w_uv || !o_heads)
    return fail(MLA_ERR_NULL, "mla_combine_out_proj: a required pointer is NULL");
  if (B < 1 || H < 1 || num_splits < 1 || d_c < 1 || d_h < 1)
    return fail(MLA_ERR_SHAPE, "mla_combine_out_proj: sizes must be >= 1");
  if (!is_dtype(part_dtype) || w_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "mla_combine_out_proj: partials F32/BF16, w_uv BF16 only");
  if (!mla::combine_uv_supported(H, num_splits, d_c, d_h, o_part, w_uv, B))
    return fail(MLA_ERR_UNSUPPORTED,
                "mla_combine_out_proj: compiled for d_c = 512, d_h = 128, at most 64 splits and "
                "16-byte aligned o_part / w_uv (got d_c=%d d_h=%d S=%d)", d_c, d_h, num_splits);
  return launched(mla::launch_combine_uv(o_part, part_dtype == MLA_BF16, lse_part, w_uv, o_heads,
                                         B, H, num_splits, as_stream(stream)),
                  "combine + W^UV");
}

mla_status_t mla_decode(const void* q_lat, const void* q_pe, const void* kv_cache,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const mla_paged_shape_t* shape, float softmax_scale,
                        int32_t num_splits, void* workspace, size_t workspace_bytes,
                        float* out, float* lse_out, mla_dtype_t dtype, void* stream) {
  if (num_splits == 1)
    return mla_decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale,
                           1, out, MLA_F32, lse_out, dtype, stream);
  mla_status_t st = check_paged_shape(shape);
  if (st != MLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_SHAPE, "num_splits %d outside [1, %d]", num_splits, kMaxSplits);
  const size_t need =
      mla_decode_workspace_bytes(shape->batch, shape->num_heads, shape->d_latent, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "mla_decode: workspace %zu bytes, need %zu",
                workspace ? workspace_bytes : static_cast<size_t>(0), need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(MLA_ERR_WORKSPACE, "mla_decode: workspace is not 16-byte aligned");
  // partials in the input precision: bf16 for bf16 caches, fp32 otherwise
  const mla_dtype_t part_dtype = dtype == MLA_BF16 ? MLA_BF16 : MLA_F32;
  const size_t rows = static_cast<size_t>(shape->batch) * shape->num_heads * num_splits;
  void* o_part = workspace;
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align256(rows * shape->d_latent * sizeof(float)));
  st = mla_decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale,
                       num_splits, o_part, part_dtype, lse_part, dtype, stream);
  if (st != MLA_OK) return st;
  return mla_splitk_combine(o_part, part_dtype, lse_part, shape->batch, shape->num_heads,
                            num_splits, shape->d_latent, out, lse_out, stream);
}

mla_status_t mla_decode_noalloc(const void* q_lat, const void* q_pe, const void* kv_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const mla_paged_shape_t* shape, float softmax_scale,
                                int32_t num_splits, float* out, float* lse_out, mla_dtype_t dtype,
                                void* stream) {
  mla_status_t st = check_paged_shape(shape);
  if (st != MLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_SHAPE, "num_splits %d outside [1, %d]", num_splits, kMaxSplits);
  if (num_splits == 1)  // no partials: the attention writes out directly
    return mla_decode(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale, 1,
                      nullptr, 0, out, lse_out, dtype, stream);
  const size_t need =
      mla_decode_workspace_bytes(shape->batch, shape->num_heads, shape->d_latent, num_splits);
  const size_t cap = mla::noalloc_scratch_bytes();
  if (need > cap)
    return fail(MLA_ERR_WORKSPACE,
                "mla_decode_noalloc: %zu bytes of split partials (B=%d H=%d d_latent=%d S=%d) "
                "exceed the %zu-byte device scratch; use fewer splits or mla_decode",
                need, shape->batch, shape->num_heads, shape->d_latent, num_splits, cap);
  void* ws = nullptr;
  const hipError_t e = mla::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return fail(MLA_ERR_LAUNCH, "mla_decode_noalloc: device scratch lookup: %s", hipGetErrorString(e));
  return mla_decode(q_lat, q_pe, kv_cache, block_table, seq_lens, shape, softmax_scale,
                    num_splits, ws, cap, out, lse_out, dtype, stream);
}

static mla_status_t absorb_q(const char* fn, const float* q_c, int64_t ld_qc, const void* w_uk,
                             const float* q_r, int64_t ld_qr, const int32_t* seq_lens,
                             float rope_base, void* q_lat, void* q_pe, int32_t B, int32_t H,
                             int32_t d_h, int32_t d_c, int32_t d_R, mla_dtype_t w_dtype,
                             mla_dtype_t out_dtype, void* stream) {
  if (!q_c || !w_uk || !q_lat) return fail(MLA_ERR_NULL, "%s: NULL q_c/w_uk/q_lat", fn);
  if (q_r && (!q_pe || !seq_lens))
    return fail(MLA_ERR_NULL, "%s: q_r given but q_pe or seq_lens is NULL", fn);
  if (B < 1 || H < 1 || d_h < 1 || d_c < 1 || (q_r && d_R < 1))
    return fail(MLA_ERR_SHAPE, "%s: sizes must be >= 1", fn);
  if (q_r && d_R % 2) return fail(MLA_ERR_SHAPE, "%s: d_R %d is odd", fn, d_R);
  if (ld_qc < static_cast<int64_t>(H) * d_h || (q_r && ld_qr < static_cast<int64_t>(H) * d_R))
    return fail(MLA_ERR_SHAPE, "%s: row strides %lld / %lld below H*d_h / H*d_R", fn,
                static_cast<long long>(ld_qc), static_cast<long long>(ld_qr));
  if (!is_dtype(w_dtype) || !is_dtype(out_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (q_r && !std::isfinite(rope_base)) return fail(MLA_ERR_SHAPE, "%s: rope_base not finite", fn);
  hipStream_t s = as_stream(stream);
  mla::GemmArgs g;
  g.x = q_c; g.ldx = ld_qc; g.sx = d_h; g.x_bf16 = 0;
  g.w = w_uk; g.ldw = d_c; g.sw = static_cast<int64_t>(d_h) * d_c; g.w_bf16 = w_dtype == MLA_BF16;
  g.w_nk = false;
  g.y = q_lat; g.ldy = static_cast<int64_t>(H) * d_c; g.sy = d_c; g.y_bf16 = out_dtype == MLA_BF16;
  g.M = B; g.N = d_c; g.K = d_h; g.batch = H;
  const bool mfma = w_dtype == MLA_BF16 && out_dtype == MLA_BF16 &&
                    mla::absorb_mfma_supported(B, H, d_h, d_c, q_c, ld_qc, w_uk, q_lat);
  // the MFMA kernel also applies the query RoPE where the shape allows (one launch)
  const bool fused = mfma && q_r && mla::absorb_rope_fusable(d_c, d_R, q_r, ld_qr, q_pe);
  mla_status_t st = launched(
      mfma ? mla::launch_absorb_mfma(q_c, ld_qc, w_uk, q_lat, B, H, d_c, fused ? q_r : nullptr,
                                     ld_qr, seq_lens, rope_base, q_pe, s)
           : mla::launch_gemm_small(g, s),
      "absorb GEMM");
  if (st != MLA_OK || !q_r || fused) return st;
  return launched(mla::launch_rope_rows(q_r, static_cast<int64_t>(B) * H, H, d_R, ld_qr, seq_lens,
                                        -1, rope_base, q_pe, out_dtype == MLA_BF16, s),
                  "query RoPE");
}

mla_status_t mla_absorb_q(const float* q_c, const void* w_uk, const float* q_r,
                          const int32_t* seq_lens, float rope_base, void* q_lat, void* q_pe,
                          int32_t B, int32_t H, int32_t d_h, int32_t d_c, int32_t d_R,
                          mla_dtype_t w_dtype, mla_dtype_t out_dtype, void* stream) {
  return absorb_q("mla_absorb_q", q_c, static_cast<int64_t>(H) * d_h, w_uk, q_r,
                  static_cast<int64_t>(H) * d_R, seq_lens, rope_base, q_lat, q_pe, B, H, d_h,
                  d_c, d_R, w_dtype, out_dtype, stream);
}

mla_status_t mla_absorb_q_strided(const float* q_c, int64_t ld_qc, const void* w_uk,
                                  const float* q_r, int64_t ld_qr, const int32_t* seq_lens,
                                  float rope_base, void* q_lat, void* q_pe, int32_t B, int32_t H,
                                  int32_t d_h, int32_t d_c, int32_t d_R, mla_dtype_t w_dtype,
                                  mla_dtype_t out_dtype, void* stream) {
  return absorb_q("mla_absorb_q_strided", q_c, ld_qc, w_uk, q_r, ld_qr, seq_lens, rope_base,
                  q_lat, q_pe, B, H, d_h, d_c, d_R, w_dtype, out_dtype, stream);
}

mla_status_t mla_pack_query_weights(const void* w_uq, const void* w_qr, const void* w_uk,
                                    int32_t H, int32_t d_cq, void* w_pack, void* stream) {
  const char* fn = "mla_pack_query_weights";
  if (!w_uq || !w_qr || !w_uk || !w_pack)
    return fail(MLA_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (H < 1 || d_cq < 384 || d_cq % 384)
    return fail(MLA_ERR_SHAPE, "%s: H %d, d_cq %d (a positive multiple of 384)", fn, H, d_cq);
  if ((reinterpret_cast<uintptr_t>(w_uq) | reinterpret_cast<uintptr_t>(w_qr) |
       reinterpret_cast<uintptr_t>(w_uk) | reinterpret_cast<uintptr_t>(w_pack)) & 15)
    return fail(MLA_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned", fn);
  return launched(mla::launch_qpath_pack(w_uq, w_qr, w_uk, H, d_cq, w_pack, as_stream(stream)),
                  "query weight packing");
}

mla_status_t mla_query_path(const float* c_q, int64_t ld_cq, const void* w_pack,
                            const int32_t* seq_lens, float rope_base, void* q_lat, void* q_pe,
                            int32_t B, int32_t H, int32_t d_h, int32_t d_R, int32_t d_c,
                            int32_t d_cq, void* stream) {
  const char* fn = "mla_query_path";
  if (!c_q || !w_pack || !seq_lens || !q_lat || !q_pe)
    return fail(MLA_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (B < 1 || H < 1 || d_h < 1 || d_R < 1 || d_c < 1 || d_cq < 1)
    return fail(MLA_ERR_SHAPE, "%s: sizes must be >= 1", fn);
  if (ld_cq < d_cq)
    return fail(MLA_ERR_SHAPE, "%s: row stride %lld below d_cq %d", fn,
                static_cast<long long>(ld_cq), d_cq);
  if (!std::isfinite(rope_base)) return fail(MLA_ERR_SHAPE, "%s: rope_base not finite", fn);
  if (!mla::qpath_supported(H, d_h, d_R, d_c, d_cq, ld_cq, c_q, w_pack, q_lat, q_pe))
    return fail(MLA_ERR_UNSUPPORTED,
                "%s: needs d_h 128, d_R 64, d_c 512, d_cq %% 384 == 0, ld_cq %% 4 == 0 and "
                "16-byte aligned pointers (got d_h %d, d_R %d, d_c %d, d_cq %d)",
                fn, d_h, d_R, d_c, d_cq);
  return launched(mla::launch_qpath(c_q, ld_cq, w_pack, seq_lens, rope_base, B, H, d_cq, q_lat,
                                    q_pe, as_stream(stream)),
                  "query path");
}

static mla_status_t kv_append(const char* fn, const float* c_kv, int64_t ld_ckv,
                              const float* k_r, int64_t ld_kr, int32_t n_new,
                              const int32_t* seq_lens_before, const int32_t* block_table,
                              void* kv_cache, float rope_base, const mla_paged_shape_t* shape,
                              mla_dtype_t cache_dtype, void* stream) {
  if (!c_kv || !k_r || !seq_lens_before || !block_table || !kv_cache)
    return fail(MLA_ERR_NULL, "%s: a required pointer is NULL", fn);
  mla_status_t st = check_paged_shape(shape);
  if (st != MLA_OK) return st;
  if (n_new < 1) return fail(MLA_ERR_SHAPE, "%s: n_new %d < 1", fn, n_new);
  if (n_new > 65535) return fail(MLA_ERR_SHAPE, "%s: n_new %d > 65535", fn, n_new);
  if (ld_ckv < shape->d_latent || ld_kr < shape->d_rope)
    return fail(MLA_ERR_SHAPE, "%s: row strides %lld / %lld below d_latent / d_rope", fn,
                static_cast<long long>(ld_ckv), static_cast<long long>(ld_kr));
  if (!is_dtype(cache_dtype) && cache_dtype != MLA_FP8)
    return fail(MLA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (!std::isfinite(rope_base)) return fail(MLA_ERR_SHAPE, "%s: rope_base", fn);
  if (cache_dtype == MLA_FP8) {
    if (shape->d_latent != 512 || shape->d_rope != 64)
      return fail(MLA_ERR_UNSUPPORTED, "%s: fp8 rows need d_latent 512, d_rope 64", fn);
    return launched(mla::launch_kv_append_fp8(c_kv, ld_ckv, k_r, ld_kr, n_new, seq_lens_before,
                                              block_table, kv_cache, rope_base, shape->batch,
                                              shape->page_size, shape->max_pages_per_seq,
                                              as_stream(stream)),
                    "cache append (fp8 rows)");
  }
  return launched(mla::launch_kv_append(c_kv, ld_ckv, k_r, ld_kr, n_new, seq_lens_before,
                                        block_table, kv_cache, cache_dtype == MLA_BF16, rope_base,
                                        shape->batch, shape->d_latent, shape->d_rope,
                                        shape->page_size, shape->max_pages_per_seq,
                                        as_stream(stream)),
                  "cache append");
}

mla_status_t mla_kv_append(const float* c_kv, const float* k_r, int32_t n_new,
                           const int32_t* seq_lens_before, const int32_t* block_table,
                           void* kv_cache, float rope_base, const mla_paged_shape_t* shape,
                           mla_dtype_t cache_dtype, void* stream) {
  if (!shape) return fail(MLA_ERR_NULL, "shape is NULL");
  return kv_append("mla_kv_append", c_kv, shape->d_latent, k_r, shape->d_rope, n_new,
                   seq_lens_before, block_table, kv_cache, rope_base, shape, cache_dtype, stream);
}

mla_status_t mla_kv_append_strided(const float* c_kv, int64_t ld_ckv, const float* k_r,
                                   int64_t ld_kr, int32_t n_new, const int32_t* seq_lens_before,
                                   const int32_t* block_table, void* kv_cache, float rope_base,
                                   const mla_paged_shape_t* shape, mla_dtype_t cache_dtype,
                                   void* stream) {
  return kv_append("mla_kv_append_strided", c_kv, ld_ckv, k_r, ld_kr, n_new, seq_lens_before,
                   block_table, kv_cache, rope_base, shape, cache_dtype, stream);
}

mla_status_t mla_prefill_attn(const void* q_c, const void* q_pe, const void* k_c,
                              const void* k_pe, const void* v_c, int32_t B, int32_t T,
                              int32_t H, int32_t d_h, int32_t d_R, float softmax_scale,
                              float* out, float* lse_out, mla_dtype_t dtype, void* stream) {
  if (!q_c || !q_pe || !k_c || !k_pe || !v_c || !out)
    return fail(MLA_ERR_NULL, "mla_prefill_attn: a required pointer is NULL");
  if (B < 1 || T < 1 || H < 1 || d_h < 1 || d_R < 1)
    return fail(MLA_ERR_SHAPE, "mla_prefill_attn: sizes must be >= 1");
  if (B > 65535 || H > 65535 || static_cast<int64_t>(B) * T * H * d_h > (static_cast<int64_t>(1) << 40))
    return fail(MLA_ERR_SHAPE, "mla_prefill_attn: B %d, H %d or the prompt is too large", B, H);
  if (!std::isfinite(softmax_scale))
    return fail(MLA_ERR_SHAPE, "mla_prefill_attn: softmax_scale is not finite");
  if (dtype != MLA_BF16 || !mla::attn_prefill_supported(d_h, d_R))
    return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_attn: BF16 inputs, d_h 128, d_R 64");
  const uintptr_t any = reinterpret_cast<uintptr_t>(q_c) | reinterpret_cast<uintptr_t>(q_pe) |
                        reinterpret_cast<uintptr_t>(k_c) | reinterpret_cast<uintptr_t>(k_pe) |
                        reinterpret_cast<uintptr_t>(v_c) | reinterpret_cast<uintptr_t>(out);
  if (any & 15) return fail(MLA_ERR_SHAPE, "mla_prefill_attn: tensors must be 16-byte aligned");
  return launched(mla::launch_attn_prefill(q_c, q_pe, k_c, k_pe, v_c, B, T, H, softmax_scale,
                                           out, lse_out, as_stream(stream)),
                  "prefill attention");
}

mla_status_t mla_quantize_cache(const void* src, mla_dtype_t src_dtype, int64_t src_ld,
                                int64_t rows, void* dst, void* stream) {
  if (!src || !dst) return fail(MLA_ERR_NULL, "mla_quantize_cache: a pointer is NULL");
  if (rows < 1 || src_ld < 576)
    return fail(MLA_ERR_SHAPE, "mla_quantize_cache: rows %lld < 1 or src_ld %lld < 576",
                static_cast<long long>(rows), static_cast<long long>(src_ld));
  if (rows > (static_cast<int64_t>(1) << 33))
    return fail(MLA_ERR_SHAPE, "mla_quantize_cache: %lld rows", static_cast<long long>(rows));
  if (!is_dtype(src_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "mla_quantize_cache: source dtype F32 or BF16");
  return launched(mla::launch_quantize_rows_fp8(src, src_dtype == MLA_BF16, src_ld, rows, dst,
                                                as_stream(stream)),
                  "fp8 row quantisation");
}

mla_status_t mla_fold_uq(const void* w_uk, const void* w_uq, int32_t H, int32_t d_h,
                         int32_t d_c, int32_t d_cq, mla_dtype_t w_dtype, void* w_out,
                         mla_dtype_t out_dtype, void* stream) {
  if (!w_uk || !w_uq || !w_out) return fail(MLA_ERR_NULL, "mla_fold_uq: a pointer is NULL");
  if (H < 1 || d_h < 1 || d_c < 1 || d_cq < 1)
    return fail(MLA_ERR_SHAPE, "mla_fold_uq: sizes must be >= 1");
  if (!is_dtype(w_dtype) || !is_dtype(out_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "mla_fold_uq: unknown dtype");
  // head i: y[i][m][n] = sum_d w_uk[i d_h + d][m] w_uq[i d_h + d][n], rows i d_c + m of w_out
  mla::GemmArgs g;
  g.x = w_uk; g.ldx = d_c; g.sx = static_cast<int64_t>(d_h) * d_c; g.x_bf16 = w_dtype == MLA_BF16;
  g.x_km = 1;
  g.w = w_uq; g.ldw = d_cq; g.sw = static_cast<int64_t>(d_h) * d_cq; g.w_bf16 = w_dtype == MLA_BF16;
  g.w_nk = false;
  g.y = w_out; g.ldy = d_cq; g.sy = static_cast<int64_t>(d_c) * d_cq; g.y_bf16 = out_dtype == MLA_BF16;
  g.M = d_c; g.N = d_cq; g.K = d_h; g.batch = H;
  return launched(mla::launch_gemm_small(g, as_stream(stream)), "W^UK^T W^UQ fold");
}

mla_status_t mla_fold_o_uv(const void* w_o, const void* w_uv, int32_t H, int32_t d_h,
                           int32_t d_c, int32_t d_model, mla_dtype_t w_dtype, void* w_out,
                           mla_dtype_t out_dtype, void* stream) {
  if (!w_o || !w_uv || !w_out) return fail(MLA_ERR_NULL, "mla_fold_o_uv: a pointer is NULL");
  if (H < 1 || d_h < 1 || d_c < 1 || d_model < 1)
    return fail(MLA_ERR_SHAPE, "mla_fold_o_uv: sizes must be >= 1");
  if (!is_dtype(w_dtype) || !is_dtype(out_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "mla_fold_o_uv: unknown dtype");
  // head i: y[i][n][c] = sum_d w_o[n][i d_h + d] w_uv[i d_h + d][c], columns i d_c + c of w_out
  mla::GemmArgs g;
  g.x = w_o; g.ldx = static_cast<int64_t>(H) * d_h; g.sx = d_h; g.x_bf16 = w_dtype == MLA_BF16;
  g.w = w_uv; g.ldw = d_c; g.sw = static_cast<int64_t>(d_h) * d_c; g.w_bf16 = w_dtype == MLA_BF16;
  g.w_nk = false;
  g.y = w_out; g.ldy = static_cast<int64_t>(H) * d_c; g.sy = d_c; g.y_bf16 = out_dtype == MLA_BF16;
  g.M = d_model; g.N = d_c; g.K = d_h; g.batch = H;
  return launched(mla::launch_gemm_small(g, as_stream(stream)), "W^O W^UV fold");
}

mla_status_t mla_out_proj(const float* o_lat, const void* w_uv, const void* w_o, int32_t B,
                          int32_t H, int32_t d_c, int32_t d_h, int32_t d_model,
                          mla_dtype_t w_dtype, float* o_heads, float* u, void* stream) {
  if (!o_lat || !w_uv || !o_heads) return fail(MLA_ERR_NULL, "mla_out_proj: NULL o_lat/w_uv/o_heads");
  if ((w_o == nullptr) != (u == nullptr))
    return fail(MLA_ERR_NULL, "mla_out_proj: w_o and u must both be given or both NULL");
  if (B < 1 || H < 1 || d_c < 1 || d_h < 1 || (w_o && d_model < 1))
    return fail(MLA_ERR_SHAPE, "mla_out_proj: sizes must be >= 1");
  if (!is_dtype(w_dtype)) return fail(MLA_ERR_UNSUPPORTED, "mla_out_proj: unknown dtype");
  hipStream_t s = as_stream(stream);
  mla::GemmArgs g;
  g.x = o_lat; g.ldx = static_cast<int64_t>(H) * d_c; g.sx = d_c; g.x_bf16 = 0;
  g.w = w_uv; g.ldw = d_c; g.sw = static_cast<int64_t>(d_h) * d_c; g.w_bf16 = w_dtype == MLA_BF16;
  g.w_nk = true;
  g.y = o_heads; g.ldy = static_cast<int64_t>(H) * d_h; g.sy = d_h; g.y_bf16 = 0;
  g.M = B; g.N = d_h; g.K = d_c; g.batch = H;
  mla_status_t st = launched(gemm(g, s), "W^UV GEMM");
  if (st != MLA_OK || !w_o) return st;
  mla::GemmArgs o;
  o.x = o_heads; o.ldx = static_cast<int64_t>(H) * d_h; o.sx = 0; o.x_bf16 = 0;
  o.w = w_o; o.ldw = static_cast<int64_t>(H) * d_h; o.sw = 0; o.w_bf16 = w_dtype == MLA_BF16;
  o.w_nk = true;
  o.y = u; o.ldy = d_model; o.sy = 0; o.y_bf16 = 0;
  o.M = B; o.N = d_model; o.K = H * d_h; o.batch = 1;
  return launched(gemm(o, s), "W^O GEMM");
}

static mla_status_t linear(const char* fn, const void* x, mla_dtype_t x_dtype, int64_t ldx,
                           const void* w, mla_dtype_t w_dtype, int32_t M, int32_t N, int32_t K,
                           float* y, int64_t ldy, int32_t accumulate, void* stream) {
  if (!x || !w || !y) return fail(MLA_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (M < 1 || N < 1 || K < 1) return fail(MLA_ERR_SHAPE, "%s: sizes must be >= 1", fn);
  if (M > 65535 * 64) return fail(MLA_ERR_SHAPE, "%s: M %d too large", fn, M);
  if (ldx < K || ldy < N)
    return fail(MLA_ERR_SHAPE, "%s: row strides ldx %lld < K or ldy %lld < N", fn,
                static_cast<long long>(ldx), static_cast<long long>(ldy));
  if (!is_dtype(x_dtype) || !is_dtype(w_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  mla::GemmArgs g;
  g.x = x; g.ldx = ldx; g.sx = 0; g.x_bf16 = x_dtype == MLA_BF16;
  g.w = w; g.ldw = K; g.sw = 0; g.w_bf16 = w_dtype == MLA_BF16; g.w_nk = true;
  g.y = y; g.ldy = ldy; g.sy = 0; g.y_bf16 = 0;
  g.M = M; g.N = N; g.K = K; g.batch = 1;
  g.accumulate = accumulate != 0;
  return launched(gemm(g, as_stream(stream)), "linear GEMM");
}

mla_status_t mla_linear(const void* x, mla_dtype_t x_dtype, const void* w,
                        mla_dtype_t w_dtype, int32_t M, int32_t N, int32_t K, float* y,
                        void* stream) {
  return linear("mla_linear", x, x_dtype, K, w, w_dtype, M, N, K, y, N, 0, stream);
}

mla_status_t mla_linear_strided(const void* x, mla_dtype_t x_dtype, int64_t ldx, const void* w,
                                mla_dtype_t w_dtype, int32_t M, int32_t N, int32_t K, float* y,
                                int64_t ldy, int32_t accumulate, void* stream) {
  return linear("mla_linear_strided", x, x_dtype, ldx, w, w_dtype, M, N, K, y, ldy, accumulate,
                stream);
}

static mla::GemmArgs det_args(const void* x, mla_dtype_t x_dtype, int64_t ldx, const void* w,
                              int32_t M, int32_t N, int32_t K, float* y, int64_t ldy,
                              int32_t accumulate) {
  mla::GemmArgs g;
  g.x = x; g.ldx = ldx; g.sx = 0; g.x_bf16 = x_dtype == MLA_BF16;
  g.w = w; g.ldw = K; g.sw = 0; g.w_bf16 = 1; g.w_nk = true;
  g.y = y; g.ldy = ldy; g.sy = 0; g.y_bf16 = 0;
  g.M = M; g.N = N; g.K = K; g.batch = 1;
  g.accumulate = accumulate != 0;
  return g;
}

size_t mla_linear_deterministic_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  // any 256-byte aligned pointers and dense strides: the size depends on the shape only
  static const char probe[1] = {0};
  const void* p = reinterpret_cast<const void*>(
      (reinterpret_cast<uintptr_t>(probe) + 255) & ~static_cast<uintptr_t>(255));
  const mla::GemmArgs g = det_args(p, MLA_F32, K, p, M, N, K, static_cast<float*>(const_cast<void*>(p)), N, 0);
  return mla::gemm_stream_det_workspace_bytes(g);
}

mla_status_t mla_linear_deterministic(const void* x, mla_dtype_t x_dtype, int64_t ldx,
                                      const void* w, mla_dtype_t w_dtype, int32_t M, int32_t N,
                                      int32_t K, float* y, int64_t ldy, int32_t accumulate,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mla_linear_deterministic";
  if (!x || !w || !y || !workspace) return fail(MLA_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (M < 1 || N < 1 || K < 1) return fail(MLA_ERR_SHAPE, "%s: sizes must be >= 1", fn);
  if (ldx < K || ldy < N)
    return fail(MLA_ERR_SHAPE, "%s: row strides ldx %lld < K or ldy %lld < N", fn,
                static_cast<long long>(ldx), static_cast<long long>(ldy));
  if (!is_dtype(x_dtype) || w_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "%s: bf16 weights required", fn);
  const mla::GemmArgs g = det_args(x, x_dtype, ldx, w, M, N, K, y, ldy, accumulate);
  const size_t need = mla::gemm_stream_det_workspace_bytes(g);
  if (need == 0 || N % 4 || ldy % 4 || (reinterpret_cast<uintptr_t>(y) & 15) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15))
    return fail(MLA_ERR_UNSUPPORTED,
                "%s: needs M <= 64, N %% 64 == 0, K %% 128 == 0, ldx %% 8 == 0, ldy %% 4 == 0 "
                "and 16-byte aligned x, w, y and workspace (M %d, N %d, K %d)", fn, M, N, K);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, workspace_bytes, need);
  return launched(mla::launch_gemm_stream_det(g, workspace, workspace_bytes, as_stream(stream)),
                  "deterministic linear GEMM");
}

mla_status_t mla_linear_deterministic_append(
    const void* x, mla_dtype_t x_dtype, int64_t ldx, const void* w, mla_dtype_t w_dtype,
    int32_t M, int32_t N, int32_t K, float* y, int64_t ldy, void* workspace,
    size_t workspace_bytes, int32_t append_col, const int32_t* seq_lens_before,
    const int32_t* block_table, void* kv_cache, float rope_base, const mla_paged_shape_t* shape,
    mla_dtype_t cache_dtype, void* stream) {
  const char* fn = "mla_linear_deterministic_append";
  if (!x || !w || !y || !workspace || !seq_lens_before || !block_table || !kv_cache)
    return fail(MLA_ERR_NULL, "%s: a required pointer is NULL", fn);
  mla_status_t st = check_paged_shape(shape);
  if (st != MLA_OK) return st;
  if (M < 1 || N < 1 || K < 1) return fail(MLA_ERR_SHAPE, "%s: sizes must be >= 1", fn);
  if (ldx < K || ldy < N)
    return fail(MLA_ERR_SHAPE, "%s: row strides ldx %lld < K or ldy %lld < N", fn,
                static_cast<long long>(ldx), static_cast<long long>(ldy));
  if (shape->batch != M)
    return fail(MLA_ERR_SHAPE, "%s: M %d rows but a batch of %d sequences", fn, M, shape->batch);
  if (append_col < 0 || static_cast<int64_t>(append_col) + shape->d_latent + shape->d_rope > N)
    return fail(MLA_ERR_SHAPE, "%s: columns %d .. %d + d_latent + d_rope outside the %d columns",
                fn, append_col, append_col, N);
  if (!std::isfinite(rope_base)) return fail(MLA_ERR_SHAPE, "%s: rope_base", fn);
  if (!is_dtype(x_dtype) || w_dtype != MLA_BF16 || cache_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "%s: bf16 weights and a bf16 cache required", fn);
  if (append_col % 4 || shape->d_latent % 4 || shape->d_rope % 4)
    return fail(MLA_ERR_UNSUPPORTED, "%s: append_col, d_latent and d_rope must be multiples of 4", fn);
  const mla::GemmArgs g = det_args(x, x_dtype, ldx, w, M, N, K, y, ldy, 0);
  const size_t need = mla::gemm_stream_det_workspace_bytes(g);
  if (need == 0 || N % 4 || ldy % 4 || (reinterpret_cast<uintptr_t>(y) & 15) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15))
    return fail(MLA_ERR_UNSUPPORTED,
                "%s: needs M <= 64, N %% 64 == 0, K %% 128 == 0, ldx %% 8 == 0, ldy %% 4 == 0 "
                "and 16-byte aligned x, w, y and workspace (M %d, N %d, K %d)", fn, M, N, K);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", fn, workspace_bytes, need);
  mla::AppendArgs app;
  app.cache = kv_cache;
  app.seq_lens_before = seq_lens_before;
  app.block_table = block_table;
  app.col = append_col;
  app.d_c = shape->d_latent;
  app.d_R = shape->d_rope;
  app.page_size = shape->page_size;
  app.max_pages = shape->max_pages_per_seq;
  app.base = rope_base;
  return launched(mla::launch_gemm_stream_det(g, workspace, workspace_bytes, as_stream(stream), app),
                  "deterministic linear GEMM with cache append");
}

mla_status_t mla_linear_planned(const void* x, mla_dtype_t x_dtype, const void* w,
                                mla_dtype_t w_dtype, int32_t M, int32_t N, int32_t K, float* y,
                                int32_t kernel, int32_t tile, int32_t split, int32_t ring,
                                void* stream) {
  if (!x || !w || !y) return fail(MLA_ERR_NULL, "mla_linear_planned: a required pointer is NULL");
  if (M < 1 || N < 1 || K < 1) return fail(MLA_ERR_SHAPE, "mla_linear_planned: sizes must be >= 1");
  if (!is_dtype(x_dtype) || w_dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "mla_linear_planned: bf16 weights required");
  mla::GemmArgs g;
  g.x = x; g.ldx = K; g.sx = 0; g.x_bf16 = x_dtype == MLA_BF16;
  g.w = w; g.ldw = K; g.sw = 0; g.w_bf16 = 1; g.w_nk = true;
  g.y = y; g.ldy = N; g.sy = 0; g.y_bf16 = 0;
  g.M = M; g.N = N; g.K = K; g.batch = 1;
  const hipStream_t s = as_stream(stream);
  if (kernel == 0) {
    if (!mla::gemm_rows_supported(g) || !mla::gemm_rows_plan_ok(g, tile, split, ring))
      return fail(MLA_ERR_UNSUPPORTED, "mla_linear_planned: tile-grid plan (%d, %d, %d) not valid here",
                  tile, split, ring);
    return launched(mla::launch_gemm_rows_with(g, tile, split, ring, s), "linear GEMM");
  }
  if (kernel == 1) {
    if (!mla::gemm_stream_supported(g) || !mla::gemm_stream_plan_ok(g, tile, split, ring))
      return fail(MLA_ERR_UNSUPPORTED, "mla_linear_planned: persistent plan (%d, %d, %d) not valid here",
                  tile, split, ring);
    return launched(mla::launch_gemm_stream_with(g, tile, split, ring, s), "linear GEMM");
  }
  if (kernel == 2) {
    if (!mla::gemm_xs_supported(g) || !mla::gemm_xs_plan_ok(g, tile, ring, split))
      return fail(MLA_ERR_UNSUPPORTED,
                  "mla_linear_planned: activation-stationary plan (%d, %d, %d) not valid here",
                  tile, split, ring);
    return launched(mla::launch_gemm_xs_with(g, tile, ring, split, s), "linear GEMM");
  }
  return fail(MLA_ERR_UNSUPPORTED, "mla_linear_planned: kernel %d unknown", kernel);
}

mla_status_t mla_validate_indices(const int32_t* block_table, const int32_t* seq_lens,
                                  const mla_paged_shape_t* shape, int32_t* dev_count,
                                  void* stream) {
  if (!block_table || !seq_lens || !dev_count)
    return fail(MLA_ERR_NULL, "mla_validate_indices: a required pointer is NULL");
  mla_status_t st = check_paged_shape(shape);
  if (st != MLA_OK) return st;
  return launched(mla::launch_validate_indices(block_table, seq_lens, shape->batch,
                                               shape->page_size, shape->max_pages_per_seq,
                                               shape->num_pages, dev_count, as_stream(stream)),
                  "index validation");
}

mla_status_t mla_stream_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink) return fail(MLA_ERR_NULL, "mla_stream_read: NULL pointer");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(MLA_ERR_SHAPE, "mla_stream_read: bytes %zu must be a positive multiple of 16", bytes);
  return launched(mla::launch_stream_read(src, bytes, sink, as_stream(stream)), "stream read");
}

mla_status_t mla_stream_read_lds(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink) return fail(MLA_ERR_NULL, "mla_stream_read_lds: NULL pointer");
  if (bytes == 0 || bytes % 1024 != 0)
    return fail(MLA_ERR_SHAPE, "mla_stream_read_lds: bytes %zu must be a positive multiple of 1024",
                bytes);
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return fail(MLA_ERR_SHAPE, "mla_stream_read_lds: src is not 16-byte aligned");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return fail(MLA_ERR_LAUNCH, "mla_stream_read_lds: cannot query the compute-unit count");
  return launched(mla::launch_stream_read_lds(src, bytes, sink, cus, as_stream(stream)),
                  "stream read (LDS DMA)");
}

}  // extern "C"
