// Host-side launchers of the libmla kernels.  Arguments are validated by the C ABI layer
// (mla_api.cpp) before any of these is called; each launcher only sizes the grid and
// enqueues on the given stream, returning the runtime's launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct PagedArgs {
  const void* q_lat;
  const void* q_pe;
  const void* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t B, H, d_c, d_R, page_size, max_pages, num_pages;
  float scale;
  int32_t num_splits;
  int32_t pages_per_split;
  void* o_part;      // fp32 or bf16 (part_bf16), [B][H][S][d_c]
  int part_bf16;     // 1: o_part elements are bf16 (round to nearest even)
  float* lse_part;
  int32_t n_q;       // query tokens per sequence (rows b n_q + t of q and of the partials)
  // In-launch merge of the splits (attn_mfma only; merge_cnt NULL = none): two counters per
  // query row (zero on entry, left zero), then one error word; out [rows][H][d_c] fp32 and
  // lse_out [rows][H] (or NULL) receive the combined result.
  int* merge_cnt = nullptr;
  float* out = nullptr;
  float* lse_out = nullptr;
};

// Decode attention, one wavefront per (sequence, head, split), fp32 VALU math.
hipError_t launch_attn_generic_f32_64_16(const PagedArgs& a, hipStream_t s);
hipError_t launch_attn_generic_bf16_512_64(const PagedArgs& a, hipStream_t s);
// Decode attention on bf16 MFMA, all heads of a (sequence, split) per workgroup.
hipError_t launch_attn_mfma_bf16_512_64(const PagedArgs& a, hipStream_t s);
bool attn_mfma_supported(const PagedArgs& a);
// The same kernel over fp8 latent rows (656 bytes: 512 E4M3 codes, 64 bf16 k^R, 4 fp32
// block scales; 128 heads), bf16 queries.
bool attn_mfma_fp8_supported(const PagedArgs& a);
hipError_t launch_attn_mfma_fp8(const PagedArgs& a, hipStream_t s);
// fp8 latent rows: rows of 576 values (bf16 or fp32, row stride src_ld) quantised into
// 656-byte rows, and the append of new tokens (c^KV quantised, k^R rotated, bf16).
hipError_t launch_quantize_rows_fp8(const void* src, int src_bf16, int64_t src_ld, int64_t rows,
                                    void* dst, hipStream_t s);
hipError_t launch_kv_append_fp8(const float* c_kv, int64_t ld_c, const float* k_r, int64_t ld_k,
                                int n_new, const int32_t* seq_lens_before,
                                const int32_t* block_table, void* cache, float base, int B,
                                int page_size, int max_pages, hipStream_t s);
// Causal prefill attention in the expanded form (d_h = 128, d_R = 64, bf16 inputs):
// q_c [B][T][H][128], q_pe [B][T][H][64], k_c [B][T][H][128], k_pe [B][T][64] (shared by the
// heads), v_c [B][T][H][128]; out [B][T][H][128] fp32, lse_out [B][T][H] or NULL.
bool attn_prefill_supported(int d_h, int d_R);
hipError_t launch_attn_prefill(const void* q_c, const void* q_pe, const void* k_c,
                               const void* k_pe, const void* v_c, int B, int T, int H,
                               float scale, float* out, float* lse_out, hipStream_t s);
// Whole grid of the head-partitioned kernel resident at once on the current device (the
// condition for its in-launch merge, whose workgroups wait for each other).
bool attn_mfma_grid_resident(const PagedArgs& a);
// The same product for 128 heads with the latent product partitioned by columns across the
// wavefronts (each LDS fragment read feeds several MFMAs).
hipError_t launch_attn_cols_bf16_512_64(const PagedArgs& a, hipStream_t s);
bool attn_cols_supported(const PagedArgs& a);
// The same products for 128 heads with four wavefronts of 32 heads on the 32 x 32 x 16
// MFMA (each LDS fragment read feeds 32 heads).
hipError_t launch_attn_wide_bf16_512_64(const PagedArgs& a, hipStream_t s);
bool attn_wide_supported(const PagedArgs& a);
// Its flattened ragged work list (as launch_attn_mfma_ragged; bf16 partials); fp8: the
// cache holds fp8 rows.
hipError_t launch_attn_wide_ragged(const PagedArgs& a, int grid, int* seq_slots, int* err,
                                   hipStream_t s, bool fp8 = false);
// The same split-grid kernel over fp8 latent rows (raw rows staged in LDS and converted to bf16 there).
hipError_t launch_attn_wide_fp8(const PagedArgs& a, hipStream_t s);

// Split-K combine fused with the W^UV up-projection (d_c = 512, d_h = 128, S <= 64, bf16
// W^UV): o_heads[b][i] = W^UV_i combine_s(o_part[b][i][s], lse_part[b][i][s]).
bool combine_uv_supported(int H, int S, int d_c, int d_h, const void* o_part, const void* w_uv,
                          int B);
hipError_t launch_combine_uv(const void* o_part, int part_bf16, const float* lse_part,
                             const void* w_uv, float* o_heads, int B, int H, int S,
                             hipStream_t s);

hipError_t launch_splitk_combine(const void* o_part, int part_bf16, const float* lse_part, int B,
                                 int H, int S, int d_c, float* out, float* lse_out, hipStream_t s);
// Combine of the flattened work list's partials (d_c = 512): with (first, count) =
// (seq_slots[2b], seq_slots[2b + 1]), head h of sequence b has rows first H + h count + i,
// i < count, of o_part [.][512] and lse_part.
hipError_t launch_combine_slots(const void* o_part, int part_bf16, const float* lse_part,
                                const int* seq_slots, int B, int H, float* out, float* lse_out,
                                hipStream_t s);
// Decode attention of a ragged batch over the flattened work list (n_q = 1): `grid`
// workgroups each take an equal page range of the batch's concatenated cached pages;
// room for (grid + B) H partial rows of 512 (o_part, part_bf16) and lse values (lse_part);
// seq_slots [2B] receives (first piece, piece count) per sequence; *err is set to 1 (and
// every count to 0) when a range would exceed 1024 pages, else to 0.
hipError_t launch_attn_mfma_ragged(const PagedArgs& a, int grid, int* seq_slots, int* err,
                                   hipStream_t s);
int attn_mfma_ragged_max_range_pages();

// Batched small-M GEMM: y[z][m][n] = sum_k x[z][m][k] * W_z(n, k), with
// W_z(n, k) = w[z*sw + n*ldw + k] when w_nk, else w[z*sw + k*ldw + n].
// x/w dtype: 0 = fp32, 1 = bf16; y dtype likewise.
// accumulate: y += the product (y holds its prior values; fp32 y only) instead of y = it.
struct GemmArgs {
  const void* x; int64_t ldx, sx; int x_bf16;
  const void* w; int64_t ldw, sw; int w_bf16; bool w_nk;
  void* y; int64_t ldy, sy; int y_bf16;
  int M, N, K, batch;
  int accumulate = 0;
  int x_km = 0;  // x[z][m][k] at x[z*sx + k*ldx + m] (launch_gemm_small only)
};
hipError_t launch_gemm_small(const GemmArgs& g, hipStream_t s);
// Same product on bf16 MFMA for bf16 nn.Linear-layout weights (w_nk), fp32 y and K a
// multiple of 128 (gemm_rows_supported); split-K results are added with fp32 atomics.
// The plan picks the tile width (tn 16-column tiles per wavefront), the k split and the
// depth of the weight ring; launch_gemm_rows_with takes them explicitly (checked by
// gemm_rows_plan_ok).
bool gemm_rows_supported(const GemmArgs& g);
void gemm_rows_plan(const GemmArgs& g, int* tn, int* ks, int* ring);
bool gemm_rows_plan_ok(const GemmArgs& g, int tn, int ks, int ring);
hipError_t launch_gemm_rows_with(const GemmArgs& g, int tn, int ks, int ring, hipStream_t s);
hipError_t launch_gemm_rows(const GemmArgs& g, hipStream_t s);
// Persistent form of the same product for M <= 64 and N a multiple of 64: one workgroup per
// CU, each streaming an equal run of (64 tn columns x 128 k) units with a continuous weight
// ring (depth `ring` k-steps); partial tile sums added into y with fp32 atomics.
bool gemm_stream_supported(const GemmArgs& g);
void gemm_stream_plan(const GemmArgs& g, int* tn, int* grid, int* ring);
bool gemm_stream_plan_ok(const GemmArgs& g, int tn, int grid, int ring);
hipError_t launch_gemm_stream_with(const GemmArgs& g, int tn, int grid, int ring, hipStream_t s);
hipError_t launch_gemm_stream(const GemmArgs& g, hipStream_t s);
// Deterministic form: partial tiles into a workspace of gemm_stream_det_workspace_bytes(g)
// (0 where the kernel does not apply), then a fixed-order sum into y.  Needs N, ldy and sy
// multiples of 4 and 16-byte aligned y and workspace.
size_t gemm_stream_det_workspace_bytes(const GemmArgs& g);
// The new token's cache row written by the second (summing) launch: row b of y holds c^KV
// at columns col .. col + d_c - 1 and k^R (before RoPE) right after it; the row
// [c^KV | RoPE(k^R, pos)] goes to the bf16 cache at position pos = seq_lens_before[b], as
// launch_kv_append writes it for one new token.  cache == nullptr: no append.
struct AppendArgs {
  void* cache = nullptr;
  const int32_t* seq_lens_before = nullptr;
  const int32_t* block_table = nullptr;
  int col = 0, d_c = 0, d_R = 0, page_size = 0, max_pages = 0;
  float base = 0.f;
};
hipError_t launch_gemm_stream_det(const GemmArgs& g, void* part, size_t bytes, hipStream_t s,
                                  const AppendArgs& app = AppendArgs());
// Activation-stationary form for M <= 64, N a multiple of 128 and K of 256: a workgroup
// stages one k slice (32 s values) of x in LDS once and streams the weights of a run of
// 128 tn-column tiles in it.  The plan picks tn (1, 2), s (8, 12, 16, 20) and the grid.
bool gemm_xs_supported(const GemmArgs& g);
bool gemm_xs_plan(const GemmArgs& g, int* tn, int* s, int* grid);
bool gemm_xs_plan_ok(const GemmArgs& g, int tn, int s, int grid);
hipError_t launch_gemm_xs_with(const GemmArgs& g, int tn, int s, int grid, hipStream_t st);
hipError_t launch_gemm_xs(const GemmArgs& g, hipStream_t st);

// Query absorption q~_i = W^UK_i^T q^C_i on bf16 MFMA (bf16 W^UK, bf16 q~, d_h = 128);
// row b of q_c starts at q_c + b ld_q, its heads d_h apart.  With q_r non-NULL (only where
// absorb_rope_fusable) the same launch writes q_pe = RoPE(q_r, seq_lens - 1) in bf16.
bool absorb_mfma_supported(int B, int H, int d_h, int d_c, const void* q_c, int64_t ld_q,
                           const void* w_uk, const void* q_lat);
bool absorb_rope_fusable(int d_c, int d_R, const float* q_r, int64_t ld_r, const void* q_pe);
hipError_t launch_absorb_mfma(const float* q_c, int64_t ld_q, const void* w_uk, void* q_lat,
                              int B, int H, int d_c, const float* q_r, int64_t ld_r,
                              const int32_t* seq_lens, float rope_base, void* q_pe,
                              hipStream_t s);

// The query side in one launch per 64-row block (qpath.hip): q^C_i and q^R_i from c^Q,
// RoPE, and q~_i = W^UK_i^T q^C_i, bf16 weights (packed by launch_qpath_pack into
// qpath_pack_elems bf16) and outputs.
bool qpath_supported(int H, int d_h, int d_R, int d_c, int d_cq, int64_t ld_q, const void* c_q,
                     const void* w_pack, const void* q_lat, const void* q_pe);
int64_t qpath_pack_elems(int H, int d_cq);
hipError_t launch_qpath_pack(const void* w_uq, const void* w_qr, const void* w_uk, int H,
                             int d_cq, void* out, hipStream_t s);
hipError_t launch_qpath(const float* c_q, int64_t ld_q, const void* w_pack,
                        const int32_t* seq_lens, float rope_base, int B, int H, int d_cq,
                        void* q_lat, void* q_pe, hipStream_t s);

hipError_t launch_rope_rows(const float* x, int64_t rows, int rows_per_seq, int d_R,
                            int64_t ld_seq, const int32_t* seq_lens, int pos_offset, float base,
                            void* out, int out_bf16, hipStream_t s);

hipError_t launch_kv_append(const float* c_kv, int64_t ld_c, const float* k_r, int64_t ld_k,
                            int n_new, const int32_t* seq_lens_before, const int32_t* block_table,
                            void* cache, int cache_bf16, float base, int B, int d_c, int d_R,
                            int page_size, int max_pages, hipStream_t s);

hipError_t launch_validate_indices(const int32_t* block_table, const int32_t* seq_lens, int B,
                                   int page_size, int max_pages, int num_pages, int32_t* count,
                                   hipStream_t s);

hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, hipStream_t s);

// The fixed device scratch of the entry point that allocates nothing: its size, and the
// current device's copy (looked up with hipGetSymbolAddress on a device's first use).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);
hipError_t launch_stream_read_lds(const void* src, size_t bytes, float* sink, int grid,
                                  hipStream_t s);

}  // namespace mla
