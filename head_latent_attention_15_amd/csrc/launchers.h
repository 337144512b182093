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
};

// Decode attention, one wavefront per (sequence, head, split), fp32 VALU math.
hipError_t launch_attn_generic_f32_64_16(const PagedArgs& a, hipStream_t s);
hipError_t launch_attn_generic_bf16_512_64(const PagedArgs& a, hipStream_t s);
// Decode attention on bf16 MFMA, all heads of a (sequence, split) per workgroup.
hipError_t launch_attn_mfma_bf16_512_64(const PagedArgs& a, hipStream_t s);
bool attn_mfma_supported(const PagedArgs& a);

// Split-K combine fused with the W^UV up-projection (d_c = 512, d_h = 128, S <= 64, bf16
// W^UV): o_heads[b][i] = W^UV_i combine_s(o_part[b][i][s], lse_part[b][i][s]).
bool combine_uv_supported(int H, int S, int d_c, int d_h, const void* o_part, const void* w_uv,
                          int B);
hipError_t launch_combine_uv(const void* o_part, int part_bf16, const float* lse_part,
                             const void* w_uv, float* o_heads, int B, int H, int S,
                             hipStream_t s);

hipError_t launch_splitk_combine(const void* o_part, int part_bf16, const float* lse_part, int B,
                                 int H, int S, int d_c, float* out, float* lse_out, hipStream_t s);

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

}  // namespace mla
