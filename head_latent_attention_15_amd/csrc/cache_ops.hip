// Cache-side kernels: query RoPE, latent-cache append, paging-index validation, and two
// streaming-read kernels (plain vector loads; LDS DMA) used as measured HBM read ceilings.
//
// RoPE ("kasblo.com/?p=4663", "分離したRoPE"; qiita.com/joule "RoPE の扱い"): pair
// (x[2k], x[2k+1]) turns by pos * base^(-2k/d_R); the decoupled key k^R is shared by all
// heads and cached after rotation next to the latent c^KV ("論文解説: DeepSeek-V2 …",
// "Decoupled RoPE": 576 elements per token per layer).
#include "device_common.h"
#include "attn_common.h"
#include "launchers.h"

namespace mla {

// out[r][:] = RoPE(x row r, seq_lens[r / rows_per_seq] + pos_offset), where row r of x starts
// at x + (r / rows_per_seq) ld_seq + (r % rows_per_seq) d_R (rows of one sequence contiguous,
// sequences ld_seq elements apart) and out is dense [rows][d_R]
template <typename OT>
__global__ __launch_bounds__(256) void rope_rows_kernel(const float* __restrict__ x,
                                                        int64_t rows, int rows_per_seq, int d_R,
                                                        int64_t ld_seq,
                                                        const int32_t* __restrict__ seq_lens,
                                                        int pos_offset, float base,
                                                        OT* __restrict__ out) {
  const int half = d_R / 2;
  const int64_t total = rows * half;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = e / half;
    const int k = static_cast<int>(e % half);
    const int64_t sq = r / rows_per_seq;
    const int64_t pos = static_cast<int64_t>(seq_lens[sq]) + pos_offset;
    const float* xr = x + sq * ld_seq + (r - sq * rows_per_seq) * d_R;
    float y0, y1;
    rope_pair(xr[2 * k], xr[2 * k + 1], pos, k, d_R, base, &y0, &y1);
    st(out + r * d_R + 2 * k, y0);
    st(out + r * d_R + 2 * k + 1, y1);
  }
}

hipError_t launch_rope_rows(const float* x, int64_t rows, int rows_per_seq, int d_R,
                            int64_t ld_seq, const int32_t* seq_lens, int pos_offset, float base,
                            void* out, int out_bf16, hipStream_t s) {
  const int64_t total = rows * (d_R / 2);
  const int blocks = static_cast<int>(total < 256 * 1024 ? (total + 255) / 256 : 1024);
  if (out_bf16) {
    hipLaunchKernelGGL(rope_rows_kernel<bf16raw>, dim3(blocks), dim3(256), 0, s, x, rows,
                       rows_per_seq, d_R, ld_seq, seq_lens, pos_offset, base,
                       static_cast<bf16raw*>(out));
  } else {
    hipLaunchKernelGGL(rope_rows_kernel<float>, dim3(blocks), dim3(256), 0, s, x, rows,
                       rows_per_seq, d_R, ld_seq, seq_lens, pos_offset, base,
                       static_cast<float*>(out));
  }
  return hipGetLastError();
}

// One workgroup per appended token: row [c^KV | RoPE(k^R, pos)] at its page and slot.  The
// inputs of token t of sequence b are rows b n_new + t of c_kv and k_r, ld_c and ld_k
// elements apart.
template <typename CT>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const float* __restrict__ c_kv, int64_t ld_c, const float* __restrict__ k_r, int64_t ld_k,
    int n_new, const int32_t* __restrict__ seq_lens_before, const int32_t* __restrict__ block_table,
    CT* __restrict__ cache, float base, int d_c, int d_R, int P, int max_pages) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int pos = seq_lens_before[b] + t;
  const int page = block_table[static_cast<int64_t>(b) * max_pages + pos / P];
  CT* row = cache + (static_cast<int64_t>(page) * P + pos % P) * (d_c + d_R);
  const float* c = c_kv + (static_cast<int64_t>(b) * n_new + t) * ld_c;
  for (int i = threadIdx.x; i < d_c; i += blockDim.x) st(row + i, c[i]);
  const float* kr = k_r + (static_cast<int64_t>(b) * n_new + t) * ld_k;
  for (int k = threadIdx.x; k < d_R / 2; k += blockDim.x) {
    float y0, y1;
    rope_pair(kr[2 * k], kr[2 * k + 1], pos, k, d_R, base, &y0, &y1);
    st(row + d_c + 2 * k, y0);
    st(row + d_c + 2 * k + 1, y1);
  }
}

hipError_t launch_kv_append(const float* c_kv, int64_t ld_c, const float* k_r, int64_t ld_k,
                            int n_new, const int32_t* seq_lens_before, const int32_t* block_table,
                            void* cache, int cache_bf16, float base, int B, int d_c, int d_R,
                            int page_size, int max_pages, hipStream_t s) {
  dim3 grid(n_new, B);
  if (cache_bf16) {
    hipLaunchKernelGGL(kv_append_kernel<bf16raw>, grid, dim3(256), 0, s, c_kv, ld_c, k_r, ld_k,
                       n_new, seq_lens_before, block_table, static_cast<bf16raw*>(cache), base,
                       d_c, d_R, page_size, max_pages);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, s, c_kv, ld_c, k_r, ld_k,
                       n_new, seq_lens_before, block_table, static_cast<float*>(cache), base,
                       d_c, d_R, page_size, max_pages);
  }
  return hipGetLastError();
}

// Single workgroup: counts invalid seq_lens and referenced out-of-pool page indices.
__global__ __launch_bounds__(256) void validate_indices_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int B, int P,
    int max_pages, int num_pages, int32_t* __restrict__ count) {
  __shared__ int red[4];
  int bad = 0;
  const int64_t cap = static_cast<int64_t>(max_pages) * P;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int L = seq_lens[b];
    if (L < 0 || L > cap) {
      ++bad;
      continue;
    }
    const int np = (L + P - 1) / P;
    for (int p = 0; p < np; ++p) {
      const int e = block_table[static_cast<int64_t>(b) * max_pages + p];
      bad += (e < 0 || e >= num_pages) ? 1 : 0;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) *count = red[0] + red[1] + red[2] + red[3];
}

hipError_t launch_validate_indices(const int32_t* block_table, const int32_t* seq_lens, int B,
                                   int page_size, int max_pages, int num_pages, int32_t* count,
                                   hipStream_t s) {
  hipLaunchKernelGGL(validate_indices_kernel, dim3(1), dim3(256), 0, s, block_table, seq_lens,
                     B, page_size, max_pages, num_pages, count);
  return hipGetLastError();
}

// Streaming read: 16-byte loads, grid-stride, one float per workgroup to defeat elision.
constexpr int kStreamBlocks = 4096;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          int64_t n16, float* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i];
    const u32x4 b = src[i + stride];
    const u32x4 c = src[i + 2 * stride];
    const u32x4 d = src[i + 3 * stride];
    const u32x4 x = a ^ b ^ c ^ d;
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = static_cast<float>(acc & 0xffff);
}

// Streaming read through LDS DMA, the copy instruction the attention kernels stage their
// cache tiles with: 8 wavefronts per workgroup, each copying 1 KB units (16 bytes per lane,
// global_load_lds_dwordx4) grid-stride into a 16-slot LDS ring with up to 15 copies in
// flight, so the chip holds ~128 KB of reads in flight per CU.  Nothing computes on the
// data; after the last copy each workgroup writes one word of its LDS to the sink.
constexpr int kDmaSlots = 16;

__global__ __launch_bounds__(512) void stream_read_lds_kernel(const char* __restrict__ src,
                                                              int64_t units,
                                                              float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char ring[8 * kDmaSlots * 1024];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint32_t base = static_cast<uint32_t>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) char*)ring)) + w * kDmaSlots * 1024;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * 8;
  int k = 0;
  for (int64_t u = blockIdx.x * 8 + w; u < units; u += nw, ++k) {
    if (k >= kDmaSlots) attn::wait_vmcnt<kDmaSlots - 1>();  // the slot's previous copy landed
    attn::dma16(src + u * 1024, static_cast<uint32_t>(lane) * 16u, base + (k % kDmaSlots) * 1024);
  }
  attn::wait_vmcnt<0>();
  attn::block_barrier();
  if (threadIdx.x == 0) sink[blockIdx.x] = static_cast<float>(*reinterpret_cast<volatile int*>(ring) & 0xffff);
}

hipError_t launch_stream_read_lds(const void* src, size_t bytes, float* sink, int grid,
                                  hipStream_t s) {
  hipLaunchKernelGGL(stream_read_lds_kernel, dim3(grid), dim3(512), 0, s,
                     static_cast<const char*>(src), static_cast<int64_t>(bytes / 1024), sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace mla
