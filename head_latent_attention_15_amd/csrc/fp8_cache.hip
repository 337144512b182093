// fp8 latent cache rows: quantisation of cache rows and the append of new tokens.
//
// A cached token is a 656-byte row: the latent c^KV (512 values) as OCP E4M3 codes, the
// rotated k^R (64 values) in bf16, and four fp32 power-of-two scales, one per 128-value
// latent block.  Block b stores x / s_b with s_b = 2^k, k the smallest integer such that
// max|x| <= 448 * 2^k (1 for an all-zero block); a code is the E4M3 value nearest to
// x / s_b, ties to the even code.  The pages name KV-cache quantisation as a companion of
// MLA's smaller cache but fix no format (kasblo.com/?p=4663, "GQA・量子化・FlashAttention
// とは何が違うのか"; "論文解説: DeepSeek-V2 …", "実装のポイント（Implementation）"); this
// one makes dequantisation exact in bf16.
//
// Every step is exact in fp32 (a power-of-two scaling and integer rounding of the
// mantissa), so the codes do not depend on how the value reached fp32.
#include "device_common.h"
#include "launchers.h"

namespace mla {
namespace {

constexpr int LAT = 512, RP = 64, FP8_ROW = 656;

// k with 2^k the block scale of a block whose largest magnitude is amax > 0: amax = m 2^E
// with m in [1, 2); 448 = 1.75 2^8, so amax <= 448 2^k  <=>  k >= E - 8 (m <= 1.75) or
// k >= E - 7 (m > 1.75).
__device__ __forceinline__ int scale_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int biased = static_cast<int>((u >> 23) & 0xff);
  if (biased == 0) {  // fp32 subnormal: normalise through frexp
    int e;
    const float m = frexpf(amax, &e);  // amax = m 2^e, m in [0.5, 1)
    return (e - 1) - 8 + (2.f * m > 1.75f ? 1 : 0);
  }
  const int E = biased - 127;
  return E - 8 + ((u & 0x7fffff) > 0x600000u ? 1 : 0);
}

// E4M3 code nearest to y (|y| <= 448), ties to even, from the fp32 bits.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 0.015625f) {  // 2^-6 and up: normal codes; round the mantissa to 3 bits
    const uint32_t ua = __float_as_uint(a);
    const uint32_t E = ((ua >> 23) & 0xff) - 127 + 7;
    const uint32_t m = ua & 0x7fffff;
    const uint32_t keep = m >> 20, rem = m & 0xfffff;
    code = (E << 3) | keep;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1))) ++code;  // carries into E
    code = min(code, 0x7eu);  // saturate at 448
  } else {                  // subnormal steps of 2^-9 (8 steps reach 2^-6, code 0x08)
    code = static_cast<uint32_t>(rintf(a * 512.f));  // exact scaling, round half to even
  }
  return code | sign;
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16raw>(bf16raw v) { return bf16_to_f32(v); }

// One wavefront quantises one row's latent: lane l holds values 8 l .. 8 l + 7 (block
// l / 16), writes their codes (8 bytes at 8 l) and, for l = 16 b, block b's scale.
__device__ __forceinline__ void quantize_latent_wave(const float (&x)[8], int lane,
                                                     unsigned char* __restrict__ row) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const int k = amax > 0.f ? scale_exponent(amax) : 0;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = e4m3_code(ldexpf(x[i], -k));
    if (i < 4) lo |= c << (8 * i);
    else hi |= c << (8 * (i - 4));
  }
  *reinterpret_cast<uint2*>(row + 8 * lane) = make_uint2(lo, hi);
  if ((lane & 15) == 0) *reinterpret_cast<float*>(row + LAT + 2 * RP + 4 * (lane >> 4)) = ldexpf(1.f, k);
}

// rows of 576 values (bf16 or fp32, row stride src_ld elements) -> 656-byte rows
template <typename T>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const T* __restrict__ src,
                                                            int64_t src_ld, int64_t rows,
                                                            unsigned char* __restrict__ dst) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const T* s = src + r * src_ld;
  unsigned char* row = dst + r * FP8_ROW;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = to_f32(s[8 * lane + i]);
  quantize_latent_wave(x, lane, row);
  // k^R: 64 bf16 values, lanes 0 .. 31 two each
  if (lane < 32) {
    const uint32_t a = f32_to_bf16(to_f32(s[LAT + 2 * lane]));
    const uint32_t b = f32_to_bf16(to_f32(s[LAT + 2 * lane + 1]));
    *reinterpret_cast<uint32_t*>(row + LAT + 4 * lane) = a | (b << 16);
  }
}

// Append n_new tokens per sequence: c^KV quantised, k^R rotated to position
// seq_lens_before[b] + t (fp64 angle) and rounded to bf16; the inputs of token t of
// sequence b are rows b n_new + t of c_kv and k_r (row strides ld_c, ld_k).  One
// wavefront per token.
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(
    const float* __restrict__ c_kv, int64_t ld_c, const float* __restrict__ k_r, int64_t ld_k,
    int n_new, const int32_t* __restrict__ seq_lens_before,
    const int32_t* __restrict__ block_table, unsigned char* __restrict__ cache, float base,
    int B, int page_size, int max_pages) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= B * n_new) return;
  const int lane = threadIdx.x & 63;
  const int b = item / n_new, t = item % n_new;
  const int64_t pos = static_cast<int64_t>(seq_lens_before[b]) + t;
  const int page = block_table[static_cast<int64_t>(b) * max_pages + pos / page_size];
  unsigned char* row = cache + (static_cast<int64_t>(page) * page_size + pos % page_size) * FP8_ROW;
  const float* c = c_kv + (static_cast<int64_t>(b) * n_new + t) * ld_c;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = c[8 * lane + i];
  quantize_latent_wave(x, lane, row);
  if (lane < RP / 2) {
    const float* kr = k_r + (static_cast<int64_t>(b) * n_new + t) * ld_k;
    float y0, y1;
    rope_pair(kr[2 * lane], kr[2 * lane + 1], pos, lane, RP, base, &y0, &y1);
    *reinterpret_cast<uint32_t*>(row + LAT + 4 * lane) =
        static_cast<uint32_t>(f32_to_bf16(y0)) | (static_cast<uint32_t>(f32_to_bf16(y1)) << 16);
  }
}

}  // namespace

hipError_t launch_quantize_rows_fp8(const void* src, int src_bf16, int64_t src_ld, int64_t rows,
                                    void* dst, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (src_bf16)
    hipLaunchKernelGGL(quantize_rows_kernel<bf16raw>, grid, dim3(256), 0, s,
                       static_cast<const bf16raw*>(src), src_ld, rows,
                       static_cast<unsigned char*>(dst));
  else
    hipLaunchKernelGGL(quantize_rows_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(src), src_ld, rows,
                       static_cast<unsigned char*>(dst));
  return hipGetLastError();
}

hipError_t launch_kv_append_fp8(const float* c_kv, int64_t ld_c, const float* k_r, int64_t ld_k,
                                int n_new, const int32_t* seq_lens_before,
                                const int32_t* block_table, void* cache, float base, int B,
                                int page_size, int max_pages, hipStream_t s) {
  const int items = B * n_new;
  hipLaunchKernelGGL(kv_append_fp8_kernel, dim3((items + 3) / 4), dim3(256), 0, s, c_kv, ld_c,
                     k_r, ld_k, n_new, seq_lens_before, block_table,
                     static_cast<unsigned char*>(cache), base, B, page_size, max_pages);
  return hipGetLastError();
}

}  // namespace mla
