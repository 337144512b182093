// Pieces shared by the MFMA attention kernels (attn_mfma.hip, attn_cols.hip, attn_wide.hip):
// the cache-tile geometry in LDS, its 16-byte-chunk swizzle, the HBM -> LDS copy issued
// from inline assembly and the explicit wait counts that go with it, and the staging of
// fp8 rows into that tile layout.
#pragma once

#include "device_common.h"

namespace mla {
namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
typedef __attribute__((address_space(3))) float lds_f32_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) int32_t lds_i32_t;

constexpr int DC = 512, DR = 64, ROW = DC + DR;
constexpr int ROW_BYTES = ROW * 2;                  // 1152
constexpr int CHUNKS = ROW_BYTES / 16;              // 72 sixteen-byte chunks per row
constexpr int TILE = 32;                            // tokens per tile
constexpr int TILE_CHUNKS = TILE * CHUNKS;          // 2304
constexpr int TILE_WAVE_COPIES = TILE_CHUNKS / 64;  // 36 wave-wide 16-byte copies per tile
constexpr int TILE_BYTES = TILE_CHUNKS * 16;        // 36864
constexpr int KSTEPS = ROW / 32;                    // 18 k-steps of the score product
constexpr float LN2 = 0.6931471805599453f;

// 16-byte-chunk swizzle of tile row t (0..31): logical chunk c of the row is stored at
// position c ^ swz(t).  Measured on gfx950, this map keeps conflict-free (full LDS read
// rate) both the ds_read_b128 of the score operand (rows 8 (r >> 2) + 4 mt + (r & 3), one
// chunk column per 16-lane group) and the transposing ds_read_b64_tr_b16 of the PV operand
// (rows 8 g + 4 r + 0..3 x 2 adjacent chunks).
__device__ __forceinline__ int swz(int t) {
  return ((((t >> 3) & 3) ^ (t & 3)) << 1) | ((t >> 2) & 1);
}

// Source offset (bytes from the tile's first row) of LDS chunk `chunk` (0..2303) of a tile:
// row t = chunk / 72, stored position p = chunk % 72, which holds logical chunk p ^ swz(t);
// rows past `last` repeat row `last`.
__device__ __forceinline__ uint32_t tile_chunk_voff(unsigned chunk, unsigned last) {
  // chunk / 72 on the full-rate 24-bit multiplier: floor(chunk * 14564 / 2^20) equals
  // chunk / 72 for every chunk below 2304
  const unsigned t = __umul24(chunk, 14564u) >> 20;
  const unsigned c = (chunk - __umul24(t, static_cast<unsigned>(CHUNKS))) ^ swz(t);
  const unsigned trow = min(t, last);
  return __umul24(trow, static_cast<unsigned>(ROW_BYTES)) + c * 16;
}

// fp8 latent rows (656 bytes: 512 E4M3 codes, 64 bf16 k^R values, 4 fp32 block scales, one
// per 128 codes) are copied into LDS raw, a tile of 32 rows as 41 chunks of 16 bytes per row
// in 21 wave-wide copies of 1 KB, and converted there into the bf16 tile layout above.
constexpr int FP8_ROW_BYTES = 656;
constexpr int FP8_ROW_CHUNKS = FP8_ROW_BYTES / 16;                  // 41
constexpr int FP8_TILE_CHUNKS = TILE * FP8_ROW_CHUNKS;               // 1312
constexpr int FP8_COPIES = (FP8_TILE_CHUNKS + 63) / 64;              // 21 wave copies
constexpr int FP8_STAGE_BYTES = FP8_COPIES * 1024;                   // 21504

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ void block_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// 16 bytes per lane from base + voff (global) to LDS address lds_addr + 16 * lane.
// lds_addr and base are wave-uniform.  M0 carries the LDS address; the s_nop covers the
// M0-write to LDS-DMA hazard.  The copy has no destination registers and is kept out of
// the compiler's view, so the compiler adds no vmcnt(0) wait in front of LDS reads; the
// kernels wait for their copies with explicit counts.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b64 = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64 >> 32));
  const void* ubase = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
  const uint32_t ulds = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(ulds), "v"(voff), "s"(ubase)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy q (0 .. 20) of a raw fp8 tile whose first row is at `base`: lane l moves chunk
// n = 64 q + l, i.e. row n / 41, bytes 16 (n % 41) .. of it, to staging byte 16 n (stage_lds
// + 1024 q + 16 l); lanes past the tile's 1312 chunks re-read its last chunk into the
// buffer's tail.  Rows past `last` repeat row `last`.
__device__ __forceinline__ void fp8_tile_copy(const char* base, unsigned last, uint32_t stage_lds,
                                              unsigned q, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));  // recomputed at every copy (no live ranges across the loop)
  const unsigned n = min(64u * q + ln, static_cast<unsigned>(FP8_TILE_CHUNKS - 1));
  const unsigned t = __umul24(n, 3197u) >> 17;  // n / 41 for n < 1312
  const unsigned c = n - __umul24(t, static_cast<unsigned>(FP8_ROW_CHUNKS));
  const unsigned row = min(t, last);
  dma16(base, __umul24(row, static_cast<unsigned>(FP8_ROW_BYTES)) + 16u * c, stage_lds + q * 1024);
}

// Latent chunk e (0 .. 2047) of a bf16 tile from the staged raw rows at src: row t = e / 64,
// logical chunk c = e % 64 (latent values 8 c .. 8 c + 7: 8 codes of block c / 16 times that
// block's power-of-two scale, exact in bf16), stored at position c ^ swz(t) of dst.
__device__ __forceinline__ void fp8_convert_latent(const lds_char_t* src, lds_char_t* dst, int e) {
  asm volatile("" : "+v"(e));
  const unsigned t = static_cast<unsigned>(e) >> 6, c = static_cast<unsigned>(e) & 63u;
  const lds_char_t* row = src + __umul24(t, static_cast<unsigned>(FP8_ROW_BYTES));
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
  const u32x2_t codes = *(const __attribute__((address_space(3))) u32x2_t*)(row + 8 * c);
  const float sc = *(const lds_f32_t*)(row + 640 + 4 * (c >> 4));
  i32x4_t v;
  v[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], sc, false));
  v[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], sc, true));
  v[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], sc, false));
  v[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], sc, true));
  *(__attribute__((address_space(3))) i32x4_t*)(dst + t * ROW_BYTES + 16 * (c ^ swz(t))) = v;
}

// k^R chunk e (0 .. 255) of a bf16 tile: row t = e / 8, logical chunk 64 + e % 8, the bf16
// bytes 16 (e % 8) .. of the raw row's k^R part as they are.
__device__ __forceinline__ void fp8_copy_rope(const lds_char_t* src, lds_char_t* dst, int e) {
  asm volatile("" : "+v"(e));
  const unsigned t = static_cast<unsigned>(e) >> 3, c = 64u + (static_cast<unsigned>(e) & 7u);
  const lds_char_t* row = src + __umul24(t, static_cast<unsigned>(FP8_ROW_BYTES));
  *(__attribute__((address_space(3))) i32x4_t*)(dst + t * ROW_BYTES + 16 * (c ^ swz(t))) =
      *(const __attribute__((address_space(3))) i32x4_t*)(row + 512 + 16 * (c - 64));
}

// Chunk e (0 .. 2303) of a bf16 tile from the staged raw rows at src: row t = e / 72,
// logical chunk c = e % 72, stored at position c ^ swz(t) of dst; c < 64 holds latent values
// 8 c .. 8 c + 7 (8 codes of block c / 16 times that block's scale: a power of two, so the
// product is exact in bf16), c >= 64 the k^R bytes 16 (c - 64) .. as they are.
__device__ __forceinline__ void fp8_convert_chunk(const lds_char_t* src, lds_char_t* dst, int e) {
  asm volatile("" : "+v"(e));
  const unsigned t = __umul24(static_cast<unsigned>(e), 7282u) >> 19;  // e / 72
  const unsigned c = static_cast<unsigned>(e) - __umul24(t, static_cast<unsigned>(CHUNKS));
  const lds_char_t* row = src + __umul24(t, static_cast<unsigned>(FP8_ROW_BYTES));
  i32x4_t v;
  if (c < 64) {
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
    const u32x2_t codes = *(const __attribute__((address_space(3))) u32x2_t*)(row + 8 * c);
    const float sc = *(const lds_f32_t*)(row + 640 + 4 * (c >> 4));
    v[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], sc, false));
    v[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], sc, true));
    v[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], sc, false));
    v[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], sc, true));
  } else {
    v = *(const __attribute__((address_space(3))) i32x4_t*)(row + 512 + 16 * (c - 64));
  }
  *(__attribute__((address_space(3))) i32x4_t*)(dst + t * ROW_BYTES + 16 * (c ^ swz(t))) = v;
}

// round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16x2_t to_bf16x2(float a, float b) {
  return __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
}

// eight bf16 ones (0x3f80 each)
__device__ __forceinline__ i32x4_t i16x4x2_ones() {
  const int one2 = 0x3f803f80;
  return i32x4_t{one2, one2, one2, one2};
}

// Exact fallback for a head block whose scores jump far above the split's fixed softmax
// reference: plain online softmax in fp32 per head (the running maximum moves every token),
// reading the rows straight from the paged cache.  One wavefront handles n_heads heads
// starting at h_begin; lane l owns features 9l .. 9l+8 of the score and latent columns
// l + 64k.
// Element k of a cache row: bf16 rows of 576 values, or (FP8) 656-byte rows of 512 E4M3
// codes, 64 bf16 values and 4 fp32 block scales (code times its block's scale).
template <bool FP8>
__device__ __forceinline__ float row_elem(const unsigned char* row, int k) {
  if constexpr (FP8) {
    if (k >= DC) return bf16_to_f32(reinterpret_cast<const bf16raw*>(row + DC)[k - DC]);
    const float sc = reinterpret_cast<const float*>(row + DC + 2 * DR)[k >> 7];
    return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(row[k]), 0) * sc;
  } else {
    return bf16_to_f32(reinterpret_cast<const bf16raw*>(row)[k]);
  }
}

// The partial of head h goes to row prow0 + h * hstride of o_part / lse_part.
template <typename OT, bool FP8 = false>
__device__ void split_exact_fallback(const bf16raw* __restrict__ q_lat,
                                     const bf16raw* __restrict__ q_pe,
                                     const bf16raw* __restrict__ cache, const int32_t* bt_row,
                                     int log2P, int j0, int j1, int bq, int H,
                                     int64_t prow0, int hstride, float scale_log2,
                                     OT* __restrict__ o_part, float* __restrict__ lse_part,
                                     int h_begin, int n_heads, int lane) {
  const int P = 1 << log2P;
  constexpr int RB = FP8 ? 656 : ROW_BYTES;
  for (int h = h_begin; h < h_begin + n_heads; ++h) {
    float q[9];
#pragma unroll
    for (int f = 0; f < 9; ++f) {
      const int k = 9 * lane + f;
      q[f] = k < DC ? bf16_to_f32(q_lat[(static_cast<int64_t>(bq) * H + h) * DC + k])
                    : bf16_to_f32(q_pe[(static_cast<int64_t>(bq) * H + h) * DR + (k - DC)]);
    }
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    for (int j = j0; j < j1; ++j) {
      const int pg = bt_row[j >> log2P];
      const unsigned char* row = reinterpret_cast<const unsigned char*>(cache) +
                                 ((static_cast<int64_t>(pg) << log2P) + (j & (P - 1))) * RB;
      float part = 0.f;
#pragma unroll
      for (int f = 0; f < 9; ++f) part += q[f] * row_elem<FP8>(row, 9 * lane + f);
      const float sc = mul_rn(wave_sum(part), scale_log2);
      const float mn = fmaxf(m, sc);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      const float p = __builtin_amdgcn_exp2f(sc - mn);
      l = l * alpha + p;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = acc[k] * alpha + p * row_elem<FP8>(row, lane + 64 * k);
      m = mn;
    }
    const int64_t ob = prow0 + static_cast<int64_t>(h) * hstride;
#pragma unroll
    for (int k = 0; k < 8; ++k) st(o_part + ob * DC + lane + 64 * k, acc[k] / l);
    if (lane == 0 && lse_part != nullptr) lse_part[ob] = (m + __log2f(l)) * LN2;
  }
}

}  // namespace attn
}  // namespace mla
