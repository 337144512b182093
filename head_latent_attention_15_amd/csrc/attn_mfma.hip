// Decode attention over the paged latent cache on bf16 MFMA (gfx950).
//
// All heads of one sequence read the same 576-wide latent rows ("論文解説: DeepSeek-V2 …",
// "Decoupled RoPE": c^KV and the shared k^R are all that is cached), so after absorbing
// W^UK into the query ("行列吸収トリック") both products of the decode step are dense
// contractions of the heads against a token tile:
//   scores  S[h][t] = sum_k [q~_h ; q^R_h][k] * row_t[k]      (k over 576)
//   latent  O[h][c] += sum_t P[h][t] * row_t[c]                (c over 512)
// followed by the W^UV up-projection outside this kernel (kasblo.com/?p=4663,
// "V側は、小さな表現の加重和を先に求める").
//
// Work decomposition.  One workgroup per (split, sequence) holds every head, so each cache
// byte crosses HBM once.  32-token tiles are copied HBM -> LDS with 16-byte
// global_load_lds_dwordx4 (no VGPR round trip) into three buffers, so two tiles' copies are
// in flight while one is consumed.  The copy is issued from inline assembly with explicit
// vmcnt waits: it has no destination registers, and keeping it out of the compiler's view
// stops the compiler from adding a full vmcnt(0) wait in front of every LDS read.
//
// The two products are split differently over the NW wavefronts of the workgroup:
//   scores: wave w owns 16 heads; S^T = K_tile (32 x 576) * Q^T (576 x 16) runs on
//           v_mfma_f32_16x16x32_bf16 with Q resident in VGPRs for the whole split and the
//           K operand read with ds_read_b128; the softmax weights P (bf16) go to LDS;
//   PV:     wave w owns 512/NW latent columns of every head; O += P (H x 32) * V (32 x cols)
//           reads P with ds_read_b128 and only its own V columns with the transposing
//           ds_read_b64_tr_b16, whose throughput is about a quarter of ds_read_b128's.
// Splitting PV by columns keeps the transposed reads to 1/NW of the tile per wave.
// LDS rows carry a 16-byte-chunk XOR swizzle so the row-strided ds_read_b128 and the
// transposed reads spread over the banks; P rows are padded to 80 bytes for the same reason.
//
// Softmax reference: each split fixes one reference maximum per head from its first tile
// (plus headroom) and never rescales the running output, which is only ever touched by
// MFMAs.  The final normalisation uses the same reference, so the result is the same
// softmax.  A tile whose maximum exceeds the reference by more than 64 (log2 units) sends
// that head block of the split to an exact VALU fallback; only inputs with very large
// score jumps take it.
//
// Tokens past the end of the split are masked to -inf before the exponent; their LDS rows
// are filled from the last valid token of the split, so no memory outside the referenced
// pages is read and P = 0 meets finite values.
#include "device_common.h"
#include "launchers.h"

#include <cstdlib>

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int DC = 512, DR = 64, ROW = DC + DR;
constexpr int ROW_BYTES = ROW * 2;                  // 1152
constexpr int CHUNKS = ROW_BYTES / 16;              // 72 sixteen-byte chunks per row
constexpr int TILE = 32;                            // tokens per tile
constexpr int TILE_CHUNKS = TILE * CHUNKS;          // 2304
constexpr int TILE_WAVE_COPIES = TILE_CHUNKS / 64;  // 36 wave-wide 16-byte copies per tile
constexpr int TILE_BYTES = TILE_CHUNKS * 16;        // 36864
constexpr int NBUF = 3;                             // tile buffers
constexpr int KSTEPS = ROW / 32;                    // 18 k-steps of the score product
constexpr int MAX_HEADS = 128;
constexpr int P_STRIDE = 80;                        // bytes per head row of a P tile (64 + pad)
constexpr int P_BYTES = MAX_HEADS * P_STRIDE;
constexpr int MAX_SPLIT_PAGES = 2048;               // block-table entries of a split in LDS
constexpr int OFF_P = NBUF * TILE_BYTES;
constexpr int OFF_PAGES = OFF_P + 2 * P_BYTES;
constexpr int OFF_L = OFF_PAGES + MAX_SPLIT_PAGES * 4;
constexpr int OFF_FLAG = OFF_L + MAX_HEADS * 4;
constexpr int LDS_BYTES = OFF_FLAG + 64;
constexpr float HEADROOM = 32.0f;  // log2 units between a split's first-tile max and its reference
constexpr float P_RANGE = 64.0f;   // a score this far above the reference takes the fallback
constexpr float LN2 = 0.6931471805599453f;

// 16-byte-chunk swizzle of tile row t (a permutation of the low three chunk bits):
//  - ds_read_b128 of one chunk column by 8 consecutive rows hits 8 distinct 16-byte bank
//    groups (the 72-chunk row pitch is a multiple of 8 chunks);
//  - the transposing reads of 4 consecutive rows x 2 adjacent chunks (one 16-lane group)
//    hit 8 distinct bank groups, because the 4 rows' swizzles differ in bits 1-2.
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

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
// M0-write to LDS-DMA hazard.
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

// round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16x2_t to_bf16x2(float a, float b) {
  return __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
}

__device__ __forceinline__ float from_bf16(__bf16 h) {
  return bf16_to_f32(__builtin_bit_cast(uint16_t, h));
}

// Exact fallback for a head block whose scores jump by more than P_RANGE above its
// reference: plain online softmax in fp32 per head (the running maximum moves every token),
// reading the rows straight from the paged cache.  One wavefront handles n_heads heads
// starting at h_begin; lane l owns features 9l .. 9l+8 of the score and latent columns
// l + 64k.
__device__ void split_exact_fallback(const bf16raw* __restrict__ q_lat,
                                     const bf16raw* __restrict__ q_pe,
                                     const bf16raw* __restrict__ cache, const int32_t* pages,
                                     int first_page, int log2P, int j0, int j1, int b, int H,
                                     int S, int s, float scale_log2, float* __restrict__ o_part,
                                     float* __restrict__ lse_part, int h_begin, int n_heads,
                                     int lane) {
  const int P = 1 << log2P;
  for (int h = h_begin; h < h_begin + n_heads; ++h) {
    float q[9];
#pragma unroll
    for (int f = 0; f < 9; ++f) {
      const int k = 9 * lane + f;
      q[f] = k < DC ? bf16_to_f32(q_lat[(static_cast<int64_t>(b) * H + h) * DC + k])
                    : bf16_to_f32(q_pe[(static_cast<int64_t>(b) * H + h) * DR + (k - DC)]);
    }
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    for (int j = j0; j < j1; ++j) {
      const int pg = pages[(j >> log2P) - first_page];
      const bf16raw* row = cache + ((static_cast<int64_t>(pg) << log2P) + (j & (P - 1))) * ROW;
      float part = 0.f;
#pragma unroll
      for (int f = 0; f < 9; ++f) part += q[f] * bf16_to_f32(row[9 * lane + f]);
      const float sc = mul_rn(wave_sum(part), scale_log2);
      const float mn = fmaxf(m, sc);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      const float p = __builtin_amdgcn_exp2f(sc - mn);
      l = l * alpha + p;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = acc[k] * alpha + p * bf16_to_f32(row[lane + 64 * k]);
      m = mn;
    }
    const int64_t ob = (static_cast<int64_t>(b) * H + h) * S + s;
#pragma unroll
    for (int k = 0; k < 8; ++k) o_part[ob * DC + lane + 64 * k] = acc[k] / l;
    if (lane == 0 && lse_part != nullptr) lse_part[ob] = (m + __log2f(l)) * LN2;
  }
}

// NW wavefronts, H = 16 * NW heads.  Scores: 16 heads per wave.  PV: 512 / NW columns of
// all H heads per wave (NHT = NW head tiles x NCT = 32 / NW column tiles = 32 tiles).
template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(
    const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int H, int log2P, int max_pages, int pages_per_split,
    int S, float scale_log2, float* __restrict__ o_part, float* __restrict__ lse_part) {
  constexpr int NT = NW * 64;
  constexpr int NHT = NW;           // head tiles in the PV product
  constexpr int NCT = 32 / NW;      // column tiles per wave in the PV product
  constexpr int CW = 16 * NCT;      // columns per wave
  constexpr int COPIES_LO = TILE_WAVE_COPIES / NW;
  constexpr int COPIES_HI = (TILE_WAVE_COPIES + NW - 1) / NW;
  static_assert(NW == 1 || NW == 2 || NW == 4 || NW == 8, "columns split evenly");
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  int32_t* pages = reinterpret_cast<int32_t*>(smem + OFF_PAGES);
  float* l_lds = reinterpret_cast<float*>(smem + OFF_L);
  int32_t* flag_lds = reinterpret_cast<int32_t*>(smem + OFF_FLAG);
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>((lds_char_t*)smem));

  const int s = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int P = 1 << log2P;
  const int h0 = 16 * w;   // score heads of this wave
  const int c0 = CW * w;   // PV columns of this wave

  const int L = seq_lens[b];
  const int j0 = s * pages_per_split * P;
  const int j1 = min(L, j0 + pages_per_split * P);

  if (j0 >= j1) {  // empty split: o = 0, lse = -inf
    for (int e = tid; e < H * DC; e += NT) {
      const int h = e / DC, c = e % DC;
      o_part[((static_cast<int64_t>(b) * H + h) * S + s) * DC + c] = 0.f;
    }
    if (lse_part != nullptr)
      for (int h = tid; h < H; h += NT) lse_part[(static_cast<int64_t>(b) * H + h) * S + s] = -INFINITY;
    return;
  }

  // stage the split's block-table entries in LDS
  const int first_page = j0 >> log2P;
  const int npg = ((j1 - 1) >> log2P) - first_page + 1;
  for (int i = tid; i < npg; i += NT)
    pages[i] = block_table[static_cast<int64_t>(b) * max_pages + first_page + i];

  // resident query fragments: B operand of S^T = K Q^T (lane: head h0 + r16, features
  // 32 kk + 8 g .. + 7)
  bf16x8_t qf[KSTEPS];
  {
    const bf16raw* qrow = q_lat + (static_cast<int64_t>(b) * H + h0 + r16) * DC + 8 * g;
    const bf16raw* prow = q_pe + (static_cast<int64_t>(b) * H + h0 + r16) * DR + 8 * g;
#pragma unroll
    for (int kk = 0; kk < DC / 32; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kk);
#pragma unroll
    for (int kk = 0; kk < DR / 32; ++kk)
      qf[DC / 32 + kk] = *reinterpret_cast<const bf16x8_t*>(prow + 32 * kk);
  }
  wait_vmcnt<0>();
  __syncthreads();  // page table visible, query fragments landed

  // this wave's share of a tile copy: wave-wide copies w, w + NW, ... (< 36)
  const int n_copies = (TILE_WAVE_COPIES - w + NW - 1) / NW;
  const char* cache_bytes = reinterpret_cast<const char*>(cache);
  // A tile starting at token tb lies inside one page (P % 32 == 0, tiles 32-aligned).
  auto issue_tile = [&](int tb, int buf) {
    const int pg = __builtin_amdgcn_readfirstlane(pages[(tb >> log2P) - first_page]);
    const char* base =
        cache_bytes + ((static_cast<int64_t>(pg) << log2P) + (tb & (P - 1))) * ROW_BYTES;
    const int last = j1 - 1 - tb;  // rows past it repeat the last valid row
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recompute the chunk coordinates each tile
#pragma unroll
    for (int r = 0; r < COPIES_HI; ++r) {
      const int q = w + NW * r;
      if (r < COPIES_LO || q < TILE_WAVE_COPIES) {
        const int chunk = 64 * q + ln;
        const int t = chunk / CHUNKS;
        const int c = (chunk - t * CHUNKS) ^ swz(t);
        const uint32_t voff = static_cast<uint32_t>(min(t, last) * ROW_BYTES + c * 16);
        dma16(base, voff, smem_lds + buf * TILE_BYTES + q * 64 * 16);
      }
    }
  };
  auto wait_own_copies = [&](bool next_in_flight) {
    if (!next_in_flight) {
      wait_vmcnt<0>();
    } else if (COPIES_LO == COPIES_HI || n_copies == COPIES_HI) {
      wait_vmcnt<COPIES_HI>();
    } else {
      wait_vmcnt<COPIES_LO>();
    }
  };

  f32x4_t o[NHT][NCT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o[ht][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Reference maximum of head h0 + r16 (log2 units, same in its 4 lanes) and this lane's
  // share of its softmax denominator.  The reference is fixed for the split: the first
  // tile's maximum plus HEADROOM, so the accumulators are never rescaled.
  float m_ref = -INFINITY, l_run = 0.f;
  bool out_of_range = false;  // sticky: a score of this head block left the reference range

  const int ntiles = (j1 - j0 + TILE - 1) / TILE;
  issue_tile(j0, 0);
  if (ntiles > 1) issue_tile(j0 + TILE, 1);
  for (int it = 0; it < ntiles; ++it) {
    const int tb = j0 + it * TILE;
    const int buf = it % NBUF;
    wait_own_copies(it + 1 < ntiles);
    block_barrier();  // tile it complete; every wave done with tile it-1 and P buffer it-1
    if (it + 2 < ntiles) issue_tile(tb + 2 * TILE, (it + 2) % NBUF);
    const char* tile = smem + buf * TILE_BYTES;
    char* ptile = smem + OFF_P + (it & 1) * P_BYTES;

    // ---- scores of heads h0..h0+15: S^T (2 token M-tiles x 16 heads, K = 576); the 36
    //      K fragments stream through a 4-deep register ring
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int gg = ln >> 4, rr = ln & 15;
      const int sk = swz(rr);
      const int k0 = rr * ROW_BYTES + 16 * (gg ^ sk);        // chunk 8j + g
      const int k1 = rr * ROW_BYTES + 16 * ((4 + gg) ^ sk);  // chunk 8j + 4 + g
      f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      constexpr int STEPS = KSTEPS * 2;
      constexpr int KRING = 4;
      auto k_frag = [&](int step) {
        const int kk = step >> 1, mt = step & 1;
        const int off = ((kk & 1) ? k1 : k0) + (kk >> 1) * 128 + mt * 16 * ROW_BYTES;
        return *reinterpret_cast<const bf16x8_t*>(tile + off);
      };
      bf16x8_t ka[KRING];
#pragma unroll
      for (int i = 0; i < KRING - 1; ++i) ka[i] = k_frag(i);
#pragma unroll
      for (int step = 0; step < STEPS; ++step) {
        if (step + KRING - 1 < STEPS) ka[(step + KRING - 1) % KRING] = k_frag(step + KRING - 1);
        const int kk = step >> 1, mt = step & 1;
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % KRING], qf[kk], sacc[mt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // softmax (log2 domain): lane holds head h0 + rr, tokens 16 mt + 4 gg + i
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tb + 16 * mt + 4 * gg + i;
          const float v = tok < j1 ? mul_rn(sacc[mt][i], scale_log2) : -INFINITY;
          sacc[mt][i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      if (it == 0) m_ref = tmax + HEADROOM;
      out_of_range |= tmax > m_ref + P_RANGE;
      float lsum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x2_t p01 = to_bf16x2(__builtin_amdgcn_exp2f(sacc[mt][0] - m_ref),
                                       __builtin_amdgcn_exp2f(sacc[mt][1] - m_ref));
        const bf16x2_t p23 = to_bf16x2(__builtin_amdgcn_exp2f(sacc[mt][2] - m_ref),
                                       __builtin_amdgcn_exp2f(sacc[mt][3] - m_ref));
        lsum += (from_bf16(p01[0]) + from_bf16(p01[1])) + (from_bf16(p23[0]) + from_bf16(p23[1]));
        const bf16x4_t p4 = __builtin_shufflevector(p01, p23, 0, 1, 2, 3);
        *reinterpret_cast<bf16x4_t*>(ptile + (h0 + rr) * P_STRIDE + (16 * mt + 4 * gg) * 2) = p4;
      }
      l_run += lsum;
    }
    block_barrier();  // P tile visible

    // ---- O[all heads][c0 .. c0 + CW) += P (H x 32) * V (32 x CW)
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int gg = ln >> 4, rr = ln & 15;
      bf16x8_t vb[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        i16x4_t half[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int t = 8 * gg + 4 * r + (rr >> 2);
          const int chunk = (c0 + 16 * ct) / 8 + ((rr & 3) >> 1);
          const char* p = tile + t * ROW_BYTES + 16 * (chunk ^ swz(t)) + 8 * (rr & 1);
          half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
        }
        vb[ct] = __builtin_bit_cast(bf16x8_t,
                                    __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
      constexpr int PRING = 3;
      auto p_frag = [&](int ht) {
        return *reinterpret_cast<const bf16x8_t*>(ptile + (16 * ht + rr) * P_STRIDE + 16 * gg);
      };
      bf16x8_t pa[PRING];
#pragma unroll
      for (int i = 0; i < PRING - 1 && i < NHT; ++i) pa[i] = p_frag(i);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        if (ht + PRING - 1 < NHT) pa[(ht + PRING - 1) % PRING] = p_frag(ht + PRING - 1);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          o[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[ht % PRING], vb[ct], o[ht][ct], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: denominators and fallback flags through LDS, then normalise and write
  {
    float lt = l_run + __shfl_xor(l_run, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const bool fb = __any(out_of_range);
    if (g == 0) l_lds[h0 + r16] = lt;
    if (lane == 0) flag_lds[w] = fb ? 1 : 0;
    if (!fb && lse_part != nullptr && g == 0)
      lse_part[(static_cast<int64_t>(b) * H + h0 + r16) * S + s] = (m_ref + __log2f(lt)) * LN2;
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    if (flag_lds[ht]) continue;  // that head block is recomputed by its owner below
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * ht + 4 * g + i;
      const float inv = 1.f / l_lds[h];
      float* dst = o_part + ((static_cast<int64_t>(b) * H + h) * S + s) * DC + c0 + r16;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) dst[16 * ct] = o[ht][ct][i] * inv;
    }
  }
  if (flag_lds[w])
    split_exact_fallback(q_lat, q_pe, cache, pages, first_page, log2P, j0, j1, b, H, S, s,
                         scale_log2, o_part, lse_part, h0, 16, lane);
}

template <int NW>
hipError_t launch_nw(const PagedArgs& a, hipStream_t st) {
  const float log2e = 1.4426950408889634f;
  hipLaunchKernelGGL((attn_mfma_kernel<NW>), dim3(a.num_splits, a.B), dim3(NW * 64), 0, st,
                     static_cast<const bf16raw*>(a.q_lat), static_cast<const bf16raw*>(a.q_pe),
                     static_cast<const bf16raw*>(a.cache), a.block_table, a.seq_lens, a.H,
                     __builtin_ctz(static_cast<unsigned>(a.page_size)), a.max_pages,
                     a.pages_per_split, a.num_splits, a.scale * log2e, a.o_part, a.lse_part);
  return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool attn_mfma_supported(const PagedArgs& a) {
  const bool heads_ok = a.H == 16 || a.H == 32 || a.H == 64 || a.H == 128;
  const bool page_ok = a.page_size >= TILE && (a.page_size & (a.page_size - 1)) == 0;
  return a.d_c == DC && a.d_R == DR && heads_ok && page_ok &&
         a.pages_per_split <= MAX_SPLIT_PAGES && a.B <= 65535 && aligned16(a.q_lat) &&
         aligned16(a.q_pe) && aligned16(a.cache);
}

hipError_t launch_attn_mfma_bf16_512_64(const PagedArgs& a, hipStream_t s) {
  switch (a.H) {
    case 16: return launch_nw<1>(a, s);
    case 32: return launch_nw<2>(a, s);
    case 64: return launch_nw<4>(a, s);
    case 128: return launch_nw<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
