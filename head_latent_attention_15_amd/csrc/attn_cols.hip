// Decode attention over the paged latent cache on bf16 MFMA (gfx950) for 128 heads, with
// the latent product partitioned by columns.
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
// One workgroup of 8 wavefronts per (sequence, split) holds all 128 heads, so each cache
// byte crosses HBM once; 32-token tiles go HBM -> LDS with LDS DMA (attn_common.h) into
// three buffers.  Wave w has two jobs per tile:
//   scores: the 16 heads of block w (heads 16 w .. 16 w + 15) against the whole tile,
//           S^T = K (32 x 576) Q^T (576 x 16) with the queries resident in VGPRs, then
//           their softmax; the weights P^T go to LDS (1 KB per block, double-buffered);
//   PV:     latent columns 64 w .. 64 w + 63 of all 128 heads,
//           O^T (64 x 128) += V^T (64 x 32) P^T (32 x 128): 4 V^T fragments (transposing
//           reads) x 8 P^T fragments = 32 MFMAs, so the V part of the tile is read from LDS
//           exactly once and each V fragment feeds eight MFMAs.
// The score product needs one K fragment read per MFMA, so a wavefront's score phase is
// bound by LDS latency while its PV phase is bound by the matrix core.  The two
// wavefronts sharing a SIMD (w and w + 4) therefore run the phases in opposite order:
// waves 0..3 do PV(it-1) then the scores and softmax of tile it, waves 4..7 the scores
// and softmax then PV(it-1), so one's MFMA-dense PV fills the other's LDS waits.
//
// The tile sits in LDS as 9 column blocks (32 rows x 128 bytes; blocks 0..7 the latent, 8
// the RoPE part), so the only reader of block w in the PV product is wave w: as soon as its
// V fragments of tile it-1 are in registers, wave w refills block w with tile it+2 (waves
// 0..3 also one quarter of the RoPE block each) while its MFMAs run.  The copies never
// queue up behind a barrier.
//
// One barrier per tile, A(it): it publishes tile it (every wave's copies landed) and
// P(it-1).
//
// Softmax reference (as in attn_mfma.hip): each split fixes one reference per head from its
// first tile (plus headroom) and never rescales the accumulators; the final normalisation
// uses the same reference, so the result is the same softmax.  A head block whose scores
// jump more than 64 (log2 units) above its reference is recomputed by an exact fallback.
// The denominators sum the bf16-rounded weights that the PV product consumes.
//
// Tokens past the end of the split are masked to -inf before the exponent; their LDS rows
// are filled from the last valid token of the split, so no memory outside the referenced
// pages is read and P = 0 meets finite values.
#include "attn_common.h"
#include "launchers.h"

#include <type_traits>

namespace mla {
namespace {

using namespace attn;

constexpr int NW = 8;                                // wavefronts per workgroup
constexpr int NH = 128;                              // heads: 8 blocks of 16
constexpr int NBUF = 3;                              // tile buffers
constexpr int BLOCK_BYTES = TILE * 128;              // one column block of a tile: 4 KB
constexpr int PBUF = NBUF * TILE_BYTES;              // P^T fragments, 2 x (8 blocks x 1 KB)
constexpr int STATS = PBUF + 2 * 8 * 1024;           // denominators (128 floats), block flags (8)
constexpr int PAGE_TABLE = STATS + 1024;             // block-table entries of the split
constexpr int MAX_SPLIT_PAGES = 1024;
constexpr int LDS_BYTES = PAGE_TABLE + MAX_SPLIT_PAGES * 4;
static_assert(LDS_BYTES <= 163840, "LDS per workgroup");
constexpr float HEADROOM = 32.0f;  // log2 units between a split's first-tile max and its reference
constexpr float P_RANGE = 64.0f;   // a score this far above the reference takes the fallback

// LDS offset of 16-byte chunk c (0..71) of tile row t (0..31): column block c >> 3, row t,
// slot (c & 7) ^ swz(t).  The 128-byte row stride maps rows onto the same banks as the
// 1152-byte rows of a row-major tile (1152 = 128 mod 256), so the swizzle keeps the score
// and transposing PV reads conflict-free as it does there.
__device__ __forceinline__ int chunk_offset(int t, int c) {
  return (c >> 3) * BLOCK_BYTES + t * 128 + 16 * ((c & 7) ^ swz(t));
}

// Source offset (bytes from the tile's first row) of lane l of copy q (0..35): the copy
// fills LDS bytes 1024 q .. 1024 q + 1023 of the tile, i.e. column block q >> 2, rows
// 8 (q & 3) .. + 7; lane l writes row 8 (q & 3) + (l >> 3), slot l & 7, which holds
// logical chunk 8 (q >> 2) + ((l & 7) ^ swz(row)).  Rows past `last` repeat row `last`.
__device__ __forceinline__ uint32_t block_copy_voff(int q, int l, unsigned last) {
  const unsigned t = 8 * (q & 3) + (l >> 3);
  const unsigned c = 8 * (q >> 2) + ((l & 7) ^ swz(t));
  return __umul24(min(t, last), static_cast<unsigned>(ROW_BYTES)) + c * 16;
}

// LDS stores must land before a barrier publishes them (gfx950 has no implicit wait there).
__device__ __forceinline__ void publish_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  block_barrier();
}

template <typename OT>
__global__ __launch_bounds__(NW * 64) void attn_cols_kernel(
    const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int log2P, int max_pages, int pages_per_split,
    int S, float scale_log2, OT* __restrict__ o_part, float* __restrict__ lse_part, int n_q) {
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  lds_char_t* const lsm = (lds_char_t*)smem;  // 32-bit LDS addressing
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>(lsm));

  // With the sequence index in x, all splits of a sequence (ids b, b + B, ...) land on
  // XCD b % 8 when B % 8 == 0, so its queries are fetched once into that XCD's L2.
  // Several query tokens per sequence (n_q > 1): token t = blockIdx.z sits at position
  // seq_len - n_q + t and sees the cache up to it; its queries and outputs are row
  // bq = b n_q + t.
  const int b = blockIdx.x, s = blockIdx.y, bq = b * n_q + blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int P = 1 << log2P;
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_pages;

  const int L = seq_lens[b] - (n_q - 1 - static_cast<int>(blockIdx.z));
  const int j0 = s * pages_per_split * P;
  const int j1 = min(L, j0 + pages_per_split * P);

  if (j0 >= j1) {  // empty split: o = 0, lse = -inf
    for (int e = tid; e < NH * DC; e += NT) {
      const int h = e / DC, c = e % DC;
      st(o_part + ((static_cast<int64_t>(bq) * NH + h) * S + s) * DC + c, 0.f);
    }
    if (lse_part != nullptr)
      for (int h = tid; h < NH; h += NT) lse_part[(static_cast<int64_t>(bq) * NH + h) * S + s] = -INFINITY;
    return;
  }
  const int ntiles = (j1 - j0 + TILE - 1) / TILE;

  // ---- tile copies.  Wave w owns copies 4 w .. 4 w + 3 (column block w) and waves 0..3
  //      also copy 32 + w (a quarter of the RoPE block): 5 or 4 copies per wave and tile.
  const int ncopies = w < 4 ? 5 : 4;
  const char* cache_bytes = reinterpret_cast<const char*>(cache);
  // A tile starting at token tb lies inside one page (P % 32 == 0, tiles 32-aligned).
  auto page_base = [&](int pg, int tb) {
    return cache_bytes + ((static_cast<int64_t>(pg) << log2P) + (tb & (P - 1))) * ROW_BYTES;
  };
  auto copy_q = [&](int r) { return r < 4 ? 4 * w + r : 32 + w; };
  // Inside the loop the block-table entries of the split come from an LDS copy: an LDS
  // read keeps the in-order LDS wait counts, where a scalar load would force full waits.
  auto split_page = [&](int tb) {
    return __builtin_amdgcn_readfirstlane(((const lds_i32_t*)(lsm + PAGE_TABLE))[(tb - j0) >> log2P]);
  };
  // copy r of this wave for tile it (buffer it % 3), whose rows come from `base`
  auto issue_copy = [&](const char* base, int it, int r) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per copy (no long live ranges)
    const unsigned last = static_cast<unsigned>(j1 - 1 - (j0 + it * TILE));  // rows past it repeat it
    const int q = copy_q(r);
    dma16(base, block_copy_voff(q, ln, last), smem_lds + (it % NBUF) * TILE_BYTES + q * 1024);
  };

  // ---- prologue: the split's block-table entries go to LDS first (one memory latency);
  //      then tile 0, the queries and tile 1 are requested together and the wave waits
  //      for all but tile 1 (a second latency).
  for (int e = tid; e * P < j1 - j0; e += NT)  // the pages this split reads
    ((lds_i32_t*)(lsm + PAGE_TABLE))[e] = bt_row[(j0 >> log2P) + e];
  const int tb1 = ntiles > 1 ? j0 + TILE : j0;  // a one-tile split copies its tile again
  const int page0 = __builtin_amdgcn_readfirstlane(bt_row[j0 >> log2P]);
  const int page1 = __builtin_amdgcn_readfirstlane(bt_row[tb1 >> log2P]);
  {
    const char* base = page_base(page0, j0);
    for (int r = 0; r < ncopies; ++r) issue_copy(base, 0, r);
  }

  // ---- resident query fragments (B operand of S^T = K Q^T): lane (g, r16) holds head
  //      16 w + r16, features 32 kk + 8 g .. + 7 (kk = 16, 17: the RoPE part).  Loaded in
  //      one assembly block together with the copies of tile 1, which waits for everything
  //      but those copies: two tiles are in flight while the queries arrive, and no
  //      compiler-inserted wait falls after a copy.  Here every wave issues five copies of
  //      tile 1 (waves 4..7 copy their first one twice: same source, same LDS bytes), so
  //      one wait count serves all.
  bf16x8_t qf[KSTEPS];
  {
    const int64_t row = static_cast<int64_t>(bq) * NH + 16 * w + r16;
    const bf16raw* qrow = q_lat + row * DC + 8 * g;
    const bf16raw* prow = q_pe + row * DR + 8 * g;
    const unsigned last1 = static_cast<unsigned>(j1 - 1 - tb1);
    const uint64_t b64 = reinterpret_cast<uint64_t>(page_base(page1, tb1));
    const uint32_t blo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64));
    const uint32_t bhi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64 >> 32));
    const void* base1 = reinterpret_cast<const void*>((static_cast<uint64_t>(bhi) << 32) | blo);
    uint32_t vo[5], la[5];
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      const int q = copy_q(c < ncopies ? c : 0);
      vo[c] = block_copy_voff(q, lane, last1);
      la[c] = __builtin_amdgcn_readfirstlane(smem_lds + TILE_BYTES + q * 1024);
    }
    i32x4_t r[KSTEPS];
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "global_load_dwordx4 %0, %18, off\n\t"
        "global_load_dwordx4 %1, %18, off offset:64\n\t"
        "global_load_dwordx4 %2, %18, off offset:128\n\t"
        "global_load_dwordx4 %3, %18, off offset:192\n\t"
        "global_load_dwordx4 %4, %18, off offset:256\n\t"
        "global_load_dwordx4 %5, %18, off offset:320\n\t"
        "global_load_dwordx4 %6, %18, off offset:384\n\t"
        "global_load_dwordx4 %7, %18, off offset:448\n\t"
        "global_load_dwordx4 %8, %18, off offset:512\n\t"
        "global_load_dwordx4 %9, %18, off offset:576\n\t"
        "global_load_dwordx4 %10, %18, off offset:640\n\t"
        "global_load_dwordx4 %11, %18, off offset:704\n\t"
        "global_load_dwordx4 %12, %18, off offset:768\n\t"
        "global_load_dwordx4 %13, %18, off offset:832\n\t"
        "global_load_dwordx4 %14, %18, off offset:896\n\t"
        "global_load_dwordx4 %15, %18, off offset:960\n\t"
        "global_load_dwordx4 %16, %19, off\n\t"
        "global_load_dwordx4 %17, %19, off offset:64\n\t"
        "s_mov_b32 m0, %25\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %20, %30\n\t"
        "s_mov_b32 m0, %26\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %21, %30\n\t"
        "s_mov_b32 m0, %27\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %22, %30\n\t"
        "s_mov_b32 m0, %28\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %23, %30\n\t"
        "s_mov_b32 m0, %29\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %24, %30\n\t"
        "s_waitcnt vmcnt(5)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
          "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15]), "=&v"(r[16]), "=&v"(r[17])
        : "v"(qrow), "v"(prow), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]),
          "s"(la[0]), "s"(la[1]), "s"(la[2]), "s"(la[3]), "s"(la[4]), "s"(base1)
        : "memory", "m0");
#pragma clang diagnostic pop
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = __builtin_bit_cast(bf16x8_t, r[kk]);
  }

  // O^T accumulators: o[ct][hb2] lane (g, r16) holds O[16 hb2 + r16][64 w + 16 ct + 4 g + i]
  f32x4_t o[4][8];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int h2 = 0; h2 < 8; ++h2) o[ct][h2] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // PV of tile it for this wave's 64 columns and all 8 head blocks.  V^T fragments (A
  // operand): lane (gg, rr) holds column 64 w + 16 ct + rr, tokens 8 gg .. 8 gg + 7,
  // gathered by two transposing reads of 4 rows each from column block w.  Once they are
  // in registers the block is free, and with `copies` set this wave's copies of tile it+3
  // (the next tile of this buffer, rows from base3) go out between the MFMAs.
  auto pv = [&](int it, bool copies, const char* base3) {
    const lds_char_t* blk = lsm + (it % NBUF) * TILE_BYTES + w * BLOCK_BYTES;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per tile (no long live ranges)
    const int gg = ln >> 4, rr = ln & 15;
    // Copy r of block w fills rows 8 r + x (x = lane >> 3) of the block, and since
    // swz(8 r + x) = swz(x) ^ 2 r its source chunk is 8 w + (cx ^ 2 r), cx = (lane & 7) ^ swz(x);
    // the RoPE quarter (waves 0..3) is rows 8 w + x, chunk 64 + (cx ^ 2 w).
    const unsigned cx = static_cast<unsigned>((ln & 7) ^ swz(ln >> 3));
    const unsigned xr = static_cast<unsigned>(ln >> 3);
    const unsigned last3 = static_cast<unsigned>(j1 - 1 - (j0 + (it + 3) * TILE));
    const uint32_t dst3 = smem_lds + ((it + 3) % NBUF) * TILE_BYTES;
    auto copy = [&](int r) {
      if (r < 4)
        dma16(base3, __umul24(min(8u * r + xr, last3), static_cast<unsigned>(ROW_BYTES)) +
                         16u * (8u * w + (cx ^ (2u * r))),
              dst3 + (4 * w + r) * 1024);
      else
        dma16(base3, __umul24(min(8u * w + xr, last3), static_cast<unsigned>(ROW_BYTES)) +
                         16u * (64u + (cx ^ (2u * w))),
              dst3 + (32 + w) * 1024);
    };
    // P^T fragments of the 8 head blocks, 1 KB each, lane-contiguous
    const lds_char_t* pb = lsm + PBUF + (it & 1) * 8192 + 16 * ln;
    constexpr int PRING = 2;
    bf16x8_t pf[PRING];
    pf[0] = *(const lds_bf16x8_t*)(pb);
    bf16x8_t va[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      i16x4_t half[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int t = 8 * gg + 4 * r + (rr >> 2);
        const int e = (rr & 3) >> 1;
        half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(blk + t * 128 + 16 * ((2 * ct + e) ^ swz(t)) + 8 * (rr & 1)));
      }
      va[ct] = __builtin_bit_cast(bf16x8_t,
                                  __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // the V reads have returned before any copy may overwrite their block
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int h2 = 0; h2 < 8; ++h2) {
      if (h2 + 1 < 8) pf[(h2 + 1) % PRING] = *(const lds_bf16x8_t*)(pb + 1024 * (h2 + 1));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        o[ct][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ct], pf[h2 % PRING], o[ct][h2], 0, 0, 0);
        if (ct == 1 && h2 < 5) {  // a copy between two MFMAs runs in their shadow
          __builtin_amdgcn_sched_barrier(0);
          if (copies && h2 < ncopies) copy(h2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Reference maximum of head 16 w + r16 (log2 units, same in its 4 lanes): the first
  // tile's maximum plus HEADROOM, fixed for the split.  Lane (g, r16) sums the bf16-rounded
  // weights it hands to the PV product (tokens 8 g .. 8 g + 7 of every tile); the four
  // lanes of a head are added at the end.
  float m_ref = -INFINITY;
  float l_part = 0.f;
  bool out_of_range = false;  // sticky: a score of this head block left the reference range

  // Scores of tile it for head block w (S^T: 2 token M tiles x 16 heads, k over 576; row r
  // of M tile mt is token 8 (r >> 2) + 4 mt + (r & 3), so lane (g, r16) ends with tokens
  // 8 g .. 8 g + 7 of head r16: after the softmax, exactly its P^T fragment).  The 36 K
  // fragments stream through a register ring.
  auto score = [&](int it, f32x4_t (&sacc)[2]) {
    const lds_char_t* tile = lsm + (it % NBUF) * TILE_BYTES;
    sacc[0] = sacc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // K fragment lane offsets: M tile mt, row t = 8 (r16 >> 2) + 4 mt + (r16 & 3), logical
    // chunk 4 (kk & 1) + g of column block kk >> 1 (recomputed per tile: no long live ranges)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int kb[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int t = 8 * ((ln & 15) >> 2) + 4 * mt + (ln & 3);
#pragma unroll
      for (int par = 0; par < 2; ++par) kb[mt][par] = chunk_offset(t, 4 * par + (ln >> 4));
    }
    constexpr int STEPS = 2 * KSTEPS;  // step = 2 kk + mt
    constexpr int KRING = 3;
    auto k_frag = [&](int step) {
      const int kk = step >> 1, mt = step & 1;
      return *(const lds_bf16x8_t*)(tile + kb[mt][kk & 1] + BLOCK_BYTES * (kk >> 1));
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
  };

  // softmax of tile it on the scores of the own block; stores its P^T fragment
  auto softmax = [&](int it, const f32x4_t (&so)[2]) {
    const int tb = j0 + it * TILE;
    f32x4_t sc[2] = {so[0], so[1]};
    if (tb + TILE > j1) {  // last tile of the split: tokens at or past j1 get weight 0
      asm volatile("" ::: "memory");  // a real branch: the masking runs on one tile only
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tb + 8 * g + 4 * mt + i >= j1) sc[mt][i] = -INFINITY;
    }
    if (it == 0) {  // the first tile's maximum fixes the reference
      asm volatile("" ::: "memory");
      float tmax = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      m_ref = mul_rn(tmax, scale_log2) + HEADROOM;
    }
    // each weight is 2^(s * scale - m_ref) with one rounding in the fma; the scale is
    // positive, so the raw maximum orders like the scaled one
    const float neg_m = -m_ref;
    float e[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) e[mt][i] = __builtin_fmaf(sc[mt][i], scale_log2, neg_m);
    out_of_range |= fmaxf(fmaxf(fmaxf(e[0][0], e[0][1]), fmaxf(e[0][2], e[0][3])),
                          fmaxf(fmaxf(e[1][0], e[1][1]), fmaxf(e[1][2], e[1][3]))) > P_RANGE;
    bf16x2_t pp[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf)
        pp[2 * mt + hlf] = to_bf16x2(__builtin_amdgcn_exp2f(e[mt][2 * hlf]),
                                     __builtin_amdgcn_exp2f(e[mt][2 * hlf + 1]));
    const bf16x8_t pt = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                                0, 1, 2, 3, 4, 5, 6, 7);
    *(lds_bf16x8_t*)(lsm + PBUF + (it & 1) * 8192 + w * 1024 + 16 * lane) = pt;
#pragma unroll
    for (int i = 0; i < 8; ++i) l_part += static_cast<float>(pt[i]);
  };

  // Phase it (between barriers A(it) and A(it+1)): PV(it-1) (which refills the wave's part
  // of buffer (it-1) % 3 with tile it+2), the scores and softmax of tile it, in the
  // wave group's order.  Tile 2 has no PV before it, so phase 0 requests it up front.
  publish_barrier();  // A(0): tile 0 and the page table
  if (ntiles > 2) {
    const char* base2 = page_base(split_page(j0 + 2 * TILE), j0 + 2 * TILE);
    for (int r = 0; r < ncopies; ++r) issue_copy(base2, 2, r);
  }
  // The two orders run as two separate loops: with the branch outside the tile loop each
  // loop body is straight-line code, which the register allocator fits in 256 VGPRs.
  auto phase_end = [&](int it, bool copies) {
    if (it == ntiles - 1) {  // the block's denominators and range flag for the epilogue
      const bool block_out = __any(out_of_range);  // a vote of the whole wavefront
      l_part += __shfl_xor(l_part, 16, 64);
      l_part += __shfl_xor(l_part, 32, 64);
      if (g == 0) ((lds_f32_t*)(lsm + STATS))[16 * w + r16] = l_part;
      if (lane == 0) ((lds_i32_t*)(lsm + STATS + 512))[w] = block_out ? 1 : 0;
    }
    // own copies of tile it+1 landed (those of tile it+2 may still be in flight)
    if (copies) {
      if (w < 4) wait_vmcnt<5>();
      else wait_vmcnt<4>();
    } else {
      wait_vmcnt<0>();
    }
    publish_barrier();  // A(it+1)
  };
  if (w < 4) {  // PV first
    for (int it = 0; it < ntiles; ++it) {
      const bool copies = it + 2 < ntiles;  // tile it+2 is (being) requested in this phase
      const int tb2 = j0 + (it + 2) * TILE;
      if (it > 0) pv(it - 1, copies, page_base(copies ? split_page(tb2) : page0, tb2));
      f32x4_t sacc[2];
      score(it, sacc);
      softmax(it, sacc);
      phase_end(it, copies);
    }
  } else {      // scores first
    for (int it = 0; it < ntiles; ++it) {
      const bool copies = it + 2 < ntiles;
      const int tb2 = j0 + (it + 2) * TILE;
      f32x4_t sacc[2];
      score(it, sacc);
      softmax(it, sacc);
      if (it > 0) pv(it - 1, copies, page_base(copies ? split_page(tb2) : page0, tb2));
      phase_end(it, copies);
    }
  }
  pv(ntiles - 1, false, nullptr);

  // ---- epilogue: normalise and write this wave's 64 columns of every head; the lse of the
  //      own block; a block whose scores left the reference range is recomputed exactly
  int flags = 0;
#pragma unroll
  for (int h2 = 0; h2 < 8; ++h2)
    flags |= (((const lds_i32_t*)(lsm + STATS + 512))[h2] != 0) << h2;
  flags = __builtin_amdgcn_readfirstlane(flags);
#pragma unroll
  for (int h2 = 0; h2 < 8; ++h2) {
    if (flags & (1 << h2)) continue;
    const float inv = 1.f / ((const lds_f32_t*)(lsm + STATS))[16 * h2 + r16];
    const int64_t row = (static_cast<int64_t>(bq) * NH + 16 * h2 + r16) * S + s;
    if constexpr (std::is_same<OT, float>::value) {
      float* dst = o_part + row * DC + 64 * w + 4 * g;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) *reinterpret_cast<f32x4_t*>(dst + 16 * ct) = o[ct][h2] * inv;
    } else {
      // bf16 (round to nearest even), 16 bytes per lane and store: for column tiles 2m and
      // 2m + 1 a lane pair (g, g ^ 1) trades halves, so even g writes columns
      // 32 m + 4 g .. + 7 and odd g writes 32 m + 4 g + 12 .. + 7 of the wave's 64
      const bool odd = (g & 1) != 0;
      bf16raw* dst = o_part + row * DC + 64 * w + 4 * g + (odd ? 12 : 0);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f32x4_t a = o[2 * m][h2] * inv, c = o[2 * m + 1][h2] * inv;
        const bf16x4_t pa = __builtin_shufflevector(to_bf16x2(a[0], a[1]), to_bf16x2(a[2], a[3]), 0, 1, 2, 3);
        const bf16x4_t pc = __builtin_shufflevector(to_bf16x2(c[0], c[1]), to_bf16x2(c[2], c[3]), 0, 1, 2, 3);
        const uint2 send = __builtin_bit_cast(uint2, odd ? pa : pc);
        uint2 recv;
        recv.x = __shfl_xor(send.x, 16, 64);
        recv.y = __shfl_xor(send.y, 16, 64);
        const bf16x4_t pr = __builtin_bit_cast(bf16x4_t, recv);
        const bf16x8_t v8 = odd ? __builtin_shufflevector(pr, pc, 0, 1, 2, 3, 4, 5, 6, 7)
                                : __builtin_shufflevector(pa, pr, 0, 1, 2, 3, 4, 5, 6, 7);
        *reinterpret_cast<bf16x8_t*>(dst + 32 * m) = v8;
      }
    }
  }
  if (!(flags & (1 << w))) {
    if (lse_part != nullptr && g == 0)
      lse_part[(static_cast<int64_t>(bq) * NH + 16 * w + r16) * S + s] = (m_ref + __log2f(l_part)) * LN2;
  } else {
    split_exact_fallback(q_lat, q_pe, cache, bt_row, log2P, j0, j1, bq, NH,
                         static_cast<int64_t>(bq) * NH * S + s, S, scale_log2,
                         o_part, lse_part, 16 * w, 16, lane);
  }
}

template <typename OT>
hipError_t launch_t(const PagedArgs& a, hipStream_t st) {
  const float log2e = 1.4426950408889634f;
  hipLaunchKernelGGL((attn_cols_kernel<OT>), dim3(a.B, a.num_splits, a.n_q), dim3(NW * 64), 0, st,
                     static_cast<const bf16raw*>(a.q_lat), static_cast<const bf16raw*>(a.q_pe),
                     static_cast<const bf16raw*>(a.cache), a.block_table, a.seq_lens,
                     __builtin_ctz(static_cast<unsigned>(a.page_size)), a.max_pages,
                     a.pages_per_split, a.num_splits, a.scale * log2e,
                     static_cast<OT*>(a.o_part), a.lse_part, a.n_q);
  return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool attn_cols_supported(const PagedArgs& a) {
  if (a.pages_per_split > MAX_SPLIT_PAGES) return false;
  const bool page_ok = a.page_size >= TILE && (a.page_size & (a.page_size - 1)) == 0;
  return a.d_c == DC && a.d_R == DR && a.H == NH && page_ok && a.B <= 65535 && a.n_q >= 1 &&
         a.n_q <= 65535 && aligned16(a.q_lat) && aligned16(a.q_pe) && aligned16(a.cache) &&
         aligned16(a.o_part);
}

hipError_t launch_attn_cols_bf16_512_64(const PagedArgs& a, hipStream_t s) {
  return a.part_bf16 ? launch_t<bf16raw>(a, s) : launch_t<float>(a, s);
}

}  // namespace mla
