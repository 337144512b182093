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
// three buffers.  The point of this kernel is how few LDS bytes each matrix-core operation
// needs.  Giving every wavefront 16 heads for both products (attn_mfma.hip) makes all eight
// read the whole tile twice, ~15x the staged bytes.  Here:
//
//   scores: wave w = (head group hg = w & 3, k parity fh = w >> 2) multiplies the tile by
//           the queries of 32 heads (heads 32 hg .. 32 hg + 31) over the k-steps of parity
//           fh (9 of the 18 32-wide steps), so each K fragment read from LDS feeds two
//           MFMAs and the queries stay resident without duplication (72 VGPRs).  The two
//           waves of a head group then trade the partial scores of each other's 16-head
//           block through LDS (2 KB per wave); each ends with the full scores of its own
//           block hb = 2 hg + fh, 32 tokens x 16 heads, and runs their softmax;
//   PV:     the weights P^T of the 8 head blocks go to LDS (8 KB per tile) and wave w
//           accumulates O^T for latent columns 64 w .. 64 w + 63 of all 128 heads:
//           4 V^T fragments (transposing reads) x 8 P^T fragments = 32 MFMAs, so the V part
//           of the tile is read from LDS exactly once.
//
// LDS bytes read per tile: 144 KB of K fragments, 64 KB of P, 32 KB of V and 16 KB of
// exchanged scores, against ~550 KB when every wave reads the whole tile twice.
//
// Per tile, two barriers:  A(it) publishes tile it and P(it-1); between A(it) and B(it)
// each wave runs PV(it-1) and the scores of tile it and stores its partner's partial;
// B(it) publishes the partials and retires tile it-1, whose buffer receives the copies of
// tile it+2; between B(it) and A(it+1) each wave adds the partner's partial, runs the
// softmax of its block and stores its P^T fragment.
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
constexpr int XCH = NBUF * TILE_BYTES;               // partial scores, 2 KB per wave
constexpr int PBUF = XCH + NW * 2048;                // P^T fragments, 1 KB per head block
constexpr int STATS = PBUF + 8 * 1024;               // denominators (128 floats), block flags (8)
constexpr int PAGE_TABLE = STATS + 1024;             // block-table entries of the split
constexpr int MAX_SPLIT_PAGES = 1024;                // block-table entries of one split in LDS
constexpr int LDS_BYTES = PAGE_TABLE + MAX_SPLIT_PAGES * 4;
static_assert(LDS_BYTES <= 163840, "LDS per workgroup");
constexpr float HEADROOM = 32.0f;  // log2 units between a split's first-tile max and its reference
constexpr float P_RANGE = 64.0f;   // a score this far above the reference takes the fallback

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
  constexpr int COPIES = (TILE_WAVE_COPIES + NW - 1) / NW;  // 5 tile copies per wave
  constexpr int HALF = KSTEPS / 2;                           // 9 score k-steps per wave
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
  const int hg = w & 3, fh = w >> 2;       // score roles: head group, k-step parity
  const int hb = 2 * hg + fh;              // own softmax block: heads 16 hb .. 16 hb + 15
  const int hx = 2 * hg + (fh ^ 1);        // the partner's block
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

  // ---- tile copies: wave w issues copies q = w, w + 8, ... of each tile (36 in all); a
  //      wave without a fifth copy repeats its first (same source, same LDS bytes), so every
  //      wave counts COPIES copies per tile.
  const char* cache_bytes = reinterpret_cast<const char*>(cache);
  // A tile starting at token tb lies inside one page (P % 32 == 0, tiles 32-aligned).
  auto page_base = [&](int pg, int tb) {
    return cache_bytes + ((static_cast<int64_t>(pg) << log2P) + (tb & (P - 1))) * ROW_BYTES;
  };
  auto copy_index = [&](int r) { return w + NW * r < TILE_WAVE_COPIES ? w + NW * r : w; };
  // Inside the loop the block-table entries of the split come from an LDS copy, read ahead
  // of the barrier that precedes the copies: an LDS read keeps the in-order LDS wait
  // counts, where a scalar load would force full waits.  Each copy's source offsets are
  // computed in place (a few VALU operations, no memory round trip).
  auto split_page = [&](int tb) {
    return __builtin_amdgcn_readfirstlane(((const lds_i32_t*)(lsm + PAGE_TABLE))[(tb - j0) >> log2P]);
  };
  auto issue_tile = [&](int it, int page) {
    const int tb = j0 + it * TILE;
    const char* base = page_base(page, tb);
    const unsigned last = static_cast<unsigned>(j1 - 1 - tb);  // rows past it repeat it
    const uint32_t dst = smem_lds + (it % NBUF) * TILE_BYTES;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per tile (no long live ranges)
#pragma unroll
    for (int r = 0; r < COPIES; ++r)
      dma16(base, tile_chunk_voff(64u * copy_index(r) + ln, last), dst + copy_index(r) * 64 * 16);
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
    const unsigned last = static_cast<unsigned>(j1 - 1 - j0);
#pragma unroll
    for (int r = 0; r < COPIES; ++r)
      dma16(base, tile_chunk_voff(64u * copy_index(r) + lane, last),
            smem_lds + copy_index(r) * 64 * 16);
  }

  // ---- resident query fragments (B operand of the score product): qo for the own block
  //      hb, qx for the partner's block hx; fragment i is k-step 2 i + fh, lane (g, r16)
  //      holding features 32 (2 i + fh) + 8 g .. + 7 of head 16 blk + r16 (i = 8: the RoPE
  //      part).  Loaded in one assembly block together with the copies of tile 1, which
  //      waits for everything but those copies: two tiles are in flight while the
  //      queries arrive, and no compiler-inserted wait falls after a copy.
  bf16x8_t qo[HALF], qx[HALF];
  {
    const int64_t rowo = static_cast<int64_t>(bq) * NH + 16 * hb + r16;
    const int64_t rowx = static_cast<int64_t>(bq) * NH + 16 * hx + r16;
    const bf16raw* qrow_o = q_lat + rowo * DC + 32 * fh + 8 * g;
    const bf16raw* qrow_x = q_lat + rowx * DC + 32 * fh + 8 * g;
    const bf16raw* prow_o = q_pe + rowo * DR + 32 * fh + 8 * g;
    const bf16raw* prow_x = q_pe + rowx * DR + 32 * fh + 8 * g;
    const unsigned last1 = static_cast<unsigned>(j1 - 1 - tb1);
    const uint64_t b64 = reinterpret_cast<uint64_t>(page_base(page1, tb1));
    const uint32_t blo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64));
    const uint32_t bhi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64 >> 32));
    const void* base1 = reinterpret_cast<const void*>((static_cast<uint64_t>(bhi) << 32) | blo);
    static_assert(COPIES == 5, "the assembly block issues five copies");
    uint32_t vo[5], la[5];
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      vo[c] = tile_chunk_voff(64u * copy_index(c) + lane, last1);
      la[c] = __builtin_amdgcn_readfirstlane(smem_lds + TILE_BYTES + copy_index(c) * 64 * 16);
    }
    i32x4_t r[2 * HALF];
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "global_load_dwordx4 %0, %18, off\n\t"
        "global_load_dwordx4 %1, %18, off offset:128\n\t"
        "global_load_dwordx4 %2, %18, off offset:256\n\t"
        "global_load_dwordx4 %3, %18, off offset:384\n\t"
        "global_load_dwordx4 %4, %18, off offset:512\n\t"
        "global_load_dwordx4 %5, %18, off offset:640\n\t"
        "global_load_dwordx4 %6, %18, off offset:768\n\t"
        "global_load_dwordx4 %7, %18, off offset:896\n\t"
        "global_load_dwordx4 %8, %20, off\n\t"
        "global_load_dwordx4 %9, %19, off\n\t"
        "global_load_dwordx4 %10, %19, off offset:128\n\t"
        "global_load_dwordx4 %11, %19, off offset:256\n\t"
        "global_load_dwordx4 %12, %19, off offset:384\n\t"
        "global_load_dwordx4 %13, %19, off offset:512\n\t"
        "global_load_dwordx4 %14, %19, off offset:640\n\t"
        "global_load_dwordx4 %15, %19, off offset:768\n\t"
        "global_load_dwordx4 %16, %19, off offset:896\n\t"
        "global_load_dwordx4 %17, %21, off\n\t"
        "s_mov_b32 m0, %27\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %22, %32\n\t"
        "s_mov_b32 m0, %28\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %23, %32\n\t"
        "s_mov_b32 m0, %29\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %24, %32\n\t"
        "s_mov_b32 m0, %30\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %25, %32\n\t"
        "s_mov_b32 m0, %31\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %26, %32\n\t"
        "s_waitcnt vmcnt(5)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
          "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15]), "=&v"(r[16]), "=&v"(r[17])
        : "v"(qrow_o), "v"(qrow_x), "v"(prow_o), "v"(prow_x), "v"(vo[0]), "v"(vo[1]),
          "v"(vo[2]), "v"(vo[3]), "v"(vo[4]), "s"(la[0]), "s"(la[1]), "s"(la[2]), "s"(la[3]),
          "s"(la[4]), "s"(base1)
        : "memory", "m0");
#pragma clang diagnostic pop
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      qo[i] = __builtin_bit_cast(bf16x8_t, r[i]);
      qx[i] = __builtin_bit_cast(bf16x8_t, r[HALF + i]);
    }
  }

  // K fragment lane offsets (the same for every tile): M tile mt, row
  // t = 8 (r16 >> 2) + 4 mt + (r16 & 3), logical chunk 4 fh + g of each 128-byte group;
  // k-step 2 i + fh adds 128 i.
  int kb[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int t = 8 * (r16 >> 2) + 4 * mt + (r16 & 3);
    kb[mt] = t * ROW_BYTES + 16 * ((4 * fh + g) ^ swz(t));
  }

  // Partial scores of tile it over this wave's k-steps: so = own block, sx = partner's
  // block; row r of M tile mt is token 8 (r >> 2) + 4 mt + (r & 3), so lane (g, r16) ends
  // with tokens 8 g .. 8 g + 7 of head r16 of the block: after the softmax, exactly the
  // P^T operand of the PV product.  The 18 K fragments stream through a register ring.
  auto score = [&](int it, f32x4_t (&so)[2], f32x4_t (&sx)[2]) {
    const lds_char_t* tile = lsm + (it % NBUF) * TILE_BYTES;
    so[0] = so[1] = sx[0] = sx[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int STEPS = 2 * HALF;  // step = 2 i + mt
    constexpr int KRING = 3;
    auto k_frag = [&](int step) {
      return *(const lds_bf16x8_t*)(tile + kb[step & 1] + 128 * (step >> 1));
    };
    bf16x8_t ka[KRING];
#pragma unroll
    for (int i = 0; i < KRING - 1; ++i) ka[i] = k_frag(i);
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
      if (step + KRING - 1 < STEPS) ka[(step + KRING - 1) % KRING] = k_frag(step + KRING - 1);
      const int mt = step & 1, i = step >> 1;
      so[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % KRING], qo[i], so[mt], 0, 0, 0);
      sx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % KRING], qx[i], sx[mt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // O^T accumulators: o[ct][hb2] lane (g, r16) holds O[16 hb2 + r16][64 w + 16 ct + 4 g + i]
  f32x4_t o[4][8];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int h2 = 0; h2 < 8; ++h2) o[ct][h2] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // PV of tile it for this wave's 64 columns and all 8 head blocks.  V^T fragments (A
  // operand): lane (gg, rr) holds column 64 w + 16 ct + rr, tokens 8 gg .. 8 gg + 7,
  // gathered by two transposing reads of 4 rows each (column tile 4 w + ct sits in chunks
  // 8 w + 2 ct, + 1; the row swizzle moves only the low three chunk bits).
  auto pv = [&](int it) {
    const lds_char_t* tile = lsm + (it % NBUF) * TILE_BYTES + 128 * w;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per tile (no long live ranges)
    const int gg = ln >> 4, rr = ln & 15;
    bf16x8_t va[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      i16x4_t half[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int t = 8 * gg + 4 * r + (rr >> 2);
        const int e = (rr & 3) >> 1;
        half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(tile + t * ROW_BYTES + 16 * ((2 * ct + e) ^ swz(t)) + 8 * (rr & 1)));
      }
      va[ct] = __builtin_bit_cast(bf16x8_t,
                                  __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // P^T fragments of the 8 head blocks, 1 KB each, lane-contiguous
    const lds_char_t* pb = lsm + PBUF + 16 * ln;
    constexpr int PRING = 2;
    bf16x8_t pf[PRING];
    pf[0] = *(const lds_bf16x8_t*)(pb);
#pragma unroll
    for (int h2 = 0; h2 < 8; ++h2) {
      if (h2 + 1 < 8) pf[(h2 + 1) % PRING] = *(const lds_bf16x8_t*)(pb + 1024 * (h2 + 1));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        o[ct][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ct], pf[h2 % PRING], o[ct][h2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Reference maximum of head 16 hb + r16 (log2 units, same in its 4 lanes): the first
  // tile's maximum plus HEADROOM, fixed for the split.  The denominators accumulate on the
  // matrix core as ones (16 x 32) * P^T (32 x 16): every entry of lane (g, r16) holds the
  // sum of head 16 hb + r16, exactly over the bf16 weights the PV product consumes.
  float m_ref = -INFINITY;
  f32x4_t l_acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool out_of_range = false;  // sticky: a score of this head block left the reference range

  // softmax of tile it on the full scores of the own block; stores its P^T fragment
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
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, i16x4x2_ones());
    l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pt, l_acc, 0, 0, 0);
    *(lds_bf16x8_t*)(lsm + PBUF + hb * 1024 + 16 * lane) = pt;
  };

  publish_barrier();  // A(0): tile 0 and the tables
  for (int it = 0; it < ntiles; ++it) {
    if (it > 0) pv(it - 1);
    f32x4_t so[2], sx[2];
    score(it, so, sx);
    *(lds_f32x4_t*)(lsm + XCH + w * 2048 + 16 * lane) = sx[0];
    *(lds_f32x4_t*)(lsm + XCH + w * 2048 + 1024 + 16 * lane) = sx[1];
    const int page2 = it + 2 < ntiles ? split_page(j0 + (it + 2) * TILE) : 0;  // read ahead
    publish_barrier();  // B(it)
    if (it + 2 < ntiles) issue_tile(it + 2, page2);
    {
      const lds_char_t* xp = lsm + XCH + (w ^ 4) * 2048 + 16 * lane;
      so[0] += *(const lds_f32x4_t*)(xp);
      so[1] += *(const lds_f32x4_t*)(xp + 1024);
    }
    softmax(it, so);
    if (it == ntiles - 1) {  // the block's denominators and range flag for the epilogue
      const bool block_out = __any(out_of_range);  // a vote of the whole wavefront
      if (g == 0) ((lds_f32_t*)(lsm + STATS))[16 * hb + r16] = l_acc[0];
      if (lane == 0) ((lds_i32_t*)(lsm + STATS + 512))[hb] = block_out ? 1 : 0;
    }
    if (it + 2 < ntiles) wait_vmcnt<COPIES>();  // own copies of tile it+1 landed
    else wait_vmcnt<0>();
    publish_barrier();  // A(it+1)
  }
  pv(ntiles - 1);

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
  if (!(flags & (1 << hb))) {
    if (lse_part != nullptr && g == 0)
      lse_part[(static_cast<int64_t>(bq) * NH + 16 * hb + r16) * S + s] = (m_ref + __log2f(l_acc[0])) * LN2;
  } else {
    split_exact_fallback(q_lat, q_pe, cache, bt_row, log2P, j0, j1, bq, NH, S, s, scale_log2,
                         o_part, lse_part, 16 * hb, 16, lane);
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
