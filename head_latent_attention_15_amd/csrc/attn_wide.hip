// Decode attention over the paged latent cache for 128 heads with 32 heads per wavefront on
// the 32 x 32 x 16 bf16 MFMA (gfx950).
//
// Same method and products as attn_mfma.hip ("論文解説: DeepSeek-V2 …", "Decoupled RoPE" and
// "行列吸収トリック": after absorption both products of the decode step contract the heads
// against the shared 576-wide latent rows):
//   scores  S[h][t] = sum_k [q~_h ; q^R_h][k] * row_t[k]      (k over 576)
//   latent  O[h][c] += sum_t P[h][t] * row_t[c]                (c over 512)
// with the W^UV up-projection outside (kasblo.com/?p=4663, "V側は、小さな表現の加重和を先に求める").
//
// Why a second kernel.  With 16 heads per wavefront every K and V fragment read from LDS
// feeds one 16 x 16 x 32 MFMA, so the 8 wavefronts of a workgroup read each 36 KB tile
// ~15 times (544 KB of LDS reads per tile) and issue 68 MFMAs each per tile.  Here four
// wavefronts (one per SIMD) own 32 heads each, and each fragment feeds one 32 x 32 x 16
// MFMA: half the LDS bytes per tile (272 KB) and half the MFMA instructions for the same
// matrix-core time.  The price is registers: a wavefront keeps its 32 heads' O^T (512 x 32
// fp32, 256 accumulator registers) and Q (576 x 32 bf16, 144 registers) for the whole
// split, which one wavefront per SIMD can hold.
//
// Per tile of 32 tokens and wavefront:
//   scores: S^T (32 tokens x 32 heads) = K_tile (32 x 576) Q^T, 36 MFMAs in two
//           accumulation chains, the K operand read with ds_read_b128 (row = token);
//   PV:     O^T (512 x 32) += V^T (512 x 32 tokens) P^T, 16 column tiles x 2 token steps,
//           the V^T operand read with two transposing ds_read_b64_tr_b16 per fragment.
// In the C layout of S^T lane (hf, n) holds head n and tokens 8 j + 4 hf + i (j, i < 4):
// exactly the tokens its B operand of P^T needs for the two 16-token steps of the PV product
// (token step ks takes j = 2 ks, 2 ks + 1), so the weights never leave registers; the V^T
// fragments read the same tokens.  One wavefront per SIMD means no other wavefront hides
// its softmax, so the softmax of tile it runs between the PV MFMAs of tile it-1 (software
// pipelining inside the wavefront).
//
// Staging as in attn_mfma.hip: 32-token tiles go HBM -> LDS by global_load_lds_dwordx4 into
// four buffers (the copies of tiles it+1 and it+2 are in flight while tiles it-1 and it are
// read; the prologue waits only for tile 0 and the queries), rows carry the same 16-byte-chunk swizzle, which keeps both the row reads of 16
// consecutive tokens and the transposing reads conflict-free, and one barrier per tile
// publishes tile it and retires tile it-2.  Softmax with a fixed per-split reference (the
// first tile's maximum plus headroom, never rescaled) and the exact VALU fallback for a head
// block whose scores leave its range, as in attn_mfma.hip.  The denominators sum the
// bf16-rounded weights the PV product consumes (v_dot2 with ones).
#include "attn_common.h"
#include "launchers.h"
#include "ragged_plan.h"

#include <type_traits>

namespace mla {
namespace {

using namespace attn;

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int WW = 4;                                  // wavefronts per workgroup
constexpr int WH = 32;                                 // heads per wavefront
constexpr int W_NBUF = 4;                              // tile buffers
constexpr int W_PAGE_TABLE = W_NBUF * TILE_BYTES;      // LDS block table of the split
constexpr int W_MAX_SPLIT_PAGES = 1024;
constexpr int W_LDS_BYTES = W_PAGE_TABLE + W_MAX_SPLIT_PAGES * 4;
static_assert(W_LDS_BYTES <= 163840, "LDS per workgroup");
// fp8 rows: three bf16 tile buffers, two raw staging buffers, then the block table
constexpr int W8_NBUF = 3;
constexpr int W8_STAGE = W8_NBUF * TILE_BYTES;
constexpr int W8_PAGE_TABLE = W8_STAGE + 2 * FP8_STAGE_BYTES;
constexpr int W8_LDS_BYTES = W8_PAGE_TABLE + W_MAX_SPLIT_PAGES * 4;
static_assert(W8_LDS_BYTES <= 163840, "LDS per workgroup (fp8 rows)");
constexpr int W8_COPIES = (FP8_COPIES + WW - 1) / WW;  // 6 raw copies per tile and wave
constexpr int W_COPIES = TILE_WAVE_COPIES / WW;        // 9 wave-wide copies per tile and wave
static_assert(W_COPIES * WW == TILE_WAVE_COPIES, "copies split evenly");
constexpr int W_KSTEPS = ROW / 16;                     // 36 score k-steps of 16 features
constexpr int W_CT = DC / 32;                          // 16 PV column tiles of 32 columns
constexpr float W_HEADROOM = 32.0f;  // log2 units between a split's first-tile max and its reference
constexpr float W_P_RANGE = 64.0f;   // a score this far above the reference takes the fallback

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The score chains accumulate in VGPRs.  O^T takes all 256 accumulation registers, and the
// builtin's accumulation form would put the chains there too (the compiler then moves two
// column tiles of O^T in and out every tile), so these two are written out: the first of a
// chain starts from the inline constant 0, the others accumulate in place.  A chain's last
// result is read only after chain_drain, which gives the 16-pass MFMA's result the wait
// states a VALU read needs and carries the chains as operands, so no read moves above it.
__device__ __forceinline__ f32x16_t mfma32_v_first(bf16x8_t a, bf16x8_t b) {
  f32x16_t d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma32_v(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void chain_drain(f32x16_t& x, f32x16_t& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(x), "+v"(y));
}

// The attention of one split: tokens j0 .. j1-1 of sequence b (j1 = split_end(), read after
// the query loads are issued) with the queries of row bq; the partial of head h goes to row
// prow0 + h * hstride of o_part / lse_part.  Every thread of the workgroup calls it with the
// same arguments.  Wavefront w owns heads 32 w .. 32 w + 31.  KRING: K fragments in flight
// in the score loop (6; 4 where the caller keeps more state live, as the ragged kernel).
// FP8: the cache holds fp8 rows (656 bytes); each tile is copied raw into one of two
// staging buffers, all of its copies right after the barrier two tiles ahead of its use,
// and converted by the whole workgroup into one of three bf16 tile buffers one tile ahead,
// spread over the score steps of the tile before (code times its block's power-of-two
// scale, exact in bf16), so the score and PV steps are the bf16 ones.
template <typename OT, int KRING, bool FP8, typename SplitEnd>
__device__ __forceinline__ void wide_split(
    const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ cache, const int32_t* __restrict__ block_table, int H,
    int log2P, int max_pages, float scale_log2, OT* __restrict__ o_part,
    float* __restrict__ lse_part, int b, int bq, int j0, SplitEnd split_end, int64_t prow0,
    int hstride) {
  constexpr int NB = FP8 ? W8_NBUF : W_NBUF;             // bf16 tile buffers
  constexpr int PTAB = FP8 ? W8_PAGE_TABLE : W_PAGE_TABLE;
  constexpr int SRC_ROW = FP8 ? FP8_ROW_BYTES : ROW_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[FP8 ? W8_LDS_BYTES : W_LDS_BYTES];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>(lsm));

  // the thread index is made opaque here, so that when this runs in a loop over pieces
  // nothing derived from it is hoisted out of the loop and kept live across the pieces
  int tid_opaque = threadIdx.x;
  asm volatile("" : "+v"(tid_opaque));
  const int tid = tid_opaque, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, n32 = lane & 31;
  const int h0 = WH * w;

  // The queries need neither the sequence length nor the block table, so their loads go out
  // first, with those two scalar loads in flight beside them.  The B operand of S^T = K Q^T
  // for k-step kk wants lane (hf, n32) to hold head h0 + n32, features 16 kk + 8 hf .. + 7:
  // two lanes per head, so loading it in place touches 32 rows per instruction.  Instead each
  // wave loads its 32 query rows in order, 1 KB per instruction, in three parts (q~ features
  // 0-255 and 256-511: two half rows per load; q^R: eight rows per load), and transposes them
  // through LDS below.
  constexpr int QA = 16, QC = 4;  // loads per wave: each q~ part, q^R
  bf16x8_t rawa[QA], rawb[QA], rawc[QC];
  {
    const int64_t qrow0 = static_cast<int64_t>(bq) * H + h0;
    const bf16raw* ql = q_lat + (qrow0 + (lane >> 5)) * DC + 8 * (lane & 31);  // rows 2 i + hf
    const bf16raw* qp = q_pe + (qrow0 + (lane >> 3)) * DR + 8 * (lane & 7);     // rows 8 i + lane / 8
#pragma unroll
    for (int i = 0; i < QA; ++i) rawa[i] = *reinterpret_cast<const bf16x8_t*>(ql + 2 * DC * i);
#pragma unroll
    for (int i = 0; i < QA; ++i) rawb[i] = *reinterpret_cast<const bf16x8_t*>(ql + 2 * DC * i + DC / 2);
#pragma unroll
    for (int i = 0; i < QC; ++i) rawc[i] = *reinterpret_cast<const bf16x8_t*>(qp + 8 * DR * i);
  }
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_pages;
  const int pg0 = __builtin_amdgcn_readfirstlane((j0 >> log2P) < max_pages ? bt_row[j0 >> log2P] : 0);

  const int j1 = split_end();
  const int P = 1 << log2P;

  if (j0 >= j1) {  // empty split: o = 0, lse = -inf
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the query loads land before the exit
    for (int e = tid; e < H * DC; e += WW * 64) {
      const int h = e / DC, c = e % DC;
      st(o_part + (prow0 + static_cast<int64_t>(h) * hstride) * DC + c, 0.f);
    }
    if (lse_part != nullptr)
      for (int h = tid; h < H; h += WW * 64) lse_part[prow0 + static_cast<int64_t>(h) * hstride] = -INFINITY;
    return;
  }

  const char* cache_bytes = reinterpret_cast<const char*>(cache);
  auto page_base = [&](int pg, int tb) {
    return cache_bytes + ((static_cast<int64_t>(pg) << log2P) + (tb & (P - 1))) * SRC_ROW;
  };
  const int ntiles = (j1 - j0 + TILE - 1) / TILE;
  const int npages = (j1 - j0 + P - 1) >> log2P;

  // Copy r of this wave fills LDS chunk 64 (w + 4 r) + lane of a tile buffer: row t, stored
  // position p, which holds logical chunk p ^ swz(t).  Its source offset in a full tile is the
  // same for every tile (kept in registers); in a tile past the split's last token (TAIL) the
  // rows past it repeat it, and the offset is recomputed with that clamp.
  uint32_t cfull[W_COPIES];
#pragma unroll
  for (int r = 0; r < W_COPIES; ++r) cfull[r] = tile_chunk_voff(64u * (w + WW * r) + lane, TILE - 1);
  auto issue_copy = [&](const char* base, unsigned last, uint32_t lds_tile, int r, auto tail) {
    uint32_t voff = cfull[r];
    if constexpr (decltype(tail)::value) voff = tile_chunk_voff(64u * (w + WW * r) + lane, last);
    dma16(base, voff, lds_tile + (w + WW * r) * 1024);
  };
  const std::true_type clamped;
  const std::false_type unclamped;
  // fp8 rows: this wave's copies q = w, w + 4, ... (the 21st repeated) of the raw tile at
  // token tb into staging buffer `stage`
  auto fp8_issue_tile = [&](const char* base, int tb, int stage) {
#pragma unroll
    for (int r = 0; r < W8_COPIES; ++r)
      fp8_tile_copy(base, static_cast<unsigned>(j1 - 1 - tb), smem_lds + W8_STAGE + stage * FP8_STAGE_BYTES,
                    min(static_cast<unsigned>(w + WW * r), static_cast<unsigned>(FP8_COPIES - 1)), lane);
  };
  // fp8 rows: this thread's 9 chunks of the bf16 tile in buffer buf from staging buffer
  // stage: eight latent chunks, then one of k^R (so no wavefront branches on the kind)
  auto fp8_convert = [&](int stage, int buf) {
    static_assert(TILE * 64 == 8 * WW * 64 && TILE * 8 == WW * 64, "conversion chunks split evenly");
    const lds_char_t* src = lsm + W8_STAGE + stage * FP8_STAGE_BYTES;
    lds_char_t* dst = lsm + buf * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fp8_convert_latent(src, dst, tid + WW * 64 * i);
      __builtin_amdgcn_sched_barrier(0);  // one chunk at a time: registers are full
    }
    fp8_copy_rope(src, dst, tid);
  };

  // ---- prologue.  Tile 0's copies go out behind the queries, then the split's block-table
  //      entries into LDS; the first barrier waits for all of it.  The copies of tiles 1 and
  //      2 go out during tile 0's score steps, so no prologue wait covers a tile that is not
  //      read yet.  The queries are transposed through LDS (tile buffers 1-3 are free until
  //      tile 0's score steps): row n's chunk c of a q~ part at slot 33 n + c of the wave's
  //      first area, of q^R at slot 9 n + c of its second; one slot of padding per row keeps
  //      the reads of the B layout conflict-free.
  //      With fp8 rows the raw tiles 0 and 1 go to the staging buffers instead, and the
  //      queries are transposed through the bf16 tile buffers from their start (tile 0 is
  //      converted after the first barrier).
  constexpr int QSA = 33 * 16 * WH, QSC = 9 * 16 * WH;  // staging bytes per wave
  constexpr int QBASE = FP8 ? 0 : TILE_BYTES;
  static_assert(QBASE + WW * (QSA + QSC) <= NB * TILE_BYTES, "query staging fits the free tile buffers");
  bf16x8_t qf[W_KSTEPS];
  {
    if constexpr (FP8) {
      fp8_issue_tile(page_base(pg0, j0), j0, 0);
      if (ntiles > 1) {
        const int tb1 = j0 + TILE;
        fp8_issue_tile(page_base(__builtin_amdgcn_readfirstlane(bt_row[tb1 >> log2P]), tb1), tb1, 1);
      }
    } else {
      const char* base0 = page_base(pg0, j0);
#pragma unroll
      for (int r = 0; r < W_COPIES; ++r)
        issue_copy(base0, static_cast<unsigned>(j1 - 1 - j0), smem_lds, r, clamped);
    }
    lds_char_t* const qa = lsm + QBASE + w * QSA;
    lds_char_t* const qc = lsm + QBASE + WW * QSA + w * QSC;
    // load i of a q~ part holds row 2 i + hf, chunk n32; of q^R, row 8 i + lane / 8, chunk lane % 8
    auto stage_a = [&](const bf16x8_t* raw) {
#pragma unroll
      for (int i = 0; i < QA; ++i) *(lds_bf16x8_t*)(qa + 16 * (33 * (2 * i + hf) + n32)) = raw[i];
    };
    auto unstage_a = [&](int k0) {  // k-steps k0 .. k0 + 15: chunks 2 k + hf of row n32
#pragma unroll
      for (int k = 0; k < 16; ++k) qf[k0 + k] = *(const lds_bf16x8_t*)(qa + 16 * (33 * n32 + 2 * k + hf));
    };
    // in the order the loads were issued (and land): q~ features 0-255, 256-511, then q^R
    stage_a(rawa);
    unstage_a(0);  // (LDS operations of one wave complete in order: no wait between)
    stage_a(rawb);
    unstage_a(16);
#pragma unroll
    for (int i = 0; i < QC; ++i) *(lds_bf16x8_t*)(qc + 16 * (9 * (8 * i + (lane >> 3)) + (lane & 7))) = rawc[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) qf[32 + k] = *(const lds_bf16x8_t*)(qc + 16 * (9 * n32 + 2 * k + hf));
  }
  lds_i32_t* const ptab = (lds_i32_t*)(lsm + PTAB);
  // tile buffer of tile it; with three buffers the offset is made opaque, since the compiler
  // otherwise strength-reduces every fragment address of the loop into registers of its own
  auto tile_at = [&](int it) -> const lds_char_t* {
    int off = (it % NB) * TILE_BYTES;
    if constexpr (NB != W_NBUF) asm volatile("" : "+s"(off));
    return lsm + off;
  };
  for (int e = tid; e < npages; e += WW * 64) ptab[e] = bt_row[(j0 >> log2P) + e];
  auto split_page = [&](int tb) {
    return __builtin_amdgcn_readfirstlane(ptab[(tb - j0) >> log2P]);
  };

  // Lane offsets inside a tile buffer, the same for every tile:
  //   kb[j]: K fragment of k-step kk (kk & 3 == j): row n32, logical chunk 2 kk + hf; k-step
  //     kk adds 128 (kk >> 2).
  //   vb[r][c1]: V^T fragment of column tile ct (ct & 1 == c1), token step 0, read r: rows
  //     8 r + 4 hf + (n >> 2) (n = lane & 15), columns 32 ct + 16 g1 + 4 (n & 3) .. + 3
  //     (g1 = lane >> 4 & 1); column tile ct adds 128 (ct >> 1).  Token step 1 reads rows 16
  //     further down, where the swizzle flips chunk bit 2: vb[r][c1 ^ 1] + 16 rows.
  int kb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kb[j] = n32 * ROW_BYTES + 16 * ((2 * j + hf) ^ swz(n32));
  int vb[2][2];
  {
    const int n = lane & 15, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = 8 * r + 4 * hf + (n >> 2);
#pragma unroll
      for (int c1 = 0; c1 < 2; ++c1)
        vb[r][c1] = t * ROW_BYTES + 16 * ((4 * c1 + 2 * g1 + ((n >> 1) & 1)) ^ swz(t)) + 8 * (n & 1);
    }
  }

  f32x16_t o[W_CT];
#pragma unroll
  for (int ct = 0; ct < W_CT; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[ct][i] = 0.f;
  float m_ref = -INFINITY;
  float lsum = 0.f;            // this lane's 16 tokens of head h0 + n32, summed over the tiles
  bool out_of_range = false;   // sticky: a score of this head block left the reference range
  const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);

  // Scores of tile it (two accumulation chains, summed), with this wave's copies of tile it+2
  // (or, near the end of the split, tile it again into the retired buffer, so every tile
  // issues the same copies and every wait counts alike) spread over the k-steps.
  // Tile tb's copy source and its last valid row (rows past the split's end repeat it).
  auto copy_src = [&](int tb) { return page_base(split_page(tb), tb); };
  // Scores of tile it (two accumulation chains, summed), with this wave's copies of tile it+2
  // (or, near the end of the split, tile it again into the retired buffer, so every tile
  // issues the same copies and every wait counts alike) spread over the k-steps.  Tile 0's
  // score steps (FIRST) issue the copies of tiles 1 and 2, one every second step.  TAIL:
  // some copied tile reaches past the split's last token (its rows are clamped).
  auto copy_tb = [&](int it) { return j0 + (it + 2 < ntiles ? it + 2 : min(it, ntiles - 1)) * TILE; };
  auto scores = [&](int it, auto first, auto tail, auto conv) -> f32x16_t {
    constexpr bool FIRST = decltype(first)::value;
    const lds_char_t* tile = tile_at(it);
    const int tb2 = copy_tb(it);
    const char* base2 = copy_src(tb2);
    const unsigned last2 = static_cast<unsigned>(j1 - 1 - tb2);
    const uint32_t lds2 = smem_lds + ((it + 2) % W_NBUF) * TILE_BYTES;
    const int tb1 = ntiles > 1 ? j0 + TILE : j0;  // FIRST: a one-tile split copies its tile again
    const char* base1 = FIRST ? copy_src(tb1) : base2;
    const unsigned last1 = static_cast<unsigned>(j1 - 1 - tb1);
    f32x16_t s0, s1;
    auto k_frag = [&](int kk) {
      return *(const lds_bf16x8_t*)(tile + kb[kk & 3] + 128 * (kk >> 2));
    };
    bf16x8_t ka[KRING];
#pragma unroll
    for (int i = 0; i < KRING - 1; ++i) ka[i] = k_frag(i);
#pragma unroll
    for (int kk = 0; kk < W_KSTEPS; ++kk) {
      if (kk + KRING - 1 < W_KSTEPS) ka[(kk + KRING - 1) % KRING] = k_frag(kk + KRING - 1);
      if (kk == 0) s0 = mfma32_v_first(ka[0], qf[0]);
      else if (kk == 1) s1 = mfma32_v_first(ka[1], qf[1]);
      else if (kk & 1) mfma32_v(s1, ka[kk % KRING], qf[kk]);
      else mfma32_v(s0, ka[kk % KRING], qf[kk]);
      if constexpr (FP8) {
        // fp8 rows: the raw copies are issued at the barrier, not here
      } else if constexpr (FIRST) {
        if (kk % 2 == 0 && kk / 2 < W_COPIES) issue_copy(base1, last1, smem_lds + TILE_BYTES, kk / 2, tail);
        else if (kk % 2 == 0) issue_copy(base2, last2, lds2, kk / 2 - W_COPIES, tail);
      } else if (kk % 4 == 0) {
        issue_copy(base2, last2, lds2, kk / 4, tail);
      }
      conv(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
    chain_drain(s0, s1);
    return s0 + s1;
  };

  // fp8 rows: the conversion of raw tile `it` into its bf16 buffer spread over the score
  // steps (latent chunk u at step 4 u, the k^R chunk at step 32)
  auto conv_of = [&](int it, bool on) {
    const lds_char_t* csrc = lsm + W8_STAGE + (it & 1) * FP8_STAGE_BYTES;
    lds_char_t* cdst = const_cast<lds_char_t*>(tile_at(it));
    return [=](int kk) {
      if (on && (kk & 3) == 0) {
        if (kk < 32) fp8_convert_latent(csrc, cdst, tid + WW * 64 * (kk >> 2));
        else fp8_copy_rope(csrc, cdst, tid);
      }
    };
  };
  const auto no_conv = [](int) {};

  // tokens at or past j1 (last tile of the split only) get weight 0
  auto mask_tail = [&](f32x16_t& sc, int it) {
    const int tb = j0 + it * TILE;
    if (tb + TILE > j1) {
      compiler_fence();  // a real branch: the masking runs on one tile only
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (tb + 8 * (r >> 2) + 4 * hf + (r & 3) >= j1) sc[r] = -INFINITY;
    }
  };

  // Softmax pieces on the raw scores (log2 domain): weight 2^(s scale - m_ref), one rounding
  // in the fma.  Register r of S^T feeds P^T operand r >> 3 (token step), element r & 7.
  float ex[16];
  bf16x2_t pk[8];
  float emax = -INFINITY;
  auto soft_exp = [&](const f32x16_t& sc, int r) {
    const float e = __builtin_fmaf(sc[r], scale_log2, -m_ref);
    emax = fmaxf(emax, e);
    ex[r] = __builtin_amdgcn_exp2f(e);
  };
  auto soft_pack = [&](int i) {
    pk[i] = to_bf16x2(ex[2 * i], ex[2 * i + 1]);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(pk[i], ones2, lsum, false);
  };
  auto soft_done = [&](bf16x8_t& p0, bf16x8_t& p1) {
    out_of_range |= emax > W_P_RANGE;
    emax = -INFINITY;
    p0 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(
             __builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
             __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7));
    p1 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(
             __builtin_shufflevector(pk[4], pk[5], 0, 1, 2, 3),
             __builtin_shufflevector(pk[6], pk[7], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // PV of tile it with P^T operands p0 (token step 0) and p1; with SOFT the softmax of the
  // next tile's scores sc runs between the first 16 MFMAs (an exponent per step, a packed
  // pair every second step), leaving its operands in n0, n1.
  auto v_frag = [&](const lds_char_t* tile, int st) {
    const int ct = st >> 1, ks = st & 1;
    i16x4_t half[2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
      half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(tile + vb[r][(ct & 1) ^ ks] + 128 * (ct >> 1) + 16 * ROW_BYTES * ks));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pv = [&](int it, bf16x8_t p0, bf16x8_t p1, auto soft, const f32x16_t& sc, bf16x8_t& n0,
                bf16x8_t& n1) {
    constexpr bool SOFT = decltype(soft)::value;
    const lds_char_t* tile = tile_at(it);
    constexpr int VRING = 4;
    constexpr int NST = 2 * W_CT;
    bf16x8_t va[VRING];
#pragma unroll
    for (int i = 0; i < VRING - 1; ++i) va[i] = v_frag(tile, i);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + VRING - 1 < NST) va[(st + VRING - 1) % VRING] = v_frag(tile, st + VRING - 1);
      o[st >> 1] = mfma32(va[st % VRING], (st & 1) ? p1 : p0, o[st >> 1]);
      if constexpr (SOFT) {
        if (st < 16) {
          soft_exp(sc, st);
          if (st & 1) soft_pack(st >> 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SOFT) soft_done(n0, n1);
  };

  // ---- main loop.  Barrier it publishes tile it (every wave's copies landed) and retires
  //      tile it-2, whose buffer the copies issued during scores(it) overwrite.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // block table in LDS
  wait_vmcnt<0>();                                    // tile 0 and the queries
  block_barrier();
  if constexpr (FP8) {
    // raw tile 0 into bf16 buffer 0 (every wave's query reads of the buffers are done);
    // then raw tile 2 into the staging buffer tile 0 left
    fp8_convert(0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
    if (ntiles > 2) fp8_issue_tile(copy_src(j0 + 2 * TILE), j0 + 2 * TILE, 0);
  }
  bf16x8_t p0, p1;
  {
    f32x16_t sc;
    if constexpr (FP8) sc = scores(0, std::true_type(), clamped, conv_of(1, ntiles > 1));
    else sc = scores(0, std::true_type(), clamped, no_conv);
    mask_tail(sc, 0);
    float tmax = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sc[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    m_ref = mul_rn(tmax, scale_log2) + W_HEADROOM;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      soft_exp(sc, r);
      if (r & 1) soft_pack(r >> 1);
    }
    soft_done(p0, p1);
  }
  for (int it = 1; it < ntiles; ++it) {
    f32x16_t sc;
    if constexpr (FP8) {
      // Barrier it publishes bf16 tile it (converted during tile it-1) and raw tile it+1
      // (copied since barrier it-1).  Then raw tile it+2 goes to the staging buffer raw tile
      // it left, and raw tile it+1 is converted into the buffer tile it-2 left during the
      // score steps of tile it.
      wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      block_barrier();
      if (it + 2 < ntiles) fp8_issue_tile(copy_src(j0 + (it + 2) * TILE), j0 + (it + 2) * TILE, it & 1);
      sc = scores(it, std::false_type(), unclamped, conv_of(it + 1, it + 1 < ntiles));
    } else {
      wait_vmcnt<W_COPIES>();  // own copies of tile it landed (tile it+1's may be in flight)
      block_barrier();
      sc = j1 - copy_tb(it) >= TILE ? scores(it, std::false_type(), unclamped, no_conv)
                                    : scores(it, std::false_type(), clamped, no_conv);
    }
    mask_tail(sc, it);
    bf16x8_t n0, n1;
    pv(it - 1, p0, p1, std::integral_constant<bool, true>(), sc, n0, n1);
    p0 = n0;
    p1 = n1;
  }
  wait_vmcnt<0>();  // no copy may still be writing LDS at the end
  {
    const f32x16_t none = {};
    bf16x8_t n0, n1;
    pv(ntiles - 1, p0, p1, std::integral_constant<bool, false>(), none, n0, n1);
  }

  // ---- epilogue: lane (hf, n32) holds head h0 + n32, columns 32 ct + 8 j + 4 hf + i of
  //      register 4 j + i of o[ct]; a head block whose scores left the reference range is
  //      recomputed exactly.  The partials go through LDS (the tile buffers are free now), so
  //      each store writes 1 KB of one row: wave w's 32 rows sit at 32 KB w; for bf16, row
  //      h's chunk c (columns 8 c .. 8 c + 7) at position c ^ h.
  const bool fallback = __any(out_of_range);
  const float lt = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = 1.f / lt;
  if (!fallback && lse_part != nullptr && hf == 0)
    lse_part[prow0 + static_cast<int64_t>(h0 + n32) * hstride] = (m_ref + __log2f(lt)) * LN2;
  if constexpr (std::is_same<OT, float>::value) {
    // fp32: the same in two halves of 256 columns (32 KB per wave each); row h's chunk c
    // (columns 4 c .. 4 c + 3 of the half) at position c ^ h
    block_barrier();  // every wave's last tile reads are done
    if (!fallback) {
      lds_char_t* const stage = lsm + w * (WH * DC * 2);
      float* dst = o_part + prow0 * DC + 4 * lane;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int ct = 0; ct < W_CT / 2; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16_t& a = o[8 * half + ct];
            *(lds_f32x4_t*)(stage + n32 * (DC * 2) + 16 * ((8 * ct + 2 * j + hf) ^ n32)) =
                f32x4_t{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]} * inv;
          }
#pragma unroll
        for (int h = 0; h < WH; ++h) {
          const f32x4_t v = *(const lds_f32x4_t*)(stage + h * (DC * 2) + 16 * (lane ^ h));
          *reinterpret_cast<f32x4_t*>(dst + static_cast<int64_t>(h0 + h) * hstride * DC + 256 * half) = v;
        }
      }
    }
  } else {
    block_barrier();  // every wave's last tile reads are done
    if (!fallback) {
      lds_char_t* const stage = lsm + w * (WH * DC * 2);
#pragma unroll
      for (int ct = 0; ct < W_CT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t v = f32x4_t{o[ct][4 * j], o[ct][4 * j + 1], o[ct][4 * j + 2], o[ct][4 * j + 3]} * inv;
          *(lds_bf16x4_t*)(stage + n32 * (DC * 2) + 16 * ((4 * ct + j) ^ n32) + 8 * hf) =
              __builtin_shufflevector(to_bf16x2(v[0], v[1]), to_bf16x2(v[2], v[3]), 0, 1, 2, 3);
        }
      bf16raw* dst = o_part + prow0 * DC + 8 * lane;
#pragma unroll
      for (int h = 0; h < WH; ++h) {
        const bf16x8_t v = *(const lds_bf16x8_t*)(stage + h * (DC * 2) + 16 * (lane ^ h));
        *reinterpret_cast<bf16x8_t*>(dst + static_cast<int64_t>(h0 + h) * hstride * DC) = v;
      }
    }
  }
  if (fallback)
    split_exact_fallback<OT, FP8>(q_lat, q_pe, cache, bt_row, log2P, j0, j1, bq, H, prow0,
                                  hstride, scale_log2, o_part, lse_part, h0, WH, lane);
}

// One workgroup of four wavefronts per (sequence, split) (blockIdx.x, blockIdx.y) and query
// token (blockIdx.z), as attn_mfma_kernel: token t of n_q sits at position seq_len - n_q + t,
// its queries and partials are row bq = b n_q + t, and the splits of a sequence share its
// XCD.  FP8: the cache holds fp8 rows.
template <typename OT, bool FP8>
__global__ __launch_bounds__(WW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_wide_kernel(const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
                      const bf16raw* __restrict__ cache, const int32_t* __restrict__ block_table,
                      const int32_t* __restrict__ seq_lens, int H, int log2P, int max_pages,
                      int pages_per_split, int S, float scale_log2, OT* __restrict__ o_part,
                      float* __restrict__ lse_part, int n_q) {
  const int b = blockIdx.x, s = blockIdx.y, z = blockIdx.z, bq = b * n_q + z;
  const int j0 = s * (pages_per_split << log2P);
  wide_split<OT, 6, FP8>(q_lat, q_pe, cache, block_table, H, log2P, max_pages, scale_log2, o_part,
                    lse_part, b, bq, j0,
                 [&] { return min(seq_lens[b] - (n_q - 1 - z), j0 + (pages_per_split << log2P)); },
                 static_cast<int64_t>(bq) * H * S + s, S);
}

// Flattened work list for ragged batches (ragged_plan.h): range r of the batch's cached
// pages goes to one workgroup, which runs wide_split on each sequence piece inside it; the
// partial of head h from piece i of sequence b is row first_b H + h count_b + i, as in
// attn_mfma_ragged_kernel, so the same slot-table combine merges them.  FP8: fp8 cache rows.
template <typename OT, bool FP8>
__global__ __launch_bounds__(WW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_wide_ragged_kernel(const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
                             const bf16raw* __restrict__ cache,
                             const int32_t* __restrict__ block_table,
                             const int32_t* __restrict__ seq_lens, int B, int H, int log2P,
                             int max_pages, float scale_log2, OT* __restrict__ o_part,
                             float* __restrict__ lse_part, int* __restrict__ seq_slots,
                             int* __restrict__ err) {
  int W = 0, tot = 0;
  if (ragged::plan_ranges(seq_lens, B, log2P, W_MAX_SPLIT_PAGES, seq_slots, err, W, tot)) return;
  // the plan's scalars wait in LDS between pieces (registers are full inside the split body)
  __shared__ int plan[2];
  if (threadIdx.x == 0) {
    plan[0] = W;
    plan[1] = tot;
  }
  __syncthreads();
  for (int k = 0;; ++k) {
    const int Wk = __builtin_amdgcn_readfirstlane(
        *static_cast<volatile __attribute__((address_space(3))) int*>(
            (__attribute__((address_space(3))) int*)plan));
    const int tk = __builtin_amdgcn_readfirstlane(
        *static_cast<volatile __attribute__((address_space(3))) int*>(
            (__attribute__((address_space(3))) int*)plan + 1));
    const int rk = __builtin_amdgcn_readfirstlane(ragged::range_of(blockIdx.x, gridDim.x));
    const int lo = rk * Wk, hi = min(lo + Wk, tk);
    ragged::Piece pc;
    if (!ragged::ragged_piece(seq_lens, B, log2P, Wk, rk, lo, hi, k, &pc)) break;
    // the previous piece's partial stores are done, and its last LDS reads too, before this
    // piece's loads and copies reuse the registers and buffers
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int j1 = pc.j1;
    wide_split<OT, 4, FP8>(q_lat, q_pe, cache, block_table, H, log2P, max_pages, scale_log2, o_part,
                      lse_part, pc.b, pc.b, pc.j0, [&] { return j1; },
                   static_cast<int64_t>(pc.first) * H + pc.index, pc.count);
  }
}

template <typename OT, bool FP8>
hipError_t launch_wide_t(const PagedArgs& a, hipStream_t st) {
  const float log2e = 1.4426950408889634f;
  hipLaunchKernelGGL((attn_wide_kernel<OT, FP8>), dim3(a.B, a.num_splits, a.n_q), dim3(WW * 64), 0, st,
                     static_cast<const bf16raw*>(a.q_lat), static_cast<const bf16raw*>(a.q_pe),
                     static_cast<const bf16raw*>(a.cache), a.block_table, a.seq_lens, a.H,
                     __builtin_ctz(static_cast<unsigned>(a.page_size)), a.max_pages,
                     a.pages_per_split, a.num_splits, a.scale * log2e,
                     static_cast<OT*>(a.o_part), a.lse_part, a.n_q);
  return hipGetLastError();
}

bool aligned16w(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool attn_wide_supported(const PagedArgs& a) {
  const bool page_ok = a.page_size >= TILE && (a.page_size & (a.page_size - 1)) == 0;
  return a.d_c == DC && a.d_R == DR && a.H == WW * WH && page_ok &&
         a.pages_per_split <= W_MAX_SPLIT_PAGES && a.B <= 65535 && a.n_q >= 1 &&
         a.n_q <= 65535 && aligned16w(a.q_lat) && aligned16w(a.q_pe) && aligned16w(a.cache) &&
         aligned16w(a.o_part);
}

hipError_t launch_attn_wide_ragged(const PagedArgs& a, int grid, int* seq_slots, int* err,
                                   hipStream_t st, bool fp8) {
  if (!attn_wide_supported(a) || !a.part_bf16) return hipErrorInvalidValue;
  const float log2e = 1.4426950408889634f;
  const auto kernel = fp8 ? attn_wide_ragged_kernel<bf16raw, true> : attn_wide_ragged_kernel<bf16raw, false>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(WW * 64), 0, st,
                     static_cast<const bf16raw*>(a.q_lat), static_cast<const bf16raw*>(a.q_pe),
                     static_cast<const bf16raw*>(a.cache), a.block_table, a.seq_lens, a.B, a.H,
                     __builtin_ctz(static_cast<unsigned>(a.page_size)), a.max_pages,
                     a.scale * log2e, static_cast<bf16raw*>(a.o_part), a.lse_part, seq_slots, err);
  return hipGetLastError();
}

hipError_t launch_attn_wide_bf16_512_64(const PagedArgs& a, hipStream_t s) {
  if (!attn_wide_supported(a)) return hipErrorInvalidValue;
  return a.part_bf16 ? launch_wide_t<bf16raw, false>(a, s) : launch_wide_t<float, false>(a, s);
}

hipError_t launch_attn_wide_fp8(const PagedArgs& a, hipStream_t s) {
  if (!attn_wide_supported(a)) return hipErrorInvalidValue;
  return a.part_bf16 ? launch_wide_t<bf16raw, true>(a, s) : launch_wide_t<float, true>(a, s);
}

}  // namespace mla
