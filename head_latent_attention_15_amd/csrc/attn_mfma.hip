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
// Work decomposition.  One workgroup per (sequence, split) holds every head, so each cache
// byte crosses HBM once.  32-token tiles are copied HBM -> LDS with 16-byte
// global_load_lds_dwordx4 (no VGPR round trip) into four buffers: while tile it is consumed,
// the copies of tiles it+1 and it+2 are in flight.  The copy is issued from inline assembly
// with explicit vmcnt waits: it has no destination registers, and keeping it out of the
// compiler's view stops the compiler from adding a full vmcnt(0) wait in front of every LDS
// read.  Each lane's source offset for each copy comes from a small LDS table written once
// per workgroup.
//
// Each of the NW wavefronts owns 16 heads for both products, so its softmax weights never
// leave its registers:
//   scores: S^T = K_tile (32 x 576) * Q^T (576 x 16) on v_mfma_f32_16x16x32_bf16, Q resident
//           in VGPRs for the whole split, the K operand read with ds_read_b128;
//   PV:     O^T (512 x 16) += V^T (512 x 32) * P^T (32 x 16), the V^T operand read with the
//           transposing ds_read_b64_tr_b16.
// Tokens are the M dimension of the score product, so the C layout of S^T is, up to a fixed
// token permutation inside each tile, the B layout P^T needs in the PV product.  LDS rows
// carry a 16-byte-chunk XOR swizzle that keeps both the row-strided ds_read_b128 of K and
// the transposed reads of V conflict-free.  Half the wavefronts run the PV product of a
// tile while the other half compute the next scores, so the two wavefronts sharing a SIMD
// alternate between LDS-heavy and matrix-core-heavy work.
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
#include "attn_common.h"
#include "combine_row.h"
#include "launchers.h"
#include "ragged_plan.h"

#include <cstdlib>
#include <type_traits>

namespace mla {
namespace {

using namespace attn;

constexpr int NBUF = 4;                             // tile buffers
constexpr int VOFF_TABLE = NBUF * TILE_BYTES;      // LDS offset of the copy offset table
constexpr int PAGE_TABLE = VOFF_TABLE + TILE_WAVE_COPIES * 64 * 4;  // after 36 x 64 offsets
constexpr int MAX_SPLIT_PAGES = 1024;               // block-table entries of one split in LDS
constexpr int LDS_BYTES = PAGE_TABLE + MAX_SPLIT_PAGES * 4;
static_assert(LDS_BYTES <= 163840, "LDS per workgroup");
// fp8 latent rows are staged raw and converted into the same bf16 tile buffers: three of
// those, two staging buffers, then the block table.
constexpr int FP8_NBUF = 3;
constexpr int FP8_STAGE = FP8_NBUF * TILE_BYTES;
constexpr int FP8_PAGE_TABLE = FP8_STAGE + 2 * FP8_STAGE_BYTES;
constexpr int FP8_LDS_BYTES = FP8_PAGE_TABLE + MAX_SPLIT_PAGES * 4;
static_assert(FP8_LDS_BYTES <= 163840, "LDS per workgroup");
constexpr float HEADROOM = 32.0f;  // log2 units between a split's first-tile max and its reference
constexpr float P_RANGE = 64.0f;   // a score this far above the reference takes the fallback

// In-launch merge of the S splits of query row bq, after this workgroup (split s) wrote
// its partial: the workgroup counts its arrival in merge_cnt[2 bq], waits until all S
// splits of the row have arrived, then combines heads s, s + S, s + 2 S, ... of the row
// (one wavefront per head, combine_row.h) into out / lse_out.  The second counter
// merge_cnt[2 bq + 1] counts the workgroups past the wait; the last one clears both, so
// the counters are zero again for the next launch.  Workgroups wait for each other here,
// so the launcher only asks for the merge when the whole grid is resident at once; the
// wait is bounded all the same, and a wait that runs out sets *merge_err.
constexpr int MERGE_SPIN_LIMIT = 1 << 20;

template <int NW, typename OT>
__device__ void merge_splits(const OT* __restrict__ o_part, const float* __restrict__ lse_part,
                             int H, int S, int s, int bq, int* __restrict__ merge_cnt,
                             int* __restrict__ merge_err, float* __restrict__ out,
                             float* __restrict__ lse_out, int tid) {
  int* const arrived = merge_cnt + 2 * bq;
  int* const passed = arrived + 1;
  // Each wavefront waits for its partial stores to complete (reach L2), then the barrier
  // orders them all before thread 0's device-scope release.  That fence (an L2 write-back)
  // and the acquire after the wait (an L2 and L1 invalidate) are cache-wide, so one thread
  // issues each for the whole workgroup: the same fences issued by every wavefront cost
  // about as much again as the attention.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(arrived, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int n = 0;
    // polled without acquire (an acquire per poll would invalidate the caches every time)
    while (__hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < S) {
      if (++n == MERGE_SPIN_LIMIT) {
        __hip_atomic_store(merge_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  const int lane = tid & 63, w = tid >> 6;
  for (int h = s + S * w; h < H; h += S * NW) {
    const int64_t row = static_cast<int64_t>(bq) * H + h;
    combine512_wave(o_part + row * S * DC, lse_part + row * S, S, out + row * DC,
                    lse_out != nullptr ? lse_out + row : nullptr, lane);
  }
  if (tid == 0 &&
      __hip_atomic_fetch_add(passed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1) {
    __hip_atomic_store(arrived, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(passed, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// NW wavefronts, H = 16 * NW heads; wave w owns heads h0 = 16 w .. h0 + 15 for both
// products, so a wave's softmax weights never leave its registers:
//   scores: S^T = K_tile (32 x 576) * Q^T (576 x 16), Q resident in VGPRs for the split;
//   PV:     O^T (512 x 16) += V^T (512 x 32) * P^T (32 x 16), 32 column tiles, the V^T
//           operand read with the transposing ds_read_b64_tr_b16.
// One barrier per tile: it publishes tile it (every wave's copies landed) and retires tile
// it-2, whose buffer then receives the copies of tile it+2.  Between barriers the waves run
// free, so the two waves sharing a SIMD overlap one's softmax arithmetic with the other's
// matrix-core work.
//
// attn_split runs this for tokens j0 .. j1-1 of sequence b with the queries of row bq and
// writes the split's partial of head h to row prow0 + h * hstride of o_part / lse_part;
// every thread of the workgroup calls it with the same arguments.
//
// With FP8 the cache holds fp8 latent rows: each tile is copied raw into a staging buffer
// one tile ahead and, during the previous tile, converted by every wavefront into the bf16
// tile buffer the products read (E4M3 code times its block's power-of-two scale is exact in
// bf16), so the score and PV steps are the bf16 ones.
template <int NW, typename OT, bool FP8 = false>
__device__ __forceinline__ void attn_split(
    const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ cache, const int32_t* __restrict__ block_table, int H,
    int log2P, int max_pages, float scale_log2, OT* __restrict__ o_part,
    float* __restrict__ lse_part, int b, int bq, int j0, int j1, int64_t prow0, int hstride) {
  constexpr int NT = NW * 64;
  constexpr int NCT = DC / 16;                                    // PV column tiles
  constexpr int STEPS = KSTEPS * 2;                               // score MFMA steps per tile
  constexpr int COPIES = FP8 ? (FP8_COPIES + NW - 1) / NW          // tile copies per wave
                             : (TILE_WAVE_COPIES + NW - 1) / NW;
  constexpr int COPY_EVERY = STEPS / COPIES;                      // score steps between copies
  constexpr int NB = FP8 ? FP8_NBUF : NBUF;                       // bf16 tile buffers
  constexpr int PTAB = FP8 ? FP8_PAGE_TABLE : PAGE_TABLE;         // LDS block table
  constexpr int SRC_ROW = FP8 ? FP8_ROW_BYTES : ROW_BYTES;        // cache row bytes
  static_assert(NW == 1 || NW == 2 || NW == 4 || NW == 8, "16 to 128 heads");
  static_assert(KSTEPS == 18, "query loader covers 512 + 64 features");
  static_assert(!FP8 || NW == 8, "fp8 rows: 128 heads");
  __shared__ __attribute__((aligned(16))) char smem[FP8 ? FP8_LDS_BYTES : LDS_BYTES];
  lds_char_t* const lsm = (lds_char_t*)smem;  // 32-bit LDS addressing for the tile reads
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>(lsm));

  // the thread index is made opaque here, so that when this runs in a loop over pieces
  // nothing derived from it is hoisted out of the loop and kept live across the pieces
  int tid_opaque = threadIdx.x;
  asm volatile("" : "+v"(tid_opaque));
  const int tid = tid_opaque, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int P = 1 << log2P;
  const int h0 = 16 * w;   // heads of this wave
  const int32_t* bt_row = block_table + static_cast<int64_t>(b) * max_pages;

  if (j0 >= j1) {  // empty split: o = 0, lse = -inf
    for (int e = tid; e < H * DC; e += NT) {
      const int h = e / DC, c = e % DC;
      st(o_part + (prow0 + static_cast<int64_t>(h) * hstride) * DC + c, 0.f);
    }
    if (lse_part != nullptr)
      for (int h = tid; h < H; h += NT) lse_part[prow0 + static_cast<int64_t>(h) * hstride] = -INFINITY;
    return;
  }

  // resident query fragments: B operand of S^T = K Q^T (lane (g, r16): head h0 + r16,
  // features 32 kk + 8 g .. + 7); loaded after the first tile's copies are issued
  bf16x8_t qf[KSTEPS];

  // Wave w issues copies q = w, w + NW, ... of each tile; lane l of copy q fills LDS chunk
  // 64 q + l, i.e. row t, stored position p, which holds logical chunk p ^ swz(t) of the row.
  // When 36 copies do not split evenly, a wave without a last copy repeats its first (same
  // source, same LDS bytes), so every wave counts COPIES copies per tile.
  const char* cache_bytes = reinterpret_cast<const char*>(cache);
  // A tile starting at token tb lies inside one page (P % 32 == 0, tiles 32-aligned).
  auto tile_page = [&](int tb) { return __builtin_amdgcn_readfirstlane(bt_row[tb >> log2P]); };
  auto page_base = [&](int pg, int tb) {
    return cache_bytes + ((static_cast<int64_t>(pg) << log2P) + (tb & (P - 1))) * SRC_ROW;
  };
  auto tile_base = [&](int tb) { return page_base(tile_page(tb), tb); };
  // source offset of lane l of copy q (LDS chunk 64 q + l); rows past the split's end
  // (t > last) repeat its last valid row
  auto copy_voff = [&](int q, int l, unsigned last) {
    return tile_chunk_voff(64u * q + l, last);
  };
  auto copy_index = [&](int r) { return w + NW * r < TILE_WAVE_COPIES ? w + NW * r : w; };
  // copy r of this wave for the tile at token tb into buffer buf, offsets computed in place
  // (the form that clamps rows at the split's end)
  auto issue_copy = [&](const char* base, int tb, int buf, int r) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recompute the copy coordinates each time (no live ranges)
    const int q = copy_index(r);
    dma16(base, copy_voff(q, ln, static_cast<unsigned>(j1 - 1 - tb)), smem_lds + buf * TILE_BYTES + q * 64 * 16);
  };
  auto issue_tile = [&](int tb, int buf) {
    const char* base = tile_base(tb);
#pragma unroll
    for (int r = 0; r < COPIES; ++r) issue_copy(base, tb, buf, r);
  };
  // fp8 rows: copy r of this wave moves chunks n = 64 q + lane (q = w + NW r, copies past
  // the 21st repeat the 21st: same source, same bytes) of the tile's raw rows, chunk n being
  // row n / 41, bytes 16 (n % 41) .. of it, to staging byte 16 n; the lanes past the tile's
  // 1312 chunks re-read its last chunk into the buffer's tail.  Rows past the split's end
  // repeat its last valid row.
  auto fp8_copy = [&](const char* base, int tb, int stage, int r) {
    const unsigned q = min(static_cast<unsigned>(w + NW * r), static_cast<unsigned>(FP8_COPIES - 1));
    fp8_tile_copy(base, static_cast<unsigned>(j1 - 1 - tb),
                  smem_lds + FP8_STAGE + stage * FP8_STAGE_BYTES, q, lane);
  };
  auto fp8_issue_tile = [&](int tb, int stage) {
    const char* base = tile_base(tb);
#pragma unroll
    for (int r = 0; r < COPIES; ++r) fp8_copy(base, tb, stage, r);
  };
  // Converts the staged raw rows of a tile into bf16 buffer buf (fp8_convert_chunk); thread
  // tid takes chunks tid, tid + NT, ...
  constexpr int CONV = (TILE_CHUNKS + NT - 1) / NT;  // chunks per thread and tile
  auto fp8_convert_chunk_i = [&](int stage, int buf, int i) {
    const int e = tid + NT * i;
    if (TILE_CHUNKS % NT != 0 && e >= TILE_CHUNKS) return;
    fp8_convert_chunk(lsm + FP8_STAGE + stage * FP8_STAGE_BYTES, lsm + buf * TILE_BYTES, e);
  };
  auto fp8_convert = [&](int stage, int buf) {
#pragma unroll
    for (int i = 0; i < CONV; ++i) fp8_convert_chunk_i(stage, buf, i);
  };
  // The copy coordinates do not depend on the tile: the workgroup writes them once to an
  // LDS table, row t << 16 | chunk byte offset, and a copy inside the loop reads its lane's
  // entry there (one LDS read, then clamp and multiply) instead of recomputing them.
  auto table_entry = [&](int r) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return FP8 ? 0u : *((const __attribute__((address_space(3))) uint32_t*)(lsm + VOFF_TABLE) + copy_index(r) * 64 + ln);
  };
  auto entry_voff = [&](uint32_t e, unsigned last) {
    return __umul24(min(e >> 16, last), static_cast<unsigned>(ROW_BYTES)) + (e & 0xffffu);
  };


  const int ntiles = (j1 - j0 + TILE - 1) / TILE;

  // O^T accumulators: o[ct] lane (g, r16) holds O[h0 + r16][16 ct + 4 g + i]
  f32x4_t o[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Reference maximum of head h0 + r16 (log2 units, same in its 4 lanes): the first tile's
  // maximum plus HEADROOM, fixed for the split, so the accumulators are never rescaled.
  // The softmax denominators accumulate on the matrix core as ones (16 x 32) * P^T
  // (32 x 16): every entry of lane (g, r16) holds the sum of head h0 + r16, exactly over the
  // bf16 weights the PV product consumes.
  float m_ref = -INFINITY;
  f32x4_t l_acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, i16x4x2_ones());
  bool out_of_range = false;  // sticky: a score of this head block left the reference range

  // Lane offsets of the K fragments inside a tile buffer, the same for every tile (kept in
  // registers):
  //   kb[mt][par]: the K fragment of k-step par (0 / 1) for M tile mt: row
  //     8 (r16 >> 2) + 4 mt + (r16 & 3), logical chunk 4 par + g; k-step kk adds 128 (kk >> 1);
  int kb[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int t = 8 * (r16 >> 2) + 4 * mt + (r16 & 3);
#pragma unroll
    for (int par = 0; par < 2; ++par) kb[mt][par] = t * ROW_BYTES + 16 * ((4 * par + g) ^ swz(t));
  }

  // Scores and softmax of tile it, returning this wave's P^T operand.  This wave's copies of
  // tile it+2 are spread over the score steps.  Near the end of the split, where there is no
  // tile it+2, the same copies re-fetch tile it (just read, so served by L2) into the retired
  // buffer instead: every score step then issues the same copies and every wait counts
  // alike.
  // the tile whose copies score(it) issues: it+2, or it itself near the end of the split
  auto copy_tile = [&](int it) { return j0 + (it + 2 < ntiles ? it + 2 : min(it, ntiles - 1)) * TILE; };
  // Inside the loop the block-table entries of the split come from an LDS copy: an LDS read
  // keeps the in-order LDS wait counts, where a scalar load (same counter, out of order)
  // would force a full wait in front of the next tile read.
  auto split_page = [&](int tb) {
    return __builtin_amdgcn_readfirstlane(
        ((const __attribute__((address_space(3))) int32_t*)(lsm + PTAB))[(tb - j0) >> log2P]);
  };
  auto score = [&](int it) {
    // The two waves of a SIMD are in different phases; the sequencer favours the older
    // wave, which left the other group behind at every barrier.  Giving the score phase
    // (K reads, softmax arithmetic, copies) the higher issue priority balances them.
    __builtin_amdgcn_s_setprio(1);
    const int tb = j0 + it * TILE;
    const lds_char_t* tile = lsm + (it % NB) * TILE_BYTES;
    const int tb2 = copy_tile(it);
    const bool copy_fp8 = FP8 && it + 2 < ntiles;  // fp8: only real tiles, into staging
    const char* base2 = page_base(split_page(tb2), tb2);
    const unsigned last2 = static_cast<unsigned>(j1 - 1 - tb2);  // rows past it repeat it
    // table reads this many score steps ahead of their copy (0: just before it)
    constexpr int LEAD = COPY_EVERY > 3 ? 3 : COPY_EVERY - 1;
    uint32_t enext = table_entry(0);

    // ---- scores S^T (2 token M-tiles x 16 heads, K = 576).  Row r of M-tile mt is token
    //      8 (r >> 2) + 4 mt + (r & 3), so lane (gg, rr) ends up with tokens 8 gg .. 8 gg + 7
    //      of head h0 + rr: after the softmax, exactly its P^T operand of the PV product.
    //      The 36 K fragments stream through a 4-deep register ring.
    f32x4_t sacc[2];  // one accumulation chain per M tile (dependent MFMAs issue back to back)
    {
      sacc[0] = sacc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      constexpr int KRING = 4;
      auto k_frag = [&](int step) {
        const int kk = step >> 1, mt = step & 1;
        return *(const lds_bf16x8_t*)(tile + kb[mt][kk & 1] + (kk >> 1) * 128);
      };
      bf16x8_t ka[KRING];
#pragma unroll
      for (int i = 0; i < KRING - 1; ++i) ka[i] = k_frag(i);
#pragma unroll
      for (int step = 0; step < STEPS; ++step) {
        if (step + KRING - 1 < STEPS) ka[(step + KRING - 1) % KRING] = k_frag(step + KRING - 1);
        const int kk = step >> 1, mt = step & 1;
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[step % KRING], qf[kk], sacc[mt], 0, 0, 0);
        if (LEAD == 0 && step > 0 && step % COPY_EVERY == 0 && step / COPY_EVERY < COPIES)
          enext = table_entry(step / COPY_EVERY);
        if constexpr (FP8) {
          if (copy_fp8 && step % COPY_EVERY == 0 && step / COPY_EVERY < COPIES)
            fp8_copy(base2, tb2, (it + 2) & 1, step / COPY_EVERY);
        } else if (step % COPY_EVERY == 0 && step / COPY_EVERY < COPIES) {
          dma16(base2, entry_voff(enext, last2),
                smem_lds + ((it + 2) % NB) * TILE_BYTES + copy_index(step / COPY_EVERY) * 64 * 16);
        }
        if (LEAD > 0 && step + LEAD >= COPY_EVERY && (step + LEAD) % COPY_EVERY == 0 &&
            (step + LEAD) / COPY_EVERY < COPIES)
          enext = table_entry((step + LEAD) / COPY_EVERY);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- softmax (log2 domain) on the raw scores: lane holds head h0 + rr, tokens
    //      8 gg + 4 mt + i.  The scale is positive, so the raw maximum orders like the
    //      scaled one; each weight is 2^(s * scale - m_ref) with one rounding in the fma.
    f32x4_t sc[2] = {sacc[0], sacc[1]};
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
    const float neg_m = -m_ref;
    float e[2][4];  // exponents s * scale - m_ref
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) e[mt][i] = __builtin_fmaf(sc[mt][i], scale_log2, neg_m);
    // a weight above 2^P_RANGE leaves the reference range
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
    l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pt, l_acc, 0, 0, 0);
    return pt;
  };

  // PV of tile it with this wave's P^T operand pt.
  auto pv = [&](int it, bf16x8_t pt) {
    __builtin_amdgcn_s_setprio(0);
    const lds_char_t* tile = lsm + (it % NB) * TILE_BYTES;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per tile (no long live ranges)
    const int gg = ln >> 4, rr = ln & 15;
    // ---- V^T fragments (A operand): lane (gg, rr) holds column 16 ct + rr, tokens
    //      8 gg .. 8 gg + 7, gathered by two transposing reads of 4 rows each.  Column tile ct
    //      sits in chunks 2 ct, 2 ct + 1; with the row swizzle only the low three chunk bits
    //      move, so 8 lane offsets (read r, ct & 3) plus the immediate 128 (ct >> 2) cover all.
    {
      int vb[2][4];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int t = 8 * gg + 4 * r + (rr >> 2);
        const int e = (rr & 3) >> 1;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          vb[r][c4] = t * ROW_BYTES + 16 * ((2 * c4 + e) ^ swz(t)) + 8 * (rr & 1);
      }
      auto v_frag = [&](int ct) {
        i16x4_t half[2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(tile + vb[r][ct & 3] + 128 * (ct >> 2)));
        return __builtin_bit_cast(bf16x8_t,
                                  __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int VRING = 4;
      bf16x8_t va[VRING];
#pragma unroll
      for (int i = 0; i < VRING - 1; ++i) va[i] = v_frag(i);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if (ct + VRING - 1 < NCT) va[(ct + VRING - 1) % VRING] = v_frag(ct + VRING - 1);
        o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ct % VRING], pt, o[ct], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // The 18 query fragments of this wave in one assembly block that also waits for them
  // (and, being issued after them, for this wave's copies of the first tile), so the two
  // latencies overlap and no compiler-inserted wait falls after a later copy.
  auto load_query = [&]() {
    const bf16raw* qrow = q_lat + (static_cast<int64_t>(bq) * H + h0 + r16) * DC + 8 * g;
    const bf16raw* prow = q_pe + (static_cast<int64_t>(bq) * H + h0 + r16) * DR + 8 * g;
    i32x4_t r[KSTEPS];
    asm volatile("global_load_dwordx4 %0, %18, off\n\tglobal_load_dwordx4 %1, %18, off offset:64\n\tglobal_load_dwordx4 %2, %18, off offset:128\n\tglobal_load_dwordx4 %3, %18, off offset:192\n\tglobal_load_dwordx4 %4, %18, off offset:256\n\tglobal_load_dwordx4 %5, %18, off offset:320\n\tglobal_load_dwordx4 %6, %18, off offset:384\n\tglobal_load_dwordx4 %7, %18, off offset:448\n\tglobal_load_dwordx4 %8, %18, off offset:512\n\tglobal_load_dwordx4 %9, %18, off offset:576\n\tglobal_load_dwordx4 %10, %18, off offset:640\n\tglobal_load_dwordx4 %11, %18, off offset:704\n\tglobal_load_dwordx4 %12, %18, off offset:768\n\tglobal_load_dwordx4 %13, %18, off offset:832\n\tglobal_load_dwordx4 %14, %18, off offset:896\n\tglobal_load_dwordx4 %15, %18, off offset:960\n\tglobal_load_dwordx4 %16, %19, off\n\tglobal_load_dwordx4 %17, %19, off offset:64\n\ts_waitcnt vmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15]), "=&v"(r[16]), "=&v"(r[17])
                 : "v"(qrow), "v"(prow)
                 : "memory");
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = __builtin_bit_cast(bf16x8_t, r[kk]);
  };
  // With eight wavefronts (five copies per tile and wave) the copies of the second tile
  // join the same block, issued after the query loads, and the block waits for everything
  // but them: two tiles are then in flight while the queries arrive.  A one-tile split
  // copies its tile again into the unused second buffer, so the wait counts stay alike.
  auto load_query_tile1 = [&]() {
    const bf16raw* qrow = q_lat + (static_cast<int64_t>(bq) * H + h0 + r16) * DC + 8 * g;
    const bf16raw* prow = q_pe + (static_cast<int64_t>(bq) * H + h0 + r16) * DR + 8 * g;
    const int tb1 = ntiles > 1 ? j0 + TILE : j0;
    const unsigned last1 = static_cast<unsigned>(j1 - 1 - tb1);
    const uint64_t b64 = reinterpret_cast<uint64_t>(tile_base(tb1));
    const uint32_t blo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64));
    const uint32_t bhi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64 >> 32));
    const void* base1 = reinterpret_cast<const void*>((static_cast<uint64_t>(bhi) << 32) | blo);
    uint32_t vo[5], la[5];  // called with COPIES == 5 only
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      vo[c] = copy_voff(copy_index(c), lane, last1);
      la[c] = __builtin_amdgcn_readfirstlane(smem_lds + TILE_BYTES + copy_index(c) * 64 * 16);
    }
    i32x4_t r[KSTEPS];
    asm volatile("global_load_dwordx4 %0, %18, off\n\tglobal_load_dwordx4 %1, %18, off offset:64\n\tglobal_load_dwordx4 %2, %18, off offset:128\n\tglobal_load_dwordx4 %3, %18, off offset:192\n\tglobal_load_dwordx4 %4, %18, off offset:256\n\tglobal_load_dwordx4 %5, %18, off offset:320\n\tglobal_load_dwordx4 %6, %18, off offset:384\n\tglobal_load_dwordx4 %7, %18, off offset:448\n\tglobal_load_dwordx4 %8, %18, off offset:512\n\tglobal_load_dwordx4 %9, %18, off offset:576\n\tglobal_load_dwordx4 %10, %18, off offset:640\n\tglobal_load_dwordx4 %11, %18, off offset:704\n\tglobal_load_dwordx4 %12, %18, off offset:768\n\tglobal_load_dwordx4 %13, %18, off offset:832\n\tglobal_load_dwordx4 %14, %18, off offset:896\n\tglobal_load_dwordx4 %15, %18, off offset:960\n\tglobal_load_dwordx4 %16, %19, off\n\tglobal_load_dwordx4 %17, %19, off offset:64\n\t"
                 "s_mov_b32 m0, %25\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %20, %30\n\t"
                 "s_mov_b32 m0, %26\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %21, %30\n\t"
                 "s_mov_b32 m0, %27\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %22, %30\n\t"
                 "s_mov_b32 m0, %28\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %23, %30\n\t"
                 "s_mov_b32 m0, %29\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %24, %30\n\t"
                 "s_waitcnt vmcnt(5)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15]), "=&v"(r[16]), "=&v"(r[17])
                 : "v"(qrow), "v"(prow), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]),
                   "s"(la[0]), "s"(la[1]), "s"(la[2]), "s"(la[3]), "s"(la[4]), "s"(base1)
                 : "memory", "m0");
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = __builtin_bit_cast(bf16x8_t, r[kk]);
  };
  if constexpr (FP8) {
    // raw tiles 0 and 1 into the two staging buffers, the block table, the queries (whose
    // wait covers the copies too); then tile 0 converted before barrier 0
    fp8_issue_tile(j0, 0);
    if (ntiles > 1) fp8_issue_tile(j0 + TILE, 1);
    for (int e = tid; e * P < j1 - j0; e += NT)  // the pages this split reads
      ((__attribute__((address_space(3))) int32_t*)(lsm + PTAB))[e] = bt_row[(j0 >> log2P) + e];
    load_query();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
    fp8_convert(0, 0);
  } else {
    issue_tile(j0, 0);
    for (int e = tid; e < TILE_WAVE_COPIES * 64; e += NT) {
      const unsigned chunk = static_cast<unsigned>(e);
      const unsigned t = chunk / CHUNKS, c = (chunk % CHUNKS) ^ swz(t);
      ((__attribute__((address_space(3))) uint32_t*)(lsm + VOFF_TABLE))[e] = (t << 16) | (c * 16);
    }
    for (int e = tid; e * P < j1 - j0; e += NT)  // the pages this split reads
      ((__attribute__((address_space(3))) int32_t*)(lsm + PTAB))[e] = bt_row[(j0 >> log2P) + e];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // table written before barrier 0
    if constexpr (COPIES == 5) {
      load_query_tile1();
    } else {
      load_query();
      if (ntiles > 1) issue_tile(j0 + TILE, 1);
    }
  }
  // Waves 0 .. NW/2-1 (group 0) take each tile as scores then PV; waves NW/2 .. NW-1
  // (group 1) run half a tile behind, as PV of the previous tile then scores.  A SIMD holds
  // one wave of each group, so while one scores (K reads, softmax arithmetic) the other feeds
  // the matrix core with its PV product.  Barrier it (before the work on tile it) publishes
  // tile it, copied by every wave, and retires tile it-2, whose buffer the copies of tile it+2
  // overwrite; both groups pass ntiles + 1 barriers.
  auto tile_barrier = [&](int it) {
    if constexpr (FP8) {
      // the raw tile it+1 (copied during tile it-1) has landed, and the conversion of tile
      // it (during tile it-1) is in LDS: barrier it publishes both; then this wave converts
      // its share of tile it+1 (spread over the score steps instead, it costs spills inside
      // the loop and runs slower)
      wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      block_barrier();
      if (it + 1 < ntiles) fp8_convert((it + 1) & 1, (it + 1) % NB);
    } else {
      if (it < ntiles) wait_vmcnt<COPIES>();  // own copies of tile it landed
      else wait_vmcnt<0>();                   // no copy may still be writing LDS at the end
      block_barrier();
    }
  };
  if (NW == 1 || w < NW / 2) {
    for (int it = 0; it < ntiles; ++it) {
      tile_barrier(it);
      const bf16x8_t pt = score(it);
      pv(it, pt);
    }
    tile_barrier(ntiles);
  } else {
    tile_barrier(0);
    bf16x8_t pt = score(0);
    for (int it = 1; it < ntiles; ++it) {
      tile_barrier(it);
      pv(it - 1, pt);
      pt = score(it);
    }
    tile_barrier(ntiles);
    pv(ntiles - 1, pt);
  }

  // ---- epilogue: normalise and write four consecutive columns per lane; a head block
  //      whose scores left the reference range is recomputed exactly
  if (!__any(out_of_range)) {
    const int64_t row = prow0 + static_cast<int64_t>(h0 + r16) * hstride;
    if (lse_part != nullptr && g == 0) lse_part[row] = (m_ref + __log2f(l_acc[0])) * LN2;
    const float inv = 1.f / l_acc[0];
    if constexpr (std::is_same<OT, float>::value) {
      float* dst = o_part + row * DC + 4 * g;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) *reinterpret_cast<f32x4_t*>(dst + 16 * ct) = o[ct] * inv;
    } else {
      // bf16 (round to nearest even), 16 bytes per lane and store: for column tiles 2m and
      // 2m + 1 a lane pair (g, g ^ 1) trades halves, so even g writes columns
      // 32 m + 4 g .. + 7 and odd g writes 32 m + 4 g + 12 .. + 7 (half the store
      // instructions of four-column stores)
      const bool odd = (g & 1) != 0;
      bf16raw* dst = o_part + row * DC + 4 * g + (odd ? 12 : 0);
#pragma unroll
      for (int m = 0; m < NCT / 2; ++m) {
        const f32x4_t a = o[2 * m] * inv, c = o[2 * m + 1] * inv;
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
  } else {
    split_exact_fallback<OT, FP8>(q_lat, q_pe, cache, bt_row, log2P, j0, j1, bq, H, prow0,
                                  hstride, scale_log2, o_part, lse_part, h0, 16, lane);
  }
}

// One workgroup per (sequence, split) (blockIdx.x, blockIdx.y), and per query token
// (blockIdx.z) when n_q > 1.  Consecutive workgroup ids go to the 8 XCDs in turn; with the
// sequence index in x, all splits of a sequence (ids b, b + B, ...) land on XCD b % 8 when
// B % 8 == 0, so the sequence's queries are fetched once into that XCD's L2.  Token t of n_q
// sits at position seq_len - n_q + t and sees the cache up to it; its queries and outputs are
// row bq = b n_q + t, and its workgroups share the sequence's XCD and read the same tiles.
template <int NW, typename OT, bool FP8 = false>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(
    const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int H, int log2P, int max_pages, int pages_per_split,
    int S, float scale_log2, OT* __restrict__ o_part, float* __restrict__ lse_part, int n_q,
    int* __restrict__ merge_cnt, int* __restrict__ merge_err, float* __restrict__ out,
    float* __restrict__ lse_out) {
  const int b = blockIdx.x, s = blockIdx.y, bq = b * n_q + blockIdx.z;
  const int L = seq_lens[b] - (n_q - 1 - static_cast<int>(blockIdx.z));
  const int j0 = s * (pages_per_split << log2P);
  const int j1 = min(L, j0 + (pages_per_split << log2P));
  attn_split<NW, OT, FP8>(q_lat, q_pe, cache, block_table, H, log2P, max_pages, scale_log2,
                          o_part, lse_part, b, bq, j0, j1, static_cast<int64_t>(bq) * H * S + s, S);
  if (merge_cnt != nullptr)
    merge_splits<NW>(o_part, lse_part, H, S, s, bq, merge_cnt, merge_err, out, lse_out,
                     static_cast<int>(threadIdx.x));
}

template <int NW, typename OT>
__global__ __launch_bounds__(NW * 64) void attn_mfma_ragged_kernel(
    const bf16raw* __restrict__ q_lat, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int B, int H, int log2P, int max_pages,
    float scale_log2, OT* __restrict__ o_part, float* __restrict__ lse_part,
    int* __restrict__ seq_slots, int* __restrict__ err) {
  int W = 0, tot = 0;
  if (ragged::plan_ranges(seq_lens, B, log2P, MAX_SPLIT_PAGES, seq_slots, err, W, tot)) return;
  // The plan's scalars wait in LDS between pieces: kept in registers across the split body
  // they push it over the register file (scratch spills inside the tile loop).
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
    // The previous piece's partial stores leave the vector-memory counter (the prologue's
    // explicit waits count only its own loads and copies), and its last LDS reads are done
    // before this piece's copies overwrite the buffers.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    attn_split<NW, OT>(q_lat, q_pe, cache, block_table, H, log2P, max_pages, scale_log2,
                       o_part, lse_part, pc.b, pc.b, pc.j0, pc.j1,
                       static_cast<int64_t>(pc.first) * H + pc.index, pc.count);
  }
}

template <int NW, typename OT>
hipError_t launch_ragged_nw_t(const PagedArgs& a, int grid, int* seq_slots, int* err,
                              hipStream_t st) {
  const float log2e = 1.4426950408889634f;
  hipLaunchKernelGGL((attn_mfma_ragged_kernel<NW, OT>), dim3(grid), dim3(NW * 64), 0, st,
                     static_cast<const bf16raw*>(a.q_lat), static_cast<const bf16raw*>(a.q_pe),
                     static_cast<const bf16raw*>(a.cache), a.block_table, a.seq_lens, a.B, a.H,
                     __builtin_ctz(static_cast<unsigned>(a.page_size)), a.max_pages,
                     a.scale * log2e, static_cast<OT*>(a.o_part), a.lse_part, seq_slots, err);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_ragged_nw(const PagedArgs& a, int grid, int* seq_slots, int* err,
                            hipStream_t st) {
  return a.part_bf16 ? launch_ragged_nw_t<NW, bf16raw>(a, grid, seq_slots, err, st)
                     : launch_ragged_nw_t<NW, float>(a, grid, seq_slots, err, st);
}

template <int NW, typename OT, bool FP8 = false>
hipError_t launch_nw_t(const PagedArgs& a, hipStream_t st) {
  const float log2e = 1.4426950408889634f;
  hipLaunchKernelGGL((attn_mfma_kernel<NW, OT, FP8>), dim3(a.B, a.num_splits, a.n_q), dim3(NW * 64), 0, st,
                     static_cast<const bf16raw*>(a.q_lat), static_cast<const bf16raw*>(a.q_pe),
                     static_cast<const bf16raw*>(a.cache), a.block_table, a.seq_lens, a.H,
                     __builtin_ctz(static_cast<unsigned>(a.page_size)), a.max_pages,
                     a.pages_per_split, a.num_splits, a.scale * log2e,
                     static_cast<OT*>(a.o_part), a.lse_part, a.n_q, a.merge_cnt,
                     a.merge_cnt != nullptr ? a.merge_cnt + 2 * a.B * a.n_q : nullptr, a.out,
                     a.lse_out);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_nw(const PagedArgs& a, hipStream_t st) {
  return a.part_bf16 ? launch_nw_t<NW, bf16raw>(a, st) : launch_nw_t<NW, float>(a, st);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool attn_mfma_supported(const PagedArgs& a) {
  const bool heads_ok = a.H == 16 || a.H == 32 || a.H == 64 || a.H == 128;
  if (a.pages_per_split > MAX_SPLIT_PAGES) return false;
  const bool page_ok = a.page_size >= TILE && (a.page_size & (a.page_size - 1)) == 0;
  return a.d_c == DC && a.d_R == DR && heads_ok && page_ok &&
         a.B <= 65535 && a.n_q >= 1 && a.n_q <= 65535 && aligned16(a.q_lat) &&
         aligned16(a.q_pe) && aligned16(a.cache);
}

bool attn_mfma_grid_resident(const PagedArgs& a) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  hipError_t e = hipErrorInvalidValue;
  switch (a.H) {
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_kernel<1, float>, 64, 0); break;
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_kernel<2, float>, 128, 0); break;
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_kernel<4, float>, 256, 0); break;
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_kernel<8, float>, 512, 0); break;
    default: break;
  }
  if (e != hipSuccess) return false;
  return static_cast<int64_t>(a.B) * a.num_splits * a.n_q <= static_cast<int64_t>(cus) * per_cu;
}

int attn_mfma_ragged_max_range_pages() { return MAX_SPLIT_PAGES; }

hipError_t launch_attn_mfma_ragged(const PagedArgs& a, int grid, int* seq_slots, int* err,
                                   hipStream_t s) {
  switch (a.H) {
    case 16: return launch_ragged_nw<1>(a, grid, seq_slots, err, s);
    case 32: return launch_ragged_nw<2>(a, grid, seq_slots, err, s);
    case 64: return launch_ragged_nw<4>(a, grid, seq_slots, err, s);
    case 128: return launch_ragged_nw<8>(a, grid, seq_slots, err, s);
    default: return hipErrorInvalidValue;
  }
}

bool attn_mfma_fp8_supported(const PagedArgs& a) { return a.H == 128 && attn_mfma_supported(a); }

hipError_t launch_attn_mfma_fp8(const PagedArgs& a, hipStream_t s) {
  if (a.H != 128) return hipErrorInvalidValue;
  return a.part_bf16 ? launch_nw_t<8, bf16raw, true>(a, s) : launch_nw_t<8, float, true>(a, s);
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

