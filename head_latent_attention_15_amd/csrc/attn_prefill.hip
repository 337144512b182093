// Prefill attention in the expanded form: a prompt of T tokens per sequence attends
// causally to itself through the up-projected keys and values.
//
// For many query tokens the pages give the naive order, keys and values up-projected once
// per prompt ([perforder] "極限最適化の代償：MLA特有の学習負荷と独自Tritonカーネルという障壁"
// on the prefill cost; kasblo.com/?p=4663, "「キャッシュを減らせた」と「その割合だけ速い」は
// 別の評価"): with k^C_{j,i} = W^UK_i c_j and v^C_{j,i} = W^UV_i c_j (two GEMMs over the
// prompt, mla_linear), head i of query t computes
//   s_tj = scale [q^C_{t,i}; q_pe_{t,i}] . [k^C_{j,i}; k^R_j]   for j <= t (192-wide)
//   o_{t,i} = sum_j softmax_j(s_tj) v^C_{j,i}                      (128-wide)
// ("論文解説: DeepSeek-V2 …", "Decoupled RoPE": the rotated k^R is shared by the heads;
// qiita.com/joule "Attention 計算": the sum runs to the query's own position).
//
// One workgroup of 8 wavefronts per (sequence, head, block of 256 queries), wavefront w
// owning queries 32 w .. 32 w + 31 of the block as two 16-query tiles.  Keys go through LDS
// in 64-key blocks, one 640-byte row per key [k^C_i (128) | k^R (64) | v^C_i (128)] with the
// 16-byte-chunk XOR swizzle of the decode tiles (a row stride of 128 mod 256 bytes, as
// there), so the row-strided K reads and the transposing V reads are conflict-free.  Per
// key block a wave computes S^T = K Q^T (tokens as the MFMA M dimension, 4 key tiles x 6
// k-steps x 2 query tiles = 48 MFMAs, each K fragment feeding both query tiles, Q resident
// in VGPRs; the key permutation inside each 32-key half makes the C layout of S^T the B
// layout of P^T), an online softmax per query (running maximum, accumulators rescaled when
// it moves), and O^T += V^T P^T (32 MFMAs, each V^T fragment feeding both query tiles).
// Blocks are staged with plain global loads double-buffered through registers.  Workgroups
// of late query blocks (the most keys) are numbered first.
#include "attn_common.h"
#include "launchers.h"

namespace mla {
namespace {

using namespace attn;

constexpr int PF_DH = 128, PF_DR = 64, PF_DQK = PF_DH + PF_DR;  // 192
constexpr int PF_ROW = (PF_DQK + PF_DH) * 2;                     // 640 bytes: k^C | k^R | v^C
constexpr int PF_ROW_CHUNKS = PF_ROW / 16;                       // 40
constexpr int PF_KB = 64;                                        // keys per block
constexpr int PF_TILE = PF_KB * PF_ROW;                          // 40960 bytes
constexpr int PF_CHUNKS = PF_KB * PF_ROW_CHUNKS;                 // 2560
constexpr int PF_NW = 8, PF_NT = PF_NW * 64;
constexpr int PF_QT = 2;                                         // 16-query tiles per wave
constexpr int PF_QB = 16 * PF_QT * PF_NW;                        // 256 queries per workgroup
constexpr int PF_LOADS = (PF_CHUNKS + PF_NT - 1) / PF_NT;        // 5 chunks per thread
constexpr int PF_KSTEPS = PF_DQK / 32;                           // 6
constexpr int PF_MT = PF_KB / 16;                                // 4 key M tiles
constexpr int PF_CT = PF_DH / 16;                                // 8 value column tiles

__global__ __launch_bounds__(PF_NT) void attn_prefill_kernel(
    const bf16raw* __restrict__ q_c, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ k_c, const bf16raw* __restrict__ k_pe,
    const bf16raw* __restrict__ v_c, int T, int H, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) char smem[2 * PF_TILE];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const int nqb = (T + PF_QB - 1) / PF_QB;
  // heads in x: the first workgroups are the last query blocks (the most keys) of every
  // head, so the longest work starts first
  const int qb = nqb - 1 - static_cast<int>(blockIdx.y);
  const int h = blockIdx.x, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int q0 = qb * PF_QB;                         // first query of the workgroup
  const int qw = q0 + 16 * PF_QT * w;                // first query of this wave
  const int q_last = min(q0 + PF_QB, T) - 1;         // last query of the workgroup
  const int nkb = q_last / PF_KB + 1;                // key blocks the workgroup needs
  const int64_t tok0 = static_cast<int64_t>(b) * T;  // first token row of the sequence

  // ---- query fragments (B operand of S^T = K Q^T): query tile qt, lane (g, r16) holds query
  //      qw + 16 qt + r16, features 32 kk + 8 g .. + 7 (kk < 4: q^C, else q_pe); queries
  //      past T repeat T - 1
  bf16x8_t qf[PF_QT][PF_KSTEPS];
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    const int q = min(qw + 16 * qt + r16, T - 1);
    const bf16raw* qc = q_c + ((tok0 + q) * H + h) * PF_DH + 8 * g;
    const bf16raw* qp = q_pe + ((tok0 + q) * H + h) * PF_DR + 8 * g;
#pragma unroll
    for (int kk = 0; kk < PF_KSTEPS; ++kk)
      qf[qt][kk] = *reinterpret_cast<const bf16x8_t*>(kk < 4 ? qc + 32 * kk : qp + 32 * (kk - 4));
  }

  // ---- staging: thread tid moves LDS chunks e = tid + 512 i (i < 5) of a block: row
  //      t = e / 40 (key kb*64 + t, keys past T repeat T - 1), stored position p = e % 40
  //      holding logical chunk c = p ^ swz(t): c < 16 k^C, c < 24 k^R, else v^C
  auto chunk_src = [&](int kb, int e) -> const bf16raw* {
    const int t = e / PF_ROW_CHUNKS, p = e - t * PF_ROW_CHUNKS;
    const int c = p ^ swz(t & 31);
    const int64_t key = tok0 + min(kb * PF_KB + t, T - 1);
    if (c < 16) return k_c + (key * H + h) * PF_DH + 8 * c;
    if (c < 24) return k_pe + key * PF_DR + 8 * (c - 16);
    return v_c + (key * H + h) * PF_DH + 8 * (c - 24);
  };
  i32x4_t stage[PF_LOADS];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int i = 0; i < PF_LOADS; ++i) {
      const int e = tid + PF_NT * i;
      if (e < PF_CHUNKS) stage[i] = *reinterpret_cast<const i32x4_t*>(chunk_src(kb, e));
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PF_LOADS; ++i) {
      const int e = tid + PF_NT * i;
      if (e < PF_CHUNKS) *(__attribute__((address_space(3))) i32x4_t*)(lsm + buf * PF_TILE + 16 * e) = stage[i];
    }
  };

  // K fragments: row r of key M tile mt is key 32 (mt >> 1) + 8 (r >> 2) + 4 (mt & 1) + (r & 3),
  // logical chunk 4 par + g (k-step kk adds 128 (kk >> 1)); the 32-key halves repeat the
  // decode tile's rows (the swizzle period is 32 rows), so half (mt >> 1) adds 32 rows.
  // V^T fragments: key half ks, rows 32 ks + 8 gg + 4 r + (rr >> 2), chunks 24 + 2 ct (+1).
  int kb_off[2][2];
#pragma unroll
  for (int m1 = 0; m1 < 2; ++m1) {
    const int t = 8 * (r16 >> 2) + 4 * m1 + (r16 & 3);
#pragma unroll
    for (int par = 0; par < 2; ++par) kb_off[m1][par] = t * PF_ROW + 16 * ((4 * par + g) ^ swz(t));
  }
  int vb[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 8 * g + 4 * r + (r16 >> 2);
    const int e = (r16 & 3) >> 1;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) vb[r][c4] = t * PF_ROW + 16 * ((2 * c4 + e) ^ swz(t)) + 8 * (r16 & 1);
  }

  f32x4_t o[PF_QT][PF_CT];
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt)
#pragma unroll
    for (int ct = 0; ct < PF_CT; ++ct) o[qt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[PF_QT], l_run[PF_QT];  // of query qw + 16 qt + r16, alike in its four lanes
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }

  load_block(0);
  store_block(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) load_block(kb + 1);  // in flight while this block is consumed
    const lds_char_t* tile = lsm + (kb & 1) * PF_TILE;
    if (kb * PF_KB <= qw + 16 * PF_QT - 1) {  // this wave's queries see some key of the block
      // ---- S^T (64 keys x 16 queries per query tile): each K fragment feeds both tiles
      f32x4_t sacc[PF_QT][PF_MT];
#pragma unroll
      for (int qt = 0; qt < PF_QT; ++qt)
#pragma unroll
        for (int mt = 0; mt < PF_MT; ++mt) sacc[qt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < PF_KSTEPS; ++kk)
#pragma unroll
        for (int mt = 0; mt < PF_MT; ++mt) {
          const bf16x8_t kf = *(const lds_bf16x8_t*)(tile + (mt >> 1) * 32 * PF_ROW +
                                                     kb_off[mt & 1][kk & 1] + (kk >> 1) * 128);
#pragma unroll
          for (int qt = 0; qt < PF_QT; ++qt)
            sacc[qt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qt][kk], sacc[qt][mt], 0, 0, 0);
        }
      // ---- online softmax (log2 domain) per query tile: lane (g, r16) holds keys
      //      32 (mt >> 1) + 8 g + 4 (mt & 1) + i of its query; keys after it get weight 0
      bf16x8_t pt[PF_QT][2];  // P^T operands of the two 32-key halves
      const bool diagonal = kb * PF_KB + PF_KB - 1 > qw;  // some key after some query
#pragma unroll
      for (int qt = 0; qt < PF_QT; ++qt) {
        const int my_q = qw + 16 * qt + r16;
        float bmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < PF_MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[qt][mt][i] *= scale_log2;
        if (diagonal) {
#pragma unroll
          for (int mt = 0; mt < PF_MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kb * PF_KB + 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
              if (key > my_q) sacc[qt][mt][i] = -INFINITY;
            }
        }
#pragma unroll
        for (int mt = 0; mt < PF_MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, sacc[qt][mt][i]);
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const float m_new = fmaxf(m_run[qt], bmax);  // finite: key 0 is seen by every query
        const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
        float psum = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x2_t pp[4];
#pragma unroll
          for (int m1 = 0; m1 < 2; ++m1)
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
              const f32x4_t& sv = sacc[qt][2 * ks + m1];
              pp[2 * m1 + hlf] = to_bf16x2(__builtin_amdgcn_exp2f(sv[2 * hlf] - m_new),
                                           __builtin_amdgcn_exp2f(sv[2 * hlf + 1] - m_new));
              psum += static_cast<float>(pp[2 * m1 + hlf][0]) + static_cast<float>(pp[2 * m1 + hlf][1]);
            }
          pt[qt][ks] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                               __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run[qt] = l_run[qt] * alpha + psum;
        m_run[qt] = m_new;
        if (__any(alpha != 1.f)) {  // the running maximum moved for some query
#pragma unroll
          for (int ct = 0; ct < PF_CT; ++ct) o[qt][ct] *= alpha;
        }
      }
      // ---- O^T (128 x 16) += V^T (128 x 32) P^T (32 x 16) per key half and query tile; each
      //      V^T fragment feeds both query tiles
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < PF_CT; ++ct) {
          i16x4_t half[2];
#pragma unroll
          for (int r = 0; r < 2; ++r)
            half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(tile + ks * 32 * PF_ROW + vb[r][ct & 3] + 128 * (3 + (ct >> 2))));
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qt = 0; qt < PF_QT; ++qt)
            o[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pt[qt][ks], o[qt][ct], 0, 0, 0);
        }
    }
    if (kb + 1 < nkb) {
      // buffer (kb + 1) & 1 was last read in block kb - 1, before the previous barrier
      store_block((kb + 1) & 1);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __syncthreads();  // publishes block kb + 1; every wave is past its reads of block kb
    }
  }

  // ---- epilogue: lane (g, r16) holds dims 16 ct + 4 g .. + 3 of its query in each tile
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    const int my_q = qw + 16 * qt + r16;
    if (my_q < T) {
      const float inv = 1.f / l_run[qt];
      float* dst = out + ((tok0 + my_q) * H + h) * PF_DH + 4 * g;
#pragma unroll
      for (int ct = 0; ct < PF_CT; ++ct) *reinterpret_cast<f32x4_t*>(dst + 16 * ct) = o[qt][ct] * inv;
      if (lse_out != nullptr && g == 0)
        lse_out[(tok0 + my_q) * H + h] = (m_run[qt] + __log2f(l_run[qt])) * LN2;
    }
  }
}

}  // namespace

bool attn_prefill_supported(int d_h, int d_R) { return d_h == PF_DH && d_R == PF_DR; }

hipError_t launch_attn_prefill(const void* q_c, const void* q_pe, const void* k_c,
                               const void* k_pe, const void* v_c, int B, int T, int H,
                               float scale, float* out, float* lse_out, hipStream_t s) {
  const float log2e = 1.4426950408889634f;
  const dim3 grid(H, (T + PF_QB - 1) / PF_QB, B);
  hipLaunchKernelGGL(attn_prefill_kernel, grid, dim3(PF_NT), 0, s,
                     static_cast<const bf16raw*>(q_c), static_cast<const bf16raw*>(q_pe),
                     static_cast<const bf16raw*>(k_c), static_cast<const bf16raw*>(k_pe),
                     static_cast<const bf16raw*>(v_c), T, H, scale * log2e, out, lse_out);
  return hipGetLastError();
}

}  // namespace mla
