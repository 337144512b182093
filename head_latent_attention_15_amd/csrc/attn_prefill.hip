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
// in 64-key blocks of three regions, one per source tensor: k^C_i rows (256 bytes), k^R rows
// (128 bytes) and v^C_i rows (256 bytes), each row's 16-byte chunks XOR-permuted by its row
// index so that the row-strided K reads and the transposing V reads are conflict-free.  The
// regions are filled by LDS-DMA copies (1 KB of consecutive LDS per wave-wide copy, the
// permutation carried by the per-lane source addresses) into three buffers, two blocks
// ahead of their use, so one barrier per block both publishes block kb+1 and retires block
// kb.  Per key block a wave computes S^T = K Q^T (tokens as the MFMA M dimension, 4 key
// tiles x 6 k-steps x 2 query tiles = 48 MFMAs, each K fragment feeding both query tiles,
// Q resident in VGPRs; the key permutation inside each 32-key half makes the C layout of
// S^T the B layout of P^T), an online softmax per query (a reference that moves with the
// running maximum when that passes it by a set margin, accumulators rescaled then), and
// O^T += V^T P^T (32 MFMAs, each V^T fragment feeding both query tiles).  Workgroups of late query blocks (the most keys) are numbered first.
#include "attn_common.h"
#include "launchers.h"

namespace mla {
namespace {

using namespace attn;

constexpr int PF_DH = 128, PF_DR = 64, PF_DQK = PF_DH + PF_DR;  // 192
constexpr int PF_KB = 64;                                        // keys per block
constexpr int PF_KC = 0;                                         // k^C region: 64 rows x 256 B
constexpr int PF_KR = PF_KC + PF_KB * PF_DH * 2;                 // k^R region: 64 rows x 128 B
constexpr int PF_V = PF_KR + PF_KB * PF_DR * 2;                  // v^C region: 64 rows x 256 B
constexpr int PF_TILE = PF_V + PF_KB * PF_DH * 2;                // 40960 bytes per block
constexpr int PF_NBUF = 3;
constexpr int PF_NW = 8, PF_NT = PF_NW * 64;
constexpr int PF_QT = 2;                                         // 16-query tiles per wave
constexpr int PF_QB = 16 * PF_QT * PF_NW;                        // 256 queries per workgroup
constexpr int PF_COPIES = PF_TILE / 1024 / PF_NW;                // 5 wave-wide copies per block
static_assert(PF_COPIES * PF_NW * 1024 == PF_TILE, "copies split evenly over the waves");
constexpr int PF_KSTEPS = PF_DQK / 32;                           // 6
constexpr float PF_SLACK = 8.0f;  // log2 units a block maximum may exceed the reference by
constexpr int PF_MT = PF_KB / 16;                                // 4 key M tiles
constexpr int PF_CT = PF_DH / 16;                                // 8 value column tiles

__global__ __launch_bounds__(PF_NT) void attn_prefill_kernel(
    const bf16raw* __restrict__ q_c, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ k_c, const bf16raw* __restrict__ k_pe,
    const bf16raw* __restrict__ v_c, int T, int H, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) char smem[PF_NBUF * PF_TILE];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>(lsm));
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

  // ---- staging.  Row t of a block is key kb*64 + t (keys past T repeat T - 1); stored
  //      position p of a row holds logical chunk p ^ f(t):
  //        k^C (16 chunks): fk(t) = (t & 3) | ((t >> 3) & 3) << 2
  //        k^R (8 chunks):  fr(t) = ((t >> 1) & 1) | ((t >> 3) & 3) << 1
  //        v^C (16 chunks): fv(t) = 2 (t & 3)
  //      (the 16 rows a K fragment read touches get 16 different positions; the 4 rows of a
  //      transposing V read, 4 different 32-byte pieces).  Copy r of wave w: r = 0, 1: k^C
  //      rows 4 q .. 4 q + 3 (q = w + 8 r); r = 2: k^R rows 8 w .. 8 w + 7; r = 3, 4: v^C rows
  //      4 q .. 4 q + 3 (q = w + 8 (r - 3)); lane l fills 16 bytes of the 1 KB it covers.
  auto fk = [](int t) { return (t & 3) | (((t >> 3) & 3) << 2); };
  auto fr = [](int t) { return ((t >> 1) & 1) | (((t >> 3) & 3) << 1); };
  auto fv = [](int t) { return 2 * (t & 3); };
  auto issue_block = [&](int kb, int buf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed at every block (no live ranges across the loop)
    const int last = T - 1 - kb * PF_KB;  // rows past it repeat it
    const int64_t key0 = tok0 + static_cast<int64_t>(kb) * PF_KB;
    const char* kc_base = reinterpret_cast<const char*>(k_c + (key0 * H + h) * PF_DH);
    const char* kr_base = reinterpret_cast<const char*>(k_pe + key0 * PF_DR);
    const char* v_base = reinterpret_cast<const char*>(v_c + (key0 * H + h) * PF_DH);
    const uint32_t hrow = static_cast<uint32_t>(H) * PF_DH * 2;  // bytes between keys (k^C, v^C)
    const uint32_t lds = smem_lds + buf * PF_TILE;
#pragma unroll
    for (int r = 0; r < 2; ++r) {  // k^C
      const int q = w + PF_NW * r, t = 4 * q + (ln >> 4), p = ln & 15;
      dma16(kc_base, static_cast<uint32_t>(min(t, last)) * hrow + 16u * (p ^ fk(t)),
            lds + PF_KC + q * 1024);
    }
    {  // k^R
      const int t = 8 * w + (ln >> 3), p = ln & 7;
      dma16(kr_base, static_cast<uint32_t>(min(t, last)) * (PF_DR * 2) + 16u * (p ^ fr(t)),
            lds + PF_KR + w * 1024);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {  // v^C
      const int q = w + PF_NW * r, t = 4 * q + (ln >> 4), p = ln & 15;
      dma16(v_base, static_cast<uint32_t>(min(t, last)) * hrow + 16u * (p ^ fv(t)),
            lds + PF_V + q * 1024);
    }
  };

  // K fragments: row r of key M tile mt is key 32 (mt >> 1) + 8 (r >> 2) + 4 (mt & 1) + (r & 3);
  // k-step kk reads logical chunk 4 kk + g of k^C (kk < 4) or 4 (kk - 4) + g of k^R; the
  // 32-key halves add 32 rows (the permutations depend on t mod 32 only).
  // V^T fragments: key half ks, rows 32 ks + 8 g + 4 r + (r16 >> 2), logical chunks
  // 8 (ct >> 2) + 2 (ct & 3) + e (e = (r16 & 3) >> 1), byte 8 (r16 & 1) of the chunk; the
  // permutation fv flips chunk bits 1-2 only, so the 8 (ct >> 2) stays an added offset.
  int kc_row[2], kc_x[2], kr_row[2], kr_x[2];
#pragma unroll
  for (int m1 = 0; m1 < 2; ++m1) {
    const int t = 8 * (r16 >> 2) + 4 * m1 + (r16 & 3);
    kc_row[m1] = PF_KC + t * PF_DH * 2;
    kc_x[m1] = fk(t);
    kr_row[m1] = PF_KR + t * PF_DR * 2;
    kr_x[m1] = fr(t);
  }
  auto k_off = [&](int mt, int kk) {
    const int m1 = mt & 1;
    return kk < 4 ? kc_row[m1] + (mt >> 1) * 32 * PF_DH * 2 + 16 * ((4 * kk + g) ^ kc_x[m1])
                  : kr_row[m1] + (mt >> 1) * 32 * PF_DR * 2 + 16 * ((4 * (kk - 4) + g) ^ kr_x[m1]);
  };
  int vb[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 8 * g + 4 * r + (r16 >> 2);
    const int e = (r16 & 3) >> 1;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      vb[r][c4] = PF_V + t * PF_DH * 2 + 16 * ((2 * c4 + e) ^ fv(t)) + 8 * (r16 & 1);
  }

  f32x4_t o[PF_QT][PF_CT];
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt)
#pragma unroll
    for (int ct = 0; ct < PF_CT; ++ct) o[qt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // of query qw + 16 qt + r16: the softmax reference (alike in its four lanes) and this
  // lane's part of the denominator
  float m_run[PF_QT], l_run[PF_QT];
  const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }

  // blocks 0 and 1 (behind the query loads, so waiting for block 0 covers those too)
  issue_block(0, 0);
  if (nkb > 1) {
    issue_block(1, 1);
    wait_vmcnt<PF_COPIES>();
  } else {
    wait_vmcnt<0>();
  }
  block_barrier();
  for (int kb = 0; kb < nkb; ++kb) {
    // block kb+2 into the buffer block kb-1 left (every wave finished it before barrier kb)
    if (kb + 2 < nkb) issue_block(kb + 2, (kb + 2) % PF_NBUF);
    const lds_char_t* tile = lsm + (kb % PF_NBUF) * PF_TILE;
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
          const bf16x8_t kf = *(const lds_bf16x8_t*)(tile + k_off(mt, kk));
#pragma unroll
          for (int qt = 0; qt < PF_QT; ++qt)
            sacc[qt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qt][kk], sacc[qt][mt], 0, 0, 0);
        }
      // ---- online softmax (log2 domain) per query tile: lane (g, r16) holds keys
      //      32 (mt >> 1) + 8 g + 4 (mt & 1) + i of its query; keys after it get weight 0.
      //      The maximum is taken on the raw scores (the scale is positive); each weight is
      //      2^(s scale - m) with one rounding in the fma.  The reference m moves only when a
      //      block's maximum passes it by more than PF_SLACK (log2 units), so weights stay
      //      below 2^PF_SLACK and the accumulators are rescaled rarely; every lane keeps its
      //      own part of the denominator (summed over the four lanes of a query at the end),
      //      summing the bf16-rounded weights the PV product consumes.
      bf16x8_t pt[PF_QT][2];  // P^T operands of the two 32-key halves
      const bool diagonal = kb * PF_KB + PF_KB - 1 > qw;  // some key after some query
#pragma unroll
      for (int qt = 0; qt < PF_QT; ++qt) {
        const int my_q = qw + 16 * qt + r16;
        if (diagonal) {
#pragma unroll
          for (int mt = 0; mt < PF_MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kb * PF_KB + 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
              if (key > my_q) sacc[qt][mt][i] = -INFINITY;
            }
        }
        float bmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < PF_MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, sacc[qt][mt][i]);
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        // finite: key 0 is seen by every query
        const float cand = mul_rn(bmax, scale_log2);
        const float m_new = cand > m_run[qt] + PF_SLACK ? cand : m_run[qt];
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
              pp[2 * m1 + hlf] =
                  to_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * hlf], scale_log2, -m_new)),
                            __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * hlf + 1], scale_log2, -m_new)));
              psum = __builtin_amdgcn_fdot2_f32_bf16(pp[2 * m1 + hlf], ones2, psum, false);
            }
          pt[qt][ks] = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                               __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
        }
        l_run[qt] = l_run[qt] * alpha + psum;
        m_run[qt] = m_new;
        if (__any(alpha != 1.f)) {  // the reference moved for some query
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
                (lds_i16x4_t*)(tile + ks * 32 * PF_DH * 2 + vb[r][ct & 3] + 128 * (ct >> 2)));
          const bf16x8_t vf = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qt = 0; qt < PF_QT; ++qt)
            o[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pt[qt][ks], o[qt][ct], 0, 0, 0);
        }
    }
    if (kb + 1 < nkb) {
      // this wave's copies of block kb+1 landed (block kb+2's may still be in flight)
      if (kb + 2 < nkb) wait_vmcnt<PF_COPIES>();
      else wait_vmcnt<0>();
      block_barrier();  // publishes block kb + 1; every wave is past its reads of block kb
    }
  }

  // ---- epilogue: lane (g, r16) holds dims 16 ct + 4 g .. + 3 of its query in each tile
#pragma unroll
  for (int qt = 0; qt < PF_QT; ++qt) {
    const int my_q = qw + 16 * qt + r16;
    float l = l_run[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (my_q < T) {
      const float inv = 1.f / l;
      float* dst = out + ((tok0 + my_q) * H + h) * PF_DH + 4 * g;
#pragma unroll
      for (int ct = 0; ct < PF_CT; ++ct) *reinterpret_cast<f32x4_t*>(dst + 16 * ct) = o[qt][ct] * inv;
      if (lse_out != nullptr && g == 0)
        lse_out[(tok0 + my_q) * H + h] = (m_run[qt] + __log2f(l)) * LN2;
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
