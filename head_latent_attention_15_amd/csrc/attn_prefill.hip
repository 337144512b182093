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
// One workgroup of 8 wavefronts per (sequence, head, block of 128 queries), wavefront w
// owning queries 16 w .. 16 w + 15 of the block.  Keys go through LDS in 32-key blocks, one
// 640-byte row per key [k^C_i (128) | k^R (64) | v^C_i (128)] with the 16-byte-chunk XOR
// swizzle of the decode tiles (a row stride of 128 mod 256 bytes, as there), so the
// row-strided K reads and the transposing V reads are conflict-free.  Per key block a wave
// computes S^T = K Q^T (tokens as the MFMA M dimension, 2 x 6 MFMAs, Q resident in VGPRs;
// the key permutation inside the block makes the C layout of S^T the B layout of P^T),
// an online softmax per query (running maximum, accumulators rescaled when it moves), and
// O^T += V^T P^T (8 MFMAs, V^T by transposing reads).  Blocks are staged with plain global
// loads double-buffered through registers.  Workgroups of late query blocks (the most
// keys) are numbered first.
#include "attn_common.h"
#include "launchers.h"

namespace mla {
namespace {

using namespace attn;

constexpr int PF_DH = 128, PF_DR = 64, PF_DQK = PF_DH + PF_DR;  // 192
constexpr int PF_ROW = (PF_DQK + PF_DH) * 2;                     // 640 bytes: k^C | k^R | v^C
constexpr int PF_ROW_CHUNKS = PF_ROW / 16;                       // 40
constexpr int PF_KB = 32;                                        // keys per block
constexpr int PF_TILE = PF_KB * PF_ROW;                          // 20480 bytes
constexpr int PF_CHUNKS = PF_KB * PF_ROW_CHUNKS;                 // 1280
constexpr int PF_NW = 8, PF_NT = PF_NW * 64;
constexpr int PF_QB = 16 * PF_NW;                                // 128 queries per workgroup
constexpr int PF_LOADS = (PF_CHUNKS + PF_NT - 1) / PF_NT;        // 3 chunks per thread
constexpr int PF_KSTEPS = PF_DQK / 32;                           // 6

__global__ __launch_bounds__(PF_NT) void attn_prefill_kernel(
    const bf16raw* __restrict__ q_c, const bf16raw* __restrict__ q_pe,
    const bf16raw* __restrict__ k_c, const bf16raw* __restrict__ k_pe,
    const bf16raw* __restrict__ v_c, int T, int H, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) char smem[2 * PF_TILE];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const int nqb = (T + PF_QB - 1) / PF_QB;
  const int qb = nqb - 1 - static_cast<int>(blockIdx.x);  // most keys first
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int q0 = qb * PF_QB;                         // first query of the workgroup
  const int qw = q0 + 16 * w;                        // first query of this wave
  const int q_last = min(q0 + PF_QB, T) - 1;         // last query of the workgroup
  const int nkb = q_last / PF_KB + 1;                // key blocks the workgroup needs
  const int64_t tok0 = static_cast<int64_t>(b) * T;  // first token row of the sequence

  // ---- query fragments (B operand of S^T = K Q^T): lane (g, r16) holds query qw + r16,
  //      features 32 kk + 8 g .. + 7 (kk < 4: q^C, else q_pe); queries past T repeat T - 1
  bf16x8_t qf[PF_KSTEPS];
  {
    const int q = min(qw + r16, T - 1);
    const bf16raw* qc = q_c + ((tok0 + q) * H + h) * PF_DH + 8 * g;
    const bf16raw* qp = q_pe + ((tok0 + q) * H + h) * PF_DR + 8 * g;
#pragma unroll
    for (int kk = 0; kk < PF_KSTEPS; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8_t*>(kk < 4 ? qc + 32 * kk : qp + 32 * (kk - 4));
  }

  // ---- staging: thread tid moves LDS chunks e = tid + 512 i (i < 3, e < 1280) of a block:
  //      row t = e / 40 (key kb*32 + t, keys past T repeat T - 1), stored position p = e % 40
  //      holding logical chunk c = p ^ swz(t): c < 16 k^C, c < 24 k^R, else v^C
  auto chunk_src = [&](int kb, int e) -> const bf16raw* {
    const int t = e / PF_ROW_CHUNKS, p = e - t * PF_ROW_CHUNKS;
    const int c = p ^ swz(t);
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

  // K fragment lane offsets (row 8 (r16 >> 2) + 4 mt + (r16 & 3), logical chunk 4 par + g;
  // k-step kk adds 128 (kk >> 1)), V^T fragment offsets (rows 8 gg + 4 r + (rr >> 2),
  // chunks 24 + 2 ct (+1)), as in the decode kernel
  int kb_off[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int t = 8 * (r16 >> 2) + 4 * mt + (r16 & 3);
#pragma unroll
    for (int par = 0; par < 2; ++par) kb_off[mt][par] = t * PF_ROW + 16 * ((4 * par + g) ^ swz(t));
  }
  int vb[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 8 * g + 4 * r + (r16 >> 2);
    const int e = (r16 & 3) >> 1;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) vb[r][c4] = t * PF_ROW + 16 * ((2 * c4 + e) ^ swz(t)) + 8 * (r16 & 1);
  }

  f32x4_t o[PF_DH / 16];
#pragma unroll
  for (int ct = 0; ct < PF_DH / 16; ++ct) o[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // of query qw + r16, alike in its four lanes
  const int my_q = qw + r16;

  load_block(0);
  store_block(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) load_block(kb + 1);  // in flight while this block is consumed
    const lds_char_t* tile = lsm + (kb & 1) * PF_TILE;
    if (kb * PF_KB <= qw + 15) {  // this wave's queries see some key of the block
      // ---- S^T (32 keys x 16 queries): row r of M tile mt is key 8 (r >> 2) + 4 mt + (r & 3)
      f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < PF_KSTEPS; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8_t kf = *(const lds_bf16x8_t*)(tile + kb_off[mt][kk & 1] + (kk >> 1) * 128);
          sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], sacc[mt], 0, 0, 0);
        }
      // ---- online softmax (log2 domain): lane (g, r16) holds keys 8 g + 4 mt + i of query
      //      my_q; keys after the query (and past T) get weight 0
      float e2[2][4];
      float bmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb * PF_KB + 8 * g + 4 * mt + i;
          const float sv = key <= my_q ? sacc[mt][i] * scale_log2 : -INFINITY;
          e2[mt][i] = sv;
          bmax = fmaxf(bmax, sv);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float m_new = fmaxf(m_run, bmax);  // finite: key kb*32 <= my_q or an earlier block
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      bf16x2_t pp[4];
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          pp[2 * mt + hlf] = to_bf16x2(__builtin_amdgcn_exp2f(e2[mt][2 * hlf] - m_new),
                                       __builtin_amdgcn_exp2f(e2[mt][2 * hlf + 1] - m_new));
          psum += static_cast<float>(pp[2 * mt + hlf][0]) + static_cast<float>(pp[2 * mt + hlf][1]);
        }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int ct = 0; ct < PF_DH / 16; ++ct) o[ct] *= alpha;
      const bf16x8_t pt = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                  __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
      // ---- O^T (128 x 16) += V^T (128 x 32) P^T (32 x 16); V^T column tile ct sits in chunks
      //      24 + 2 ct, 24 + 2 ct + 1: group 3 + (ct >> 2) of the row
#pragma unroll
      for (int ct = 0; ct < PF_DH / 16; ++ct) {
        i16x4_t half[2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t*)(tile + vb[r][ct & 3] + 128 * (3 + (ct >> 2))));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pt, o[ct], 0, 0, 0);
      }
    }
    if (kb + 1 < nkb) {
      // buffer (kb + 1) & 1 was last read in block kb - 1, before the previous barrier
      store_block((kb + 1) & 1);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __syncthreads();  // publishes block kb + 1; every wave is past its reads of block kb
    }
  }

  // ---- epilogue: lane (g, r16) holds dims 16 ct + 4 g .. + 3 of query my_q
  if (my_q < T) {
    const float inv = 1.f / l_run;
    float* dst = out + ((tok0 + my_q) * H + h) * PF_DH + 4 * g;
#pragma unroll
    for (int ct = 0; ct < PF_DH / 16; ++ct) *reinterpret_cast<f32x4_t*>(dst + 16 * ct) = o[ct] * inv;
    if (lse_out != nullptr && g == 0) lse_out[(tok0 + my_q) * H + h] = (m_run + __log2f(l_run)) * LN2;
  }
}

}  // namespace

bool attn_prefill_supported(int d_h, int d_R) { return d_h == PF_DH && d_R == PF_DR; }

hipError_t launch_attn_prefill(const void* q_c, const void* q_pe, const void* k_c,
                               const void* k_pe, const void* v_c, int B, int T, int H,
                               float scale, float* out, float* lse_out, hipStream_t s) {
  const float log2e = 1.4426950408889634f;
  const dim3 grid((T + PF_QB - 1) / PF_QB, H, B);
  hipLaunchKernelGGL(attn_prefill_kernel, grid, dim3(PF_NT), 0, s,
                     static_cast<const bf16raw*>(q_c), static_cast<const bf16raw*>(q_pe),
                     static_cast<const bf16raw*>(k_c), static_cast<const bf16raw*>(k_pe),
                     static_cast<const bf16raw*>(v_c), T, H, scale * log2e, out, lse_out);
  return hipGetLastError();
}

}  // namespace mla
