// Decode attention over the paged latent cache, one wavefront per (sequence, head, split).
//
// Plain fp32 VALU version: each lane owns a strided slice of the 576-wide row
// ([c^KV | k^R]), the score is a wave-wide sum, and an online softmax keeps the running
// maximum, denominator and latent sum.  Used for the small fp32 shape (d_c = 64, d_R = 16)
// and for bf16 head counts the MFMA kernel does not tile.
//
// Method: scores (q~_i . c_j + q^R_i . k^R_j) * scale over the cached tokens, softmax,
// latent weighted sum o~_i = sum_j p_ij c_j (qiita.com/joule "Attention 計算" in the
// absorbed order of "論文解説: DeepSeek-V2 …" section "行列吸収トリック"; kasblo.com/?p=4663
// "V側は、小さな表現の加重和を先に求める").
#include "device_common.h"
#include "launchers.h"

namespace mla {

template <typename T, typename OT, int DC, int DR>
__global__ __launch_bounds__(64) void attn_generic_kernel(
    const T* __restrict__ q_lat, const T* __restrict__ q_pe, const T* __restrict__ cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int H,
    int P, int max_pages, int pages_per_split, int S, float scale_log2, OT* __restrict__ o_part,
    float* __restrict__ lse_part, int n_q) {
  static_assert(DR <= 64, "rope part must fit one lane each");
  constexpr int ROW = DC + DR;
  constexpr int NC = (DC + 63) / 64;
  // query row bq = b n_q + t: token t of sequence b, at position seq_len - n_q + t
  const int s = blockIdx.x, h = blockIdx.y, bq = blockIdx.z, b = bq / n_q, t = bq - b * n_q;
  const int lane = threadIdx.x;

  float qc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int idx = lane + 64 * k;
    qc[k] = idx < DC ? ld(q_lat + (static_cast<int64_t>(bq) * H + h) * DC + idx) : 0.f;
  }
  const float qr = lane < DR ? ld(q_pe + (static_cast<int64_t>(bq) * H + h) * DR + lane) : 0.f;

  const int L = seq_lens[b] - (n_q - 1 - t);
  const int j0 = s * pages_per_split * P;
  const int j1 = min(L, (s + 1) * pages_per_split * P);
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_pages;

  float m = -INFINITY, l = 0.f;
  float acc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) acc[k] = 0.f;

  for (int j = j0; j < j1; ++j) {
    const int page = bt[j / P];
    const T* row = cache + (static_cast<int64_t>(page) * P + (j % P)) * ROW;
    float v[NC];
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int idx = lane + 64 * k;
      v[k] = idx < DC ? ld(row + idx) : 0.f;
      part += qc[k] * v[k];
    }
    if (lane < DR) part += qr * ld(row + DC + lane);
    // log2 domain: the score is rounded once, so the maximum and the exponent see the same
    // value, and exp2(0) is exactly 1 (a single-token context returns its latent exactly)
    const float sc = mul_rn(wave_sum(part), scale_log2);
    const float mn = fmaxf(m, sc);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    const float p = __builtin_amdgcn_exp2f(sc - mn);
    l = l * alpha + p;
#pragma unroll
    for (int k = 0; k < NC; ++k) acc[k] = acc[k] * alpha + p * v[k];
    m = mn;
  }

  const int64_t ob = (static_cast<int64_t>(bq) * H + h) * S + s;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int idx = lane + 64 * k;
    if (idx < DC) st(o_part + ob * DC + idx, acc[k] * inv);
  }
  if (lane == 0 && lse_part != nullptr)
    lse_part[ob] = l > 0.f ? (m + __log2f(l)) * 0.6931471805599453f : -INFINITY;
}

template <typename T, typename OT, int DC, int DR>
static hipError_t launch_generic_t(const PagedArgs& a, hipStream_t st) {
  dim3 grid(a.num_splits, a.H, a.B * a.n_q);
  hipLaunchKernelGGL((attn_generic_kernel<T, OT, DC, DR>), grid, dim3(64), 0, st,
                     static_cast<const T*>(a.q_lat), static_cast<const T*>(a.q_pe),
                     static_cast<const T*>(a.cache), a.block_table, a.seq_lens, a.H,
                     a.page_size, a.max_pages, a.pages_per_split, a.num_splits,
                     a.scale * 1.4426950408889634f, static_cast<OT*>(a.o_part), a.lse_part,
                     a.n_q);
  return hipGetLastError();
}

template <typename T, int DC, int DR>
static hipError_t launch_generic(const PagedArgs& a, hipStream_t st) {
  return a.part_bf16 ? launch_generic_t<T, bf16raw, DC, DR>(a, st)
                     : launch_generic_t<T, float, DC, DR>(a, st);
}

hipError_t launch_attn_generic_f32_64_16(const PagedArgs& a, hipStream_t s) {
  return launch_generic<float, 64, 16>(a, s);
}

hipError_t launch_attn_generic_bf16_512_64(const PagedArgs& a, hipStream_t s) {
  return launch_generic<bf16raw, 512, 64>(a, s);
}

}  // namespace mla
