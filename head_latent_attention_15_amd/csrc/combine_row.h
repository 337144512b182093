// Log-sum-exp combine of the S split partials of one (query row, head), d_c = 512, on one
// wavefront.  Shared by the combine kernel (combine.hip) and the attention kernel's
// in-launch merge (attn_mfma.hip), so both give the same bits.
//
// Split s saw a disjoint token range and produced its own normalised latent sum o_s and
// lse_s = ln sum_j e^{score_j}; weighting each split by e^{lse_s - M} (M = max lse)
// recovers the softmax over all tokens, because its denominator is a sum over the tokens
// (qiita.com/joule "Attention 計算").  Empty splits (lse = -inf) get weight exactly 0.
#pragma once

#include "device_common.h"

namespace mla {

typedef __attribute__((ext_vector_type(4))) float cr_f32x4_t;

// eight consecutive partial values of one split, fp32 or bf16
template <typename PT> struct Part8;
template <> struct Part8<bf16raw> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16raw* p) {
    u = *reinterpret_cast<const uint4*>(p);
  }
  __device__ __forceinline__ float at(int i) const {
    const unsigned w = (i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w;
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <> struct Part8<float> {
  cr_f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const cr_f32x4_t*>(p);
    b = *reinterpret_cast<const cr_f32x4_t*>(p + 4);
  }
  __device__ __forceinline__ float at(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

// part: the row's S partials of 512 values, part_stride elements apart (16-byte aligned);
// lse: its S lses, lse_stride apart; out: 512 fp32 (16-byte aligned); lse_out: one float or
// NULL.  1 <= S <= 64.  Lane l owns columns
// 8 l .. 8 l + 7 (one 16-byte load per split for bf16 partials), lane s holds split s's lse
// and weight.  Every load of a chunk of 8 splits goes out before anything waits (split
// indices past S re-read split S - 1 and get weight 0, so the loads carry no branch that
// would make each wait for its own data); the weights reach the lanes by readlane.
template <typename PT>
__device__ __forceinline__ void combine512_wave(const PT* __restrict__ part,
                                                const float* __restrict__ lse, int S,
                                                float* __restrict__ out,
                                                float* __restrict__ lse_out, int lane,
                                                int64_t part_stride = 512, int lse_stride = 1) {
  const float xraw = lse[static_cast<int64_t>(min(lane, S - 1)) * lse_stride];
  const PT* base = part + 8 * lane;
  Part8<PT> v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j].load(base + min(j, S - 1) * part_stride);
  __builtin_amdgcn_sched_barrier(0);

  const float x = lane < S ? xraw : -INFINITY;
  const float m = wave_max(x);
  const float msafe = (m == -INFINITY) ? 0.f : m;
  const float wl = (x == -INFINITY) ? 0.f : expf(x - msafe);  // 0 for lanes >= S
  const float den = wave_sum(wl);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0;;) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s0 + j));
#pragma unroll
      for (int i = 0; i < 8; ++i)  // an empty split adds exactly 0 (and no NaN)
        acc[i] = fmaf(w, w != 0.f ? v[j].at(i) : 0.f, acc[i]);
    }
    s0 += 8;
    if (s0 >= S) break;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j].load(base + min(s0 + j, S - 1) * part_stride);
  }
  float* dst = out + 8 * lane;
  *reinterpret_cast<cr_f32x4_t*>(dst) = cr_f32x4_t{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  *reinterpret_cast<cr_f32x4_t*>(dst + 4) = cr_f32x4_t{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  if (lane == 0 && lse_out != nullptr) *lse_out = den > 0.f ? msafe + logf(den) : -INFINITY;
}

}  // namespace mla
