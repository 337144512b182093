// Log-sum-exp combine of split-K partials.
//
// Split s of a (sequence, head) saw a disjoint token range and produced its own
// normalised latent sum o_s and lse_s = ln sum_j e^{score_j}.  The softmax over all tokens
// is recovered exactly by weighting each split with e^{lse_s - M} (M = max lse): the
// softmax denominator is a sum over the tokens (qiita.com/joule "Attention 計算").
//
// One workgroup per (sequence, head), numbered sequence-fastest: consecutive workgroup ids
// go to the 8 XCDs in turn, so (with B a multiple of 8) the workgroups of sequence b run on
// XCD b % 8, the one whose attention workgroups wrote b's partials, and can find them in
// that XCD's L2.  Each thread owns 4 consecutive latent columns
// (one 16-byte load per split for fp32 partials, 8 bytes for bf16), the weights live in
// LDS.  Deterministic: fixed summation order, no atomics.
#include "combine_row.h"
#include "device_common.h"
#include "launchers.h"

namespace mla {

constexpr int kCombineThreads = 128;

typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned short u16x4_t;

__device__ __forceinline__ f32x4_t load4(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}
__device__ __forceinline__ f32x4_t load4(const bf16raw* p) {
  const u16x4_t v = *reinterpret_cast<const u16x4_t*>(p);
  return f32x4_t{bf16_to_f32(v[0]), bf16_to_f32(v[1]), bf16_to_f32(v[2]), bf16_to_f32(v[3])};
}

template <typename PT>
__global__ __launch_bounds__(kCombineThreads) void splitk_combine_kernel(
    const PT* __restrict__ o_part, const float* __restrict__ lse_part, int B, int H, int S,
    int d_c, float* __restrict__ out, float* __restrict__ lse_out) {
  extern __shared__ float w_lds[];  // S weights
  __shared__ float red[kCombineThreads / 64];
  const int bh = (blockIdx.x % B) * H + blockIdx.x / B;
  const int tid = threadIdx.x;
  const float* lse = lse_part + static_cast<int64_t>(bh) * S;

  float m = -INFINITY;
  for (int s = tid; s < S; s += kCombineThreads) m = fmaxf(m, lse[s]);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();

  const float msafe = (m == -INFINITY) ? 0.f : m;
  float part = 0.f;
  for (int s = tid; s < S; s += kCombineThreads) {
    const float x = lse[s];
    const float w = (x == -INFINITY) ? 0.f : expf(x - msafe);
    w_lds[s] = w;
    part += w;
  }
  part = wave_sum(part);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) den += red[w];
  const float inv = den > 0.f ? 1.f / den : 0.f;

  const PT* base = o_part + static_cast<int64_t>(bh) * S * d_c;
  for (int c = tid * 4; c < d_c; c += kCombineThreads * 4) {
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const float w = w_lds[s];
      if (w != 0.f) {
        const f32x4_t v = load4(base + static_cast<int64_t>(s) * d_c + c);
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
      }
    }
    acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
    *reinterpret_cast<f32x4_t*>(out + static_cast<int64_t>(bh) * d_c + c) = acc;
  }
  if (tid == 0 && lse_out != nullptr) lse_out[bh] = den > 0.f ? msafe + logf(den) : -INFINITY;
}

// d_c = 512, at most 64 splits: one wavefront per (sequence, head) (combine_row.h).
template <typename PT>
__global__ __launch_bounds__(256) void combine512_kernel(
    const PT* __restrict__ o_part, const float* __restrict__ lse_part, int B, int H, int S,
    float* __restrict__ out, float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= B * H) return;
  const int bh = (item % B) * H + item / B;  // sequence-fastest, as in splitk_combine_kernel
  combine512_wave(o_part + static_cast<int64_t>(bh) * S * 512, lse_part + static_cast<int64_t>(bh) * S,
                  S, out + static_cast<int64_t>(bh) * 512, lse_out != nullptr ? lse_out + bh : nullptr,
                  lane);
}

// Combine for the flattened work list of ragged batches: the count_b <= 64 partials of
// sequence b, head h are rows first_b H + h count_b + i (i < count_b) of o_part [.][512] /
// lse_part, with (first_b, count_b) = (seq_slots[2b], seq_slots[2b + 1]).  One wavefront
// per (sequence, head); a sequence without tokens gets o = 0, lse = -inf.
template <typename PT>
__global__ __launch_bounds__(256) void combine512_slots_kernel(
    const PT* __restrict__ o_part, const float* __restrict__ lse_part,
    const int* __restrict__ seq_slots, int B, int H, float* __restrict__ out,
    float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= B * H) return;
  const int b = item / H, h = item % H;
  const int first = seq_slots[2 * b], count = seq_slots[2 * b + 1];
  if (count == 0) {
    float* dst = out + static_cast<int64_t>(item) * 512 + 8 * lane;
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (lane == 0 && lse_out != nullptr) lse_out[item] = -INFINITY;
    return;
  }
  const int64_t row0 = static_cast<int64_t>(first) * H + static_cast<int64_t>(h) * count;
  combine512_wave(o_part + row0 * 512, lse_part + row0, count,
                  out + static_cast<int64_t>(item) * 512,
                  lse_out != nullptr ? lse_out + item : nullptr, lane);
}

hipError_t launch_combine_slots(const void* o_part, int part_bf16, const float* lse_part,
                                const int* seq_slots, int B, int H, float* out, float* lse_out,
                                hipStream_t st) {
  const int items = B * H;
  if (part_bf16)
    hipLaunchKernelGGL(combine512_slots_kernel<bf16raw>, dim3((items + 3) / 4), dim3(256), 0, st,
                       static_cast<const bf16raw*>(o_part), lse_part, seq_slots, B, H, out, lse_out);
  else
    hipLaunchKernelGGL(combine512_slots_kernel<float>, dim3((items + 3) / 4), dim3(256), 0, st,
                       static_cast<const float*>(o_part), lse_part, seq_slots, B, H, out, lse_out);
  return hipGetLastError();
}

hipError_t launch_splitk_combine(const void* o_part, int part_bf16, const float* lse_part, int B,
                                 int H, int S, int d_c, float* out, float* lse_out, hipStream_t st) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(o_part) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  if (d_c == 512 && S <= 64 && aligned) {
    const int items = B * H;
    if (part_bf16)
      hipLaunchKernelGGL(combine512_kernel<bf16raw>, dim3((items + 3) / 4), dim3(256), 0, st,
                         static_cast<const bf16raw*>(o_part), lse_part, B, H, S, out, lse_out);
    else
      hipLaunchKernelGGL(combine512_kernel<float>, dim3((items + 3) / 4), dim3(256), 0, st,
                         static_cast<const float*>(o_part), lse_part, B, H, S, out, lse_out);
    return hipGetLastError();
  }
  const size_t lds = static_cast<size_t>(S) * sizeof(float);
  if (part_bf16)
    hipLaunchKernelGGL(splitk_combine_kernel<bf16raw>, dim3(B * H), dim3(kCombineThreads), lds,
                       st, static_cast<const bf16raw*>(o_part), lse_part, B, H, S, d_c, out, lse_out);
  else
    hipLaunchKernelGGL(splitk_combine_kernel<float>, dim3(B * H), dim3(kCombineThreads), lds, st,
                       static_cast<const float*>(o_part), lse_part, B, H, S, d_c, out, lse_out);
  return hipGetLastError();
}

}  // namespace mla
