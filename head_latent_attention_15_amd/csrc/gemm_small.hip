// Batched small GEMM with fp32 accumulation, for the projections around the attention and
// the offline weight folds:
//   y[z][m][n] = sum_k x[z][m][k] * W_z(n, k)
// x[z][m][k] is x[z*sx + m*ldx + k], or x[z*sx + k*ldx + m] with x_km (a weight read
// transposed, as W^UK_i^T in the fold W^UK_i^T W^UQ_i).
// W_z(n, k) is w[z*sw + n*ldw + k] for nn.Linear-layout weights ([out, in], used by
// y = x W^T: W^DQ, W^UQ, W^QR, W^DKV, W^KR, W^UV_i, W^O) and w[z*sw + k*ldw + n] for the
// query absorption q~_i = W^UK_i^T q^C_i ("論文解説: DeepSeek-V2 …", "行列吸収トリック").
//
// 64x64 output tile per workgroup, 32-deep k slices staged in LDS as fp32, 4x4 outputs per
// thread.  Inputs are read once per M tile; M (the batch) is at most a few tiles here, so
// the weights stream from HBM about once.
#include "device_common.h"
#include "launchers.h"

namespace mla {

constexpr int GT_M = 64, GT_N = 64, GT_K = 32;

template <typename XT, typename WT, typename YT, bool W_NK>
__global__ __launch_bounds__(256) void gemm_small_kernel(
    const XT* __restrict__ x, int64_t ldx, int64_t sx, const WT* __restrict__ w, int64_t ldw,
    int64_t sw, YT* __restrict__ y, int64_t ldy, int64_t sy, int M, int N, int K,
    int accumulate, int x_km) {
  __shared__ float xs[GT_K][GT_M + 4];
  __shared__ float ws[GT_K][GT_N + 4];
  const int z = blockIdx.z;
  x += z * sx;
  w += z * sw;
  y += z * sy;
  const int m0 = blockIdx.y * GT_M, n0 = blockIdx.x * GT_N;
  const int tid = threadIdx.x;
  const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += GT_K) {
    for (int e = tid; e < GT_M * GT_K; e += 256) {
      const int mm = e / GT_K, kk = e % GT_K;
      const int gm = m0 + mm, gk = k0 + kk;
      xs[kk][mm] = (gm < M && gk < K) ? ld(x + (x_km ? gk * ldx + gm : gm * ldx + gk)) : 0.f;
    }
    for (int e = tid; e < GT_N * GT_K; e += 256) {
      int nn, kk;
      if (W_NK) {
        nn = e / GT_K;
        kk = e % GT_K;
      } else {
        kk = e / GT_N;
        nn = e % GT_N;
      }
      const int gn = n0 + nn, gk = k0 + kk;
      float v = 0.f;
      if (gn < N && gk < K) v = W_NK ? ld(w + gn * ldw + gk) : ld(w + gk * ldw + gn);
      ws[kk][nn] = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < GT_K; ++kk) {
      float a[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][tm + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ws[kk][tn + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + tm + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tn + j;
      if (gn >= N) continue;
      YT* dst = y + gm * ldy + gn;
      st(dst, accumulate ? acc[i][j] + ld(dst) : acc[i][j]);
    }
  }
}

template <typename XT, typename WT, typename YT>
static hipError_t launch3(const GemmArgs& g, hipStream_t s) {
  dim3 grid((g.N + GT_N - 1) / GT_N, (g.M + GT_M - 1) / GT_M, g.batch);
  if (g.w_nk) {
    hipLaunchKernelGGL((gemm_small_kernel<XT, WT, YT, true>), grid, dim3(256), 0, s,
                       static_cast<const XT*>(g.x), g.ldx, g.sx, static_cast<const WT*>(g.w),
                       g.ldw, g.sw, static_cast<YT*>(g.y), g.ldy, g.sy, g.M, g.N, g.K,
                       g.accumulate, g.x_km);
  } else {
    hipLaunchKernelGGL((gemm_small_kernel<XT, WT, YT, false>), grid, dim3(256), 0, s,
                       static_cast<const XT*>(g.x), g.ldx, g.sx, static_cast<const WT*>(g.w),
                       g.ldw, g.sw, static_cast<YT*>(g.y), g.ldy, g.sy, g.M, g.N, g.K,
                       g.accumulate, g.x_km);
  }
  return hipGetLastError();
}

template <typename XT, typename WT>
static hipError_t launch2(const GemmArgs& g, hipStream_t s) {
  return g.y_bf16 ? launch3<XT, WT, bf16raw>(g, s) : launch3<XT, WT, float>(g, s);
}

template <typename XT>
static hipError_t launch1(const GemmArgs& g, hipStream_t s) {
  return g.w_bf16 ? launch2<XT, bf16raw>(g, s) : launch2<XT, float>(g, s);
}

hipError_t launch_gemm_small(const GemmArgs& g, hipStream_t s) {
  return g.x_bf16 ? launch1<bf16raw>(g, s) : launch1<float>(g, s);
}

}  // namespace mla
