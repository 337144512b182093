// Weight-streaming GEMM for the projections around the attention, on bf16 MFMA:
//   y[z][m][n] = sum_k x[z][m][k] * w[z][n][k]
// with w in nn.Linear layout ([out, in], k contiguous): W^DQ, W^UQ, W^QR, W^DKV, W^KR
// ("論文解説: DeepSeek-V2 …", "Low-Rank Key-Value Joint Compression" and the query
// compression beside it), the per-head W^UV_i and W^O ("行列吸収トリック"; kasblo.com/?p=4663,
// "V側は、小さな表現の加重和を先に求める").  M is the decode batch (a few tens of rows), so the
// weights are the traffic: every weight byte is read once, from HBM straight into MFMA
// B-operand registers (lane (g, r) takes w[n + r][k + 8 g .. + 7], 16 contiguous bytes).
//
// The activations x are small and shared by every workgroup; a workgroup stages them
// through LDS in 128-wide k chunks as bf16, split as x = hi + lo (both bf16, lo the
// rounding remainder) when x is fp32, so the products keep about 16 significant bits of x
// and every product of a bf16 weight is exact in the fp32 accumulator.
//
// Work decomposition: 4 wavefronts, wave w owns TN column tiles of 16 (64 TN columns per
// workgroup) and all four 16-row tiles of a 64-row block of x.  Long k ranges are split over
// KS workgroups, which add their results into y with fp32 atomics (y is zeroed first,
// unless the caller accumulates into its prior contents), so the sum order, and with it
// the last bits of y, can differ between runs.  Each wave keeps
// the weight fragments of the next R - 1 k-steps in flight: at these sizes the loaded HBM
// latency is several microseconds, and the bytes outstanding across the chip, not the
// access pattern, set the rate.
#include "device_common.h"
#include "launchers.h"

#include <algorithm>
#include <type_traits>

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int KC = 128;                 // k per staged chunk (4 MFMA k-steps)
constexpr int XROW = KC * 2 + 16;       // LDS bytes per staged row: bf16, padded (banks)
constexpr int XPLANE = 64 * XROW;       // one plane (hi or lo) of 64 rows
constexpr int GR_LDS = 2 * 2 * XPLANE;  // two chunk buffers x (hi, lo)

// two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, a in the low half;
// branch-free, so the loops around it keep exact memory wait counts
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <typename XT, int TN, int R>
__global__ __launch_bounds__(256, 2) void gemm_rows_kernel(
    const XT* __restrict__ x, int64_t ldx, int64_t sx, const bf16raw* __restrict__ w,
    int64_t ldw, int64_t sw, float* __restrict__ y, int64_t ldy, int64_t sy, int M, int N,
    int K, int KS, int kper, int atomic_out) {
  constexpr bool SPLIT_X = std::is_same<XT, float>::value;  // fp32 x: hi + lo planes
  __shared__ __attribute__((aligned(16))) char smem[GR_LDS];
  lds_char_t* const lsm = (lds_char_t*)smem;

  const int z = blockIdx.z / KS, ks = blockIdx.z % KS;
  x += z * sx;
  w += z * sw;
  y += z * sy;
  const int m0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int n0 = blockIdx.x * 64 * TN + wv * 16 * TN;  // this wave's first column
  const int kb = ks * kper;
  const int nchunks = kper / KC;

  // ---- staging of one 128-wide chunk of x: thread t converts row t / 4, columns
  //      32 (t % 4) .. + 31 (rows past M are zero)
  const int srow = tid >> 2, scol = (tid & 3) * 32;
  const bool srow_ok = m0 + srow < M;
  const XT* xsrc = x + static_cast<int64_t>(m0 + (srow_ok ? srow : 0)) * ldx + scol;
  float xv[32];
  auto stage_load = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      if constexpr (SPLIT_X) {
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(xsrc + kc + i);
        if (!srow_ok) v = f32x4_t{0.f, 0.f, 0.f, 0.f};
        xv[i] = v[0]; xv[i + 1] = v[1]; xv[i + 2] = v[2]; xv[i + 3] = v[3];
      } else {
        uint2 v = *reinterpret_cast<const uint2*>(xsrc + kc + i);
        if (!srow_ok) v = uint2{0u, 0u};
        xv[i] = __uint_as_float(v.x << 16); xv[i + 1] = __uint_as_float(v.x & 0xffff0000u);
        xv[i + 2] = __uint_as_float(v.y << 16); xv[i + 3] = __uint_as_float(v.y & 0xffff0000u);
      }
    }
  };
  auto stage_store = [&](int buf) {
    lds_char_t* hi = lsm + buf * 2 * XPLANE + srow * XROW + scol * 2;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      u32x4_t h, l;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = xv[i + 2 * j], b = xv[i + 2 * j + 1];
        h[j] = pack_bf16(a, b);
        if constexpr (SPLIT_X) {
          const float ah = __uint_as_float(h[j] << 16), bh = __uint_as_float(h[j] & 0xffff0000u);
          l[j] = pack_bf16(a - ah, b - bh);
        }
      }
      *(lds_u32x4_t*)(hi + 2 * i) = h;
      if constexpr (SPLIT_X) *(lds_u32x4_t*)(hi + XPLANE + 2 * i) = l;
    }
  };

  // ---- weight rows of this lane (clamped to N - 1; those columns are not stored)
  const bf16raw* wrow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = min(n0 + 16 * j + r, N - 1);
    wrow[j] = w + static_cast<int64_t>(n) * ldw + kb + 8 * g;
  }
  const int nsteps = nchunks * 4;
  auto w_frag = [&](int step, int j) {
    return *reinterpret_cast<const bf16x8_t*>(wrow[j] + 32 * step);
  };

  f32x4_t acc[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // W fragments of the next R - 1 k-steps in flight (ring of R k-steps, R a multiple of
  // the 4 steps of a chunk).  Every step issues TN loads (clamped to the last step near the
  // end), so the wait before each MFMA is an exact count.  The chunk loop is unrolled over
  // one turn of the ring (R / 4 chunks; the plan makes the chunk count a multiple of it), so
  // every ring slot is a fixed register.
  static_assert(R % 4 == 0 && R >= 4, "ring of whole chunks");
  constexpr int CPT = R / 4;  // chunks per turn of the ring
  bf16x8_t wf[R][TN];
#pragma unroll
  for (int i = 0; i < R - 1; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) wf[i][j] = w_frag(min(i, nsteps - 1), j);

  stage_load(kb);
  stage_store(0);
  for (int c0 = 0; c0 < nchunks; c0 += CPT) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = c0 + u;
      __syncthreads();  // chunk c staged; the other buffer is free
      stage_load(kb + min(c + 1, nchunks - 1) * KC);
      const lds_char_t* xa = lsm + (c & 1) * 2 * XPLANE + r * XROW + g * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int step = 4 * c + i, slot = 4 * u + i;  // slot == step % R
#pragma unroll
        for (int j = 0; j < TN; ++j) wf[(slot + R - 1) % R][j] = w_frag(min(step + R - 1, nsteps - 1), j);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8_t ah = *(const lds_bf16x8_t*)(xa + mt * 16 * XROW + i * 64);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wf[slot][j], acc[j][mt], 0, 0, 0);
          if constexpr (SPLIT_X) {
            const bf16x8_t al = *(const lds_bf16x8_t*)(xa + XPLANE + mt * 16 * XROW + i * 64);
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wf[slot][j], acc[j][mt], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c + 1 < nchunks) stage_store((c + 1) & 1);
    }
  }

  // ---- lane (g, r) of tile (j, mt) holds y[m0 + 16 mt + 4 g + i][n0 + 16 j + r]
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + 16 * j + r;
    if (n >= N) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * mt + 4 * g + i;
        if (m >= M) continue;
        float* dst = y + static_cast<int64_t>(m) * ldy + n;
        if (atomic_out) atomicAdd(dst, acc[j][mt][i]);
        else *dst = acc[j][mt][i];
      }
  }
}

// zero y[z][m][n] for the atomic accumulation: rows (z, m) over grid.y, 16-byte stores
// along n where the row is aligned
__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ y, int64_t ldy,
                                                        int64_t sy, int M, int N, int batch) {
  const int64_t rows = static_cast<int64_t>(M) * batch;
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
    const int64_t z = row / M, m = row - z * M;
    float* p = y + z * sy + m * ldy;
    const bool vec = (reinterpret_cast<uintptr_t>(p) & 15) == 0;
    for (int n = (blockIdx.x * 256 + threadIdx.x) * 4; n < N; n += gridDim.x * 1024) {
      if (vec && n + 4 <= N) {
        *reinterpret_cast<float4*>(p + n) = make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        for (int k = n; k < min(n + 4, N); ++k) p[k] = 0.f;
      }
    }
  }
}

template <typename XT, int TN, int R>
hipError_t launch_t(const GemmArgs& g, int KS, hipStream_t s) {
  const int kper = g.K / KS;
  const int nb = (g.N + 64 * TN - 1) / (64 * TN), mb = (g.M + 63) / 64;
  if (KS > 1 && !g.accumulate) {
    const int64_t rows = static_cast<int64_t>(g.batch) * g.M;
    const int gx = static_cast<int>(std::min<int64_t>((g.N + 1023) / 1024, 64));
    const int gy = static_cast<int>(std::min<int64_t>(rows, 4096));
    hipLaunchKernelGGL(zero_rows_kernel, dim3(gx, gy), dim3(256), 0, s, static_cast<float*>(g.y),
                       g.ldy, g.sy, g.M, g.N, g.batch);
  }
  hipLaunchKernelGGL((gemm_rows_kernel<XT, TN, R>), dim3(nb, mb, g.batch * KS), dim3(256), 0, s,
                     static_cast<const XT*>(g.x), g.ldx, g.sx, static_cast<const bf16raw*>(g.w),
                     g.ldw, g.sw, static_cast<float*>(g.y), g.ldy, g.sy, g.M, g.N, g.K, KS,
                     kper, KS > 1 || g.accumulate ? 1 : 0);
  return hipGetLastError();
}

// ring depths compiled per tile width: the ring holds 4 R TN registers per lane
template <typename XT, int TN>
hipError_t launch_r(const GemmArgs& g, int KS, int R, hipStream_t s) {
  switch (R) {
    case 4: return launch_t<XT, TN, 4>(g, KS, s);
    case 8: return launch_t<XT, TN, 8>(g, KS, s);
    case 12: if constexpr (TN <= 2) return launch_t<XT, TN, 12>(g, KS, s); else break;
    case 16: if constexpr (TN <= 2) return launch_t<XT, TN, 16>(g, KS, s); else break;
    case 20: if constexpr (TN == 1) return launch_t<XT, TN, 20>(g, KS, s); else break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename XT>
hipError_t launch_x(const GemmArgs& g, int TN, int KS, int R, hipStream_t s) {
  switch (TN) {
    case 4: return launch_r<XT, 4>(g, KS, R, s);
    case 2: return launch_r<XT, 2>(g, KS, R, s);
    case 1: return launch_r<XT, 1>(g, KS, R, s);
    default: return hipErrorInvalidValue;
  }
}

bool ring_ok(int tn, int r) {
  return r == 4 || r == 8 || ((r == 12 || r == 16) && tn <= 2) || (r == 20 && tn == 1);
}

}  // namespace

bool gemm_rows_supported(const GemmArgs& g) {
  return g.w_bf16 && g.w_nk && !g.y_bf16 && g.K % KC == 0 && g.K > 0 && g.M > 0 && g.N > 0 &&
         g.batch > 0 && g.batch <= 65535 && (g.M + 63) / 64 <= 65535 &&
         (reinterpret_cast<uintptr_t>(g.w) & 15) == 0 && (g.ldw % 8) == 0 && (g.sw % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(g.x) & 15) == 0 && (g.ldx % 8) == 0 && (g.sx % 8) == 0;
}

// Tile width, k split and ring depth.  Wide tiles (fewer re-reads of x per weight byte)
// pay off when both N and the k range are long; otherwise narrower tiles spread better.
// The k split is the smallest divisor of the chunk count whose grid fills about 3/4 of the
// 256 CUs.  The ring is the deepest compiled one that turns a whole number of times over a
// workgroup's chunks: the weight bytes in flight per CU, not the access pattern, bound
// these short streams (the fragment pattern itself streams at full HBM rate once enough
// loads are outstanding).  (Chosen from measurements at the DeepSeek-V2 projection shapes
// with M = 64.)
void gemm_rows_plan(const GemmArgs& g, int* tn, int* ks, int* ring) {
  const int chunks = g.K / KC;
  const int64_t mb = (g.M + 63) / 64;
  const int t = (g.N >= 4096 && g.K >= 8192) ? 4 : (g.N >= 4096 ? 2 : 1);
  const int64_t nb = (g.N + 64 * t - 1) / (64 * t);
  *tn = t;
  *ks = 1;
  for (int d = 1; d <= chunks; ++d) {
    if (chunks % d != 0) continue;
    if (static_cast<int64_t>(g.batch) * d > 65535) break;
    *ks = d;
    if (nb * mb * g.batch * d >= 192) break;
  }
  const int per = chunks / *ks;
  *ring = 4;
  if (t < 4)  // four-tile waves already hold 12 KB in flight per wave with the shallow ring
    for (int r = 20; r > 4; r -= 4)
      if (ring_ok(t, r) && per % (r / 4) == 0) { *ring = r; break; }
}

bool gemm_rows_plan_ok(const GemmArgs& g, int tn, int ks, int ring) {
  const int chunks = g.K / KC;
  return (tn == 1 || tn == 2 || tn == 4) && ks >= 1 && chunks % ks == 0 &&
         static_cast<int64_t>(g.batch) * ks <= 65535 && ring_ok(tn, ring) &&
         (chunks / ks) % (ring / 4) == 0;
}

hipError_t launch_gemm_rows_with(const GemmArgs& g, int tn, int ks, int ring, hipStream_t s) {
  if (!gemm_rows_plan_ok(g, tn, ks, ring)) return hipErrorInvalidValue;
  return g.x_bf16 ? launch_x<bf16raw>(g, tn, ks, ring, s) : launch_x<float>(g, tn, ks, ring, s);
}

hipError_t launch_gemm_rows(const GemmArgs& g, hipStream_t s) {
  int tn = 1, ks = 1, ring = 4;
  gemm_rows_plan(g, &tn, &ks, &ring);
  return launch_gemm_rows_with(g, tn, ks, ring, s);
}

}  // namespace mla
