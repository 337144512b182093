// Activation-stationary weight-streaming GEMM for the projections around the attention:
//   y[m][n] = sum_k x[m][k] * w[n][k]      (M <= 64 rows, w in nn.Linear layout, bf16)
// for W^UQ, W^QR and W^O ("論文解説: DeepSeek-V2 …", query compression; "行列吸収トリック";
// kasblo.com/?p=4663, "V側は、小さな表現の加重和を先に求める").
//
// The k range is cut into slices of KR = 32 S values; a workgroup (one per CU) takes one
// slice of x and a run of consecutive column tiles (128 TN output columns each) in it.  x's
// slice is copied into LDS once (LDS DMA), converted in place into two bf16 planes (hi +
// rounding remainder, about 16 significant bits, so every product with a bf16 weight is
// exact in fp32; bf16 x is copied as is), and then stays: the loop streams only weights.
// All eight wavefronts own TN column tiles of 16 and all four 16-row tiles of x; the bf16
// weight rows go from HBM straight into MFMA B-operand registers (lane (g, r): row n + r,
// 16 contiguous bytes), one tile's S k-steps ahead, so the ring runs on across tiles and
// never restarts.  After each tile the partial sums are added into y (fp32 atomics, y
// zeroed first unless the caller accumulates; the slices of one tile add up there).  The
// loop issues no other global loads and has no barrier: every wait is the exact count of
// the fragment it needs.
#include "device_common.h"
#include "launchers.h"

#include <algorithm>
#include <type_traits>

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int XS_LDS = 160 * 1024;  // x slice: 64 rows x KR values x 4 bytes at most
constexpr int XS_CUS = 256;

// two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, a in the low half
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// 16 bytes per lane from base + voff to LDS address lds_addr + 16 * lane (LDS DMA: no
// destination registers, completion counted by vmcnt); base and lds_addr wave-uniform
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b64 = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b64 >> 32));
  const void* ubase = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
  const uint32_t ulds = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(ulds), "v"(voff), "s"(ubase)
      : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct XsArgs {
  int64_t ldx, ldw, ldy;
  int M, N;
  int NT;   // column tiles
  int nt;   // tiles per workgroup (a run inside one k slice)
  int K;
};

// Plane layout in LDS: row t of plane p (0 hi, 1 lo) starts at t * ROWB + p * HALF, with
// HALF = 2 KR bytes (KR bf16 values) and ROWB = 2 HALF for fp32 x (the raw fp32 row is
// converted in place into its hi and lo halves) or HALF for bf16 x.  Inside a half row the
// 16-byte pieces are XOR-swizzled by the row: piece q sits at q ^ (t & 15), so the 16 rows
// an A-fragment read touches hit 16 different bank groups.
template <typename XT, int TN, int S>
__global__ __launch_bounds__(512) void gemm_xs_kernel(const XT* x, const bf16raw* w, float* y,
                                                      XsArgs a) {
  constexpr bool SPLIT_X = std::is_same<XT, float>::value;
  constexpr int KR = 32 * S;                 // k values per slice
  constexpr int HALF = KR * 2;               // bytes of one bf16 plane row
  constexpr int ROWB = SPLIT_X ? 2 * HALF : HALF;
  constexpr int RAWROW = KR * static_cast<int>(sizeof(XT));  // bytes of one raw x row
  static_assert(RAWROW == ROWB, "in-place layout");
  static_assert(64 * ROWB <= XS_LDS, "x slice fits in LDS");
  constexpr int CW = 128 * TN;               // columns per tile (8 waves x 16 TN)
  constexpr int R = S;                       // weight ring: one tile's k-steps
  __shared__ __attribute__((aligned(16))) char smem[64 * ROWB];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>(lsm));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  // workgroup -> (k slice, first tile); consecutive workgroups walk the tiles of one slice
  const int runs_per_slice = a.NT / a.nt;
  const int slice = blockIdx.x / runs_per_slice;
  const int tile0 = (blockIdx.x - slice * runs_per_slice) * a.nt;
  const int k0 = slice * KR;
  const int ntl = a.nt;
  const int nsteps = S * ntl;

  // ---- weights: lane (g, r) of wave wv reads rows tile * CW + 16 (TN wv + j) + r
  const bf16raw* wlane[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
    wlane[j] = w + static_cast<int64_t>(16 * (TN * wave + j) + r) * a.ldw + k0 + 8 * g;
  // step s of the run: tile tile0 + s / S, k-step s % S.  Past the run the ring still loads
  // (so every wait count stays the same) but from one lane-uniform 16-byte address, the
  // first bytes of w: a broadcast of one line instead of 16 rows of the last tile again.
  auto w_frag = [&](int tl, int ks, int j) {
    const bf16raw* p =
        tl < ntl ? wlane[j] + static_cast<int64_t>(tile0 + tl) * CW * a.ldw + 32 * ks : w;
    return *reinterpret_cast<const bf16x8_t*>(p);
  };
  bf16x8_t wf[R][TN];
#pragma unroll
  for (int i = 0; i < R - 1; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) wf[i][j] = w_frag(0, i, j);

  // ---- x slice: raw rows by LDS DMA.  The slab (row t at t * RAWROW) is filled by 1 KB
  //      copies in order; lane l of copy i fills bytes 1024 i + 16 l, i.e. row t = that /
  //      RAWROW, from x[min(t, M - 1)][k0 ..] (a copy may span two rows)
  constexpr int NCOPY = 64 * RAWROW / 1024;
  static_assert(NCOPY % 8 == 0, "copies split evenly over the waves");
  {
    const char* xb = reinterpret_cast<const char*>(x + k0);
#pragma unroll
    for (int i = 0; i < NCOPY / 8; ++i) {
      const int cp = wave * (NCOPY / 8) + i;
      const int byte = cp * 1024 + lane * 16;
      const int t = byte / RAWROW, o = byte - t * RAWROW;
      const int srow = min(t, a.M - 1);
      dma16(xb, static_cast<uint32_t>(srow * a.ldx * sizeof(XT)) + static_cast<uint32_t>(o),
            smem_lds + cp * 1024);
    }
  }
  asm volatile("" ::: "memory");  // the copies stay behind the weight prefetches

  // ---- wait for everything this wave issued (the weight prefetches went out first, so
  //      they are in flight beside the copies), then for everyone's copies; convert in
  //      place.  Counting to zero keeps the wait independent of how many loads the
  //      compiler emits for the prefetch.
  wait_vmcnt<0>();
  __syncthreads();
  if constexpr (SPLIT_X) {
    // thread t converts 16-byte raw pieces q = t + 512 i (4 floats each) of the slab,
    // row-major: all reads first, a barrier, then the writes (the halves overlap the raw row)
    constexpr int PIECES = 64 * KR / 4;
    constexpr int PER = PIECES / 512;
    f32x4_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 512 * i, t = q / (KR / 4), c = q % (KR / 4);
      v[i] = *(const __attribute__((address_space(3))) f32x4_t*)(lsm + t * ROWB + 16 * c);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 512 * i, t = q / (KR / 4), c = q % (KR / 4);
      // floats 4 c .. 4 c + 3 -> bf16 4 c .. + 3: half of 16-byte piece c / 2
      u32x2_t h, l;
      h[0] = pack_bf16(v[i][0], v[i][1]);
      h[1] = pack_bf16(v[i][2], v[i][3]);
      l[0] = pack_bf16(v[i][0] - __uint_as_float(h[0] << 16), v[i][1] - __uint_as_float(h[0] & 0xffff0000u));
      l[1] = pack_bf16(v[i][2] - __uint_as_float(h[1] << 16), v[i][3] - __uint_as_float(h[1] & 0xffff0000u));
      const int off = t * ROWB + 16 * ((c >> 1) ^ (t & 15)) + 8 * (c & 1);
      *(lds_u32x2_t*)(lsm + off) = h;
      *(lds_u32x2_t*)(lsm + off + HALF) = l;
    }
  } else {
    // bf16 x: swizzle the pieces in place (piece q of row t to position q ^ (t & 15)) --
    // each 16-row group is permuted among its own positions
    constexpr int PIECES = 64 * KR / 8;
    constexpr int PER = PIECES / 512;
    u32x4_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 512 * i, t = q / (KR / 8), c = q % (KR / 8);
      v[i] = *(const lds_u32x4_t*)(lsm + t * ROWB + 16 * c);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + 512 * i, t = q / (KR / 8), c = q % (KR / 8);
      *(lds_u32x4_t*)(lsm + t * ROWB + 16 * (c ^ (t & 15))) = v[i];
    }
  }
  __syncthreads();

  // ---- the run: tile after tile, one turn of the ring per tile
  f32x4_t acc[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const lds_char_t* xa = lsm + r * ROWB;
  for (int tl = 0; tl < ntl; ++tl) {
#pragma unroll
    for (int ks = 0; ks < S; ++ks) {
      // prefetch step tl * S + ks + R - 1 = tile tl + 1, k-step ks - 1 (ks > 0) or tile tl,
      // k-step S - 1 (ks == 0)
      const int ptl = ks == 0 ? tl : tl + 1;
      const int pks = ks == 0 ? S - 1 : ks - 1;
#pragma unroll
      for (int j = 0; j < TN; ++j) wf[(ks + R - 1) % R][j] = w_frag(ptl, pks, j);
      const int piece = (4 * ks + g) ^ r;  // A fragment piece of k-step ks, swizzled by row
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8_t ah = *(const lds_bf16x8_t*)(xa + mt * 16 * ROWB + 16 * piece);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wf[ks][j], acc[j][mt], 0, 0, 0);
        if constexpr (SPLIT_X) {
          const bf16x8_t al = *(const lds_bf16x8_t*)(xa + mt * 16 * ROWB + HALF + 16 * piece);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wf[ks][j], acc[j][mt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // this tile's slice sum into y
    float* yt = y + static_cast<int64_t>(tile0 + tl) * CW + 16 * TN * wave + r;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (16 * mt < a.M) {  // wave-uniform: 16-row tiles wholly past M add nothing
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 16 * mt + 4 * g + e;
            if (m < a.M) atomicAdd(yt + static_cast<int64_t>(m) * a.ldy + 16 * j, acc[j][mt][e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][mt][e] = 0.f;
      }
    // keep the accumulators in their own registers across tiles (folded into the next
    // MFMA as a zero operand, they were renamed into registers the weight ring uses, and
    // the first MFMA of every tile then waited for nearly the whole ring)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) asm volatile("" : "+v"(acc[j][mt]));
  }
}

__global__ __launch_bounds__(256) void zero_rows_xs(float* __restrict__ y, int64_t ldy, int M,
                                                    int N) {
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    float* p = y + static_cast<int64_t>(m) * ldy;
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

template <typename XT, int TN, int S>
hipError_t launch_t(const GemmArgs& g, const XsArgs& a, int grid, hipStream_t s) {
  const int gx = std::min((g.N + 1023) / 1024, 64);
  if (!g.accumulate)
    hipLaunchKernelGGL(zero_rows_xs, dim3(gx, std::min(g.M, 4096)), dim3(256), 0, s,
                       static_cast<float*>(g.y), g.ldy, g.M, g.N);
  hipLaunchKernelGGL((gemm_xs_kernel<XT, TN, S>), dim3(grid), dim3(512), 0, s,
                     static_cast<const XT*>(g.x), static_cast<const bf16raw*>(g.w),
                     static_cast<float*>(g.y), a);
  return hipGetLastError();
}

// compiled (x type, tile, slice) combinations: the slice (fp32 x, 4 bytes per value) or
// (bf16 x) fits in LDS and the ring of S k-steps fits in registers
bool xs_combo_ok(bool x_bf16, int tn, int s) {
  if (tn == 1) return x_bf16 ? (s == 8 || s == 16 || s == 20) : (s == 8 || s == 12 || s == 16);
  if (tn == 2) return x_bf16 ? (s == 8 || s == 16) : (s == 8 || s == 12 || s == 16);
  return false;
}

template <typename XT>
hipError_t launch_x(const GemmArgs& g, const XsArgs& a, int tn, int s, int grid, hipStream_t st) {
  constexpr bool F = std::is_same<XT, float>::value;
  if (tn == 1) {
    switch (s) {
      case 8: return launch_t<XT, 1, 8>(g, a, grid, st);
      case 16: return launch_t<XT, 1, 16>(g, a, grid, st);
      case 12: if constexpr (F) return launch_t<XT, 1, 12>(g, a, grid, st); else break;
      case 20: if constexpr (!F) return launch_t<XT, 1, 20>(g, a, grid, st); else break;
      default: break;
    }
  } else if (tn == 2) {
    switch (s) {
      case 8: return launch_t<XT, 2, 8>(g, a, grid, st);
      case 16: return launch_t<XT, 2, 16>(g, a, grid, st);
      case 12: if constexpr (F) return launch_t<XT, 2, 12>(g, a, grid, st); else break;
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool gemm_xs_supported(const GemmArgs& g) {
  return g.w_bf16 && g.w_nk && !g.y_bf16 && g.batch == 1 && g.M > 0 && g.M <= 64 &&
         g.N > 0 && g.N % 128 == 0 && g.K > 0 && g.K % 256 == 0 &&
         (reinterpret_cast<uintptr_t>(g.w) & 15) == 0 && (g.ldw % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(g.x) & 15) == 0 && (g.ldx % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(g.y) & 3) == 0 &&
         g.ldx * 64 * (g.x_bf16 ? 2 : 4) < (int64_t{1} << 31);  // 32-bit copy offsets
}

bool gemm_xs_plan_ok(const GemmArgs& g, int tn, int s, int grid) {
  if (!xs_combo_ok(g.x_bf16 != 0, tn, s) || g.N % (128 * tn) != 0 || g.K % (32 * s) != 0)
    return false;
  const int64_t nt = g.N / (128 * tn), slices = g.K / (32 * s);
  if (grid < 1 || grid > XS_CUS || (nt * slices) % grid != 0) return false;
  const int64_t run = nt * slices / grid;
  return nt % run == 0;  // a run stays inside one slice
}

// The plan: for each compiled slice the largest workgroup count up to one per CU whose
// runs stay inside a slice; the score is workgroups x slice length (the weight k-steps in
// flight per CU scale with the slice), ties going to the longer slice (x staged fewer
// times, fewer partial sums; at W^UQ 192 workgroups of 512-wide slices measured 22 us
// against 25 us for 256 of 384).  One-tile waves only: with two tiles per wave the compiler places a wait for
// nearly the whole weight ring at the start of every tile (measured in its code), which
// the plan avoids; the two-tile form stays available to mla_linear_planned.
bool gemm_xs_plan(const GemmArgs& g, int* tn, int* s, int* grid) {
  // First choice: the longest slice (12 k-steps or more) whose run is at least 4 tiles with
  // at least 3/4 of the CUs busy: measured on [W^UQ; W^QR] (24576 columns, k = 1536) at
  // 192 x 12-step slices (4 tiles each) against 192 x 16 (3 tiles each), 34.0 against 35.3
  // us, since each workgroup stages its x slice once and then streams a longer run.
  for (int sl : {20, 16, 12}) {
    if (!xs_combo_ok(g.x_bf16 != 0, 1, sl) || g.N % 128 != 0 || g.K % (32 * sl) != 0) continue;
    const int64_t nt = g.N / 128, units = nt * (g.K / (32 * sl));
    for (int gd = static_cast<int>(std::min<int64_t>(units, XS_CUS)); gd >= XS_CUS * 3 / 4; --gd)
      if (units % gd == 0 && nt % (units / gd) == 0 && units / gd >= 4) {
        *tn = 1; *s = sl; *grid = gd;
        return true;
      }
  }
  // Otherwise: the most weight bytes in flight (workgroups x slice length)
  int64_t best = -1;
  for (int t : {1})
    for (int sl : {20, 16, 12, 8}) {
      if (!xs_combo_ok(g.x_bf16 != 0, t, sl) || g.N % (128 * t) != 0 || g.K % (32 * sl) != 0)
        continue;
      const int64_t nt = g.N / (128 * t), units = nt * (g.K / (32 * sl));
      for (int gd = static_cast<int>(std::min<int64_t>(units, XS_CUS)); gd >= 1; --gd) {
        if (units % gd != 0 || nt % (units / gd) != 0) continue;
        const int64_t score = static_cast<int64_t>(gd) * sl * 64 + sl;
        if (score > best) { best = score; *tn = t; *s = sl; *grid = gd; }
        break;
      }
    }
  return best >= 0;
}

hipError_t launch_gemm_xs_with(const GemmArgs& g, int tn, int s, int grid, hipStream_t st) {
  if (!gemm_xs_plan_ok(g, tn, s, grid)) return hipErrorInvalidValue;
  XsArgs a;
  a.ldx = g.ldx; a.ldw = g.ldw; a.ldy = g.ldy;
  a.M = g.M; a.N = g.N; a.K = g.K;
  a.NT = g.N / (128 * tn);
  a.nt = static_cast<int>(static_cast<int64_t>(a.NT) * (g.K / (32 * s)) / grid);
  return g.x_bf16 ? launch_x<bf16raw>(g, a, tn, s, grid, st) : launch_x<float>(g, a, tn, s, grid, st);
}

hipError_t launch_gemm_xs(const GemmArgs& g, hipStream_t st) {
  int tn = 1, s = 8, grid = 1;
  if (!gemm_xs_plan(g, &tn, &s, &grid)) return hipErrorInvalidValue;
  return launch_gemm_xs_with(g, tn, s, grid, st);
}

}  // namespace mla
