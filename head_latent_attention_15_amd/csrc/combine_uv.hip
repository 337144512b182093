// Split-K combine fused with the W^UV up-projection: for every sequence b and head i
//   o~_{b,i} = sum_s e^{lse_s - M} o_part[b][i][s] / sum_s e^{lse_s - M}     (M = max_s lse_s)
//   o_heads[b][i][:] = W^UV_i o~_{b,i}
// The combine re-assembles one softmax whose token sum was cut into disjoint ranges
// (qiita.com/joule "Attention 計算"); applying W^UV_i only after the weighted sum of latents
// is the value side of the absorbed order ("論文解説: DeepSeek-V2 …", "行列吸収トリック";
// kasblo.com/?p=4663, "V側は、小さな表現の加重和を先に求める").  Fusing the two keeps o~ on
// the chip: it is never written to HBM and read back.
//
// One workgroup (8 wavefronts) per (head, block of ROWS = 16 or 32 sequences; 32 once
// 16-row blocks would need more than one workgroup per CU).  Phase 1: the 512 / ROWS lanes
// of a sequence each merge ROWS latent columns (16-byte loads per split), with the split
// weights computed once per sequence across those lanes and passed around by shuffle; the
// result is stored in LDS as two bf16 planes (hi + rounding remainder: about 16
// significant bits, so every product with a bf16 weight is exact in fp32).  Phase 2:
// wavefront w computes output columns 16 w .. 16 w + 15 of all ROWS sequences on
// v_mfma_f32_16x16x32_bf16 (A = o~ from LDS, B = W^UV_i rows straight from HBM into
// registers, 16 contiguous bytes per lane and k-step); those loads go out right after the
// partial loads, so they are in flight during the combine.
//
// Workgroups go to the 8 XCDs in turn; with H a multiple of 8 the blocks of one head are
// numbered so that they share an XCD (and run at about the same time): W^UV_i comes from
// HBM about once and from that XCD's L2 for the others.  Deterministic: fixed summation
// orders, no atomics.
#include "device_common.h"
#include "launchers.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int CU_DC = 512;                 // latent width
constexpr int CU_DH = 128;                 // head width: 8 wavefronts x 16 columns
constexpr int CU_MAXS = 64;                // splits handled
constexpr int CU_ROWB = CU_DC * 2 + 16;    // LDS bytes per row of one plane (padded)

// two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, a in the low half
__device__ __forceinline__ unsigned pack2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// N consecutive partial values of one split as loaded (bf16: N / 8 16-byte loads, kept
// packed until use; fp32: N / 4)
template <typename PT, int N> struct RawN;
template <int N> struct RawN<bf16raw, N> {
  uint4 u[N / 8];
  __device__ __forceinline__ void load(const bf16raw* p) {
#pragma unroll
    for (int i = 0; i < N / 8; ++i) u[i] = *reinterpret_cast<const uint4*>(p + 8 * i);
  }
  __device__ __forceinline__ float at(int i) const {
    const uint4 h = u[i >> 3];
    const int k = (i >> 1) & 3;
    const unsigned w = k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <int N> struct RawN<float, N> {
  f32x4_t u[N / 4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) u[i] = *reinterpret_cast<const f32x4_t*>(p + 4 * i);
  }
  __device__ __forceinline__ float at(int i) const { return u[i >> 2][i & 3]; }
};

// ROWS sequences per workgroup (16 or 32): TPR = 512 / ROWS lanes per sequence, each
// merging ROWS consecutive latent columns; lane q of a sequence's lane group holds the lse
// of splits q + TPR k; CHUNK splits' loads in flight at a time.
template <typename PT, int ROWS>
__global__ __launch_bounds__(512) void combine_uv_kernel(const PT* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         const bf16raw* __restrict__ w_uv,
                                                         float* __restrict__ o_heads, int B,
                                                         int H, int S) {
  constexpr int TPR = 512 / ROWS, CPT = ROWS, NL = CU_MAXS / TPR, MT = ROWS / 16;
  constexpr int CHUNK = ROWS == 16 ? 4 : 2;
  constexpr int PLANE = ROWS * CU_ROWB;
  static_assert(CU_MAXS % CHUNK == 0 && TPR * CPT == CU_DC, "layout");
  __shared__ __attribute__((aligned(16))) char smem[2 * PLANE];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const int nbb = (B + ROWS - 1) / ROWS;
  int head, bb;
  if (H % 8 == 0) {  // blocks of head i on XCD i % 8, consecutive on it
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    head = xcd + 8 * (slot / nbb);
    bb = slot - (slot / nbb) * nbb;
  } else {
    head = blockIdx.x / nbb;
    bb = blockIdx.x - head * nbb;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;

  // ---- phase 1 inputs: sequence rr = t / TPR of the block (rows past B re-read row B - 1
  //      and store nothing), columns CPT q .. CPT q + CPT - 1.  Every load of the first
  //      CHUNK splits and of W^UV_i is issued before anything waits (indices past S re-read
  //      split S - 1; such splits get weight 0), in this order: lse, partials, W^UV.
  const int rr = tid / TPR, q = tid % TPR;
  const int b = min(bb * ROWS + rr, B - 1);
  const int64_t bh = static_cast<int64_t>(b) * H + head;
  float lraw[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) lraw[k] = lse_part[bh * S + min(q + TPR * k, S - 1)];
  const PT* src = o_part + bh * S * CU_DC + CPT * q;
  RawN<PT, CPT> v[CHUNK];
#pragma unroll
  for (int j = 0; j < CHUNK; ++j) v[j].load(src + static_cast<int64_t>(min(j, S - 1)) * CU_DC);
  // W^UV_i rows 16 wv + r: lane (g, r) takes columns 32 ks + 8 g .. + 7 for every k-step
  const bf16raw* wsrc =
      w_uv + (static_cast<int64_t>(head) * CU_DH + 16 * wv + r) * CU_DC + 8 * g;
  uint4 wreg[CU_DC / 32];
#pragma unroll
  for (int ks = 0; ks < CU_DC / 32; ++ks)
    wreg[ks] = *reinterpret_cast<const uint4*>(wsrc + 32 * ks);
  __builtin_amdgcn_sched_barrier(0);

  // ---- split weights of the sequence: max and sum over its TPR lanes
  float l[NL], wgt[NL];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    l[k] = q + TPR * k < S ? lraw[k] : -INFINITY;
    m = fmaxf(m, l[k]);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float msafe = (m == -INFINITY) ? 0.f : m;
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    wgt[k] = (l[k] == -INFINITY) ? 0.f : expf(l[k] - msafe);
    den += wgt[k];
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
  const float inv = den > 0.f ? 1.f / den : 0.f;

  // ---- weighted sum of the partials, CHUNK splits at a time
  float acc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) acc[i] = 0.f;
  const int rowbase = lane & (64 - TPR);
  for (int s0 = 0;;) {
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) {
      const int s = s0 + j;  // < 64: CHUNK divides CU_MAXS
      float w = 0.f;  // 0 for s >= S and for empty splits
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        const float t = __shfl(wgt[k], rowbase + s % TPR, 64);
        w = s / TPR == k ? t : w;
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i)  // a weight-0 split adds exactly 0 (never its values)
        acc[i] = fmaf(w, w != 0.f ? v[j].at(i) : 0.f, acc[i]);
    }
    s0 += CHUNK;
    if (s0 >= S) break;
#pragma unroll
    for (int j = 0; j < CHUNK; ++j)
      v[j].load(src + static_cast<int64_t>(min(s0 + j, S - 1)) * CU_DC);
  }

  // ---- o~ -> LDS as hi and lo bf16 planes, row rr, bytes 2 CPT q .. + 2 CPT - 1
  {
    lds_char_t* dst = lsm + rr * CU_ROWB + 2 * CPT * q;
#pragma unroll
    for (int c = 0; c < CPT / 8; ++c) {
      u32x4_t hi, lo;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = acc[8 * c + 2 * p] * inv, e = acc[8 * c + 2 * p + 1] * inv;
        const unsigned h2 = pack2(a, e);
        hi[p] = h2;
        lo[p] = pack2(a - __uint_as_float(h2 << 16), e - __uint_as_float(h2 & 0xffff0000u));
      }
      *(lds_u32x4_t*)(dst + 16 * c) = hi;
      *(lds_u32x4_t*)(dst + PLANE + 16 * c) = lo;
    }
  }
  __syncthreads();

  // ---- phase 2: C[b][j] = sum_c o~[b][c] W^UV_i[j][c], wave wv: j = 16 wv .. 16 wv + 15
  f32x4_t c4[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) c4[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < CU_DC / 32; ++ks) {
    const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, wreg[ks]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const lds_char_t* ap = lsm + (16 * mt + r) * CU_ROWB + 64 * ks + 16 * g;
      const bf16x8_t ah = *(const lds_bf16x8_t*)ap;
      const bf16x8_t al = *(const lds_bf16x8_t*)(ap + PLANE);
      c4[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, c4[mt], 0, 0, 0);
      c4[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, c4[mt], 0, 0, 0);
    }
  }
  // lane (g, r): rows 16 mt + 4 g .. + 3 of the block, column 16 wv + r
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bo = bb * ROWS + 16 * mt + 4 * g + e;
      if (bo < B)
        o_heads[(static_cast<int64_t>(bo) * H + head) * CU_DH + 16 * wv + r] = c4[mt][e];
    }
}

}  // namespace

bool combine_uv_supported(int H, int S, int d_c, int d_h, const void* o_part, const void* w_uv,
                          int B) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(o_part) | reinterpret_cast<uintptr_t>(w_uv);
  const int64_t blocks = static_cast<int64_t>(H) * ((B + 15) / 16);
  return d_c == CU_DC && d_h == CU_DH && S >= 1 && S <= CU_MAXS && (a & 15) == 0 &&
         blocks <= 0x7fffffff;
}

// 16-sequence blocks while they fit one workgroup per CU in one round; 32 beyond (the
// kernel's registers allow one workgroup per CU)
template <typename PT>
static hipError_t launch_rows(const PT* o_part, const float* lse_part, const bf16raw* w_uv,
                              float* o_heads, int B, int H, int S, hipStream_t s) {
  const int64_t blocks16 = static_cast<int64_t>(H) * ((B + 15) / 16);
  if (blocks16 > 256 && B > 16)
    hipLaunchKernelGGL((combine_uv_kernel<PT, 32>), dim3(H * ((B + 31) / 32)), dim3(512), 0, s,
                       o_part, lse_part, w_uv, o_heads, B, H, S);
  else
    hipLaunchKernelGGL((combine_uv_kernel<PT, 16>), dim3(static_cast<unsigned>(blocks16)),
                       dim3(512), 0, s, o_part, lse_part, w_uv, o_heads, B, H, S);
  return hipGetLastError();
}

hipError_t launch_combine_uv(const void* o_part, int part_bf16, const float* lse_part,
                             const void* w_uv, float* o_heads, int B, int H, int S,
                             hipStream_t s) {
  if (part_bf16)
    return launch_rows(static_cast<const bf16raw*>(o_part), lse_part,
                       static_cast<const bf16raw*>(w_uv), o_heads, B, H, S, s);
  return launch_rows(static_cast<const float*>(o_part), lse_part,
                     static_cast<const bf16raw*>(w_uv), o_heads, B, H, S, s);
}

}  // namespace mla
