// Split-K combine fused with the W^UV up-projection: for every sequence b and head i
//   o~_{b,i} = sum_s e^{lse_s - M} o_part[b][i][s] / sum_s e^{lse_s - M}     (M = max_s lse_s)
//   o_heads[b][i][:] = W^UV_i o~_{b,i}
// The combine re-assembles one softmax whose token sum was cut into disjoint ranges
// (qiita.com/joule "Attention 計算"); applying W^UV_i only after the weighted sum of latents
// is the value side of the absorbed order ("論文解説: DeepSeek-V2 …", "行列吸収トリック";
// kasblo.com/?p=4663, "V側は、小さな表現の加重和を先に求める").  Fusing the two keeps o~ on
// the chip: it is never written to HBM and read back.
//
// One workgroup (8 wavefronts) per (head, block of 16 sequences).  Phase 1: thread t
// combines row t / 32 of the block over 16 latent columns (two 16-byte bf16 loads per
// split), with the split weights computed once per row across its 32 lanes and passed
// around by shuffle; the result is stored in LDS as two bf16 planes (hi + rounding
// remainder: about 16 significant bits, so every product with a bf16 weight is exact in
// fp32).  Phase 2: wavefront w computes output columns 16 w .. 16 w + 15 of all 16 rows on
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
constexpr int CU_ROWS = 16;                // sequences per workgroup
constexpr int CU_ROWB = CU_DC * 2 + 16;    // LDS bytes per row of one plane (padded)
constexpr int CU_PLANE = CU_ROWS * CU_ROWB;
constexpr int CU_MAXS = 64;                // splits handled (two per lane of a row group)
constexpr int CU_CHUNK = 4;                // splits whose loads are issued together

// two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, a in the low half
__device__ __forceinline__ unsigned pack2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// 16 consecutive partial values of one split as loaded (bf16: two 16-byte loads, kept
// packed until use; fp32: four)
template <typename PT> struct Raw16;
template <> struct Raw16<bf16raw> {
  uint4 u[2];
  __device__ __forceinline__ void load(const bf16raw* p) {
    u[0] = *reinterpret_cast<const uint4*>(p);
    u[1] = *reinterpret_cast<const uint4*>(p + 8);
  }
  __device__ __forceinline__ float at(int i) const {
    const uint4 h = u[i >> 3];
    const unsigned w = ((i >> 1) & 3) == 0 ? h.x : ((i >> 1) & 3) == 1 ? h.y
                     : ((i >> 1) & 3) == 2 ? h.z : h.w;
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <> struct Raw16<float> {
  f32x4_t u[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = *reinterpret_cast<const f32x4_t*>(p + 4 * i);
  }
  __device__ __forceinline__ float at(int i) const { return u[i >> 2][i & 3]; }
};

template <typename PT>
__global__ __launch_bounds__(512) void combine_uv_kernel(const PT* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         const bf16raw* __restrict__ w_uv,
                                                         float* __restrict__ o_heads, int B,
                                                         int H, int S) {
  __shared__ __attribute__((aligned(16))) char smem[2 * CU_PLANE];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const int nbb = (B + CU_ROWS - 1) / CU_ROWS;
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

  // ---- phase 1 inputs: row rr = t / 32 of the block (rows past B re-read row B - 1 and
  //      store nothing), columns 16 q .. 16 q + 15; lane q of the row group holds the lse
  //      of splits q and q + 32.  Every load of the first CU_CHUNK splits and of W^UV_i is
  //      issued before anything waits (indices past S re-read split S - 1; such splits get
  //      weight 0), in this order: lse, partials, W^UV.
  const int rr = tid >> 5, q = tid & 31;
  const int b = min(bb * CU_ROWS + rr, B - 1);
  const int64_t bh = static_cast<int64_t>(b) * H + head;
  const float l0raw = lse_part[bh * S + min(q, S - 1)];
  const float l1raw = lse_part[bh * S + min(q + 32, S - 1)];
  const PT* src = o_part + bh * S * CU_DC + 16 * q;
  Raw16<PT> v[CU_CHUNK];
#pragma unroll
  for (int j = 0; j < CU_CHUNK; ++j)
    v[j].load(src + static_cast<int64_t>(min(j, S - 1)) * CU_DC);
  // W^UV_i rows 16 wv + r: lane (g, r) takes columns 32 ks + 8 g .. + 7 for every k-step
  const bf16raw* wsrc =
      w_uv + (static_cast<int64_t>(head) * CU_DH + 16 * wv + r) * CU_DC + 8 * g;
  uint4 wreg[CU_DC / 32];
#pragma unroll
  for (int ks = 0; ks < CU_DC / 32; ++ks)
    wreg[ks] = *reinterpret_cast<const uint4*>(wsrc + 32 * ks);
  __builtin_amdgcn_sched_barrier(0);

  // ---- split weights of the row: max and sum over the 32 lanes of the row group
  const float l0 = q < S ? l0raw : -INFINITY;
  const float l1 = q + 32 < S ? l1raw : -INFINITY;
  float m = fmaxf(l0, l1);
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float msafe = (m == -INFINITY) ? 0.f : m;
  const float w0 = (l0 == -INFINITY) ? 0.f : expf(l0 - msafe);
  const float w1 = (l1 == -INFINITY) ? 0.f : expf(l1 - msafe);
  float den = w0 + w1;
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
  const float inv = den > 0.f ? 1.f / den : 0.f;

  // ---- weighted sum of the partials, CU_CHUNK splits at a time
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int rowbase = lane & 32;
  for (int s0 = 0;;) {
#pragma unroll
    for (int j = 0; j < CU_CHUNK; ++j) {
      const int s = s0 + j;  // < 64: CU_CHUNK divides CU_MAXS
      const float wa = __shfl(w0, rowbase + (s & 31), 64);
      const float wb = __shfl(w1, rowbase + (s & 31), 64);
      const float w = s < 32 ? wa : wb;  // 0 for s >= S and for empty splits
#pragma unroll
      for (int i = 0; i < 16; ++i)  // a weight-0 split adds exactly 0 (never its values)
        acc[i] = fmaf(w, w != 0.f ? v[j].at(i) : 0.f, acc[i]);
    }
    s0 += CU_CHUNK;
    if (s0 >= S) break;
#pragma unroll
    for (int j = 0; j < CU_CHUNK; ++j)
      v[j].load(src + static_cast<int64_t>(min(s0 + j, S - 1)) * CU_DC);
  }

  // ---- o~ -> LDS as hi and lo bf16 planes, row rr, bytes 32 q .. 32 q + 31
  {
    u32x4_t hi[2], lo[2];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float a = acc[2 * p] * inv, c = acc[2 * p + 1] * inv;
      const unsigned h2 = pack2(a, c);
      hi[p >> 2][p & 3] = h2;
      lo[p >> 2][p & 3] =
          pack2(a - __uint_as_float(h2 << 16), c - __uint_as_float(h2 & 0xffff0000u));
    }
    lds_char_t* dst = lsm + rr * CU_ROWB + 32 * q;
    *(lds_u32x4_t*)dst = hi[0];
    *(lds_u32x4_t*)(dst + 16) = hi[1];
    *(lds_u32x4_t*)(dst + CU_PLANE) = lo[0];
    *(lds_u32x4_t*)(dst + CU_PLANE + 16) = lo[1];
  }
  __syncthreads();

  // ---- phase 2: C[b][j] = sum_c o~[b][c] W^UV_i[j][c], wave wv: j = 16 wv .. 16 wv + 15
  f32x4_t c4 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < CU_DC / 32; ++ks) {
    const lds_char_t* ap = lsm + r * CU_ROWB + 64 * ks + 16 * g;
    const bf16x8_t ah = *(const lds_bf16x8_t*)ap;
    const bf16x8_t al = *(const lds_bf16x8_t*)(ap + CU_PLANE);
    const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, wreg[ks]);
    c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, c4, 0, 0, 0);
    c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, c4, 0, 0, 0);
  }
  // lane (g, r): rows 4 g .. 4 g + 3 of the block, column 16 wv + r
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bo = bb * CU_ROWS + 4 * g + e;
    if (bo < B)
      o_heads[(static_cast<int64_t>(bo) * H + head) * CU_DH + 16 * wv + r] = c4[e];
  }
}

}  // namespace

bool combine_uv_supported(int H, int S, int d_c, int d_h, const void* o_part, const void* w_uv,
                          int B) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(o_part) | reinterpret_cast<uintptr_t>(w_uv);
  const int64_t blocks = static_cast<int64_t>(H) * ((B + CU_ROWS - 1) / CU_ROWS);
  return d_c == CU_DC && d_h == CU_DH && S >= 1 && S <= CU_MAXS && (a & 15) == 0 &&
         blocks <= 0x7fffffff;
}

hipError_t launch_combine_uv(const void* o_part, int part_bf16, const float* lse_part,
                             const void* w_uv, float* o_heads, int B, int H, int S,
                             hipStream_t s) {
  const int blocks = H * ((B + CU_ROWS - 1) / CU_ROWS);
  if (part_bf16)
    hipLaunchKernelGGL(combine_uv_kernel<bf16raw>, dim3(blocks), dim3(512), 0, s,
                       static_cast<const bf16raw*>(o_part), lse_part,
                       static_cast<const bf16raw*>(w_uv), o_heads, B, H, S);
  else
    hipLaunchKernelGGL(combine_uv_kernel<float>, dim3(blocks), dim3(512), 0, s,
                       static_cast<const float*>(o_part), lse_part,
                       static_cast<const bf16raw*>(w_uv), o_heads, B, H, S);
  return hipGetLastError();
}

}  // namespace mla
