// Query absorption on bf16 MFMA: q~_i = W^UK_i^T q^C_i for every head i
// ("論文解説: DeepSeek-V2 …", "行列吸収トリック"; kasblo.com/?p=4663, "K側は…Qを変換する"):
//   q~[b][i][c] = sum_j q^C[b][i][j] * W^UK[i d_h + j][c]
// W^UK is stored [H d_h][d_c] (the nn.Linear layout of the up-projection), so for the
// absorption the contraction index j runs down its rows.  One workgroup per (head,
// 128-column block of c, 64-row block of b) copies its 128 x d_h block of W^UK into LDS
// transposed ([c][j], so an MFMA operand is one 16-byte read) and q^C_i as two bf16 planes
// (x = hi + lo, about 16 significant bits of the fp32 input; every product with a bf16
// weight is exact in fp32), then computes the 128 x 64 block of q~^T on
// v_mfma_f32_16x16x32_bf16: A = W^UK_i^T (c x j), B = q^C_i^T (j x b).  Each lane's C
// entries are four consecutive c of one b, written as one 8-byte bf16 store.  At the
// DeepSeek-V2 sizes the same launch also rotates the query's RoPE part (qiita.com/joule,
// "RoPE の扱い"), so the absorption step is one kernel.
#include "device_common.h"
#include "launchers.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) unsigned short lds_u16_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int AB_DH = 128;                 // d_h (the contraction length)
constexpr int AB_ROW = AB_DH * 2 + 16;     // LDS bytes per [c] or [b] row: bf16, padded
constexpr int AB_W = 128 * AB_ROW;         // W^UK_i^T block: 128 columns c
constexpr int AB_X = 64 * AB_ROW;          // one plane of q^C_i: 64 rows b
constexpr int AB_LDS = AB_W + 2 * AB_X;

// two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, a in the low half;
// branch-free, so the loops around it keep exact memory wait counts
__device__ __forceinline__ unsigned pack2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// The query RoPE rides along when ROPE: for d_c = 512 (four column blocks) and d_R = 64,
// column block x of (row block, head) rotates q^R rows b0 + 16 x .. + 15, two pairs per
// thread; their loads go out before the weight and q^C loads and the fp64 rotation runs
// while those are in flight.
struct AbsorbRope {
  const float* q_r;
  int64_t ld_r;
  const int32_t* seq_lens;
  float base;
  bf16raw* q_pe;
};
constexpr int AB_DR = 64;

template <bool ROPE>
__global__ __launch_bounds__(256) void absorb_kernel(const float* __restrict__ q_c,
                                                     const bf16raw* __restrict__ w_uk,
                                                     bf16raw* __restrict__ q_lat, int B, int H,
                                                     int d_c, int64_t ld_q, AbsorbRope rp) {
  __shared__ __attribute__((aligned(16))) char smem[AB_LDS];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const int c0 = blockIdx.x * 128, b0 = blockIdx.y * 64, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;

  // ---- RoPE inputs: pair e = tid + 256 p is row b0 + 16 blockIdx.x + e / 32, pair e % 32
  //      (rows past B load row B - 1 and store nothing: unconditional loads keep the wait
  //      for them apart from the weight loads issued next)
  float2 rv[2] = {};
  int rpos[2] = {};
  if constexpr (ROPE) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = tid + 256 * p, k = e & 31;
      const int b = min(b0 + 16 * static_cast<int>(blockIdx.x) + (e >> 5), B - 1);
      rv[p] = *reinterpret_cast<const float2*>(rp.q_r + static_cast<int64_t>(b) * rp.ld_r +
                                               h * AB_DR + 2 * k);
      rpos[p] = rp.seq_lens[b] - 1;
    }
  }

  // ---- W^UK_i rows j, columns c0 .. c0 + 127 -> LDS [c][j]: thread t moves 16-byte
  //      pieces q = t + 256 e (row j = q / 16, columns 8 (q % 16) .. + 7)
  const bf16raw* wsrc = w_uk + static_cast<int64_t>(h) * AB_DH * d_c + c0;
  uint4 wv8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = tid + 256 * e, j = q >> 4, cc = (q & 15) * 8;
    wv8[e] = *reinterpret_cast<const uint4*>(wsrc + static_cast<int64_t>(j) * d_c + cc);
  }
  // ---- q^C_i rows b0 .. b0 + 63 (zero past B) -> two bf16 planes [b][j]: thread t converts
  //      row t / 4, columns 32 (t % 4) .. + 31
  const int xr = tid >> 2, xc = (tid & 3) * 32;
  const bool xr_ok = b0 + xr < B;
  const float* xsrc =
      q_c + static_cast<int64_t>(b0 + (xr_ok ? xr : 0)) * ld_q + h * AB_DH + xc;
  f32x4_t xv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xv[i] = *reinterpret_cast<const f32x4_t*>(xsrc + 4 * i);
    if (!xr_ok) xv[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // ---- RoPE while the weight and q^C loads are in flight (the scheduling barrier keeps
  //      its arithmetic, and so its wait, below the last load)
  if constexpr (ROPE) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = tid + 256 * p, b = b0 + 16 * blockIdx.x + (e >> 5), k = e & 31;
      float y0, y1;
      rope_pair(rv[p].x, rv[p].y, rpos[p], k, AB_DR, rp.base, &y0, &y1);
      if (b < B)
        *reinterpret_cast<unsigned*>(rp.q_pe + (static_cast<int64_t>(b) * H + h) * AB_DR +
                                     2 * k) = pack2(y0, y1);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = tid + 256 * e, j = q >> 4, cc = (q & 15) * 8;
    const unsigned u[4] = {wv8[e].x, wv8[e].y, wv8[e].z, wv8[e].w};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      *(lds_u16_t*)(lsm + (cc + k) * AB_ROW + 2 * j) =
          static_cast<unsigned short>((k & 1) ? (u[k >> 1] >> 16) : (u[k >> 1] & 0xffffu));
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    u32x4_t hi, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = xv[i + (p >> 1)][2 * (p & 1)], bb = xv[i + (p >> 1)][2 * (p & 1) + 1];
      hi[p] = pack2(a, bb);
      lo[p] = pack2(a - __uint_as_float(hi[p] << 16), bb - __uint_as_float(hi[p] & 0xffff0000u));
    }
    lds_char_t* dst = lsm + AB_W + xr * AB_ROW + 2 * (xc + 4 * i);
    *(lds_u32x4_t*)dst = hi;
    *(lds_u32x4_t*)(dst + AB_X) = lo;
  }
  __syncthreads();

  // ---- wave wv: column tiles 2 wv, 2 wv + 1 (of 16 c), all four row tiles of 16 b
  f32x4_t acc[2][4];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[n][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < AB_DH / 32; ++ks) {
    bf16x8_t a[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
      a[n] = *(const lds_bf16x8_t*)(lsm + (32 * wv + 16 * n + r) * AB_ROW + 64 * ks + 16 * g);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const lds_char_t* xp = lsm + AB_W + (16 * m + r) * AB_ROW + 64 * ks + 16 * g;
      const bf16x8_t xh = *(const lds_bf16x8_t*)xp;
      const bf16x8_t xl = *(const lds_bf16x8_t*)(xp + AB_X);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        acc[n][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[n], xh, acc[n][m], 0, 0, 0);
        acc[n][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[n], xl, acc[n][m], 0, 0, 0);
      }
    }
  }
  // ---- lane (g, r) of tile (n, m): q~[b0 + 16 m + r][h][c0 + 32 wv + 16 n + 4 g + 0..3]
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int b = b0 + 16 * m + r;
    if (b >= B) continue;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int c = c0 + 32 * wv + 16 * n + 4 * g;
      uint2 v;
      v.x = pack2(acc[n][m][0], acc[n][m][1]);
      v.y = pack2(acc[n][m][2], acc[n][m][3]);
      *reinterpret_cast<uint2*>(q_lat + (static_cast<int64_t>(b) * H + h) * d_c + c) = v;
    }
  }
}

}  // namespace

bool absorb_mfma_supported(int B, int H, int d_h, int d_c, const void* q_c, int64_t ld_q,
                           const void* w_uk, const void* q_lat) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(q_c) | reinterpret_cast<uintptr_t>(w_uk) |
                      reinterpret_cast<uintptr_t>(q_lat);
  return d_h == AB_DH && d_c % 128 == 0 && B >= 1 && (B + 63) / 64 <= 65535 && H <= 65535 &&
         (a & 15) == 0 && ld_q % 4 == 0;
}

bool absorb_rope_fusable(int d_c, int d_R, const float* q_r, int64_t ld_r, const void* q_pe) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(q_r) | reinterpret_cast<uintptr_t>(q_pe);
  return d_c == 4 * 128 && d_R == AB_DR && (a & 7) == 0 && ld_r % 2 == 0;
}

hipError_t launch_absorb_mfma(const float* q_c, int64_t ld_q, const void* w_uk, void* q_lat,
                              int B, int H, int d_c, const float* q_r, int64_t ld_r,
                              const int32_t* seq_lens, float rope_base, void* q_pe,
                              hipStream_t s) {
  const dim3 grid(d_c / 128, (B + 63) / 64, H);
  const AbsorbRope rp{q_r, ld_r, seq_lens, rope_base, static_cast<bf16raw*>(q_pe)};
  if (q_r)
    hipLaunchKernelGGL(absorb_kernel<true>, grid, dim3(256), 0, s, q_c,
                       static_cast<const bf16raw*>(w_uk), static_cast<bf16raw*>(q_lat), B, H,
                       d_c, ld_q, rp);
  else
    hipLaunchKernelGGL(absorb_kernel<false>, grid, dim3(256), 0, s, q_c,
                       static_cast<const bf16raw*>(w_uk), static_cast<bf16raw*>(q_lat), B, H,
                       d_c, ld_q, rp);
  return hipGetLastError();
}

}  // namespace mla
