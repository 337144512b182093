// Persistent weight-streaming GEMM for the projections around the attention, on bf16 MFMA:
//   y[z][m][n] = sum_k x[z][m][k] * w[z][n][k]      (M <= 64 rows, w in nn.Linear layout)
// for W^DQ, W^UQ, W^QR, W^DKV, W^KR ("論文解説: DeepSeek-V2 …", "Low-Rank Key-Value Joint
// Compression" and the query compression beside it), the per-head W^UV_i and W^O
// ("行列吸収トリック"; kasblo.com/?p=4663, "V側は、小さな表現の加重和を先に求める").
//
// At decode batch sizes the weights are the traffic, read once, and the loaded HBM latency
// is several microseconds: the rate is set by the weight bytes in flight across the chip and
// by keeping every CU busy for the whole launch.  So the work is cut into units of one
// column tile (64 TN output columns) by 128 k, numbered tile-major, and each workgroup (one
// per CU) takes an equal run of consecutive units.  Its weight stream never restarts: the
// ring of weight fragments runs on across unit and tile boundaries, and the partial sums of
// a tile are flushed when the run leaves the tile: into y with fp32 atomics (y zeroed first
// unless the caller accumulates), or, in the deterministic form, with plain stores into the
// tile's own slot of a caller workspace, which gemm_stream_reduce then sums in one fixed
// order (slice, then run) into y.  For [W^DQ; W^DKV; W^KR] h that summing launch can also
// write the new token's cache row [c^KV | RoPE(k^R)] (qiita.com/joule "RoPE の扱い";
// "論文解説: DeepSeek-V2 …", "Decoupled RoPE"): it is the first point where whole rows of
// c^KV and k^R exist, since the product splits their k range over workgroups.
//
// A workgroup has two roles.  Waves 0-3 (consumers) own TN column tiles of 16 each and all
// four 16-row tiles of x; the bf16 weight rows go from HBM straight into MFMA B-operand
// registers (lane (g, r): w[n + r][k + 8 g .. + 7]), R - 1 k-steps ahead.  Waves 4-7
// (producers) stage x through LDS, each 16 rows, two units ahead: fp32 x as two bf16 terms
// (hi + rounding remainder, about 16 significant bits, so every product with a bf16 weight
// is exact in fp32), bf16 x as is.  The consumers issue no other global loads, so every
// wait in their loop is the exact count for the fragment it needs.  One barrier per unit
// hands a staged chunk of x from producers to consumers.
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
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int KC = 128;                  // k per unit (4 MFMA k-steps)
constexpr int XROW = KC * 2;             // LDS bytes per staged bf16 row
constexpr int XPLANE = 64 * XROW;        // one plane (hi or lo) of 64 rows: 16 KB
constexpr int RAWROW = KC * 4;           // LDS bytes per raw fp32 row
constexpr int RAWUNIT = 64 * RAWROW;     // raw fp32 x of one unit: 32 KB
// fp32 x: two hi + lo plane buffers and three raw units in flight; bf16 x: four planes
// filled by the copies directly
constexpr int PLANES_F32 = 2, RAWS_F32 = 3, PLANES_BF16 = 4;
constexpr int GS_LDS = PLANES_F32 * 2 * XPLANE + RAWS_F32 * RAWUNIT;  // 160 KB
static_assert(GS_LDS <= 163840 && PLANES_BF16 * XPLANE <= GS_LDS, "LDS per workgroup");
constexpr int GS_CUS = 256;              // workgroups per launch at most (one per CU)

// Staged rows are stored with their 16-byte pieces XOR-swizzled by the row index: piece q
// of row t sits at position q ^ (t & 15).  The 16 lanes that read or write one piece index
// across 16 consecutive rows then hit 16 different bank groups.
__device__ __forceinline__ int swz(int q, int t) { return q ^ (t & 15); }

// 16 bytes per lane from base + voff (global) to LDS address lds_addr + 16 * lane, on the
// LDS DMA path (no destination registers; completion counted by vmcnt).  base and lds_addr
// are wave-uniform; M0 carries the LDS address and the s_nop covers the M0 write hazard.
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

// two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, a in the low half
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

struct StreamArgs {
  int64_t ldx, sx, ldw, sw, ldy, sy;
  int M, N;
  int NB;   // column tiles per batch entry
  int NCH;  // units (128-wide k chunks) per tile
  int nu;   // units per workgroup
  int ksl;  // k slices (1, 2, 4 or 8): workgroup g works in slice (g % 8) % ksl
  // deterministic form (part != nullptr): the partial tile of run q of slice sl for tile t
  // goes to slot (sl * ntiles + t) * jmax + q - (t * cps) / nu, M rows of 64 TN floats
  float* part;
  int ntiles, jmax;
};

// Work units.  Workgroups go to the 8 XCDs in turn (g -> XCD g % 8).  The k chunks are cut
// into ksl slices and slice s is worked by the XCDs x with x % ksl == s, over all column
// tiles, so an XCD's workgroups re-read only 1 / ksl of x, which then stays in that XCD's
// L2.  Inside a slice the units are numbered tile-major; workgroup g takes run q of them.
struct Unit {
  int z, cb, ch;  // batch entry, column tile, k chunk
  bool tile_end;  // last unit of its tile inside the slice
};
struct UnitMap {
  int slice, cps, run, v0, nu, NB;
  __device__ UnitMap(const StreamArgs& a, int g)
      : slice((g & 7) % a.ksl), cps(a.NCH / a.ksl), run((g >> 3) * (8 / a.ksl) + (g & 7) / a.ksl),
        v0(run * a.nu), nu(a.nu), NB(a.NB) {}
  // unit i of the run; past the run it repeats the last unit
  __device__ Unit operator()(int i) const {
    const int v = v0 + min(i, nu - 1);
    const int tile = v / cps;
    const int c = v - tile * cps;
    const int z = tile / NB;
    return Unit{z, tile - z * NB, slice * cps + c, c == cps - 1};
  }
};

// ---------------- consumers ----------------
// (they end with a full wait on their own memory operations: the compiler lays the role
// split out with a path from the end of this code into the producers', and would otherwise
// merge this role's outstanding loads into the producers' wait counts)
template <typename XT, int TN, int R, bool DET>
__device__ __forceinline__ void consume(const XT* x, const bf16raw* w, float* y,
                                        const StreamArgs& a, lds_char_t* lsm, int wave, int g,
                                        int r, int nu, const UnitMap& unit_of) {
  constexpr bool SPLIT_X = std::is_same<XT, float>::value;
  constexpr int CW = 64 * TN;
  constexpr int UPT = R / 4;
  constexpr int NPL = SPLIT_X ? PLANES_F32 : PLANES_BF16;
  const int col = wave * 16 * TN + r;  // + 16 j: this lane's weight row inside the tile
  const int nsteps = 4 * nu;
  // scalar element offset of unit i's weights (tile rows from cb * CW, k from ch * KC)
  auto unit_w = [&](int i) {
    const Unit u = unit_of(i);
    return u.z * a.sw + static_cast<int64_t>(u.cb) * CW * a.ldw + u.ch * KC;
  };
  const bf16raw* wlane[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) wlane[j] = w + static_cast<int64_t>(col + 16 * j) * a.ldw + 8 * g;
  auto w_frag = [&](int64_t base, int kstep, int j) {
    return *reinterpret_cast<const bf16x8_t*>(wlane[j] + base + 32 * kstep);
  };

  f32x4_t acc[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prefetch steps 0 .. R - 2 (units 0 .. UPT - 1; clamped past the run)
  bf16x8_t wf[R][TN];
  {
    int64_t ub[UPT];
#pragma unroll
    for (int q = 0; q < UPT; ++q) ub[q] = unit_w(q);
#pragma unroll
    for (int i = 0; i < R - 1; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) wf[i][j] = w_frag(ub[i >> 2], min(i, nsteps - 1) & 3, j);
  }
  __syncthreads();

  for (int t0 = 0; t0 < nu; t0 += UPT) {
    // weight bases of the units whose fragments this turn prefetches: step 4 t0 + s + R - 1
    // for s < R lies in unit t0 + UPT - 1 + (s + 3) / 4, i.e. units t0 + UPT - 1 .. t0 + 2 UPT - 1
    int64_t pb[UPT + 1];
#pragma unroll
    for (int q = 0; q <= UPT; ++q) pb[q] = unit_w(t0 + UPT - 1 + q);
#pragma unroll
    for (int uu = 0; uu < UPT; ++uu) {
      const int i = t0 + uu;
      // A fragment of k-step k, row tile mt: row 16 mt + r, piece 4 k + g (swizzled by r)
      const lds_char_t* xa = lsm + (i % NPL) * (SPLIT_X ? 2 : 1) * XPLANE + r * XROW;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int slot = 4 * uu + k;               // == step % R
        const int ps = slot + R - 1;               // prefetched step, relative to 4 t0
        const int pstep = 4 * t0 + ps;
        // past the last step the prefetch repeats the last fragment (L2-resident)
        const int pk = pstep < nsteps ? (ps & 3) : 3;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          wf[(slot + R - 1) % R][j] = w_frag(pb[(ps >> 2) - (UPT - 1)], pk, j);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8_t ah = *(const lds_bf16x8_t*)(xa + mt * 16 * XROW + 16 * swz(4 * k + g, r));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wf[slot][j], acc[j][mt], 0, 0, 0);
          if constexpr (SPLIT_X) {
            const bf16x8_t al = *(const lds_bf16x8_t*)(xa + XPLANE + mt * 16 * XROW + 16 * swz(4 * k + g, r));
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wf[slot][j], acc[j][mt], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the run leaves this tile after unit i: add its partial sums into y, or store them
      // in the tile's slot of the workspace
      const Unit u = unit_of(i);
      if (i == nu - 1 || u.tile_end) {
        if constexpr (DET) {
          const int t = u.z * a.NB + u.cb;
          const int q = unit_of.run - (t * unit_of.cps) / nu;
          float* pt = a.part +
                      ((static_cast<int64_t>(unit_of.slice) * a.ntiles + t) * a.jmax + q) * a.M * CW + col;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int m = 16 * mt + 4 * g + e;
                if (m < a.M) pt[m * CW + 16 * j] = acc[j][mt][e];
                acc[j][mt][e] = 0.f;
              }
        } else {
          float* yt = y + u.z * a.sy + static_cast<int64_t>(u.cb) * CW + col;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int m = 16 * mt + 4 * g + e;
                if (m < a.M) atomicAdd(yt + static_cast<int64_t>(m) * a.ldy + 16 * j, acc[j][mt][e]);
                acc[j][mt][e] = 0.f;
              }
        }
      }
      __syncthreads();
    }
  }
  wait_vmcnt<0>();
}

template <typename XT, int TN, int R, bool DET>
__global__ __launch_bounds__(512) void gemm_stream_kernel(const XT* x, const bf16raw* w,
                                                          float* y, StreamArgs a) {
  constexpr bool SPLIT_X = std::is_same<XT, float>::value;  // fp32 x: hi + lo planes
  constexpr int CW = 64 * TN;                                // columns per tile
  constexpr int UPT = R / 4;                                 // units per turn of the ring
  static_assert(R % 4 == 0 && R >= 4, "ring of whole units");
  __shared__ __attribute__((aligned(16))) char smem[GS_LDS];
  lds_char_t* const lsm = (lds_char_t*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int nu = a.nu;
  const UnitMap unit_of(a, blockIdx.x);

  constexpr int NPL = SPLIT_X ? PLANES_F32 : PLANES_BF16;  // plane buffers
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<size_t>(lsm));

  if (wave < 4) {
    consume<XT, TN, R, DET>(x, w, y, a, lsm, wave, g, r, nu, unit_of);
  } else {
    // ---------------- producers: x of unit i -> plane buffer i % NPL ----------------
    // Wave p stages rows 16 p .. 16 p + 15 with LDS DMA copies of 1 KB (its only global
    // accesses, so its waits are exact counts).  fp32 x: each copy brings two 512-byte rows
    // into a raw buffer (three units in flight); after its own copies land the wave converts
    // its rows into the hi and lo planes.  bf16 x: each copy brings four 256-byte rows
    // straight into a plane buffer (three units in flight, four buffers).  Rows past M copy
    // row M - 1: their products land in rows of y that are never written.
    const int p = wave - 4;
    constexpr int CPU_ = SPLIT_X ? 8 : 4;                     // copies per wave and unit
    constexpr int RPC = SPLIT_X ? 2 : 4;                      // rows per copy
    constexpr int PPR = SPLIT_X ? RAWROW / 16 : XROW / 16;    // 16-byte pieces per row
    auto issue = [&](int i) {
      const Unit u = unit_of(i);
      const char* base = reinterpret_cast<const char*>(x + u.z * a.sx + u.ch * KC);
      const uint32_t dst = SPLIT_X ? smem_lds + NPL * 2 * XPLANE + (i % RAWS_F32) * RAWUNIT
                                   : smem_lds + (i % NPL) * XPLANE;
#pragma unroll
      for (int e = 0; e < CPU_; ++e) {
        const int t = 16 * p + RPC * e + lane / PPR;       // row of this lane's piece
        const int pos = lane % PPR;                        // stored position in the row
        const int srow = min(t, a.M - 1);
        const uint32_t voff = static_cast<uint32_t>(srow * a.ldx * sizeof(XT)) +
                              static_cast<uint32_t>(swz(pos, t) * 16);
        dma16(base, voff, dst + (16 * p + RPC * e) * PPR * 16);
      }
    };
    // fp32: convert this wave's 16 raw rows of unit i into the planes of buffer i % NPL;
    // lane l takes row 16 p + (l & 15), floats 32 (l >> 4) .. + 31
    auto convert = [&](int i) {
      const int t = 16 * p + (lane & 15), h = lane >> 4;
      const lds_char_t* raw = lsm + NPL * 2 * XPLANE + (i % RAWS_F32) * RAWUNIT + t * RAWROW;
      lds_char_t* hi = lsm + (i % NPL) * 2 * XPLANE + t * XROW;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // 8 floats -> one 16-byte piece of each plane
        const f32x4_t f0 = *(const __attribute__((address_space(3))) f32x4_t*)(raw + 16 * swz(8 * h + 2 * e, t));
        const f32x4_t f1 = *(const __attribute__((address_space(3))) f32x4_t*)(raw + 16 * swz(8 * h + 2 * e + 1, t));
        const float f[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
        u32x4_t hv, lv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hv[j] = pack_bf16(f[2 * j], f[2 * j + 1]);
          lv[j] = pack_bf16(f[2 * j] - __uint_as_float(hv[j] << 16),
                            f[2 * j + 1] - __uint_as_float(hv[j] & 0xffff0000u));
        }
        const int q = swz(4 * h + e, t);
        *(lds_u32x4_t*)(hi + 16 * q) = hv;
        *(lds_u32x4_t*)(hi + XPLANE + 16 * q) = lv;
      }
    };
    // units 0, 1, 2 in flight; unit 0 staged before the first barrier
    issue(0);
    issue(1);
    issue(2);
    wait_vmcnt<2 * CPU_>();
    if constexpr (SPLIT_X) convert(0);
    __syncthreads();
    // iteration i: unit i + 1 lands (unit i + 2 may still be in flight) and is staged into
    // buffer (i + 1) % NPL, whose previous unit the consumers finished before this barrier;
    // then the copies of unit i + 3 go out (into the raw buffer of unit i, converted last
    // round, or the plane buffer of unit i - 1)
    for (int i = 0; i < nu; ++i) {
      wait_vmcnt<CPU_>();
      if constexpr (SPLIT_X) convert(i + 1);
      issue(i + 3);
      __syncthreads();
    }
    wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup ends
  }
}

// zero y[z][m][n] (rows over grid.y, 16-byte stores where the row is aligned)
__global__ __launch_bounds__(256) void zero_rows_stream(float* __restrict__ y, int64_t ldy,
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

// Deterministic form, second pass: y[z][m][n] (+)= the partial tiles of column tile
// t = z * NB + n / CW summed slice by slice, run by run (runs q0 .. q1 of each slice cover
// the tile's units t * cps .. (t + 1) * cps - 1).  One thread per 4 columns; the slots are
// loaded eight at a time (independent loads in flight together) and added in that order.
// With app.cache set (batch 1), the quads of row m inside [c^KV | k^R] also go to the new
// token's cache row (AppendArgs): the same fp32 sums, rounded to bf16, k^R pairs rotated
// first, exactly as the separate append kernel does with them.
__global__ __launch_bounds__(256) void gemm_stream_reduce(const float* __restrict__ part,
                                                          float* __restrict__ y, StreamArgs a,
                                                          int CW, int batch, int accumulate,
                                                          AppendArgs app) {
  const int cps = a.NCH / a.ksl;
  const int64_t quads = static_cast<int64_t>(batch) * a.M * (a.N / 4);
  for (int64_t id = blockIdx.x * 256ll + threadIdx.x; id < quads; id += static_cast<int64_t>(gridDim.x) * 256) {
    const int n = static_cast<int>(id % (a.N / 4)) * 4;
    const int64_t zm = id / (a.N / 4);
    const int m = static_cast<int>(zm % a.M), z = static_cast<int>(zm / a.M);
    const int t = z * a.NB + n / CW, c = n % CW;
    const int q0 = (t * cps) / a.nu, nq = ((t + 1) * cps - 1) / a.nu - q0 + 1;
    const int slots = a.ksl * nq;  // slot i: slice i / nq, run q0 + i % nq
    const float* base = part + static_cast<int64_t>(t) * a.jmax * a.M * CW +
                        static_cast<int64_t>(m) * CW + c;
    const int64_t slice_stride = static_cast<int64_t>(a.ntiles) * a.jmax * a.M * CW;
    float* yp = y + z * a.sy + static_cast<int64_t>(m) * a.ldy + n;
    // a quad of k^R to append: its two rotations are computed first, while the slot loads
    // below are in flight
    const int ac = n - app.col;  // column inside [c^KV | k^R]
    const bool app_row = app.cache != nullptr && ac >= 0 && ac < app.d_c + app.d_R;
    const bool app_rope = app_row && ac >= app.d_c;  // quads never straddle c^KV and k^R
    int pos = 0;
    double rs[2] = {0.0, 0.0}, rc[2] = {1.0, 1.0};
    if (app_row) pos = app.seq_lens_before[m];
    if (app_rope) {
      const int k = (ac - app.d_c) / 2;
      rope_angle(pos, k, app.d_R, app.base, &rs[0], &rc[0]);
      rope_angle(pos, k + 1, app.d_R, app.base, &rs[1], &rc[1]);
    }
    float4 sum = accumulate ? *reinterpret_cast<const float4*>(yp) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = 0; i0 < slots; i0 += 8) {
      float4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = min(i0 + k, slots - 1);
        v[k] = *reinterpret_cast<const float4*>(base + (i / nq) * slice_stride +
                                                static_cast<int64_t>(i % nq) * a.M * CW);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (i0 + k < slots) {
          sum.x += v[k].x; sum.y += v[k].y; sum.z += v[k].z; sum.w += v[k].w;
        }
    }
    *reinterpret_cast<float4*>(yp) = sum;
    if (app_row) {
      const int page = app.block_table[static_cast<int64_t>(m) * app.max_pages + pos / app.page_size];
      bf16raw* row = static_cast<bf16raw*>(app.cache) +
                     (static_cast<int64_t>(page) * app.page_size + pos % app.page_size) * (app.d_c + app.d_R);
      float v[4] = {sum.x, sum.y, sum.z, sum.w};
      if (app_rope) {
        rope_rotate(sum.x, sum.y, rs[0], rc[0], &v[0], &v[1]);
        rope_rotate(sum.z, sum.w, rs[1], rc[1], &v[2], &v[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) st(row + ac + i, v[i]);
    }
  }
}

template <typename XT, int TN, int R, bool DET>
hipError_t launch_t(const GemmArgs& g, const StreamArgs& a, int grid, hipStream_t s,
                    const AppendArgs& app) {
  const int64_t rows = static_cast<int64_t>(g.batch) * g.M;
  const int gx = static_cast<int>(std::min<int64_t>((g.N + 1023) / 1024, 64));
  const int gy = static_cast<int>(std::min<int64_t>(rows, 4096));
  if (!g.accumulate && !a.part)
    hipLaunchKernelGGL(zero_rows_stream, dim3(gx, gy), dim3(256), 0, s,
                       static_cast<float*>(g.y), g.ldy, g.sy, g.M, g.N, g.batch);
  hipLaunchKernelGGL((gemm_stream_kernel<XT, TN, R, DET>), dim3(grid), dim3(512), 0, s,
                     static_cast<const XT*>(g.x), static_cast<const bf16raw*>(g.w),
                     static_cast<float*>(g.y), a);
  if constexpr (DET) {
    const int64_t quads = rows * (g.N / 4);
    const int rg = static_cast<int>(std::min<int64_t>((quads + 255) / 256, 4096));
    hipLaunchKernelGGL(gemm_stream_reduce, dim3(rg), dim3(256), 0, s, a.part,
                       static_cast<float*>(g.y), a, 64 * TN, g.batch, g.accumulate ? 1 : 0, app);
  }
  return hipGetLastError();
}

template <typename XT, int TN>
hipError_t launch_r(const GemmArgs& g, const StreamArgs& a, int grid, int R, hipStream_t s,
                    const AppendArgs& app) {
  if (a.part)  // the deterministic form is built for the planned ring only
    return R == 4 ? launch_t<XT, TN, 4, true>(g, a, grid, s, app) : hipErrorInvalidValue;
  if (app.cache != nullptr) return hipErrorInvalidValue;  // the append rides on the summing launch
  switch (R) {
    case 4: return launch_t<XT, TN, 4, false>(g, a, grid, s, app);
    case 8: return launch_t<XT, TN, 8, false>(g, a, grid, s, app);
    case 12: if constexpr (TN <= 2) return launch_t<XT, TN, 12, false>(g, a, grid, s, app); else break;
    case 16: if constexpr (TN <= 2) return launch_t<XT, TN, 16, false>(g, a, grid, s, app); else break;
    case 20: if constexpr (TN <= 2) return launch_t<XT, TN, 20, false>(g, a, grid, s, app); else break;
    default: break;
  }
  return hipErrorInvalidValue;
}

bool ring_ok(int tn, int r) {
  return r == 4 || r == 8 || ((r == 12 || r == 16 || r == 20) && tn <= 2);
}

}  // namespace

bool gemm_stream_supported(const GemmArgs& g) {
  return g.w_bf16 && g.w_nk && !g.y_bf16 && g.K % KC == 0 && g.K > 0 && g.M > 0 &&
         g.M <= 64 && g.N > 0 && g.N % 64 == 0 && g.batch > 0 &&
         (reinterpret_cast<uintptr_t>(g.w) & 15) == 0 && (g.ldw % 8) == 0 && (g.sw % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(g.x) & 15) == 0 && (g.ldx % 8) == 0 && (g.sx % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(g.y) & 3) == 0 &&
         g.ldx * 64 * (g.x_bf16 ? 2 : 4) < (int64_t{1} << 31) &&  // 32-bit copy offsets
         static_cast<int64_t>(g.batch) * (g.N / 64) * (g.K / KC) < (int64_t{1} << 30);
}

bool gemm_stream_plan_ok(const GemmArgs& g, int tn, int grid, int ring) {
  if (!(tn == 1 || tn == 2 || tn == 4) || g.N % (64 * tn) != 0 || !ring_ok(tn, ring)) return false;
  const int64_t units = static_cast<int64_t>(g.batch) * (g.N / (64 * tn)) * (g.K / KC);
  if (grid < 1 || grid > GS_CUS || units % grid != 0) return false;
  return (units / grid) % (ring / 4) == 0;
}

// Tile width, workgroups and ring depth.  For each tile width the workgroup count is the
// largest divisor of the unit count up to one per CU (a multiple of 8 if one is close).
// Measured at the DeepSeek-V2 shapes (W^O: 64 x 5120 x 16384; [W^DQ; W^DKV; W^KR]:
// 64 x 2112 x 5120) with the weights streaming from HBM: the shallowest ring (4 k-steps,
// three in flight per wave) beats the deeper ones by 2-6 %, and 128-column tiles beat 256-
// and 64-column ones; so tile 2 is preferred, then 4, then 1, as long as its workgroup
// count is within 7/8 of the best.
void gemm_stream_plan(const GemmArgs& g, int* tn, int* grid, int* ring) {
  int gds[3] = {0, 0, 0};
  const int order[3] = {2, 4, 1};
  int best_gd = 0;
  for (int i = 0; i < 3; ++i) {
    const int t = order[i];
    if (g.N % (64 * t) != 0) continue;
    const int64_t units = static_cast<int64_t>(g.batch) * (g.N / (64 * t)) * (g.K / KC);
    int gd = 1;
    for (int d = static_cast<int>(std::min<int64_t>(units, GS_CUS)); d >= 1; --d)
      if (units % d == 0) { gd = d; break; }
    for (int d = gd - gd % 8; d >= 8 && d * 8 >= gd * 7; d -= 8)
      if (units % d == 0) { gd = d; break; }
    gds[i] = gd;
    best_gd = std::max(best_gd, gd);
  }
  for (int i = 0; i < 3; ++i)
    if (gds[i] > 0 && gds[i] * 8 >= best_gd * 7) {
      *tn = order[i]; *grid = gds[i]; *ring = 4;
      return;
    }
  *tn = 1; *grid = 1; *ring = 4;
}

namespace {
StreamArgs stream_args(const GemmArgs& g, int tn, int grid) {
  StreamArgs a;
  a.ldx = g.ldx; a.sx = g.sx; a.ldw = g.ldw; a.sw = g.sw; a.ldy = g.ldy; a.sy = g.sy;
  a.M = g.M; a.N = g.N;
  a.NB = g.N / (64 * tn);
  a.NCH = g.K / KC;
  a.nu = static_cast<int>(static_cast<int64_t>(g.batch) * a.NB * a.NCH / grid);
  a.ksl = 1;
  if (g.batch == 1 && grid % 8 == 0)
    for (int k = 8; k > 1; k /= 2)
      if (a.NCH % k == 0) { a.ksl = k; break; }
  a.part = nullptr;
  a.ntiles = g.batch * a.NB;
  const int cps = a.NCH / a.ksl;
  a.jmax = (cps + a.nu - 1) / a.nu + 1;  // runs that can meet one tile inside a slice
  return a;
}

size_t part_bytes(const GemmArgs& g, const StreamArgs& a, int tn) {
  return static_cast<size_t>(a.ksl) * a.ntiles * a.jmax * g.M * 64 * tn * sizeof(float);
}

hipError_t launch_args(const GemmArgs& g, const StreamArgs& a, int tn, int grid, int ring,
                       hipStream_t s, const AppendArgs& app = AppendArgs()) {
  if (g.x_bf16) {
    switch (tn) {
      case 4: return launch_r<bf16raw, 4>(g, a, grid, ring, s, app);
      case 2: return launch_r<bf16raw, 2>(g, a, grid, ring, s, app);
      default: return launch_r<bf16raw, 1>(g, a, grid, ring, s, app);
    }
  }
  switch (tn) {
    case 4: return launch_r<float, 4>(g, a, grid, ring, s, app);
    case 2: return launch_r<float, 2>(g, a, grid, ring, s, app);
    default: return launch_r<float, 1>(g, a, grid, ring, s, app);
  }
}
}  // namespace

size_t gemm_stream_det_workspace_bytes(const GemmArgs& g) {
  if (!gemm_stream_supported(g)) return 0;
  int tn = 1, grid = 1, ring = 4;
  gemm_stream_plan(g, &tn, &grid, &ring);
  return part_bytes(g, stream_args(g, tn, grid), tn);
}

hipError_t launch_gemm_stream_det(const GemmArgs& g, void* part, size_t bytes, hipStream_t s,
                                  const AppendArgs& app) {
  int tn = 1, grid = 1, ring = 4;
  gemm_stream_plan(g, &tn, &grid, &ring);
  if (!gemm_stream_plan_ok(g, tn, grid, ring)) return hipErrorInvalidValue;
  StreamArgs a = stream_args(g, tn, grid);
  if (!part || bytes < part_bytes(g, a, tn) || (reinterpret_cast<uintptr_t>(part) & 15) ||
      g.N % 4 || (g.ldy % 4) || (g.sy % 4) || (reinterpret_cast<uintptr_t>(g.y) & 15))
    return hipErrorInvalidValue;
  if (app.cache != nullptr &&
      (g.batch != 1 || app.col % 4 || app.d_c % 4 || app.d_R % 4 || app.col + app.d_c + app.d_R > g.N))
    return hipErrorInvalidValue;
  a.part = static_cast<float*>(part);
  return launch_args(g, a, tn, grid, ring, s, app);
}

hipError_t launch_gemm_stream_with(const GemmArgs& g, int tn, int grid, int ring, hipStream_t s) {
  if (!gemm_stream_plan_ok(g, tn, grid, ring)) return hipErrorInvalidValue;
  const StreamArgs a = stream_args(g, tn, grid);
  return launch_args(g, a, tn, grid, ring, s);
}

hipError_t launch_gemm_stream(const GemmArgs& g, hipStream_t s) {
  int tn = 1, grid = 1, ring = 4;
  gemm_stream_plan(g, &tn, &grid, &ring);
  return launch_gemm_stream_with(g, tn, grid, ring, s);
}

}  // namespace mla
