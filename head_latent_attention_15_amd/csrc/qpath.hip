// The query side of a decode step in one launch: up-projection of the compressed query,
// query RoPE and absorption of W^UK, per head.
//   q^C_i = W^UQ_i c^Q,  q^R_i = W^QR_i c^Q          (qiita.com/joule, "Query の圧縮")
//   q_pe_i = RoPE(q^R_i, pos = seq_len - 1)           (qiita.com/joule, "RoPE の扱い")
//   q~_i  = W^UK_i^T q^C_i                            (qiita.com/joule, "Absorption Trick による最適化")
// A head's absorption needs only that head's d_h = 128 values of q^C, so one workgroup can
// hold the whole contraction over d_c^Q and apply W^UK_i in the same launch: q^C never goes
// to HBM, and no k range is split over workgroups, so there are no atomics and every
// result is the same on every run.
//
// The weights come packed once at load time (qpath_pack_kernel).  [W^UQ_i; W^QR_i] (192 rows)
// is cut into 12 tiles of 16 rows and d_c^Q / 32 k-steps; each (tile, k-step) is one 1 KB
// MFMA operand fragment (lane 16 g + n: row n, k 8 g .. 8 g + 7), and the fragments are
// ordered 128-wide chunk of k, head, tile, k-step within the chunk: everything a head needs
// for one chunk is one contiguous 48 KB block, read in full by the head's two workgroups
// together, and the blocks all heads read at about the same time form one contiguous
// region, spread over every HBM channel.  Row-major weights would be read 256 bytes per row
// per chunk across 160 rows, which the DRAM serves far more slowly.  W^UK_i follows as two 64 KB images, one per
// half, laid out exactly as the workgroup keeps it in LDS, so it is copied in linear 1 KB
// blocks.
//
// Workgroup (head i, half hf) of 12 wavefronts, 64 rows b (one block of the batch):
// hf = blockIdx.x / H, so the two halves of a head run on one XCD (consecutive ids go to
// the 8 XCDs in turn; H % 8 == 0 at the DeepSeek-V2 sizes) and W^UQ_i, which both read,
// comes from HBM once.
//   phase 1: the 10 columns tiles of 16 (q^C_i: tiles 0..7; this half's 32 columns of q^R_i:
//            tiles 8, 9) in pairs: wave w < 10 computes tiles 2 p, 2 p + 1 (p = w % 5) over
//            the k-steps 2 kh, 2 kh + 1 (kh = w / 5) of every 128-wide chunk of d_c^Q.
//            C = X W^T on v_mfma_f32_16x16x32_bf16 with A = c^Q from LDS as two bf16 planes
//            (hi + rounding remainder: ~16 significant bits of the fp32 input, so each
//            product with a bf16 weight is exact in fp32), each A fragment feeding both
//            tiles, and B = the weight fragments streamed from HBM straight into registers,
//            12 fragments (three chunks) ahead.  The two k halves of a tile are added at the
//            end, in one fixed order.  LDS read traffic bounds this loop: every wave reads
//            its k half of each chunk, so pairing the tiles halves it against one tile per
//            wave.
//            Waves 10, 11 only stage c^Q: each chunk converted to the two planes into a
//            double buffer, one barrier per chunk.  The split keeps each wave's loads of one
//            kind: a wave's memory counter retires in issue order, so a wave that waited for
//            c^Q loads would also wait for every weight load issued before them.
//   phase 2: q^C_i to LDS as hi / lo planes; the q^R tiles are rotated with the cos / sin
//            table built at the start (fp64 angles) and stored as q_pe.
//   phase 3: q~_i columns 256 hf .. + 255 = W^UK_i^T q^C_i on waves 0..7 (4 column groups x
//            2 row groups), A = W^UK_i^T read with the transposing ds_read_b64_tr_b16 from
//            W^UK_i as stored ([j][c], copied HBM -> LDS during chunks 1..7 without a
//            register round trip), B = the q^C planes.
#include "attn_common.h"
#include "device_common.h"
#include "launchers.h"

#include <algorithm>
#include <type_traits>

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x2_t lds_f32x2_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
typedef __attribute__((address_space(3))) unsigned lds_u32_t;
typedef __attribute__((address_space(3))) unsigned short lds_u16_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int QP_NC = 10;                     // computing waves
constexpr int QP_NW = QP_NC + 2, QP_NT = QP_NW * 64;  // + two c^Q staging waves
constexpr int QP_CT = QP_NC * 64;             // threads of the computing waves
constexpr int QP_M = 64;                      // rows b per workgroup
constexpr int QP_DH = 128, QP_DR = 64, QP_DC = 512;
constexpr int QP_KC = 128;                    // k per chunk of c^Q (4 MFMA k-steps)
constexpr int QP_ROW = QP_KC * 2 + 16;        // LDS bytes per padded bf16 row (272)
constexpr int QP_PLANE = QP_M * QP_ROW;       // one plane of 64 rows
constexpr int QP_CHUNK = 2 * QP_PLANE;        // hi and lo planes of one chunk
constexpr int QP_WUK = 2 * QP_CHUNK;          // W^UK_i, this half's 256 columns: [j][c]
constexpr int QP_UROW = 256 * 2;              // its row: 32 chunks of 16 bytes, swizzled
constexpr int QP_TAB = QP_WUK + QP_DH * QP_UROW;  // RoPE {cos, sin}: [64 b][16 pairs]
constexpr int QP_LDS = QP_TAB + QP_M * 16 * 8;    // 147,456 bytes
constexpr int QP_RING = 12;                   // weight fragments in flight per wave (3 chunks)
constexpr int QP_UNROLL = QP_RING / 4;        // chunks per turn of the ring
constexpr int QP_XLOADS = 16;                 // 16-byte c^Q loads per staging thread and chunk
constexpr int QP_UCOPIES = QP_DH * QP_UROW / 1024;  // wave-wide 1 KB copies of W^UK_i (64)
static_assert(QP_LDS <= 163840, "LDS per workgroup");
static_assert(QP_NC * 4096 <= 2 * QP_CHUNK, "k-half exchange fits in the chunk buffers");

// stored position of 16-byte chunk c of W^UK row j: conflict-free transposing reads of
// four consecutive rows (and of two such groups eight rows apart) at one chunk pair
__device__ __forceinline__ int qp_uswz(int j) { return ((j & 3) << 1) | (((j >> 3) & 1) << 3); }

__device__ __forceinline__ unsigned qp_pack2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__global__ __launch_bounds__(QP_NT) void qpath_kernel(
    const float* __restrict__ c_q, int64_t ld_q, const bf16raw* __restrict__ w_pack,
    const int32_t* __restrict__ seq_lens, float rope_base, int B, int H, int d_cq,
    bf16raw* __restrict__ q_lat, bf16raw* __restrict__ q_pe) {
  __shared__ __attribute__((aligned(16))) char smem[QP_LDS];
  lds_char_t* const lsm = (lds_char_t*)smem;
  const int h = blockIdx.x % H, hf = blockIdx.x / H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int nchunks = d_cq / QP_KC;
  // phase 2 puts q^C_i in the chunk buffer the last chunk does not read
  lds_char_t* const qc = lsm + (nchunks & 1) * QP_CHUNK;

  if (w >= QP_NC) {
    // ---- c^Q staging: thread p = tid - 640 moves row p / 2, k 64 (p % 2) .. + 63 of each
    //      chunk (rows past B read row B - 1: their products land in rows never stored).
    //      Two chunks are in flight: chunk ch + 1, loaded two barriers earlier, is converted
    //      and stored after the barrier that ends chunk ch - 1's reads, then chunk ch + 3 is
    //      loaded into the registers it leaves.  Past the end the last chunk is loaded and
    //      stored again (into a buffer nobody reads before it is rewritten after a
    //      barrier): no branch around the loads, so each wait is the exact one
    const int p = tid - QP_CT, xrow = p >> 1;
    const float* xsrc = c_q + static_cast<int64_t>(min(xrow, B - 1)) * ld_q + 64 * (p & 1);
    lds_char_t* const xdst = lsm + xrow * QP_ROW + 128 * (p & 1);
    f32x4_t xa[QP_XLOADS], xb[QP_XLOADS];
    auto load_x = [&](f32x4_t (&xv)[QP_XLOADS], int ch) {
      ch = min(ch, nchunks - 1);
#pragma unroll
      for (int i = 0; i < QP_XLOADS; ++i)
        xv[i] = *reinterpret_cast<const f32x4_t*>(xsrc + ch * QP_KC + 4 * i);
    };
    auto store_x = [&](const f32x4_t (&xv)[QP_XLOADS], int buf) {
#pragma unroll
      for (int i = 0; i < QP_XLOADS; i += 2) {
        u32x4_t hi, lo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a = xv[i + (q >> 1)][2 * (q & 1)], bb = xv[i + (q >> 1)][2 * (q & 1) + 1];
          hi[q] = qp_pack2(a, bb);
          lo[q] = qp_pack2(a - __uint_as_float(hi[q] << 16),
                           bb - __uint_as_float(hi[q] & 0xffff0000u));
        }
        *(lds_u32x4_t*)(xdst + buf * QP_CHUNK + 8 * i) = hi;
        *(lds_u32x4_t*)(xdst + buf * QP_CHUNK + QP_PLANE + 8 * i) = lo;
        // one group of eight values at a time: with two chunks in flight, converting the
        // whole chunk ahead of its stores would not fit in the registers
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    load_x(xa, 0);
    load_x(xb, 1);
    store_x(xa, 0);
    load_x(xa, 2);
    __syncthreads();
    // buffer (ch + 1) & 1 was last read in chunk ch - 1, before the previous barrier
    int ch = 0;
    for (; ch + 1 < nchunks; ch += 2) {
      store_x(xb, (ch + 1) & 1);  // chunk ch + 1
      load_x(xb, ch + 3);
      __syncthreads();
      store_x(xa, (ch + 2) & 1);  // chunk ch + 2
      load_x(xa, ch + 4);
      __syncthreads();
    }
    if (ch < nchunks) {
      store_x(xb, (ch + 1) & 1);
      __syncthreads();
    }
    __syncthreads();  // the k-half exchange (below) writes
    __syncthreads();  // and reads
  } else {
    const int pr = w % 5, kh = w / 5;  // tile pair, k half

    // ---- positions of the RoPE table entries e = tid + 640 q < 1024 (row b = e / 16),
    //      loaded first, without a branch, so that the wait for them leaves the loads below
    //      in flight (entries past 1024 load a valid position they never use)
    int pos[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      pos[q] = seq_lens[min((tid + QP_CT * q) >> 4, B - 1)] - 1;
    __builtin_amdgcn_sched_barrier(0);  // both go out before the weight loads

    // ---- packed tiles 2 pr + tt of this half: q^C tiles 0..7 of head i, then q^R tiles
    //      8 + 2 hf, 9 + 2 hf.  Ring fragment n: chunk n / 4, k-step 2 kh + (n % 4) / 2 of
    //      the chunk, tile n % 2; a (chunk, head) block holds 12 tiles x 4 k-steps of 512 bf16
    const bf16raw* fbase[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 2 * pr + tt, pt = t < 8 ? t : t + 2 * hf;
      fbase[tt] = w_pack + ((static_cast<int64_t>(h) * 12 + pt) * 4 + 2 * kh) * 512 + 8 * lane;
    }
    const int64_t chunk_stride = static_cast<int64_t>(H) * 48 * 512;
    auto frag_src = [&](int n) {
      return reinterpret_cast<const bf16x8_t*>(fbase[n & 1] + chunk_stride * (n >> 2) + 512 * ((n >> 1) & 1));
    };
    bf16x8_t wf[QP_RING];
#pragma unroll
    for (int n = 0; n < QP_RING - 2; ++n) wf[n] = *frag_src(n);

    // ---- RoPE table while the loads are in flight: entry e = row b, pair k = 16 hf + e % 16
    //      (angle pos * base^(-2k/d_R) and its sine and cosine in fp64)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + QP_CT * q;
      if (e < QP_M * 16) {
        const double theta = pow(static_cast<double>(rope_base),
                                 -2.0 * static_cast<double>(16 * hf + (e & 15)) / QP_DR);
        double sn, cs;
        sincos(static_cast<double>(pos[q]) * theta, &sn, &cs);
        *(lds_f32x2_t*)(lsm + QP_TAB + 8 * e) =
            f32x2_t{static_cast<float>(cs), static_cast<float>(sn)};
      }
    }
    __syncthreads();

    // ---- W^UK_i rows j, columns 256 hf .. + 255 -> LDS [j][c], chunk c of row j at position
    //      c ^ qp_uswz(j), from its packed image (the same bytes in the same order): copy i
    //      moves 1 KB, rows 2 i and 2 i + 1.  Wave w issues copy w + 10 (ch - 1) in chunk
    //      ch = 1 .. 7, after the first weight loads have gone out; copies a short d_c^Q
    //      leaves over go after the loop
    const bf16raw* ubase = w_pack + static_cast<int64_t>(H) * 192 * d_cq +
                           static_cast<int64_t>(2 * h + hf) * QP_DH * 256;
    const uint32_t ulds = static_cast<uint32_t>(reinterpret_cast<size_t>(lsm)) + QP_WUK;
    auto copy_uk = [&](int i) {
      attn::dma16(ubase, static_cast<uint32_t>(i * 1024 + 16 * lane), ulds + i * 1024);
    };
    const int uk_chunks = min(7, nchunks - 1);

    // ---- phase 1: acc[tt][mt], lane (g, n), entry e: C[16 mt + 4 g + e][column n of tile
    //      2 pr + tt], this wave's k half
    f32x4_t acc[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[tt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // A fragments of one k-step: plane pl, row tile mt of k-step sl of chunk ch (this wave's
    // k half).  They are read one k-step ahead, each right after the last product that uses
    // the registers it replaces, so the LDS reads run under the products; the barrier of
    // chunk ch sits between its two k-steps: every read of chunk ch is done by then (its
    // buffer can be refilled) and chunk ch + 1, written during chunk ch - 1's second half and
    // chunk ch's first, is complete
    auto a_src = [&](int ch, int sl, int pl, int mt) {
      return (const lds_bf16x8_t*)(lsm + (ch & 1) * QP_CHUNK + (16 * mt + r) * QP_ROW +
                                   64 * (2 * kh + sl) + 16 * g + pl * QP_PLANE);
    };
    bf16x8_t xf[2][4];
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) xf[pl][mt] = *a_src(0, 0, pl, mt);
    // chunk ch (cu = ch % 3): weight fragment n = 4 ch + q sits in slot 4 cu + q.  Before
    // k-step sl uses fragments n = 4 ch + 2 sl and n + 1, the wave loads fragments n + 10 and
    // n + 11 into the slots that fragments n - 2 and n - 1 (the previous k-step) freed.  In
    // the last turn only the first k-step's loads are fragments that exist
    auto chunk = [&](int ch, auto cu_c, auto tail_c) {
      constexpr int cu = decltype(cu_c)::value;
      constexpr bool tail = decltype(tail_c)::value;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        if (!tail || (cu == 0 && sl == 0)) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            wf[(4 * cu + 2 * sl + tt + QP_RING - 2) % QP_RING] =
                *frag_src(4 * ch + 2 * sl + tt + QP_RING - 2);
        }
        __builtin_amdgcn_sched_barrier(0);  // issued here, not sunk below the products
        if (sl == 0 && ch >= 1 && ch <= uk_chunks && w + QP_NC * (ch - 1) < QP_UCOPIES)
          copy_uk(w + QP_NC * (ch - 1));
        const bf16x8_t wk0 = wf[(4 * cu + 2 * sl) % QP_RING];
        const bf16x8_t wk1 = wf[(4 * cu + 2 * sl + 1) % QP_RING];
        const bool next = sl == 0 || !(tail && cu == QP_UNROLL - 1);  // a k-step follows
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            acc[0][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[pl][mt], wk0, acc[0][mt], 0, 0, 0);
            acc[1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[pl][mt], wk1, acc[1][mt], 0, 0, 0);
            if (next) xf[pl][mt] = *a_src(sl == 0 ? ch : ch + 1, sl ^ 1, pl, mt);
          }
        if (sl == 0) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // k-step 1 of chunk ch is read
          __syncthreads();
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using NoTail = std::false_type;
    using Tail = std::true_type;
    for (int c0 = 0; c0 < nchunks - QP_UNROLL; c0 += QP_UNROLL) {
      chunk(c0, I0{}, NoTail{});
      chunk(c0 + 1, I1{}, NoTail{});
      chunk(c0 + 2, I2{}, NoTail{});
    }
    chunk(nchunks - 3, I0{}, Tail{});
    chunk(nchunks - 2, I1{}, Tail{});
    chunk(nchunks - 1, I2{}, Tail{});
    static_assert(QP_UNROLL == 3, "the turn above is written out for three chunks");
    for (int i = w + QP_NC * uk_chunks; i < QP_UCOPIES; i += QP_NC) copy_uk(i);

    // ---- k-half exchange through the chunk buffers (no wave reads them after the last
    //      chunk's barrier; the staging waves' last, unused copy went in before it): wave w
    //      sends its partial of the tile it does not finish (4 KB) and adds the partner's
    //      partial of the tile it finishes, tile 2 pr + kh: k half 0's sum plus k half 1's
    //      (float addition is commutative: one result in both waves)
    lds_char_t* const xs = lsm + w * 4096 + 16 * lane;
    const int partner = kh ? pr : pr + 5;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      *(lds_f32x4_t*)(xs + mt * 1024) = kh ? acc[0][mt] : acc[1][mt];
    __syncthreads();
    f32x4_t fin[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4_t other = *(const lds_f32x4_t*)(lsm + partner * 4096 + 16 * lane + mt * 1024);
      fin[mt] = kh ? acc[1][mt] + other : acc[0][mt] + other;
    }
    // the copies of W^UK_i are complete before the barrier that precedes phase 3
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- phase 2: tile t = 2 pr + kh: q^C_i columns 16 t + n (t < 8) to LDS planes [b][j];
    //      q^R (t = 8, 9): lanes n and n ^ 1 hold the pair (even, odd) of one row; the even
    //      lane stores both rotated values
    const int t = 2 * pr + kh;
    if (t < 8) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b = 16 * mt + 4 * g + e;
          const float v = fin[mt][e];
          const unsigned hb = qp_pack2(v, 0.f) & 0xffffu;
          *(lds_u16_t*)(qc + b * QP_ROW + 2 * (16 * t + r)) = static_cast<unsigned short>(hb);
          *(lds_u16_t*)(qc + QP_PLANE + b * QP_ROW + 2 * (16 * t + r)) =
              static_cast<unsigned short>(qp_pack2(v - __uint_as_float(hb << 16), 0.f));
        }
    } else {
      const int kl = 8 * (t - 8) + (r >> 1);  // this lane's pair in this half's table
      const bool even = (r & 1) == 0;
      f32x2_t cs[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cs[mt][e] = *(const lds_f32x2_t*)(lsm + QP_TAB + 8 * (16 * (16 * mt + 4 * g + e) + kl));
      bf16raw* const dst = q_pe + static_cast<int64_t>(h) * QP_DR + 32 * hf + 16 * (t - 8) + r;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // quad_perm [1, 0, 3, 2]: the value of lane n ^ 1
          const float mine = fin[mt][e];
          const float other = __int_as_float(
              __builtin_amdgcn_mov_dpp(__float_as_int(mine), 0xB1, 0xF, 0xF, true));
          const float x0 = even ? mine : other, x1 = even ? other : mine;
          const float y0 = fmaf(x0, cs[mt][e].x, -x1 * cs[mt][e].y);
          const float y1 = fmaf(x0, cs[mt][e].y, x1 * cs[mt][e].x);
          const int b = 16 * mt + 4 * g + e;
          if (even && b < B)
            *reinterpret_cast<unsigned*>(dst + static_cast<int64_t>(b) * H * QP_DR) = qp_pack2(y0, y1);
        }
    }
  }
  __syncthreads();
  if (w >= 8) return;  // phase 3 runs on waves 0..7 (no barrier follows)

  // ---- phase 3: q~^T (256 c x 64 b) = W^UK_i^T (c x j) q^C_i^T (j x b); wave w takes the
  //      16-column tiles ct = 4 (w % 4) + 0..3 and the row tiles mt = 2 (w / 4) + 0, 1; lane
  //      (g, n) of tile (ct, mt) holds c = 16 ct + 4 g + e of row b = 16 mt + n.  The A
  //      fragment of (ct, ks), lane (g, n): W^UK rows j = 32 ks + 8 g + 0..7 at column
  //      16 ct + n, as two transposing reads of four rows: in each 16-lane group lane n reads
  //      row 4 hr + n / 4, columns 16 ct + 4 (n % 4) .. + 3
  const int cg = w & 3, mg = w >> 2;
  f32x4_t o[4][2];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) o[cc][mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < QP_DH / 32; ++ks) {
    bf16x8_t xf[2][2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const lds_char_t* xp = qc + (16 * (2 * mg + mm) + r) * QP_ROW + 64 * ks + 16 * g;
      xf[mm][0] = *(const lds_bf16x8_t*)xp;
      xf[mm][1] = *(const lds_bf16x8_t*)(xp + QP_PLANE);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int ct = 4 * cg + cc;
      attn::i16x4_t half[2];
#pragma unroll
      for (int hr = 0; hr < 2; ++hr) {
        const int j = 32 * ks + 8 * g + 4 * hr + (r >> 2);
        const int chk = (2 * ct + ((r & 3) >> 1)) ^ qp_uswz(j);
        half[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (attn::lds_i16x4_t*)(lsm + QP_WUK + j * QP_UROW + 16 * chk + 8 * (r & 1)));
      }
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          o[cc][mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xf[mm][pl], o[cc][mm], 0, 0, 0);
    }
  }
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int b = 16 * (2 * mg + mm) + r;
      if (b >= B) continue;
      uint2 v;
      v.x = qp_pack2(o[cc][mm][0], o[cc][mm][1]);
      v.y = qp_pack2(o[cc][mm][2], o[cc][mm][3]);
      *reinterpret_cast<uint2*>(q_lat + (static_cast<int64_t>(b) * H + h) * QP_DC + 256 * hf +
                                16 * (4 * cg + cc) + 4 * g) = v;
    }
}

// Packing for qpath_kernel, one thread per 16 bytes.
//   fragments: q = (((c * H + i) * 12 + tile) * 4 + s4) * 64 + l holds row 16 tile + l % 16
//     of head i's [W^UQ_i; W^QR_i] at k = 32 (4 c + s4) + 8 (l / 16) .. + 7
//   W^UK images, after H * 192 * d_cq elements: u = ((2 i + hf) * 128 + j) * 32 + pos holds
//     W^UK row i * 128 + j, columns 256 hf + 8 (pos ^ qp_uswz(j)) .. + 7
__global__ __launch_bounds__(256) void qpath_pack_kernel(const bf16raw* __restrict__ w_uq,
                                                         const bf16raw* __restrict__ w_qr,
                                                         const bf16raw* __restrict__ w_uk,
                                                         int H, int d_cq,
                                                         bf16raw* __restrict__ out) {
  const int nchunks = d_cq / QP_KC;
  const int64_t nfrag = static_cast<int64_t>(H) * nchunks * 48 * 64;
  const int64_t total = nfrag + static_cast<int64_t>(H) * 2 * QP_DH * 32;
  for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < total; q += static_cast<int64_t>(gridDim.x) * 256) {
    const bf16raw* src;
    if (q < nfrag) {
      const int l = static_cast<int>(q & 63);
      const int64_t f = q >> 6;  // fragment
      const int s4 = static_cast<int>(f & 3), tile = static_cast<int>((f >> 2) % 12);
      const int64_t ci = (f >> 2) / 12;
      const int i = static_cast<int>(ci % H), c = static_cast<int>(ci / H);
      const int row = 16 * tile + (l & 15), k = 32 * (4 * c + s4) + 8 * (l >> 4);
      src = row < QP_DH ? w_uq + (static_cast<int64_t>(i) * QP_DH + row) * d_cq + k
                        : w_qr + (static_cast<int64_t>(i) * QP_DR + row - QP_DH) * d_cq + k;
    } else {
      const int64_t u = q - nfrag;
      const int pos = static_cast<int>(u & 31), j = static_cast<int>((u >> 5) & 127);
      const int hf = static_cast<int>((u >> 12) & 1), i = static_cast<int>(u >> 13);
      src = w_uk + (static_cast<int64_t>(i) * QP_DH + j) * QP_DC + 256 * hf + 8 * (pos ^ qp_uswz(j));
    }
    *reinterpret_cast<uint4*>(out + q * 8) = *reinterpret_cast<const uint4*>(src);
  }
}

}  // namespace

bool qpath_supported(int H, int d_h, int d_R, int d_c, int d_cq, int64_t ld_q, const void* c_q,
                     const void* w_pack, const void* q_lat, const void* q_pe) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(c_q) | reinterpret_cast<uintptr_t>(w_pack) |
                      reinterpret_cast<uintptr_t>(q_lat) | reinterpret_cast<uintptr_t>(q_pe);
  return H >= 1 && H <= 32767 && d_h == QP_DH && d_R == QP_DR && d_c == QP_DC &&
         d_cq >= QP_KC * QP_UNROLL && d_cq % (QP_KC * QP_UNROLL) == 0 && ld_q >= d_cq &&
         ld_q % 4 == 0 && (a & 15) == 0;
}

int64_t qpath_pack_elems(int H, int d_cq) {
  return static_cast<int64_t>(H) * (192 * static_cast<int64_t>(d_cq) + QP_DH * QP_DC);
}

hipError_t launch_qpath_pack(const void* w_uq, const void* w_qr, const void* w_uk, int H,
                             int d_cq, void* out, hipStream_t s) {
  const int64_t total = qpath_pack_elems(H, d_cq) / 8;
  const int grid = static_cast<int>(std::min<int64_t>((total + 255) / 256, 65535));
  hipLaunchKernelGGL(qpath_pack_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<const bf16raw*>(w_uq), static_cast<const bf16raw*>(w_qr),
                     static_cast<const bf16raw*>(w_uk), H, d_cq, static_cast<bf16raw*>(out));
  return hipGetLastError();
}

hipError_t launch_qpath(const float* c_q, int64_t ld_q, const void* w_pack,
                        const int32_t* seq_lens, float rope_base, int B, int H, int d_cq,
                        void* q_lat, void* q_pe, hipStream_t s) {
  // one launch per block of 64 rows b (each block reads the weights again)
  for (int b0 = 0; b0 < B; b0 += QP_M) {
    hipLaunchKernelGGL(qpath_kernel, dim3(2 * H), dim3(QP_NT), 0, s, c_q + b0 * ld_q, ld_q,
                       static_cast<const bf16raw*>(w_pack), seq_lens + b0, rope_base,
                       min(QP_M, B - b0), H, d_cq,
                       static_cast<bf16raw*>(q_lat) + static_cast<int64_t>(b0) * H * QP_DC,
                       static_cast<bf16raw*>(q_pe) + static_cast<int64_t>(b0) * H * QP_DR);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
