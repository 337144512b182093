// Flattened work list for ragged batches: the plan every workgroup of a ragged attention
// launch computes from seq_lens on the device (no host synchronisation, no planning
// launch), shared by the ragged kernels of attn_mfma.hip and attn_wide.hip.
#pragma once

#include "device_common.h"

namespace mla {
namespace ragged {

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// exclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_excl_scan_i(int v, int lane) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x - v;
}

// Flattened work list for ragged batches (one query token per sequence).  The cached pages
// of all sequences, concatenated in sequence order (tot pages), are cut into gridDim.x
// ranges of W = ceil(tot / gridDim.x) pages, widened to ceil(max_b pages_b / 63) if that
// cut left some sequence in more than 64 ranges; range r goes to one workgroup, which runs the
// split body of its attention kernel on each piece of a sequence inside it.  Every workgroup is busy for the same number of
// pages (but the last), whatever the mix of lengths, and no workgroup is launched empty.
// Sequence b is cut into count_b pieces (ranges floor(off_b / W) ..
// floor((off_b + pages_b - 1) / W)); with first_b the number of pieces of the sequences
// before b (at most gridDim.x + B pieces in all), the partial of head h from piece i is row
// first_b H + h count_b + i of o_part [.][512] / lse_part: a sequence's pieces of one head
// are consecutive rows, as the splits in the split-grid layout.  Each
// workgroup computes this plan from seq_lens with wave scans (every wave alike, so the loop
// over pieces is uniform); range 0's workgroup also writes (first_b, count_b) to seq_slots
// for the combine.  Workgroup ids go to the 8 XCDs in turn, so range r = (id % 8)(G / 8) +
// id / 8 gives each XCD a contiguous eighth of the tokens: a sequence's pieces and its
// queries mostly share one L2.
// Piece k (0-based, in sequence order) of range r = [lo, hi) under range width W, or
// false past the range's last piece.  A piece is the part of one sequence inside the range:
// sequence b, tokens j0 .. j1-1, and its partials' place (the sequence's first piece over
// the whole batch, its piece count, and this piece's index among them).  A fresh scan over
// seq_lens for every piece keeps no per-lane state alive across the pieces, whose split
// body needs nearly every register.
struct Piece {
  int b, j0, j1, first, count, index;
};

__device__ __forceinline__ bool ragged_piece(const int32_t* __restrict__ seq_lens, int B,
                                             int log2P, int W, int r, int lo, int hi, int k,
                                             Piece* pc) {
  const int lane = threadIdx.x & 63;
  const int P = 1 << log2P;
  int off_run = 0, first_run = 0;
  for (int base = 0; base < B; base += 64) {
    const int bb = base + lane;
    const int len = bb < B ? seq_lens[bb] : 0;
    const int pg = (len + P - 1) >> log2P;
    const int off = off_run + wave_excl_scan_i(pg, lane);
    const int cnt = pg > 0 ? (off + pg - 1) / W - off / W + 1 : 0;
    const bool in = cnt > 0 && off < hi && off + pg > lo;
    const uint64_t mask = __ballot(in);
    const int n = __builtin_popcountll(mask);
    if (k < n) {
      const int first = first_run + wave_excl_scan_i(cnt, lane);
      // the k-th lane of the mask: the one with k mask lanes below it
      const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
      const int l = __builtin_ctzll(__ballot(in && below == k));
      const int off_b = __builtin_amdgcn_readlane(off, l);
      const int pg_b = __builtin_amdgcn_readlane(pg, l);
      const int p0 = max(off_b, lo) - off_b, p1 = min(off_b + pg_b, hi) - off_b;
      // (integer division runs on the vector unit: readfirstlane keeps the fields scalar)
      pc->b = base + l;
      pc->j0 = p0 << log2P;
      pc->j1 = min(__builtin_amdgcn_readlane(len, l), p1 << log2P);
      pc->first = __builtin_amdgcn_readlane(first, l);
      pc->count = __builtin_amdgcn_readlane(cnt, l);
      pc->index = __builtin_amdgcn_readfirstlane(r - off_b / W);
      return true;
    }
    k -= n;
    off_run = __builtin_amdgcn_readfirstlane(off_run + wave_sum_i(pg));
    first_run = __builtin_amdgcn_readfirstlane(first_run + wave_sum_i(cnt));
  }
  return false;
}

// Flattened work list for ragged batches (one query token per sequence).  The cached pages
// of all sequences, concatenated in sequence order (tot pages), are cut into gridDim.x
// ranges of W = ceil(tot / gridDim.x) pages, widened to ceil(max_b pages_b / 63) if that
// cut left some sequence in more than 64 ranges; range r goes to one workgroup, which runs
// attn_split on each piece of a sequence inside it.  Every workgroup is busy for the same
// number of pages (but the last), whatever the mix of lengths, and none is launched empty.
// Sequence b is cut into count_b pieces (ranges floor(off_b / W) ..
// floor((off_b + pages_b - 1) / W)); with first_b the number of pieces of the sequences
// before b (at most gridDim.x + B pieces in all), the partial of head h from piece i is row
// first_b H + h count_b + i of o_part [.][512] / lse_part: a sequence's pieces of one head
// are consecutive rows, as the splits in the split-grid layout.  Each workgroup computes
// the plan from seq_lens with wave scans (every wave alike, so the loop over pieces is
// uniform); range 0's workgroup also writes (first_b, count_b) to seq_slots for the
// combine.  Workgroup ids go to the 8 XCDs in turn, so range r = (id % 8)(G / 8) + id / 8
// gives each XCD a contiguous eighth of the tokens: a sequence's pieces and its queries
// mostly share one L2.

// Range of workgroup id among G: consecutive ids go to the 8 XCDs in turn, so this gives
// each XCD a contiguous eighth of the ranges (of the tokens).
__device__ __forceinline__ int range_of(int id, int G) {
  return (G % 8 == 0) ? (id % 8) * (G / 8) + id / 8 : id;
}

// The plan's start, run by every workgroup alike: the total page count tot and the range
// width W (the even split, widened so that no sequence is cut into more than 64 pieces);
// range 0's workgroup writes (first_b, count_b) to seq_slots and *err = 1 when a range
// would exceed max_range pages (its block-table entries must fit LDS), else 0.  Returns
// that condition: the workgroup then writes nothing more.
__device__ __forceinline__ bool plan_ranges(const int32_t* __restrict__ seq_lens, int B, int log2P,
                                            int max_range, int* __restrict__ seq_slots,
                                            int* __restrict__ err, int& W_out, int& tot_out) {
  const int G = gridDim.x;
  const int r = __builtin_amdgcn_readfirstlane(range_of(blockIdx.x, G));
  const int lane = threadIdx.x & 63;
  const int P = 1 << log2P;
  int tot = 0, mx = 0;
  for (int base = 0; base < B; base += 64) {
    const int bb = base + lane;
    const int pg = bb < B ? (seq_lens[bb] + P - 1) >> log2P : 0;
    tot += wave_sum_i(pg);
    mx = max(mx, wave_max_i(pg));
  }
  tot = __builtin_amdgcn_readfirstlane(tot);
  mx = __builtin_amdgcn_readfirstlane(mx);
  // the even split, unless it cuts some sequence into more than 64 pieces (then a width of
  // ceil(max pages / 63) bounds every count by 64)
  int W = __builtin_amdgcn_readfirstlane(max((tot + G - 1) / G, 1));
  {
    int off_run = 0, most = 0;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const int pg = bb < B ? (seq_lens[bb] + P - 1) >> log2P : 0;
      const int off = off_run + wave_excl_scan_i(pg, lane);
      most = max(most, wave_max_i(pg > 0 ? (off + pg - 1) / W - off / W + 1 : 0));
      off_run = __builtin_amdgcn_readfirstlane(off_run + wave_sum_i(pg));
    }
    if (__builtin_amdgcn_readfirstlane(most) > 64)
      W = __builtin_amdgcn_readfirstlane(max(W, (mx + 62) / 63));
  }
  const bool too_long = W > max_range;  // a range's block-table entries must fit LDS
  if (r == 0 && threadIdx.x < 64) {
    int off_run = 0, first_run = 0;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const int pg = bb < B ? (seq_lens[bb] + P - 1) >> log2P : 0;
      const int off = off_run + wave_excl_scan_i(pg, lane);
      const int cnt = pg > 0 && !too_long ? (off + pg - 1) / W - off / W + 1 : 0;
      if (bb < B) {
        seq_slots[2 * bb] = first_run + wave_excl_scan_i(cnt, lane);
        seq_slots[2 * bb + 1] = cnt;
      } else {
        wave_excl_scan_i(cnt, lane);  // every lane takes part in the shuffles
      }
      off_run = __builtin_amdgcn_readfirstlane(off_run + wave_sum_i(pg));
      first_run = __builtin_amdgcn_readfirstlane(first_run + wave_sum_i(cnt));
    }
    if (threadIdx.x == 0) *err = too_long ? 1 : 0;
  }
  W_out = W;
  tot_out = tot;
  return too_long;
}

}  // namespace ragged
}  // namespace mla
