// Tile walk and lane mapping of the prefill and decode kernels.  The
// probes include this same header, so what they record is what the kernels
// visit.
#pragma once

#include <limits.h>
#include <math.h>

#include "common.h"

namespace olmo3 {
namespace pf {

constexpr int kD = 128;     // head size
constexpr int kBQ = 128;    // queries per workgroup (4 wavefronts x 32)
constexpr int kBK = 64;     // keys per tile
constexpr int kWaves = 4;
constexpr int kQW = 32;     // queries per wavefront

// Key s is visible from query t ("OLMo 3's Sliding-Window Attention
// Pattern", "The sliding-window mask"): s <= t, and t - s < window on
// sliding layers.
__host__ __device__ __forceinline__ bool visible(int t, int s, int window, int sliding) {
  return s <= t && (!sliding || t - s < window);
}

// Applies the visibility predicate to one 32x32 block of scores in the
// v_mfma_f32_32x32x16 output layout (row = key, column = query): register r
// of a lane holds key kb0 + 8*(r/4) + 4*(lane/32) + r%4 for the lane's query
// tq, and is set to -inf unless visible(tq, key).  With rel = tq - kb0 -
// 4*(lane/32) and the key offset c = 8*(r/4) + r%4, tq - key = rel - c, so
// the key is visible iff 0 <= rel - c (and rel - c < window on sliding
// layers).  The prefill kernel and its probe both mask through this function.
__host__ __device__ __forceinline__ void mask_block(f32x16& s, int tq, int kb0, int lane,
                                                    int window, int sliding) {
  const int rel = tq - kb0 - 4 * (lane >> 5);
  // positions stay below 2^30: a window at least that wide is a full one;
  // then rel - c < w is the visibility test as one unsigned comparison
  // (negative differences wrap past every window)
  const unsigned w = sliding && window < (1 << 30) ? (unsigned)window : (1u << 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int c = 8 * (r >> 2) + (r & 3);
    s[r] = (unsigned)(rel - c) < w ? s[r] : -INFINITY;
  }
}

// Key tiles [kt0, kt1) that hold any key visible from queries [q0, q1):
// keys from q0 - window + 1 (sliding) or 0 (full) up to q1 - 1.
__host__ __device__ __forceinline__ void key_tiles(int q0, int q1, int window, int sliding,
                                                   int& kt0, int& kt1) {
  const int first = sliding ? (q0 - window + 1 > 0 ? q0 - window + 1 : 0) : 0;
  kt0 = first / kBK;
  kt1 = (q1 + kBK - 1) / kBK;
}

// True when every pair of queries [q0, q1) and keys [k0, k0 + kBK) is
// visible, so the tile needs no per-element mask.
__host__ __device__ __forceinline__ bool tile_interior(int k0, int q0, int q1, int window,
                                                       int sliding) {
  return k0 + kBK - 1 <= q0 && (!sliding || (q1 - 1) - k0 < window);
}

// The interior tiles of [kt0, kt1) form one run [i0, i1): the causal
// condition holds for kt <= (q0 + 1)/kBK - 1 and the window condition for
// kt >= ceil((q1 - window)/kBK).  Tiles [kt0, i0) lie on the window's far
// edge and tiles [i1, kt1) on the diagonal; only those are masked.
__host__ __device__ __forceinline__ void interior_tiles(int q0, int q1, int window, int sliding,
                                                        int kt0, int kt1, int& i0, int& i1) {
  i1 = (q0 + 1) / kBK;
  if (i1 > kt1) i1 = kt1;
  if (i1 < kt0) i1 = kt0;
  i0 = kt0;
  if (sliding) {
    const int lo = q1 - window;
    const int first = lo > 0 ? (lo + kBK - 1) / kBK : 0;
    if (first > i0) i0 = first;
  }
  if (i0 > i1) i0 = i1;
}

// Grids of fewer workgroups than this (two per CU) may split each query
// block's key tiles over kKvSplits workgroups, whose partial softmax states
// are then merged, so that the chip holds two workgroups per CU.
constexpr int kSplitBelowBlocks = 512;
constexpr int kKvSplits = 2;

struct Work {
  int b, h, qb;
};

// Grids of up to this many query blocks (16 rounds of the 512 workgroups
// the GPU holds at once) take the interleaved order of work_at: with few
// rounds the last one's imbalance shows.  Longer grids keep each (batch,
// head)'s blocks together, which keeps its keys and values in the caches.
constexpr int kInterleaveMaxBlocks = 8192;

// Query block L of the remapped order -> (batch, head, query block); BH =
// B*H pairs.  The XCD remap hands each XCD a contiguous range of L.  When
// the pairs split evenly over the 8 XCDs, XCD x takes pairs x*k .. x*k+k-1
// (k = BH/8: with grouped heads, the query heads of one key/value head).
// In a small grid it first walks the last n_even blocks of each pair (blocks
// of equal work, e.g. full sliding windows) pair after pair, then the rest
// longest causal rows first with the pairs interleaved (query block outer,
// pair inner), so that every long block starts in the first rounds while
// blocks of one pair keep their keys and values together where order does
// not matter.  Otherwise (and with n_even = n_qblk) pair after pair, each
// longest rows first.
__host__ __device__ __forceinline__ Work work_at(int L, int n_qblk, int BH, int H, int n_even) {
  if (BH % 8 == 0 && n_qblk * BH <= kInterleaveMaxBlocks) {
    const int k = BH / 8;
    const int per = k * n_qblk;
    const int x = L / per;
    int j = L % per, p, qb;
    if (j < k * n_even) {
      p = j / n_even;
      qb = n_qblk - 1 - j % n_even;
    } else {
      j -= k * n_even;
      p = j % k;
      qb = n_qblk - n_even - 1 - j / k;
    }
    const int bh = x * k + p;
    return Work{bh / H, bh % H, qb};
  }
  const int qi = L % n_qblk;
  const int bh = L / n_qblk;
  return Work{bh / H, bh % H, n_qblk - 1 - qi};
}

// Blocks a uniform prefill keeps pair after pair (work_at's n_even): on a
// sliding layer with one query head per key/value head, the blocks whose
// windows are full (equal work, the last ones); everywhere else none.
// Grouped query heads read the same keys and values, so they gain from
// running side by side; full layers measured faster interleaved.
__host__ __device__ __forceinline__ int even_blocks(int n_qblk, int H, int G, int sliding,
                                                    int window, int q_pos0) {
  if (H != G || !sliding) return 0;
  // block qb starts at q_pos0 + qb kBQ; its window is full from q0 >= window - 1
  const int64_t d = (int64_t)window - 1 - q_pos0;
  if (d <= 0) return n_qblk;
  const int64_t first = (d + kBQ - 1) / kBQ;
  return first >= n_qblk ? 0 : n_qblk - (int)first;
}

// Workgroup -> (batch, head, query block): the query blocks of a (batch,
// head) sit on one XCD (shared K/V in its L2).
__host__ __device__ __forceinline__ Work work_of(int bid, int nblk, int n_qblk, int H, int n_even) {
  return work_at(xcd_remap(bid, nblk), n_qblk, nblk / n_qblk, H, n_even);
}

// With kKvSplits workgroups per query block: workgroup -> block and split
// (the splits of a block are neighbours in the remapped order, so they share
// an XCD).
__host__ __device__ __forceinline__ Work work_of_split(int bid, int nblk, int n_qblk, int H,
                                                       int n_even, int& split) {
  const int L = xcd_remap(bid, nblk);
  split = L % kKvSplits;
  return work_at(L / kKvSplits, n_qblk, nblk / (kKvSplits * n_qblk), H, n_even);
}

// Key tiles [kta, ktb) of split `split` of the block's tiles [kt0, kt1).
__host__ __device__ __forceinline__ void split_tiles(int kt0, int kt1, int split, int& kta,
                                                     int& ktb) {
  const int n = kt1 - kt0;
  kta = kt0 + n * split / kKvSplits;
  ktb = kt0 + n * (split + 1) / kKvSplits;
}

// Query of a lane: wavefront w owns 32 consecutive queries; lanes l and
// l + 32 share a query (MFMA 32x32 output column l % 32).
__device__ __forceinline__ int lane_query(int q0, int wave, int lane) {
  return q0 + wave * kQW + (lane & 31);
}

// Key held in accumulator register r of 32-key block kb of a tile at k0
// (v_mfma_f32_32x32x16_bf16 output row: 8*(r/4) + 4*(lane/32) + r%4).
__device__ __forceinline__ int lane_key(int k0, int kb, int r, int lane) {
  return k0 + kb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace pf

namespace dec {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;             // 16 lanes x 8 bf16 cover a row
constexpr int kGroups = kThreads / kLanesPerRow;  // rows in flight per step
constexpr int kUnroll = 4;                   // steps per loop iteration
constexpr int kRowsPerIter = kGroups * kUnroll;
constexpr int kMaxSplits = 64;
constexpr int64_t kMinRowsPerSplit = 256;
// Splits per (sequence, key/value head): enough for about this many
// workgroups.  Few long workgroups stream as fast as many short ones (at
// B*G >= 512 every pair is one workgroup, which then writes its output rows
// itself and no merge runs), and fewer reach the end of the stream together.
constexpr int64_t kTargetWorkgroups = 512;

// Rows of a split at iteration i, step u, for lane group grp.
__host__ __device__ __forceinline__ int64_t row_of(int64_t r0, int64_t i, int u, int grp) {
  return r0 + i * kRowsPerIter + u * kGroups + grp;
}

}  // namespace dec
}  // namespace olmo3
