// Flash-style causal prefill, d = 128, bf16 in / out, fp32 accumulation
// (v_mfma_f32_32x32x16_bf16), and the probe that records its tile walk.
//
// Masking follows "OLMo 3's Sliding-Window Attention Pattern", "The
// sliding-window mask": key s is visible from query t iff s <= t and, on a
// sliding layer, t - s < window.  Work per query row grows with the square
// of the length on full layers and with the window on sliding layers (same
// page, "The problem"); tiles with no visible key are never visited.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace olmo3 {

namespace {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Workgroup = 4 wavefronts x 32 queries of one (batch, head).  Per key tile of
// 64 keys each wavefront computes S^T = K Q^T (two 32x32 blocks: K from LDS as
// the A operand, its queries' Q^T held in registers as B), so a lane owns one
// query column, and accumulates O^T += V^T P^T with P^T taken straight from
// the S accumulators (converted to bf16) as the B operand.
//
// The queries arrive times c = log2(e)/sqrt(d) (the prologue rounds c q to
// bf16 once), and each tile's first two S MFMAs start from -m, the running
// maximum, instead of 0: the scores leave the MFMAs as c s - m, ready for
// exp2, with no per-score multiply-add.
//
// K and V tiles go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds: lane l of a wavefront fills bytes 16 l ..
// 16 l + 15 after the wavefront's base), row-major, 256-byte rows, with XOR-swizzled
// 16-byte columns: column c of K row r sits at c ^ (r mod 16), of V row r at
// c ^ 4 (r mod 4).  The V^T operand is read with ds_read_b64_tr_b16: within a
// group of 16 lanes, lane i receives element i mod 4 of the 8-byte pieces
// addressed by lanes 4j + i/4 (j = 0..3), so lane i addressing
// V[K0 + i/4][dbase + 4 (i mod 4)] receives d = dbase + i for keys K0 .. K0+3.
// P^T and the V^T reads use the same key order (the MFMA output order: lane
// half h holds keys 4h + 0..3 and 8 + 4h + 0..3 of every 16), so no data moves
// between lanes.  Both swizzles keep these reads free of bank conflicts.
//
// Software pipeline, one barrier per tile: the step of tile j computes S for
// tile j+1 while it exponentiates tile j and multiplies it into O.  K tiles
// and V tiles each have a ring of two LDS buffers, V one tile behind K: the
// step of tile j loads K_{j+2} and V_{j+1} into the buffers that held K_j and
// V_{j-1}, which every wavefront was done with before that step's barrier.
//
// The step's instruction order is fixed by hand (scheduling fences between
// MFMA slots): each of the 16 S MFMAs is followed by the LDS read of the K
// operand four MFMAs ahead and one pair of this tile's weights (two exp2, a
// bf16 pack, a dot2 into the row sum); each of the 16 O MFMAs by the
// transposed reads of the V operand three MFMAs ahead, and the O MFMAs also
// cover the next tile's maximum.  Two choices keep the compiler's wait
// counters precise: the tile loads are MUBUF (buffer_load ... lds) rather
// than global_load_lds, whose outstanding loads make every LDS read wait for
// all of them (lgkmcnt(0)); and each LDS buffer is its own __shared__ array,
// so the transposed reads of one V buffer are known not to alias the loads
// still landing in the other buffers (one array makes the first transposed
// read of a step wait for every load issued at the step's start).
//
// The tiles of a query block split into three runs: far window edge, interior
// (every pair visible: no mask code at all) and diagonal.  The running maximum
// is rescaled lazily: O and the row sum are rescaled only when a tile's
// maximum exceeds the reference by more than 2^8 (so P <= 256), which leaves
// the result unchanged and skips the rescale on almost every tile.  The row
// sum adds the bf16 weights that enter P V, two at a time (v_dot2_f32_bf16).
// ---------------------------------------------------------------------------
constexpr int kTileBytes = pf::kBK * pf::kD * 2;  // 16 KiB
constexpr float kRescaleSlack = 8.0f;             // log2 units

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// Buffer resource for a run of rows starting at p: raw (stride 0), range
// 2^31 - 1 bytes (the per-lane offsets of one tile stay far below), dword 3
// as gfx950 takes it for untyped loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}

// 16 bytes per lane from rs + off into LDS at dst + 16 * lane (dst uniform).
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t off, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)dst, 16, off, 0, 0, 0);
}

// max(x[l], x[l ^ 32]) in every lane: v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second, so after
// swapping x with itself the two results hold, in every lane, the lane's own
// value and its partner's.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// kPrefix: keys before main_pos0 come from a ring (chunked prefill on a
// sliding layer); without it every key is a main row (main_pos0 == 0).
// kPacked: sequences of different lengths and offsets packed row after row
// (cu_seqlens, seq_pos); a workgroup past its sequence's end exits.
// kSplit (neither of the others): kKvSplits workgroups per query block, each
// taking a contiguous share of its key tiles and writing a partial state.
template <bool kPrefix, bool kPacked, bool kSplit = false>
__global__ __launch_bounds__(256, 2) void prefill_d128_kernel(AttnArgs a) {
  using namespace pf;
  // K ring and V ring, two 16 KiB buffers each, one array per buffer
  __shared__ __attribute__((aligned(512))) char sK0[kTileBytes], sK1[kTileBytes];
  __shared__ __attribute__((aligned(512))) char sV0[kTileBytes], sV1[kTileBytes];
  auto kbuf_of = [&](int b) __attribute__((always_inline)) { return b ? sK1 : sK0; };
  auto vbuf_of = [&](int b) __attribute__((always_inline)) { return b ? sV1 : sV0; };

  const int n_qblk = (a.Tq + kBQ - 1) / kBQ;
  int split = 0;
  // (packed sequences start at their own positions: all interleaved)
  const int n_even =
      kPacked ? 0 : even_blocks(n_qblk, a.H, a.G, a.sliding, a.window, (int)a.q_pos0);
  const Work w = kSplit ? work_of_split(blockIdx.x, gridDim.x, n_qblk, a.H, n_even, split)
                        : work_of(blockIdx.x, gridDim.x, n_qblk, a.H, n_even);
  const int g = w.h / (a.H / a.G);
  // this sequence: query rows row0 .. row0 + len - 1 at positions qpos0 ..,
  // keys at positions 0 .. n_keys - 1
  int64_t row0 = (int64_t)w.b * a.Tq;
  int len = a.Tq, qpos0 = (int)a.q_pos0, n_keys = (int)a.n_keys;
  if constexpr (kPacked) {
    const int64_t c0 = min(max((int64_t)a.cu_seqlens[w.b], (int64_t)0), a.n_rows);
    const int64_t c1 = min(max((int64_t)a.cu_seqlens[w.b + 1], c0), a.n_rows);
    row0 = c0;
    len = (int)min(c1 - c0, (int64_t)a.Tq);
    qpos0 = a.seq_pos ? max(a.seq_pos[w.b], 0) : 0;
    if (w.qb * kBQ >= len || (int64_t)qpos0 + len > a.key_limit) return;
    n_keys = qpos0 + len;
  }
  const int q0 = qpos0 + w.qb * kBQ;
  const int q1 = min(q0 + kBQ, qpos0 + len);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int tq = lane_query(q0, wave, lane);
  const int tql = min(tq, q1 - 1) - qpos0;  // query row of the lane

  // Q^T operand: lane holds query tq, d = 16*ks + 8*half .. +7
  bf16x8 qop[8];
  {
    const bf16* qrow = (const bf16*)a.q + ((row0 + tql) * a.H + w.h) * kD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[ks] = *(const bf16x8*)(qrow + ks * 16 + half * 8);
  }

  int kt0, kt1, i0, i1;
  key_tiles(q0, q1, a.window, a.sliding, kt0, kt1);
  interior_tiles(q0, q1, a.window, a.sliding, kt0, kt1, i0, i1);
  // this workgroup's tiles [kta, ktb): all of them, or its split's share
  int kta = kt0, ktb = kt1;
  if constexpr (kSplit) split_tiles(kt0, kt1, split, kta, ktb);

  // Direct loads: instruction i of wavefront w fills tile rows 16 i + 4 w ..
  // +3; lane l takes row 16 i + 4 w + l/16, stored column l mod 16, i.e.
  // logical column (l mod 16) ^ swizzle(row).  Positions past the last key
  // are clamped to it (such keys lie past every query of the block: masked).
  const int lrow = 4 * wave + (lane >> 4);  // row within each 16-row slab
  const int kcol = (lane & 15) ^ (lrow & 15);
  const int vcol = (lane & 15) ^ (4 * (lrow & 3));
  // A tile's loads use a buffer resource based at its first row plus 32-bit
  // per-lane byte offsets.  Tiles whose 64 rows are consecutive rows of one
  // source take that fast path; the last tile (positions past n_keys) and,
  // with a prefix, tiles that cross the prefix/main boundary or the ring's
  // wrap go row by row.
  const bool packed_main = kPacked && a.main_packed;
  const bf16* kbase = (const bf16*)a.k + (packed_main ? row0 * a.k_sr : w.b * a.k_sb) + g * a.k_sg;
  const bf16* vbase = (const bf16*)a.v + (packed_main ? row0 * a.v_sr : w.b * a.v_sb) + g * a.v_sg;
  const int main0 = kPacked ? (packed_main ? qpos0 : 0) : (kPrefix ? (int)a.main_pos0 : 0);
  const int ring = kPrefix ? (int)a.ring : 1;
  const int64_t p_sr = a.p_sr;
  const bf16* kpbase = kPrefix ? (const bf16*)a.kp + w.b * a.p_sb + g * a.p_sg : nullptr;
  const bf16* vpbase = kPrefix ? (const bf16*)a.vp + w.b * a.p_sb + g * a.p_sg : nullptr;
  // Byte offsets of this lane's rows 16 i + lrow in a run of 64 rows, so that
  // a tile's loads are one uniform base plus these.  Row strides are at most
  // G * d elements and G is capped by the prologue's head limit, so 64 rows
  // span a few MiB at most and the offsets fit 32 bits.
  uint32_t k_off[4], v_off[4], kp_off[4], vp_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    k_off[i] = (uint32_t)(((16 * i + lrow) * (int)a.k_sr + kcol * 8) * 2);
    v_off[i] = (uint32_t)(((16 * i + lrow) * (int)a.v_sr + vcol * 8) * 2);
    kp_off[i] = kPrefix ? (uint32_t)(((16 * i + lrow) * (int)p_sr + kcol * 8) * 2) : 0u;
    vp_off[i] = kPrefix ? (uint32_t)(((16 * i + lrow) * (int)p_sr + vcol * 8) * 2) : 0u;
  }
  const int slab = 4 * wave * 256;  // this wavefront's byte offset in a slab
  // slot0 = k0 mod ring (kept up to date by the caller: an integer division
  // per tile costs about as much VALU work as a tenth of the step's softmax)
  auto load_rows = [&](const bf16* base, int64_t sr, const uint32_t* off, const bf16* pbase,
                       const uint32_t* poff, int col8, int k0, int slot0,
                       char* dst) __attribute__((always_inline)) {
    if (!kPrefix || k0 >= main0) {
      if (k0 + kBK <= n_keys) {
        const auto rs = rows_rsrc(base + (int64_t)(k0 - main0) * sr);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_to_lds(rs, off[i], dst + 16 * i * 256);
        return;
      }
    } else if (k0 + kBK <= main0 && slot0 + kBK <= ring) {
      const auto rs = rows_rsrc(pbase + (int64_t)slot0 * p_sr);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_to_lds(rs, poff[i], dst + 16 * i * 256);
      return;
    }
    // row by row: each load covers four rows of 16 lanes; the lanes of each
    // row load it from a resource based at that row (uniform per row)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = min(k0 + 16 * i + 4 * wave + r, n_keys - 1);
        const bf16* row = (!kPrefix || p >= main0) ? base + (int64_t)(p - main0) * sr
                                                   : pbase + (int64_t)(p % ring) * p_sr;
        if ((lane >> 4) == r) load_to_lds(rows_rsrc(row), (uint32_t)(col8 * 2), dst + 16 * i * 256);
      }
  };
  auto load_k = [&](int k0, int slot0, int buf) __attribute__((always_inline)) {
    load_rows(kbase, a.k_sr, k_off, kpbase, kp_off, kcol * 8, k0, slot0, kbuf_of(buf) + slab);
  };
  auto load_v = [&](int k0, int slot0, int buf) __attribute__((always_inline)) {
    load_rows(vbase, a.v_sr, v_off, vpbase, vp_off, vcol * 8, k0, slot0, vbuf_of(buf) + slab);
  };
  // ring slots of the next K and V tiles a step loads (prefix only)
  int kslot = 0, vslot = 0;
  auto advance_slot = [&](int& s) __attribute__((always_inline)) {
    s += kBK;
    if (s >= ring) s = ring >= kBK ? s - ring : s % ring;
  };

  // LDS read offsets.  K (A operand of S^T): row 32 kb + col, column
  // 2 ks + half.  V^T (A operand of O^T, ds_read_b64_tr_b16): row
  // 16 kk + 8 r + 4 half + (lane mod 16)/4, d = 32 db + 16 ((lane/16) mod 2)
  // + 4 (lane mod 4), 8-byte half (lane mod 2) of its 16-byte column.
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = col * 256 + (((2 * ks + half) ^ (col & 15)) << 4);
  const int vrow = 4 * half + ((lane & 15) >> 2);
  int voff[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int c16 = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    voff[db] = vrow * 256 + ((c16 ^ (4 * (vrow & 3))) << 4) + (lane & 1) * 8;
  }

  auto qk = [&](int buf, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    const char* k = kbuf_of(buf);
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a0 = *(const bf16x8*)(k + koff[ks]);
      const bf16x8 a1 = *(const bf16x8*)(k + koff[ks] + 32 * 256);
      s0 = mfma32(a0, qop[ks], s0);
      s1 = mfma32(a1, qop[ks], s1);
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // running maximum m of c s (the -1e30 sentinel until a score is seen)
  float m = -1e30f, lsum = 0.f;
  // the current tile's scores hold c s - sb: sb = m once the lane has seen a
  // score, 0 before; negm holds -sb in all 16 entries, the accumulator input
  // of the next tile's first S MFMAs (a sentinel base would swamp the scores
  // in fp32)
  float sb = 0.f;
  f32x16 negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;
  f32x16 s0, s1;  // scores of the current tile
  // the unmasked maximum of the current tile's scores, taken during the
  // previous step (a masked tile recomputes it after masking)
  float mt_next = 0.f;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  // the maximum of a tile's 64 scores of this lane's query: a max3 tree
  // (depth 4), then the partner lane (l ^ 32)
  auto tile_max = [&](const f32x16& x0, const f32x16& x1) __attribute__((always_inline)) {
    float t1[12];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      t1[i] = fmaxf(fmaxf(x0[3 * i], x0[3 * i + 1]), x0[3 * i + 2]);
      t1[5 + i] = fmaxf(fmaxf(x1[3 * i], x1[3 * i + 1]), x1[3 * i + 2]);
    }
    t1[10] = x0[15];
    t1[11] = x1[15];
    const float t2a = fmaxf(fmaxf(t1[0], t1[1]), t1[2]), t2b = fmaxf(fmaxf(t1[3], t1[4]), t1[5]);
    const float t2c = fmaxf(fmaxf(t1[6], t1[7]), t1[8]), t2d = fmaxf(fmaxf(t1[9], t1[10]), t1[11]);
    return pair_max(fmaxf(fmaxf(t2a, t2b), fmaxf(t2c, t2d)));
  };

  // Step of tile kt.  kMask: apply the visibility predicate per element.
  // kBuf: buffers holding K_kt and V_kt ((kt - kta) mod 2, known at compile
  // time so that every LDS address is a constant offset).  Operand rings:
  // K reads run kKA MFMAs ahead of their use, V reads kVA.
  constexpr int kKA = 4, kVA = 3;
  auto step = [&](int kt, auto mask_tag, auto buf_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    constexpr int jb = decltype(buf_tag)::value;
    const int k0 = kt * kBK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 2 < ktb) load_k(k0 + 2 * kBK, kslot, jb);
    if (kt + 1 < ktb) load_v(k0 + kBK, vslot, jb ^ 1);
    if constexpr (kPrefix) {
      advance_slot(kslot);
      advance_slot(vslot);
    }

    const char* kbuf = kbuf_of(jb ^ 1);  // K of tile kt + 1
    const char* vbuf = vbuf_of(jb);      // V of tile kt
    // K operand of S MFMA i (i = 0..15): 16-dim chunk i / 2, keys 32 (i mod 2) ..
    auto kread = [&](int i) __attribute__((always_inline)) {
      return *(const bf16x8*)(kbuf + koff[i >> 1] + (i & 1) * 32 * 256);
    };
    // V^T operand of O MFMA i: keys 16 (i / 4) .., dims 32 (i mod 4) ..
    auto vread = [&](int i) __attribute__((always_inline)) {
      const int kk = i >> 2, db = i & 3;
      const bf16x4 lo4 = lds_read_tr(vbuf + voff[db] + (16 * kk) * 256);
      const bf16x4 hi4 = lds_read_tr(vbuf + voff[db] + (16 * kk + 8) * 256);
      return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    };
    // the first K reads overlap the mask, maximum and rescale test
    bf16x8 ka[kKA + 1];
#pragma unroll
    for (int i = 0; i < kKA; ++i) ka[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);

    float mt = mt_next;
    if constexpr (kMask) {
      // the two 32-key blocks of the tile start at k0 and k0 + 32
      mask_block(s0, tq, k0, lane, a.window, a.sliding);
      mask_block(s1, tq, k0 + 32, lane, a.window, a.sliding);
      mt = tile_max(s0, s1);
    }
    if (__ballot(mt + sb > m + kRescaleSlack)) {
      const float mn = fmaxf(m, mt + sb);
      float alpha = fast_exp2(m - mn);
      // keep this a real (uniform) branch: without the barrier the compiler
      // folds the condition into the multiplier and rescales every tile
      asm volatile("" : "+v"(alpha));
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      // the tile's scores and the next tile's start move to the new base
      const float nb = mn > -1e29f ? mn : 0.f;
      const float sh = sb - nb;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] += sh;
        s1[r] += sh;
        negm[r] = -nb;
      }
      sb = nb;
    }

    bf16x8 pk[4];
    // weights of key pair p of the tile (p = 0..15: 16-key chunk p / 4, pair
    // p mod 4), packed to bf16 and added to the row sum
    auto pair = [&](int p) __attribute__((always_inline)) {
      const int kk = p >> 2, e = 2 * (p & 3), r = (kk & 1) * 8 + e;
      const float x0 = (kk < 2 ? s0 : s1)[r], x1 = (kk < 2 ? s0 : s1)[r + 1];
      pk[kk][e] = (bf16)fast_exp2(x0);
      pk[kk][e + 1] = (bf16)fast_exp2(x1);
      const bf16x2 pr = {pk[kk][e], pk[kk][e + 1]};
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
    };

    // The S MFMAs carry this tile's exponentials between them: a wavefront
    // in that half of its step issues ahead of the other wavefront on its
    // SIMD (wave priority 1), whose O MFMAs then fill the MFMA pipe while
    // the first one's VALU work runs (+2-5 % against equal priorities).
    __builtin_amdgcn_s_setprio(1);
    // S of the next tile (on the last tile the result is discarded), started
    // from -sb: MFMA i, then the K read for MFMA i + kKA, then weight pair i
    // of this tile
    f32x16 n0, n1;
    bf16x8 va[kVA + 1];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & 1)
        n1 = mfma32(ka[i % (kKA + 1)], qop[i >> 1], i == 1 ? negm : n1);
      else
        n0 = mfma32(ka[i % (kKA + 1)], qop[i >> 1], i == 0 ? negm : n0);
      if (i + kKA < 16) ka[(i + kKA) % (kKA + 1)] = kread(i + kKA);
      if (i == 15) {
#pragma unroll
        for (int u = 0; u < kVA; ++u) va[u] = vread(u);
      }
      pair(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // O += P V: MFMA i, then the V reads for MFMA i + kVA; slots 8-12 also
    // take the next tile's maximum (its S MFMAs are done by then)
    float t1[12], t2[4], mx = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o[i & 3] = mfma32(va[i % (kVA + 1)], pk[i >> 2], o[i & 3]);
      if (i + kVA < 16) va[(i + kVA) % (kVA + 1)] = vread(i + kVA);
      if (i == 8 || i == 9) {
#pragma unroll
        for (int u = 5 * (i - 8); u < 5 * (i - 7); ++u) {
          t1[u] = fmaxf(fmaxf(n0[3 * u], n0[3 * u + 1]), n0[3 * u + 2]);
          t1[5 + u] = fmaxf(fmaxf(n1[3 * u], n1[3 * u + 1]), n1[3 * u + 2]);
        }
      }
      if (i == 10) {
        t1[10] = n0[15];
        t1[11] = n1[15];
        t2[0] = fmaxf(fmaxf(t1[0], t1[1]), t1[2]);
        t2[1] = fmaxf(fmaxf(t1[3], t1[4]), t1[5]);
        t2[2] = fmaxf(fmaxf(t1[6], t1[7]), t1[8]);
        t2[3] = fmaxf(fmaxf(t1[9], t1[10]), t1[11]);
      }
      if (i == 11) mx = fmaxf(fmaxf(t2[0], t2[1]), fmaxf(t2[2], t2[3]));
      if (i == 12) mt_next = pair_max(mx);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    s0 = n0;
    s1 = n1;
  };


  // (a split with no tiles skips to its empty partial state)
  if (!kSplit || kta < ktb) {
    const int slot_a = kPrefix ? (kta * kBK) % ring : 0;
    load_k(kta * kBK, slot_a, 0);
    load_v(kta * kBK, slot_a, 0);
    if constexpr (kPrefix) {
      vslot = slot_a;
      advance_slot(vslot);  // tile kta + 1
      kslot = vslot;
      advance_slot(kslot);  // tile kta + 2
    }
    if (kta + 1 < ktb) load_k((kta + 1) * kBK, vslot, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    qk(0, s0, s1);
    mt_next = tile_max(s0, s1);
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    auto run = [&](int& kt, int end, auto mask_tag) __attribute__((always_inline)) {
      if (kt < end && ((kt - kta) & 1)) step(kt++, mask_tag, B1{});
      for (; kt + 1 < end; kt += 2) {
        step(kt, mask_tag, B0{});
        step(kt + 1, mask_tag, B1{});
      }
      if (kt < end) step(kt++, mask_tag, B0{});
    };
    int kt = kta;
    run(kt, kSplit ? min(i0, ktb) : i0, std::true_type{});
    run(kt, kSplit ? min(i1, ktb) : i1, std::false_type{});
    run(kt, ktb, std::true_type{});
  }

  lsum += __shfl_xor(lsum, 32, kWave);
  if constexpr (kSplit) {
    // partial state (m, l, o[d]) of this query, head and split; lanes l and
    // l + 32 hold the same m and l and different halves of o
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    if (tq < q1) {
      float* pp = a.part +
                  (((row0 + (tq - qpos0)) * a.H + w.h) * kKvSplits + split) * (int64_t)(kD + 2);
      if (half == 0) {
        pp[0] = m;
        pp[1] = lsum;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float* po = pp + 2 + db * 32 + 8 * r4 + 4 * half;
          *(f32x2*)po = f32x2{o[db][4 * r4], o[db][4 * r4 + 1]};
          *(f32x2*)(po + 2) = f32x2{o[db][4 * r4 + 2], o[db][4 * r4 + 3]};
        }
    }
    return;
  }
  const float inv = 1.0f / lsum;
  if (tq < q1) {
    bf16* orow = (bf16*)a.out + ((row0 + (tq - qpos0)) * a.H + w.h) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v4 = {(bf16)(o[db][4 * r4] * inv), (bf16)(o[db][4 * r4 + 1] * inv),
                     (bf16)(o[db][4 * r4 + 2] * inv), (bf16)(o[db][4 * r4 + 3] * inv)};
        *(bf16x4*)(orow + db * 32 + 8 * r4 + 4 * half) = v4;
      }
  }
}

// Counts every (query, key) pair the kernel above accumulates: the same
// work mapping, tile runs, lane -> (query, key) map and mask function.
// visit[(t - pos_offset) * (pos_offset + T) + s] for query position t and key
// position s.
__global__ __launch_bounds__(256) void probe_prefill_kernel(int T, int pos_offset, int window,
                                                            int sliding, int kv_splits,
                                                            uint8_t* visit) {
  using namespace pf;
  const int n_qblk = (T + kBQ - 1) / kBQ;
  const int n_keys = pos_offset + T;
  int split = 0;
  const Work w = kv_splits > 1 ? work_of_split(blockIdx.x, gridDim.x, n_qblk, 1, 0, split)
                               : work_of(blockIdx.x, gridDim.x, n_qblk, 1, 0);
  const int q0 = pos_offset + w.qb * kBQ, q1 = min(q0 + kBQ, n_keys);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tq = lane_query(q0, wave, lane);
  int kt0, kt1, i0, i1;
  key_tiles(q0, q1, window, sliding, kt0, kt1);
  interior_tiles(q0, q1, window, sliding, kt0, kt1, i0, i1);
  int kta = kt0, ktb = kt1;
  if (kv_splits > 1) split_tiles(kt0, kt1, split, kta, ktb);
  for (int kt = kta; kt < ktb; ++kt) {
    const int k0 = kt * kBK;
    const bool interior = kt >= i0 && kt < i1;
    for (int kb = 0; kb < 2; ++kb) {
      // the kernel's own masking of this block (interior tiles unmasked)
      f32x16 sc;
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
      if (!interior) mask_block(sc, tq, k0 + 32 * kb, lane, window, sliding);
      for (int r = 0; r < 16; ++r) {
        const int s = lane_key(k0, kb, r, lane);
        // one lane owns each (query, key) pair, so the count has no race
        if (sc[r] == 0.f && tq < q1 && s < n_keys) ++visit[(int64_t)(tq - pos_offset) * n_keys + s];
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t s) {
  const int n_qblk = (a.Tq + pf::kBQ - 1) / pf::kBQ;
  const int blocks = n_qblk * a.H * a.B;
  if (a.cu_seqlens) {
    if (a.kp)
      prefill_d128_kernel<true, true><<<blocks, 256, 0, s>>>(a);
    else
      prefill_d128_kernel<false, true><<<blocks, 256, 0, s>>>(a);
  } else if (a.kp) {
    prefill_d128_kernel<true, false><<<blocks, 256, 0, s>>>(a);
  } else if (a.kv_splits == pf::kKvSplits) {
    prefill_d128_kernel<false, false, true><<<blocks * pf::kKvSplits, 256, 0, s>>>(a);
  } else {
    prefill_d128_kernel<false, false><<<blocks, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_probe_prefill(int T, int64_t pos_offset, int window, int sliding, int kv_splits,
                                uint8_t* visit, hipStream_t s) {
  hipError_t e = hipMemsetAsync(visit, 0, (size_t)T * (size_t)(pos_offset + T), s);
  if (e != hipSuccess) return e;
  const int n_qblk = (T + pf::kBQ - 1) / pf::kBQ;
  probe_prefill_kernel<<<n_qblk * kv_splits, 256, 0, s>>>(T, (int)pos_offset, window, sliding,
                                                          kv_splits, visit);
  return hipGetLastError();
}

}  // namespace olmo3
