// Causal attention kernels: a plain per-query kernel for other head sizes
// and fp32, and split-KV decode (d = 128, bf16 or e4m3 caches) with a
// log-sum-exp merge across wavefronts and, when a key range is split, across
// workgroups.
// The MFMA prefill kernel lives in prefill.hip.
//
// Masking follows "OLMo 3's Sliding-Window Attention Pattern", "The
// sliding-window mask"; decode on a ring reads exactly the `window` held
// entries ("Olmo 3 7B", "SERVICEABILITY JOIN").  Softmax uses base-2
// exponentials with log2(e)/sqrt(d) folded into the scores.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace olmo3 {

namespace {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Plain kernel: one thread per query row, keys streamed from global memory.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnArgs a) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  // this sequence: query rows row0 .. row0 + len - 1 at positions qpos0 ..
  int64_t row0 = (int64_t)b * a.Tq, len = a.Tq, qpos0 = a.q_pos0, n_keys = a.n_keys;
  if (a.cu_seqlens) {
    const int64_t c0 = min(max((int64_t)a.cu_seqlens[b], (int64_t)0), a.n_rows);
    const int64_t c1 = min(max((int64_t)a.cu_seqlens[b + 1], c0), a.n_rows);
    row0 = c0;
    len = min(c1 - c0, (int64_t)a.Tq);
    qpos0 = a.seq_pos ? max((int64_t)a.seq_pos[b], (int64_t)0) : 0;
    if (qpos0 + len > a.key_limit) return;
    n_keys = qpos0 + len;
  } else if (a.all_visible && a.seq_pos) {
    // decode, per-sequence positions: rows of the ring or the linear cache
    const int64_t p = max((int64_t)a.seq_pos[b], (int64_t)0);
    n_keys = min(a.sliding ? min(p + 1, (int64_t)a.window) : p + 1, a.key_limit);
  }
  if (t >= len) return;
  const int g = h / (a.H / a.G);
  const T* qp = (const T*)a.q + ((row0 + t) * a.H + h) * D;
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = (float)qp[e] * a.scale_log2;
    o[e] = 0.f;
  }
  const int64_t tpos = qpos0 + t;
  // positions [p0, p1) when masked; main rows [0, n_keys) when all visible
  int64_t p0 = 0, p1 = n_keys;
  if (!a.all_visible) {
    p1 = min(tpos + 1, n_keys);
    if (a.sliding) p0 = max(tpos - a.window + 1, (int64_t)0);
  }
  const bool packed_main = a.cu_seqlens && a.main_packed;
  const int64_t main0 = a.all_visible ? 0 : (a.cu_seqlens ? (packed_main ? qpos0 : 0) : a.main_pos0);
  const T* kb = (const T*)a.k + (packed_main ? row0 * a.k_sr : b * a.k_sb) + g * a.k_sg;
  const T* vb = (const T*)a.v + (packed_main ? row0 * a.v_sr : b * a.v_sb) + g * a.v_sg;
  const T* kpb = a.kp ? (const T*)a.kp + b * a.p_sb + g * a.p_sg : nullptr;
  const T* vpb = a.kp ? (const T*)a.vp + b * a.p_sb + g * a.p_sg : nullptr;
  float m = -1e30f, l = 0.f;
  for (int64_t p = p0; p < p1; ++p) {
    const T *kp, *vp;
    if (p >= main0) {
      kp = kb + (p - main0) * a.k_sr;
      vp = vb + (p - main0) * a.v_sr;
    } else {
      const int64_t slot = a.ring > 0 ? p % a.ring : p;
      kp = kpb + slot * a.p_sr;
      vp = vpb + slot * a.p_sr;
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) s += q[e] * (float)kp[e];
    const float mn = fmaxf(m, s);
    const float al = fast_exp2(m - mn);
    const float pr = fast_exp2(s - mn);
    l = l * al + pr;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = o[e] * al + pr * (float)vp[e];
    m = mn;
  }
  const float inv = 1.0f / l;
  T* op = (T*)a.out + ((row0 + t) * a.H + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = (T)(o[e] * inv);
}

// ---------------------------------------------------------------------------
// Split-KV decode, d = 128, bf16.  16 lanes read one 256-byte cache row
// (8 bf16 each); 16 lane groups per workgroup stream interleaved rows of the
// split, kUnroll rows per group in flight.  Every row is read once for all
// GRP query heads of its key/value head.  Scores are reduced across the 16
// lanes, the softmax state is kept per lane group and merged, first across
// the 4 groups of a wavefront with lane exchanges and then across
// wavefronts in LDS, into one partial (m, l, o) per head and split, or,
// when the split is the whole key range, into the output row itself.
// ---------------------------------------------------------------------------
// Sum over the 16 lanes of a DPP row, returned in all of them: neighbours,
// pairs of neighbours, the two quads of each half row (mirrored), then the
// two half rows (mirrored); each step is one add with a DPP operand.
template <int kCtrl>
__device__ __forceinline__ float dpp_operand(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                              0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_operand<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_operand<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_operand<0x141>(x);  // row_half_mirror
  x += dpp_operand<0x140>(x);  // row_mirror
  return x;
}

// Sum over the 8 lanes of each half of a 16-lane row.
__device__ __forceinline__ float row8_sum(float x) {
  x += dpp_operand<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_operand<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_operand<0x141>(x);  // row_half_mirror
  return x;
}

__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
__device__ __forceinline__ bf16x2 pair(const bf16x8& v, int i) {
  return bf16x2{v[2 * i], v[2 * i + 1]};
}

// kFp8: the caches hold e4m3 codes (a 128-byte row, 8 bytes per lane);
// k_scale is folded into the query and v_scale into the partial output, so
// each scale multiplies the result exactly once.
// Waves per SIMD the register budget is held to: enough rows in flight per
// CU to cover HBM latency (each wavefront streams 8 KiB per iteration).
constexpr float kSlack = 8.0f;  // log2 units: bf16-cache weights at most 2^8 before a rescale

template <int GRP, bool kFp8>
constexpr int decode_waves_per_eu() {
  return kFp8 ? (GRP <= 2 ? 6 : (GRP <= 3 ? 4 : 2)) : (GRP <= 1 ? 8 : (GRP <= 5 ? 4 : 2));
}

template <int GRP, bool kFp8>
__global__ __launch_bounds__(dec::kThreads)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<GRP, kFp8>()))) void decode_split_kernel(
    DecodeArgs a) {
  using namespace dec;
  const int sp = blockIdx.x % a.splits;
  const int bg = blockIdx.x / a.splits;
  const int g = bg % a.G, b = bg / a.G;
  int64_t n = a.n, rps = a.rows_per_split;
  if (a.seq_pos) {  // this sequence's rows, split evenly
    const int64_t p = max((int64_t)a.seq_pos[b], (int64_t)0);
    n = min(a.sliding ? min(p + 1, (int64_t)a.window) : p + 1, a.cap);
    rps = ((n + a.splits - 1) / a.splits + kRowsPerIter - 1) / kRowsPerIter * kRowsPerIter;
  }
  const int64_t r0 = (int64_t)sp * rps;
  const int64_t r1 = min(n, r0 + rps);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15;
  const int grp = tid >> 4;

  static_assert(kUnroll == 4, "rows are paired for the bf16 dot products");
  // queries: bf16 pairs (bf16 caches), or fp32 scaled by k_scale (e4m3)
  bf16x8 qv[GRP];
  float qf[kFp8 ? GRP : 1][8];
#pragma unroll
  for (int j = 0; j < GRP; ++j) {
    qv[j] = *(const bf16x8*)((const bf16*)a.q + ((int64_t)b * a.H + g * GRP + j) * kD + li * 8);
    if constexpr (kFp8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[j][e] = (float)qv[j][e] * a.k_scale;
    }
  }
  const float c = a.scale_log2;
  float m[GRP], l[GRP], o[GRP][8];
#pragma unroll
  for (int j = 0; j < GRP; ++j) {
    m[j] = -1e30f;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  }
  // row r of this (sequence, head): element offset (bf16) or byte offset (e4m3)
  const int64_t base = ((int64_t)b * a.G + g) * a.cap * kD + li * 8;
  const bf16* kb = (const bf16*)a.k_cache + base;
  const bf16* vb = (const bf16*)a.v_cache + base;
  const uint8_t* kb8 = (const uint8_t*)a.k_cache + base;
  const uint8_t* vb8 = (const uint8_t*)a.v_cache + base;
  typedef typename std::conditional<kFp8, u32x2, bf16x8>::type Chunk;
  // Cache rows are read once per call: non-temporal loads keep the stream
  // from being allocated in L2 and the last-level cache (+13 % bandwidth).
  auto load = [&](const bf16* p16, const uint8_t* p8, int64_t r) -> Chunk {
    if constexpr (kFp8)
      return __builtin_nontemporal_load((const u32x2*)(p8 + r * kD));
    else
      return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)(p16 + r * kD)));
  };
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  const int64_t n_iter = r1 > r0 ? (r1 - r0 + kRowsPerIter - 1) / kRowsPerIter : 0;
  if constexpr (kFp8 && GRP == 1) {
    // e4m3 codes, one query head: 16-byte loads (half the load instructions
    // of 8-byte ones).  Each 16-lane group still reads rows row_of(i, u) for
    // u = 0..3 of every iteration, as a pair of rows per step: lanes 8 h + c
    // take codes 16 c .. 16 c + 15 of row row_of(i, 2 u2 + h), u2 = 0, 1.
    // The two halves keep separate softmax states over their rows, merged
    // after the loop, then spread to the 8-elements-per-lane layout below.
    const int h = li >> 3, cc = li & 7;
    float qf16[16];
    {
      const bf16* qp = (const bf16*)a.q + ((int64_t)b * a.H + g) * kD + 16 * cc;
      const bf16x8 q0 = *(const bf16x8*)qp, q1 = *(const bf16x8*)(qp + 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf16[e] = (float)q0[e] * a.k_scale;
        qf16[8 + e] = (float)q1[e] * a.k_scale;
      }
    }
    float o16[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o16[e] = 0.f;
    const uint8_t* kr8 = (const uint8_t*)a.k_cache + ((int64_t)b * a.G + g) * a.cap * kD + 16 * cc;
    const uint8_t* vr8 = (const uint8_t*)a.v_cache + ((int64_t)b * a.G + g) * a.cap * kD + 16 * cc;
    for (int64_t i = 0; i < n_iter; ++i) {
      u32x4 kr[2], vr[2];
      bool ok[2];
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int64_t r = row_of(r0, i, 2 * u2 + h, grp);
        ok[u2] = r < r1;
        const int64_t rc = ok[u2] ? r : r0;
        kr[u2] = __builtin_nontemporal_load((const u32x4*)(kr8 + rc * kD));
        vr[u2] = __builtin_nontemporal_load((const u32x4*)(vr8 + rc * kD));
      }
      float sc[2];
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        float kf[16];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) e4m3x4_to_f32(kr[u2][w4], kf + 4 * w4);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc = fmaf(qf16[e], kf[e], acc);
        const float t = row8_sum(acc) * c;  // every lane takes part in the sum
        sc[u2] = ok[u2] ? t : -INFINITY;
      }
      const float mn = fmaxf(m[0], fmaxf(sc[0], sc[1]));
      const float al = fast_exp2(m[0] - mn);
      m[0] = mn;
      const float p0 = fast_exp2(sc[0] - mn), p1 = fast_exp2(sc[1] - mn);
      l[0] = l[0] * al + (p0 + p1);
      float vf0[16], vf1[16];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        e4m3x4_to_f32(vr[0][w4], vf0 + 4 * w4);
        e4m3x4_to_f32(vr[1][w4], vf1 + 4 * w4);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) o16[e] = fmaf(p1, vf1[e], fmaf(p0, vf0[e], o16[e] * al));
    }
    // merge the halves (lanes l and l ^ 8 hold the same elements)
    {
      const float mo = __shfl_xor(m[0], 8, kWave), lo = __shfl_xor(l[0], 8, kWave);
      const float mn = fmaxf(m[0], mo);
      const float fa = fast_exp2(m[0] - mn), fb = fast_exp2(mo - mn);
      l[0] = l[0] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < 16; ++e) o16[e] = o16[e] * fa + __shfl_xor(o16[e], 8, kWave) * fb;
      m[0] = mn;
    }
    // lane li of the group takes elements 8 li .. 8 li + 7: those of lane
    // li / 2, first or second half
    const int src = (lane & ~15) + (li >> 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float lo8 = __shfl(o16[e], src, kWave), hi8 = __shfl(o16[8 + e], src, kWave);
      o[0][e] = (li & 1) ? hi8 : lo8;
    }
  } else if constexpr (kFp8) {
    // e4m3 codes: keys and values converted to fp32, exact running maximum
    // rescaled every iteration, every row masked against r1 (the loop shape
    // that measured fastest for these half-size rows)
    for (int64_t i = 0; i < n_iter; ++i) {
      Chunk kr[kUnroll], vr[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t r = row_of(r0, i, u, grp);
        ok[u] = r < r1;
        const int64_t rc = ok[u] ? r : r0;
        kr[u] = load(kb, kb8, rc);
        vr[u] = load(vb, vb8, rc);
      }
      // scores in log2 units: this lane's 8 elements, then the row's 16 lanes
      float s[kUnroll][GRP];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float kf[8];
        e4m3x4_to_f32(kr[u][0], kf);
        e4m3x4_to_f32(kr[u][1], kf + 4);
#pragma unroll
        for (int j = 0; j < GRP; ++j) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf(qf[j][e], kf[e], acc);
          s[u][j] = acc;
        }
#pragma unroll
        for (int j = 0; j < GRP; ++j) s[u][j] = row16_sum(s[u][j]) * c;
      }
      float vf[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        e4m3x4_to_f32(vr[u][0], vf[u]);
        e4m3x4_to_f32(vr[u][1], vf[u] + 4);
      }
      float mx[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        mx[j] = -INFINITY;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (!ok[u]) s[u][j] = -INFINITY;
          mx[j] = fmaxf(mx[j], s[u][j]);
        }
      }
      float al[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const float mn = fmaxf(m[j], mx[j]);
        al[j] = fast_exp2(m[j] - mn);
        m[j] = mn;
      }
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        float p[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) p[u] = fast_exp2(s[u][j] - m[j]);
        l[j] = l[j] * al[j] + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float acc = o[j][e] * al[j];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) acc = fmaf(p[u], vf[u][e], acc);
          o[j][e] = acc;
        }
      }
    }
  } else {
    // bf16 rows.  One iteration: 4 rows per lane group; only the last
    // iteration of a split can hold rows past r1 (kTail: rows clamped to r0
    // and masked).  Scores stay unscaled until the exponent, c * s - m in one
    // fma.  Lazy rescale: m[j] is a reference maximum, moved (and o, l
    // rescaled) only when a scaled score passes it by more than 2^kSlack, so
    // the weights stay at most 2^kSlack; the merges below accept any
    // reference.
    auto iteration = [&](int64_t i, auto tail_tag) __attribute__((always_inline)) {
      constexpr bool kTail = decltype(tail_tag)::value;
      Chunk kr[kUnroll], vr[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t r = row_of(r0, i, u, grp);
        ok[u] = !kTail || r < r1;
        const int64_t rc = ok[u] ? r : r0;
        kr[u] = load(kb, kb8, rc);
        vr[u] = load(vb, vb8, rc);
      }
      // scores: this lane's 8 elements, then the row's 16 lanes
      float s[kUnroll][GRP];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
        for (int j = 0; j < GRP; ++j) {
          float acc = dot2(pair(kr[u], 0), pair(qv[j], 0), 0.f);
#pragma unroll
          for (int e = 1; e < 4; ++e) acc = dot2(pair(kr[u], e), pair(qv[j], e), acc);
          s[u][j] = row16_sum(acc);
        }
      }
      // values as bf16 pairs of rows (0, 1) and (2, 3)
      bf16x2 v01[8], v23[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v01[e] = bf16x2{vr[0][e], vr[1][e]};
        v23[e] = bf16x2{vr[2][e], vr[3][e]};
      }
      bool grow = false;
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (kTail && !ok[u]) s[u][j] = -INFINITY;
          mx = fmaxf(mx, s[u][j]);
        }
        grow |= mx * c > m[j] + kSlack;
      }
      if (__ballot(grow)) {
#pragma unroll
        for (int j = 0; j < GRP; ++j) {
          float mx = -INFINITY;
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, s[u][j]);
          const float mn = fmaxf(m[j], mx * c);
          float a1 = fast_exp2(m[j] - mn);
          // keep this a real (uniform) branch rather than a multiply per tile
          asm volatile("" : "+v"(a1));
          m[j] = mn;
          l[j] *= a1;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[j][e] *= a1;
        }
      }
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        float p[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) p[u] = fast_exp2(fmaf(s[u][j], c, -m[j]));
        // the weights enter P V as bf16; the row sum adds those same values
        const bf16x2 p01 = {(bf16)p[0], (bf16)p[1]}, p23 = {(bf16)p[2], (bf16)p[3]};
        l[j] = dot2(p23, ones, dot2(p01, ones, l[j]));
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = dot2(p23, v23[e], dot2(p01, v01[e], o[j][e]));
      }
    };
    for (int64_t i = 0; i + 1 < n_iter; ++i) iteration(i, std::false_type{});
    if (n_iter > 0) iteration(n_iter - 1, std::true_type{});
  }

  // merge the 4 lane groups of this wavefront (lanes l, l^16, l^32, l^48)
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const float mo = __shfl_xor(m[j], off, kWave);
      const float lo = __shfl_xor(l[j], off, kWave);
      const float mn = fmaxf(m[j], mo);
      const float fa = fast_exp2(m[j] - mn), fb = fast_exp2(mo - mn);
      l[j] = l[j] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[j][e], off, kWave);
        o[j][e] = o[j][e] * fa + oo * fb;
      }
      m[j] = mn;
    }
  }
  // then the 4 wavefronts, through LDS
  __shared__ float sm[4][GRP], sl[4][GRP];
  __shared__ float so[4][GRP][kD];
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (li == 0) {
        sm[wave][j] = m[j];
        sl[wave][j] = l[j];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) so[wave][j][li * 8 + e] = o[j][e];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < GRP * kD; idx += kThreads) {
    const int j = idx / kD, d = idx % kD;
    float M = sm[0][j];
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2) M = fmaxf(M, sm[w2][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const float f = fast_exp2(sm[w2][j] - M);
      L += sl[w2][j] * f;
      O += so[w2][j][d] * f;
    }
    const float Ov = kFp8 ? O * a.v_scale : O;
    const int64_t bh = (int64_t)b * a.H + g * GRP + j;
    if (a.splits == 1) {
      // the whole key range: the output row itself (the merge of one state)
      ((bf16*)a.out)[bh * kD + d] = (bf16)(Ov / L);
      continue;
    }
    float* pp = a.part + (bh * a.splits + sp) * (kD + 2);
    if (d == 0) {
      pp[0] = M;
      pp[1] = L;
    }
    pp[2 + d] = Ov;
  }
}

// Split-KV decode on MFMA, bf16 caches, GRP = H/G >= 2 query heads per
// key/value head.  Same split of the rows [r0, r1) over workgroups and the
// same partial (m, l, o) per head as decode_split_kernel; inside a split the
// 4 wavefronts take 16-row stages in turn (stage t -> wavefront t mod 4).
// Per stage a wavefront
//   - loads the stage's K straight into the MFMA A-operand layout (lane l:
//     key l mod 16, d = 32 kk + 8 (l/16) + 0..7) and its V rows coalesced
//     (lane l: row 4 i + l/16, 16-byte column l mod 16), two stages ahead
//     of the arithmetic (non-temporal: every row is read once);
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (B = Q^T: lane l holds
//     query l mod 16, zero past GRP), 4 blocks over d = 128; lane l ends with
//     query l mod 16 and keys 4 (l/16) + 0..3;
//   - softmax over the stage's 16 keys per query (maximum over the lane's 4
//     values, then lanes l ^ 16 and l ^ 32), with the lazy reference maximum
//     of the VALU kernel;
//   - writes V to its LDS tile (16-byte columns XOR-swizzled by 2 (r mod 8)
//     so the transposed reads are conflict-free) and forms O += P V with
//     v_mfma_f32_16x16x16_bf16: A = P, already in its layout (query l mod 16,
//     keys 4 (l/16) + 0..3), B = 16 keys x 16 d of V read with
//     ds_read_b64_tr_b16 (lane 4 j + t of a 16-lane group addresses row
//     4 (l/16) + j, d = 16 blk + 4 t .. + 3, and receives V[4 (l/16) + j]
//     [16 blk + l mod 16], j = 0..3), 8 blocks over d.
// Lane l then holds O for queries 4 (l/16) + r, d = 16 blk + l mod 16.
constexpr int kStageRows = 16;

typedef short i16x4 __attribute__((ext_vector_type(4)));

struct DecStage {
  bf16x8 k[4];  // A operand of block kk
  bf16x8 v[4];  // rows 4 i + l/16, column l mod 16
};
// e4m3 caches: 16-byte loads (half as many load instructions per byte as
// 8-byte ones).  k: the lane's 32 code bytes of its key row (d = 32 quad ..
// +31, block kk taking d = 32 quad + 8 kk .. +7; the Q operand is loaded
// with the same d order, which the sum over d does not see); v: code bytes
// 16 (col mod 8) .. +15 of rows 8 i + 2 quad + col / 8.
struct DecStage8 {
  u32x4 k[2];
  u32x4 v[2];
};

// Eight e4m3 codes -> their values as bf16 (exact: every e4m3 value is a
// bf16 value), two per v_cvt_scalef32_pk_bf16_fp8 (scale 1: the cache scales
// are applied to the softmax scale and the output instead).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 w) {
  const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], 1.0f, false);
  const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], 1.0f, true);
  const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], 1.0f, false);
  const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], 1.0f, true);
  return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// Two wavefronts per SIMD: the three stages in registers (96 VGPRs of K and V)
// leave no room for a third.  kFp8: e4m3 caches, converted to bf16 in
// registers (keys as the MFMA operand, values before their LDS tile);
// k_scale multiplies the softmax scale and v_scale the output.
template <int GRP, bool kFp8>
__global__ __launch_bounds__(dec::kThreads, 2) void decode_mfma_kernel(DecodeArgs a) {
  using namespace dec;
  static_assert(GRP >= 2 && GRP <= 16, "query heads per key/value head");
  __shared__ __attribute__((aligned(16))) char vtile[4][kStageRows * kD * 2];  // per wavefront
  __shared__ float sm[4][GRP], sl[4][GRP];
  __shared__ float so[4][GRP][kD];

  const int sp = blockIdx.x % a.splits;
  const int bg = blockIdx.x / a.splits;
  const int g = bg % a.G, b = bg / a.G;
  int64_t n = a.n, rps = a.rows_per_split;
  if (a.seq_pos) {  // this sequence's rows, split evenly
    const int64_t p = max((int64_t)a.seq_pos[b], (int64_t)0);
    n = min(a.sliding ? min(p + 1, (int64_t)a.window) : p + 1, a.cap);
    rps = ((n + a.splits - 1) / a.splits + kRowsPerIter - 1) / kRowsPerIter * kRowsPerIter;
  }
  const int64_t r0 = (int64_t)sp * rps;
  const int64_t r1 = min(n, r0 + rps);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, quad = lane >> 4;

  // Q^T operand: query col (zero past GRP), d = 32 kk + 8 quad .. + 7
  // (e4m3 caches: d = 32 quad + 8 kk .. + 7, the order of the key codes)
  bf16x8 qop[4];
  {
    const bool real = col < GRP;
    const bf16* qrow = (const bf16*)a.q + ((int64_t)b * a.H + g * GRP + (real ? col : 0)) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int d0 = kFp8 ? 32 * quad + 8 * kk : 32 * kk + 8 * quad;
      const bf16x8 v = *(const bf16x8*)(qrow + d0);
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[kk][e] = real ? v[e] : (bf16)0.0f;
    }
  }

  // (sequence, head) bases, uniform; rows as 32-bit byte offsets (the
  // launcher takes this kernel only while cap * 256 B fits 32 bits)
  constexpr int kEs = kFp8 ? 1 : 2;  // bytes per cache element
  // stages in flight per wavefront (8 KiB of K and V each with bf16 rows,
  // 4 KiB with e4m3 codes; 4 or 5 e4m3 stages measured no faster)
  constexpr int kStages = 3;
  typedef typename std::conditional<kFp8, DecStage8, DecStage>::type Stage;
  const char* kb = (const char*)a.k_cache + ((int64_t)b * a.G + g) * a.cap * kD * kEs;
  const char* vb = (const char*)a.v_cache + ((int64_t)b * a.G + g) * a.cap * kD * kEs;
  const uint32_t rlast = (uint32_t)(r1 - 1);
  auto fetch = [&](int64_t t, Stage& st) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(r0 + t * kStageRows);
    if constexpr (kFp8) {
      const uint32_t koff = min(base + col, rlast) * kD + 32 * quad;
      st.k[0] = __builtin_nontemporal_load((const u32x4*)(kb + koff));
      st.k[1] = __builtin_nontemporal_load((const u32x4*)(kb + koff + 16));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t voff = min(base + 8 * i + 2 * quad + (col >> 3), rlast) * kD + 16 * (col & 7);
        st.v[i] = __builtin_nontemporal_load((const u32x4*)(vb + voff));
      }
    } else {
      const uint32_t koff = min(base + col, rlast) * (kD * 2) + 16 * quad;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        st.k[kk] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)(kb + koff + 64 * kk)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t voff = min(base + 4 * i + quad, rlast) * (kD * 2) + 16 * col;
        st.v[i] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)(vb + voff)));
      }
    }
  };
  auto kop = [&](const Stage& st, int kk) __attribute__((always_inline)) -> bf16x8 {
    if constexpr (kFp8) {
      const u32x4 w = st.k[kk >> 1];
      return e4m3x8_to_bf16((kk & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]});
    } else {
      return st.k[kk];
    }
  };

  f32x4 o[kD / 16];
#pragma unroll
  for (int i = 0; i < kD / 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -1e30f, lsum = 0.f;  // of query col
  const float c = kFp8 ? a.scale_log2 * a.k_scale : a.scale_log2;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  char* const vt = vtile[wave];
  // transposed-read address of V block blk: row 4 quad + col / 4, d = 16 blk + 4 (col mod 4)
  const int vr = 4 * quad + (col >> 2);
  const int vsw = 2 * (vr & 7);

  auto compute = [&](const Stage& st, int64_t t) __attribute__((always_inline)) {
    f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(st, kk), qop[kk], s4, 0, 0, 0);
    const int64_t key0 = r0 + t * kStageRows + 4 * quad;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (key0 + r >= r1) s4[r] = -INFINITY;
    float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
    {
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    }
    const float mt = mx * c;
    if (__ballot(mt > m + kSlack)) {
      const float mn = fmaxf(m, mt);
      float al = fast_exp2(m - mn);
      asm volatile("" : "+v"(al));
      m = mn;
      lsum *= al;
      // O rows are queries 4 quad + r, whose factors sit in lanes col = 4 quad + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(al, 4 * quad + r, kWave);
#pragma unroll
        for (int i2 = 0; i2 < kD / 16; ++i2) o[i2][r] *= ar;
      }
    }
    const float nm = -m;
    bf16x4 pa;
#pragma unroll
    for (int r = 0; r < 4; ++r) pa[r] = (bf16)fast_exp2(fmaf(s4[r], c, nm));
    // the weights enter P V as bf16; the row sum adds those same values
    lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pa[0], pa[1]}, ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pa[2], pa[3]}, ones, lsum, false);
    const i16x4 pai = __builtin_bit_cast(i16x4, pa);
    // V tile: row r, 16-byte column c stored at c ^ 2 (r mod 8)
    if constexpr (kFp8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * i + 2 * quad + (col >> 3), c0 = 2 * (col & 7);
        const u32x4 w = st.v[i];
        *(bf16x8*)(vt + r * 256 + ((c0 ^ (2 * (r & 7))) * 16)) = e4m3x8_to_bf16(u32x2{w[0], w[1]});
        *(bf16x8*)(vt + r * 256 + (((c0 + 1) ^ (2 * (r & 7))) * 16)) = e4m3x8_to_bf16(u32x2{w[2], w[3]});
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + quad;
        *(bf16x8*)(vt + r * 256 + ((col ^ (2 * (r & 7))) * 16)) = st.v[i];
      }
    }
#pragma unroll
    for (int blk = 0; blk < kD / 16; ++blk) {
      const int d0 = 16 * blk + 4 * (col & 3);
      const char* pv = vt + vr * 256 + (((d0 >> 3) ^ vsw) * 16) + (d0 & 7) * 2;
      const i16x4 vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(pv));
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pai, vv, o[blk], 0, 0, 0);
    }
  };

  const int64_t n_stages = r1 > r0 ? (r1 - r0 + kStageRows - 1) / kStageRows : 0;
  const int64_t n_mine = n_stages > wave ? (n_stages - wave + 3) / 4 : 0;
  // Three stages in registers: one being used, two in flight.  The steady
  // loop has no branches, so every fetch is issued two stages ahead; fetches
  // past the wavefront's last stage read (clamped) rows that are not used.
  // Three stages in registers, named (an array of them was not kept in
  // registers): at the top of a trip stage i + j sits in s_j; each step
  // fetches two stages ahead (past the split's end, rows are clamped to its
  // last) into the register set just computed.  The trip is branch-free so
  // that every wait is an exact vmcnt.
  static_assert(kStages == 3, "the loop below holds three stages");
  if (n_mine > 0) {
    Stage s0, s1, s2;
    fetch(wave, s0);
    fetch(wave + 4, s1);
    int64_t i = 0;
    for (; i + 3 <= n_mine; i += 3) {
      const int64_t t = wave + 4 * i;
      fetch(t + 8, s2);
      compute(s0, t);
      fetch(t + 12, s0);
      compute(s1, t + 4);
      fetch(t + 16, s1);
      compute(s2, t + 8);
    }
    if (i < n_mine) compute(s0, wave + 4 * i);
    if (i + 1 < n_mine) compute(s1, wave + 4 * (i + 1));
  }

  // this wavefront's (m, l) per query (col) and O rows (queries 4 quad + r)
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (quad == 0 && col < GRP) {
    sm[wave][col] = m;
    sl[wave][col] = lsum;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = 4 * quad + r;
    if (q < GRP) {
#pragma unroll
      for (int blk = 0; blk < kD / 16; ++blk) so[wave][q][16 * blk + col] = o[blk][r];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < GRP * kD; idx += kThreads) {
    const int j = idx / kD, d = idx % kD;
    float M = sm[0][j];
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2) M = fmaxf(M, sm[w2][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const float f = fast_exp2(sm[w2][j] - M);
      L += sl[w2][j] * f;
      O += so[w2][j][d] * f;
    }
    if constexpr (kFp8) O *= a.v_scale;
    const int64_t bh = (int64_t)b * a.H + g * GRP + j;
    if (a.splits == 1) {
      ((bf16*)a.out)[bh * kD + d] = (bf16)(O / L);
      continue;
    }
    float* pp = a.part + (bh * a.splits + sp) * (kD + 2);
    if (d == 0) {
      pp[0] = M;
      pp[1] = L;
    }
    pp[2 + d] = O;
  }
}

__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  using namespace dec;
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* p = a.part + (int64_t)bh * a.splits * (kD + 2);
  float M = -1e30f;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, p[s * (kD + 2)]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float f = fast_exp2(p[s * (kD + 2)] - M);
    L += p[s * (kD + 2) + 1] * f;
    O += p[s * (kD + 2) + 2 + d] * f;
  }
  ((bf16*)a.out)[(int64_t)bh * kD + d] = (bf16)(O / L);
}

// The grouped MFMA kernel's walk: 16-row stages of the split, stage t taken
// by wavefront t mod 4.
__global__ __launch_bounds__(dec::kThreads) void probe_decode_mfma_kernel(DecodeArgs a,
                                                                         int32_t* count) {
  using namespace dec;
  const int sp = blockIdx.x;
  const int64_t r0 = (int64_t)sp * a.rows_per_split;
  const int64_t r1 = min(a.n, r0 + a.rows_per_split);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n_stages = r1 > r0 ? (r1 - r0 + kStageRows - 1) / kStageRows : 0;
  const int64_t n_mine = n_stages > wave ? (n_stages - wave + 3) / 4 : 0;
  for (int64_t i = 0; i < n_mine; ++i) {
    const int64_t r = r0 + (wave + 4 * i) * kStageRows + lane;
    if (lane < kStageRows && r < r1) atomicAdd(&count[r], 1);
  }
}

__global__ __launch_bounds__(dec::kThreads) void probe_decode_kernel(DecodeArgs a, int32_t* count) {
  using namespace dec;
  const int sp = blockIdx.x;
  const int64_t r0 = (int64_t)sp * a.rows_per_split;
  const int64_t r1 = min(a.n, r0 + a.rows_per_split);
  const int grp = threadIdx.x >> 4, li = threadIdx.x & 15;
  const int64_t n_iter = r1 > r0 ? (r1 - r0 + kRowsPerIter - 1) / kRowsPerIter : 0;
  for (int64_t i = 0; i < n_iter; ++i)
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r = row_of(r0, i, u, grp);
      if (r < r1 && li == 0) atomicAdd(&count[r], 1);
    }
}

template <typename T, int D>
hipError_t launch_generic_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.Tq + 63) / 64, a.H, a.B);
  attn_generic_kernel<T, D><<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, int d, hipStream_t s) {
#define OLMO3_GEN(T, DD) \
  if (d == DD) return launch_generic_t<T, DD>(a, s);
  if (dtype == 0) {
    OLMO3_GEN(bf16, 16) OLMO3_GEN(bf16, 32) OLMO3_GEN(bf16, 64) OLMO3_GEN(bf16, 128)
  } else {
    OLMO3_GEN(float, 16) OLMO3_GEN(float, 32) OLMO3_GEN(float, 64) OLMO3_GEN(float, 128)
  }
#undef OLMO3_GEN
  return hipErrorInvalidValue;
}

int decode_splits(int B, int G, int64_t n) {
  using namespace dec;
  const int64_t pairs = (int64_t)B * G;
  int64_t s = (kTargetWorkgroups + pairs - 1) / pairs;
  const int64_t by_rows = (n + kMinRowsPerSplit - 1) / kMinRowsPerSplit;
  if (s > by_rows) s = by_rows;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

// The grouped MFMA kernel serves bf16 and e4m3 caches with H/G >= 2 whose rows fit
// 32-bit byte offsets; the per-row kernel the rest.
bool uses_decode_mfma(const DecodeArgs& a) {
  return a.H / a.G >= 2 && a.cap < ((int64_t)1 << 24);
}

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t s) {
  const int group = a.H / a.G;
  const int blocks = a.B * a.G * a.splits;
#define OLMO3_DEC(GG)                                                                     \
  case GG:                                                                                \
    if (uses_decode_mfma(a)) {                                                            \
      if (a.fp8)                                                                          \
        decode_mfma_kernel<(GG >= 2 ? GG : 2), true><<<blocks, dec::kThreads, 0, s>>>(a); \
      else                                                                                \
        decode_mfma_kernel<(GG >= 2 ? GG : 2), false><<<blocks, dec::kThreads, 0, s>>>(a); \
    } else if (a.fp8) {                                                                   \
      decode_split_kernel<GG, true><<<blocks, dec::kThreads, 0, s>>>(a);                  \
    } else {                                                                              \
      decode_split_kernel<GG, false><<<blocks, dec::kThreads, 0, s>>>(a);                 \
    }                                                                                     \
    break;
  switch (group) {
    OLMO3_DEC(1) OLMO3_DEC(2) OLMO3_DEC(3) OLMO3_DEC(4)
    OLMO3_DEC(5) OLMO3_DEC(6) OLMO3_DEC(7) OLMO3_DEC(8)
    default:
      return hipErrorInvalidValue;
  }
#undef OLMO3_DEC
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s) {
  decode_merge_kernel<<<a.B * a.H, dec::kD, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_probe_decode(const DecodeArgs& a, int32_t* count, hipStream_t s) {
  hipError_t e = hipMemsetAsync(count, 0, (size_t)a.cap * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  if (uses_decode_mfma(a))
    probe_decode_mfma_kernel<<<a.splits, dec::kThreads, 0, s>>>(a, count);
  else
    probe_decode_kernel<<<a.splits, dec::kThreads, 0, s>>>(a, count);
  return hipGetLastError();
}

}  // namespace olmo3
