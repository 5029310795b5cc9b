// Causal attention kernels: flash-style MFMA prefill (d = 128, bf16), a
// plain per-query kernel for other head sizes and fp32, and split-KV decode
// with a log-sum-exp merge.
//
// Masking follows "OLMo 3's Sliding-Window Attention Pattern", "The
// sliding-window mask"; decode on a ring reads exactly the `window` held
// entries ("Olmo 3 7B", "SERVICEABILITY JOIN").  Softmax uses base-2
// exponentials with log2(e)/sqrt(d) folded into the scores.
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
// Prefill, d = 128.
//
// Workgroup = 4 wavefronts x 32 queries of one (batch, head).  Per key tile
// of 64 keys each wavefront computes S^T = K Q^T (two 32x32 blocks, K from
// LDS as the A operand, its queries' Q^T held in registers as B), so a lane
// owns one query column; it then accumulates O^T += V^T P^T with P^T taken
// straight from the S accumulators (converted to bf16) as the B operand.
// The key order inside each 16-key group is permuted consistently in P^T and
// in the transposed V tile in LDS, so no data moves between lanes.  K and
// V^T tiles are double-buffered in LDS; the next tile's global loads are in
// flight while the current one is used.
// LDS: K tile [64 keys][128 d] (256 B rows, 16-byte columns XOR-swizzled by
// key), V^T tile [128 d][64 keys] (128 B rows, columns swizzled by d/2).
// ---------------------------------------------------------------------------
constexpr int kTileBytes = pf::kBK * pf::kD * 2;  // 16 KiB

__device__ __forceinline__ int k_lds_off(int row, int c16) {
  return row * 256 + ((c16 ^ (row & 15)) << 4);
}
__device__ __forceinline__ int v_lds_off(int d, int c16) {
  return d * 128 + ((c16 ^ ((d >> 1) & 7)) << 4);
}

__global__ __launch_bounds__(256, 2) void prefill_d128_kernel(AttnArgs a) {
  using namespace pf;
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];
  char* const sK = smem;
  char* const sV = smem + 2 * kTileBytes;

  const int n_qblk = (a.Tq + kBQ - 1) / kBQ;
  const Work w = work_of(blockIdx.x, gridDim.x, n_qblk, a.H);
  const int g = w.h / (a.H / a.G);
  const int q0 = w.qb * kBQ;
  const int q1 = min(q0 + kBQ, a.Tq);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int tq = lane_query(q0, wave, lane);
  const int tql = min(tq, a.Tq - 1);

  // Q^T operand: lane holds query tq, d = 16*ks + 8*half .. +7
  bf16x8 qop[8];
  {
    const bf16* qrow = (const bf16*)a.q + ((int64_t)(w.b * a.Tq + tql) * a.H + w.h) * kD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[ks] = *(const bf16x8*)(qrow + ks * 16 + half * 8);
  }

  const bf16* kbase = (const bf16*)a.k + w.b * a.k_sb + g * a.k_sg;
  const bf16* vbase = (const bf16*)a.v + w.b * a.v_sb + g * a.v_sg;
  const int last = (int)a.n_keys - 1;

  // global -> registers.  K: thread -> (row tid/16 + 16 i, 16-byte column
  // tid%16).  V: thread -> (keys 4*(tid%16) .. +3, d chunk tid/16).
  bf16x8 kr[4], vr[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(k0 + (tid >> 4) + 16 * i, last);
      kr[i] = *(const bf16x8*)(kbase + (int64_t)key * a.k_sr + (tid & 15) * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(k0 + 4 * (tid & 15) + i, last);
      vr[i] = *(const bf16x8*)(vbase + (int64_t)key * a.v_sr + (tid >> 4) * 8);
    }
  };
  // registers -> LDS stage st (V transposed, keys permuted within 16-groups:
  // logical key 16c + 8q + 4hh + j sits at 16c + 8hh + 4q + j).
  auto store_tile = [&](int st) {
    char* k = sK + st * kTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 4) + 16 * i;
      *(bf16x8*)(k + k_lds_off(row, tid & 15)) = kr[i];
    }
    char* v = sV + st * kTileBytes;
    const int kg = tid & 15, dc = tid >> 4;
    const int pg = 4 * (kg >> 2) + 2 * (kg & 1) + ((kg & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dc * 8 + e;
      bf16x4 p4 = {vr[0][e], vr[1][e], vr[2][e], vr[3][e]};
      *(bf16x4*)(v + v_lds_off(d, pg >> 1) + (pg & 1) * 8) = p4;
    }
  };

  int kt0, kt1;
  key_tiles(q0, q1, a.window, a.sliding, kt0, kt1);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -1e30f, lsum = 0.f;
  const float c = a.scale_log2;

  load_tile(kt0 * kBK);
  store_tile(0);

  for (int kt = kt0; kt < kt1; ++kt) {
    const int st = (kt - kt0) & 1;
    const int k0 = kt * kBK;
    const bool more = kt + 1 < kt1;
    if (more) load_tile(k0 + kBK);
    __syncthreads();

    // S^T for keys k0 .. k0+63
    const char* k = sK + st * kTileBytes;
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a0 = *(const bf16x8*)(k + k_lds_off(col, 2 * ks + half));
      const bf16x8 a1 = *(const bf16x8*)(k + k_lds_off(32 + col, 2 * ks + half));
      s0 = mfma32(a0, qop[ks], s0);
      s1 = mfma32(a1, qop[ks], s1);
    }
    if (!tile_interior(k0, q0, q1, a.window, a.sliding)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (!visible(tq, lane_key(k0, 0, r, lane), a.window, a.sliding)) s0[r] = -INFINITY;
        if (!visible(tq, lane_key(k0, 1, r, lane), a.window, a.sliding)) s1[r] = -INFINITY;
      }
    }

    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mnew = fmaxf(m, mx * c);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = fast_exp2(fmaf(s0[r], c, -mnew));
      s1[r] = fast_exp2(fmaf(s1[r], c, -mnew));
      ps += s0[r] + s1[r];
    }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    bf16x8 pk[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pk[0][e] = (bf16)s0[e];
      pk[1][e] = (bf16)s0[8 + e];
      pk[2][e] = (bf16)s1[e];
      pk[3][e] = (bf16)s1[8 + e];
    }

    const char* v = sV + st * kTileBytes;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + col;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 va = *(const bf16x8*)(v + v_lds_off(d, 2 * kk + half));
        o[db] = mfma32(va, pk[kk], o[db]);
      }
    }
    if (more) store_tile(st ^ 1);
  }

  lsum += __shfl_xor(lsum, 32, kWave);
  const float inv = 1.0f / lsum;
  if (tq < a.Tq) {
    bf16* orow = (bf16*)a.out + ((int64_t)(w.b * a.Tq + tq) * a.H + w.h) * kD;
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

__global__ __launch_bounds__(256) void probe_prefill_kernel(int T, int window, int sliding,
                                                            uint8_t* visit) {
  using namespace pf;
  const int n_qblk = (T + kBQ - 1) / kBQ;
  const Work w = work_of(blockIdx.x, gridDim.x, n_qblk, 1);
  const int q0 = w.qb * kBQ, q1 = min(q0 + kBQ, T);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tq = lane_query(q0, wave, lane);
  int kt0, kt1;
  key_tiles(q0, q1, window, sliding, kt0, kt1);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * kBK;
    const bool interior = tile_interior(k0, q0, q1, window, sliding);
    for (int kb = 0; kb < 2; ++kb)
      for (int r = 0; r < 16; ++r) {
        const int s = lane_key(k0, kb, r, lane);
        const bool acc = interior || visible(tq, s, window, sliding);
        if (acc && tq < T && s < T) visit[(int64_t)tq * T + s] = 1;
      }
  }
}

// ---------------------------------------------------------------------------
// Plain kernel: one thread per query row, keys streamed from global memory.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnArgs a) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (t >= a.Tq) return;
  const int g = h / (a.H / a.G);
  const T* qp = (const T*)a.q + ((int64_t)(b * a.Tq + t) * a.H + h) * D;
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = (float)qp[e] * a.scale_log2;
    o[e] = 0.f;
  }
  const int64_t tpos = a.q_pos0 + t;
  int64_t r0 = 0, r1 = a.n_keys;
  if (!a.all_visible) {
    r1 = min(tpos + 1, a.n_keys);
    if (a.sliding) r0 = max(tpos - a.window + 1, (int64_t)0);
  }
  const T* kb = (const T*)a.k + b * a.k_sb + g * a.k_sg;
  const T* vb = (const T*)a.v + b * a.v_sb + g * a.v_sg;
  float m = -1e30f, l = 0.f;
  for (int64_t r = r0; r < r1; ++r) {
    const T* kp = kb + r * a.k_sr;
    const T* vp = vb + r * a.v_sr;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) s += q[e] * (float)kp[e];
    const float mn = fmaxf(m, s);
    const float al = fast_exp2(m - mn);
    const float p = fast_exp2(s - mn);
    l = l * al + p;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = o[e] * al + p * (float)vp[e];
    m = mn;
  }
  const float inv = 1.0f / l;
  T* op = (T*)a.out + ((int64_t)(b * a.Tq + t) * a.H + h) * D;
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
// wavefronts in LDS, into one partial (m, l, o) per head and split.
// ---------------------------------------------------------------------------
template <int GRP>
__global__ __launch_bounds__(dec::kThreads) void decode_split_kernel(DecodeArgs a) {
  using namespace dec;
  const int sp = blockIdx.x % a.splits;
  const int bg = blockIdx.x / a.splits;
  const int g = bg % a.G, b = bg / a.G;
  const int64_t r0 = (int64_t)sp * a.rows_per_split;
  const int64_t r1 = min(a.n, r0 + a.rows_per_split);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15;
  const int grp = tid >> 4;

  float q[GRP][8];
#pragma unroll
  for (int j = 0; j < GRP; ++j) {
    const bf16x8 qv = *(const bf16x8*)((const bf16*)a.q + ((int64_t)b * a.H + g * GRP + j) * kD + li * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[j][e] = (float)qv[e] * a.scale_log2;
  }
  float m[GRP], l[GRP], o[GRP][8];
#pragma unroll
  for (int j = 0; j < GRP; ++j) {
    m[j] = -1e30f;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  }
  const bf16* kb = (const bf16*)a.k_cache + ((int64_t)b * a.G + g) * a.cap * kD + li * 8;
  const bf16* vb = (const bf16*)a.v_cache + ((int64_t)b * a.G + g) * a.cap * kD + li * 8;

  const int64_t n_iter = r1 > r0 ? (r1 - r0 + kRowsPerIter - 1) / kRowsPerIter : 0;
  for (int64_t i = 0; i < n_iter; ++i) {
    bf16x8 kr[kUnroll], vr[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r = row_of(r0, i, u, grp);
      ok[u] = r < r1;
      const int64_t rc = ok[u] ? r : r0;
      kr[u] = *(const bf16x8*)(kb + rc * kD);
      vr[u] = *(const bf16x8*)(vb + rc * kD);
    }
    float s[kUnroll][GRP];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = (float)kr[u][e];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(q[j][e], kf[e], acc);
        s[u][j] = acc;
      }
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < GRP; ++j) s[u][j] += __shfl_xor(s[u][j], off, kWave);
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (!ok[u]) s[u][j] = -INFINITY;
        mx = fmaxf(mx, s[u][j]);
      }
      const float mn = fmaxf(m[j], mx);
      const float al = fast_exp2(m[j] - mn);
      m[j] = mn;
      float p[kUnroll], ps = 0.f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        p[u] = fast_exp2(s[u][j] - mn);
        ps += p[u];
      }
      l[j] = l[j] * al + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = o[j][e] * al;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc = fmaf(p[u], (float)vr[u][e], acc);
        o[j][e] = acc;
      }
    }
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
    float* pp = a.part + (((int64_t)b * a.H + g * GRP + j) * a.splits + sp) * (kD + 2);
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

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t s) {
  const int n_qblk = (a.Tq + pf::kBQ - 1) / pf::kBQ;
  const int blocks = n_qblk * a.H * a.B;
  prefill_d128_kernel<<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

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

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t s) {
  const int group = a.H / a.G;
  const int blocks = a.B * a.G * a.splits;
#define OLMO3_DEC(GG) \
  case GG:            \
    decode_split_kernel<GG><<<blocks, dec::kThreads, 0, s>>>(a); \
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

hipError_t launch_probe_prefill(int T, int window, int sliding, uint8_t* visit, hipStream_t s) {
  hipError_t e = hipMemsetAsync(visit, 0, (size_t)T * T, s);
  if (e != hipSuccess) return e;
  const int n_qblk = (T + pf::kBQ - 1) / pf::kBQ;
  probe_prefill_kernel<<<n_qblk, 256, 0, s>>>(T, window, sliding, visit);
  return hipGetLastError();
}

hipError_t launch_probe_decode(const DecodeArgs& a, int32_t* count, hipStream_t s) {
  hipError_t e = hipMemsetAsync(count, 0, (size_t)a.cap * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  probe_decode_kernel<<<a.splits, dec::kThreads, 0, s>>>(a, count);
  return hipGetLastError();
}

}  // namespace olmo3
