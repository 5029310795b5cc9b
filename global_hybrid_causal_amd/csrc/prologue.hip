// Fused QK-norm + RoPE + KV-cache append (one wavefront per token), for a
// uniform batch, per-sequence positions or packed sequences of any length.
//
// QK-norm: one RMS statistic over the token's whole query vector (H*d
// features) and one over its whole key vector (G*d features), then a
// per-feature gain ("Case Study: OLMo 3", architecture item 2; gains of width
// H*d and G*d per "Count OLMo 3's Parameters").  RoPE: pair (i, i + d/2)
// turns by pos * omega_i at absolute position pos = pos_offset + t ("Case
// Study: OLMo 3", item 3; "Olmo-3 End-to-End Implementation", "Inference
// Pipeline").  Append: rotated key and untouched value go to the cache slot
// of the position, ring slot pos mod window on sliding layers ("Olmo 3 7B",
// per-layer-type cache).
//
// Each lane owns "pair chunks": 16-byte pieces of the first half of a head
// and the matching piece of the second half, so a rotation never crosses
// lanes.  The lane's pair chunks all sit at the same offset inside their
// heads, so its RoPE angles are computed once per token (fp64 product and
// range reduction, fp32 sincos) and reused for every query and key head.
#include "common.h"
#include "kernels.h"

namespace olmo3 {

namespace {

constexpr int kTokensPerBlock = 4;  // one wavefront per token
constexpr int kMaxChunksPerLane = 8;

template <typename T, int D>
struct PairChunks {
  static constexpr int kVec = Io<T>::kVec;
  static constexpr int kPerHead = D / (2 * kVec);  // pair chunks per head
  static_assert(kPerHead >= 1 && kWave % kPerHead == 0, "unsupported head size");
};

template <typename T, int D>
__device__ __forceinline__ void rope_angles(int lane, int64_t pos, const RopeTable& rope,
                                            float* cs, float* sn) {
  constexpr int kVec = Io<T>::kVec;
  const int j = lane % PairChunks<T, D>::kPerHead;
  constexpr double kTwoPi = 6.283185307179586;
  constexpr double kInvTwoPi = 0.15915494309189535;
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  double f[kVec];
#pragma unroll
  for (int e = 0; e < kVec; e += 2) {
    const f64x2 v = *(const f64x2*)&rope.inv_freq[j * kVec + e];
    f[e] = v[0];
    f[e + 1] = v[1];
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const double a = (double)pos * f[e];
    const double r = a - kTwoPi * rint(a * kInvTwoPi);  // |r| <= pi
    sincosf((float)r, &sn[e], &cs[e]);
  }
}

// Normalise, rotate and emit the `nheads` heads of one token row.
// emit(h, j, y0, y1) receives pair chunk j of head h: elements j*kVec ..
// j*kVec + kVec-1 of the head (y0) and the same offsets past d/2 (y1).
// With kAngles, angles() runs once the row's loads are issued and fills cs
// and sn; otherwise they are already there.
// Row loads: plain, or (stream) non-temporal, for rows read once by a call
// too large for the last-level cache to hold them and its own outputs.
// (A compile-time choice: a runtime one lets the compiler merge the two
// loads and drop the non-temporal hint.)
template <bool kStream, typename T>
__device__ __forceinline__ typename Io<T>::vec load_row_chunk(const T* p) {
  typedef typename Io<T>::vec vec;
  if constexpr (kStream) return __builtin_bit_cast(vec, __builtin_nontemporal_load((const u32x4*)p));
  return *(const vec*)p;
}

template <typename T, int D, bool kAngles, bool kStream, typename Angles, typename Emit>
__device__ __forceinline__ void norm_rope_row(const T* __restrict__ src, const T* __restrict__ gain,
                                              int nheads, float eps, int lane, const float* cs,
                                              const float* sn, float mscale, Angles angles,
                                              Emit emit) {
  typedef typename Io<T>::vec vec;
  constexpr int kVec = Io<T>::kVec;
  constexpr int kPerHead = PairChunks<T, D>::kPerHead;
  const int n_chunks = nheads * kPerHead;
  vec a0[kMaxChunksPerLane], a1[kMaxChunksPerLane];
  auto load = [&](int k) __attribute__((always_inline)) {
    const int pc = lane + kWave * k;
    const int h = pc / kPerHead, j = pc % kPerHead;
    const T* p = src + h * D + j * kVec;
    a0[k] = load_row_chunk<kStream>(p);
    a1[k] = load_row_chunk<kStream>(p + D / 2);
  };
  float ss = 0.f;
  auto accumulate = [&](int k) __attribute__((always_inline)) {
    float f0[kVec], f1[kVec];
    Io<T>::to_f32(a0[k], f0);
    Io<T>::to_f32(a1[k], f1);
#pragma unroll
    for (int e = 0; e < kVec; ++e) ss += f0[e] * f0[e] + f1[e] * f1[e];
  };
  if constexpr (kAngles) {  // every load issued before the angle arithmetic
#pragma unroll
    for (int k = 0; k < kMaxChunksPerLane; ++k)
      if (lane + kWave * k < n_chunks) load(k);
    angles();
#pragma unroll
    for (int k = 0; k < kMaxChunksPerLane; ++k)
      if (lane + kWave * k < n_chunks) accumulate(k);
  } else {
#pragma unroll
    for (int k = 0; k < kMaxChunksPerLane; ++k)
      if (lane + kWave * k < n_chunks) {
        load(k);
        accumulate(k);
      }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)(nheads * D) + eps);
#pragma unroll
  for (int k = 0; k < kMaxChunksPerLane; ++k) {
    const int pc = lane + kWave * k;
    if (pc < n_chunks) {
      const int h = pc / kPerHead, j = pc % kPerHead;
      const T* gp = gain + h * D + j * kVec;
      float g0[kVec], g1[kVec], x0[kVec], x1[kVec], y0[kVec], y1[kVec];
      Io<T>::to_f32(*(const vec*)gp, g0);
      Io<T>::to_f32(*(const vec*)(gp + D / 2), g1);
      Io<T>::to_f32(a0[k], x0);
      Io<T>::to_f32(a1[k], x1);
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const float u = x0[e] * r * g0[e];
        const float w = x1[e] * r * g1[e];
        y0[e] = (u * cs[e] - w * sn[e]) * mscale;
        y1[e] = (w * cs[e] + u * sn[e]) * mscale;
      }
      emit(h, j, y0, y1);
    }
  }
}

// kVec consecutive values of one head: as T, or (e4m3 cache, T = bf16) as
// codes of value * inv_scale.
template <typename T>
__device__ __forceinline__ void store_chunk(T* dst, const float* y) {
  *(typename Io<T>::vec*)dst = Io<T>::from_f32(y);
}
__device__ __forceinline__ void store_chunk_e4m3(uint8_t* dst, const float* y, float inv_scale) {
  u32x2 w;
  w[0] = f32x4_to_e4m3(y[0] * inv_scale, y[1] * inv_scale, y[2] * inv_scale, y[3] * inv_scale);
  w[1] = f32x4_to_e4m3(y[4] * inv_scale, y[5] * inv_scale, y[6] * inv_scale, y[7] * inv_scale);
  *(u32x2*)dst = w;
}

// Sequence of packed row `row`: the number of b >= 1 with cu[b] <= row
// (cu[0] = 0), counted 64 entries at a time with a ballot; clamped to
// [0, B-1].  Uniform across the wavefront.
__device__ __forceinline__ int packed_sequence(const int32_t* cu, int B, int64_t row, int lane) {
  int b = 0;
  for (int j0 = 1; j0 <= B; j0 += kWave) {
    const int j = j0 + lane;
    const bool le = j <= B && (int64_t)cu[j] <= row;
    b += __popcll(__ballot(le));
  }
  return min(b, B - 1);
}

// kRoles: one workgroup per token and one wavefront per part of it (queries,
// keys, values), so that the three dependent load / reduce / store chains of
// a token overlap; used when there are too few tokens to fill the GPU (decode).
// Otherwise one wavefront per token handles all three parts in turn.
// kEarly (with kRoles, for a few hundred tokens at most): a wavefront issues
// its row's loads before the RoPE angle arithmetic, so that the two overlap;
// it keeps more registers live, which larger grids cannot afford.
// kStream: the projected rows are read with non-temporal loads.
template <typename T, int D, bool kRoles, bool kEarly, bool kStream = false>
__global__ __launch_bounds__(kWave * kTokensPerBlock) void qknorm_rope_append_kernel(
    PrologueArgs a, RopeTable rope) {
  typedef typename Io<T>::vec vec;
  constexpr int kVec = Io<T>::kVec;
  const int lane = threadIdx.x % kWave;
  const int64_t row = kRoles ? (int64_t)blockIdx.x
                             : (int64_t)blockIdx.x * kTokensPerBlock + threadIdx.x / kWave;
  const int role = kRoles ? (int)(threadIdx.x / kWave) : -1;
  const bool do_q = !kRoles || role == 0, do_k = !kRoles || role == 1, do_v = !kRoles || role == 2;
  // (sequence, index in it, its length, absolute position) of this row
  int b;
  int64_t t, len, pos;
  if (a.cu_seqlens) {
    if (row >= a.n_rows) return;
    b = packed_sequence(a.cu_seqlens, a.B, row, lane);
    const int64_t first = a.cu_seqlens[b];
    t = row - first;
    len = (int64_t)a.cu_seqlens[b + 1] - first;
    if (t < 0 || t >= len) return;  // inconsistent offsets: row belongs to no sequence
    pos = (a.seq_pos ? (int64_t)a.seq_pos[b] : 0) + t;
  } else {
    if (row >= (int64_t)a.B * a.T) return;
    b = (int)(row / a.T);
    t = row % a.T;
    len = a.T;
    pos = (a.seq_pos ? (int64_t)a.seq_pos[b] : a.pos_offset) + t;
  }
  if (pos < 0) return;

  // RoPE angles, once per wavefront: first, or (kEarly) once the row's loads
  // are issued.
  float cs[kVec], sn[kVec];
  if (!kEarly && (do_q || do_k)) rope_angles<T, D>(lane, pos, rope, cs, sn);
  auto angles = [&]() __attribute__((always_inline)) {
    if constexpr (kEarly) rope_angles<T, D>(lane, pos, rope, cs, sn);
  };

  // queries -> q_out [rows][H][D]
  if (do_q && a.q_pre) {
    const T* src = (const T*)a.q_pre + row * a.H * D;
    T* qo = (T*)a.q_out + row * a.H * D;
    norm_rope_row<T, D, kEarly, kStream>(src, (const T*)a.q_gain, a.H, a.eps, lane, cs, sn,
                                         rope.mscale * a.q_scale, angles,
                                         [&](int h, int j, const float* y0, const float* y1) {
                                  store_chunk(qo + h * D + j * kVec, y0);
                                  store_chunk(qo + h * D + D / 2 + j * kVec, y1);
                                });
  }

  const int64_t slot = a.sliding ? pos % a.window : pos;
  const bool to_cache = a.store && len - t <= a.keep_last && slot < a.cap;
  // rotated-key copy: [b][g][t] strided, or [g][row] for packed rows
  const int64_t kb_idx = a.cu_seqlens ? 0 : b, kt_idx = a.cu_seqlens ? row : t;
  constexpr bool kCanFp8 = kVec == 8;  // e4m3 caches hold bf16 rows only
  const bool fp8 = a.cache_fp8;

  // keys -> optional strided copy (prefill workspace) and the cache slot
  if (do_k) {
    const T* src = (const T*)a.k_pre + row * a.G * D;
    T* ko = (T*)a.k_out;
    norm_rope_row<T, D, kEarly, kStream>(
        src, (const T*)a.k_gain, a.G, a.eps, lane, cs, sn, rope.mscale, angles,
        [&](int h, int j, const float* y0, const float* y1) {
          if (ko) {
            T* d = ko + kb_idx * a.k_sb + h * a.k_sg + kt_idx * a.k_st;
            store_chunk(d + j * kVec, y0);
            store_chunk(d + D / 2 + j * kVec, y1);
          }
          if (!to_cache) return;
          const int64_t off = (((int64_t)b * a.G + h) * a.cap + slot) * D;
          if constexpr (kCanFp8) {
            if (fp8) {
              uint8_t* d = (uint8_t*)a.k_cache + off;
              store_chunk_e4m3(d + j * kVec, y0, a.k_inv_scale);
              store_chunk_e4m3(d + D / 2 + j * kVec, y1, a.k_inv_scale);
              return;
            }
          }
          {
            T* d = (T*)a.k_cache + off;
            store_chunk(d + j * kVec, y0);
            store_chunk(d + D / 2 + j * kVec, y1);
          }
        });
  }

  // values -> cache slot, unchanged (or as e4m3 codes of value / scale)
  if (do_v && to_cache) {
    const T* src = (const T*)a.v + row * a.G * D;
    const int n_vec = a.G * D / kVec;
    for (int c = lane; c < n_vec; c += kWave) {
      const int h = c / (D / kVec), e = c % (D / kVec);
      const int64_t off = (((int64_t)b * a.G + h) * a.cap + slot) * D + e * kVec;
      const vec x = load_row_chunk<kStream>(src + c * kVec);
      if constexpr (kCanFp8) {
        if (fp8) {
          float f[kVec];
          Io<T>::to_f32(x, f);
          store_chunk_e4m3((uint8_t*)a.v_cache + off, f, a.v_inv_scale);
          continue;
        }
      }
      *(vec*)((T*)a.v_cache + off) = x;
    }
  }
}

// Decode prologue (bf16 rows, d = 128, one token per sequence): one
// workgroup of 8 wavefronts per token.  The token's query, key and value rows
// are cut into pair chunks (8 values of a head and the 8 values d/2 further
// on, the halves that RoPE rotates together), dealt out over the 512
// threads; each thread adds up its squares, the workgroup adds the
// wavefronts' sums through LDS, and the 64 rotation angles of the token's
// position are computed once, one per lane of wavefront 0, into LDS.  Each
// thread then handles a few pair chunks instead of a wavefront a whole row,
// which shortens the token's dependent chain (a decode batch has too few
// tokens to hide it).  The squares are added in another order than in the
// row kernel above, so a key may round differently in its last place.
constexpr int kDecProThreads = 512;
constexpr int kDecProItems = 3;  // pair chunks per thread: 8 (H + 2G) <= 1536

__global__ __launch_bounds__(kDecProThreads) void decode_prologue_kernel(PrologueArgs a,
                                                                         RopeTable rope) {
  constexpr int D = 128, kVec = 8, kPer = D / (2 * kVec);  // 8 pair chunks per head
  constexpr int kWaves = kDecProThreads / kWave;
  __shared__ float s_cs[D / 2], s_sn[D / 2];
  __shared__ float s_ss[kWaves][2];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int b = blockIdx.x;
  const int64_t pos = a.seq_pos ? (int64_t)a.seq_pos[b] : a.pos_offset;
  if (pos < 0) return;  // the whole workgroup: no position for this sequence
  const int nq = a.H * kPer, nk = a.G * kPer, n = nq + 2 * nk;
  const bf16* src[3] = {(const bf16*)a.q_pre + (int64_t)b * a.H * D,
                        (const bf16*)a.k_pre + (int64_t)b * a.G * D,
                        (const bf16*)a.v + (int64_t)b * a.G * D};
  const bf16* gain[2] = {(const bf16*)a.q_gain, (const bf16*)a.k_gain};
  // item it -> part (0 queries, 1 keys, 2 values) and pair chunk pc
  auto item = [&](int it, int& part, int& pc) __attribute__((always_inline)) {
    part = it < nq ? 0 : (it < nq + nk ? 1 : 2);
    pc = it - (part == 0 ? 0 : (part == 1 ? nq : nq + nk));
  };
  bf16x8 x0[kDecProItems], x1[kDecProItems], g0[kDecProItems], g1[kDecProItems];
#pragma unroll
  for (int i = 0; i < kDecProItems; ++i) {
    const int it = tid + kDecProThreads * i;
    if (it < n) {
      int part, pc;
      item(it, part, pc);
      const int off = (pc / kPer) * D + (pc % kPer) * kVec;
      x0[i] = *(const bf16x8*)(src[part] + off);
      x1[i] = *(const bf16x8*)(src[part] + off + D / 2);
      if (part < 2) {
        g0[i] = *(const bf16x8*)(gain[part] + off);
        g1[i] = *(const bf16x8*)(gain[part] + off + D / 2);
      }
    }
  }
  if (wave == 0) {  // angle of rate `lane` at this position, as in rope_angles
    constexpr double kTwoPi = 6.283185307179586;
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double ang = (double)pos * rope.inv_freq[lane];
    const double r = ang - kTwoPi * rint(ang * kInvTwoPi);
    float sv, cv;
    sincosf((float)r, &sv, &cv);
    s_cs[lane] = cv;
    s_sn[lane] = sv;
  }
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kDecProItems; ++i) {
    const int it = tid + kDecProThreads * i;
    if (it < nq + nk) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const float f0 = (float)x0[i][e], f1 = (float)x1[i][e];
        t += f0 * f0 + f1 * f1;
      }
      ss[it < nq ? 0 : 1] += t;
    }
  }
  ss[0] = wave_sum(ss[0]);
  ss[1] = wave_sum(ss[1]);
  if (lane == 0) {
    s_ss[wave][0] = ss[0];
    s_ss[wave][1] = ss[1];
  }
  __syncthreads();
  float tot[2] = {0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    tot[0] += s_ss[w][0];
    tot[1] += s_ss[w][1];
  }
  const float rn[2] = {1.0f / sqrtf(tot[0] / (float)(a.H * D) + a.eps),
                       1.0f / sqrtf(tot[1] / (float)(a.G * D) + a.eps)};
  const int64_t slot = a.sliding ? pos % a.window : pos;
  const bool to_cache = a.store && slot < a.cap;
  const bool fp8 = a.cache_fp8;
#pragma unroll
  for (int i = 0; i < kDecProItems; ++i) {
    const int it = tid + kDecProThreads * i;
    if (it >= n) continue;
    int part, pc;
    item(it, part, pc);
    const int h = pc / kPer, j = pc % kPer;
    if (part == 2) {  // values -> cache slot, unchanged (or as e4m3 codes)
      if (!to_cache) continue;
      const int64_t off = (((int64_t)b * a.G + h) * a.cap + slot) * D + j * kVec;
      if (fp8) {
        float f0[kVec], f1[kVec];
        Io<bf16>::to_f32(x0[i], f0);
        Io<bf16>::to_f32(x1[i], f1);
        store_chunk_e4m3((uint8_t*)a.v_cache + off, f0, a.v_inv_scale);
        store_chunk_e4m3((uint8_t*)a.v_cache + off + D / 2, f1, a.v_inv_scale);
      } else {
        *(bf16x8*)((bf16*)a.v_cache + off) = x0[i];
        *(bf16x8*)((bf16*)a.v_cache + off + D / 2) = x1[i];
      }
      continue;
    }
    float y0[kVec], y1[kVec];
    const float r = rn[part];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float cs = s_cs[j * kVec + e], sn = s_sn[j * kVec + e];
      const float u = (float)x0[i][e] * r * (float)g0[i][e];
      const float w = (float)x1[i][e] * r * (float)g1[i][e];
      y0[e] = (u * cs - w * sn) * rope.mscale;
      y1[e] = (w * cs + u * sn) * rope.mscale;
    }
    if (part == 0) {
      bf16* qo = (bf16*)a.q_out + ((int64_t)b * a.H + h) * D + j * kVec;
      store_chunk(qo, y0);
      store_chunk(qo + D / 2, y1);
    } else if (to_cache) {
      const int64_t off = (((int64_t)b * a.G + h) * a.cap + slot) * D + j * kVec;
      if (fp8) {
        store_chunk_e4m3((uint8_t*)a.k_cache + off, y0, a.k_inv_scale);
        store_chunk_e4m3((uint8_t*)a.k_cache + off + D / 2, y1, a.k_inv_scale);
      } else {
        store_chunk((bf16*)a.k_cache + off, y0);
        store_chunk((bf16*)a.k_cache + off + D / 2, y1);
      }
    }
  }
}

// Whether decode_prologue_kernel serves this call: one bf16 token per
// sequence with d = 128, queries present, no rotated-key copy.
bool decode_prologue_fits(const PrologueArgs& a, int dtype, int d) {
  return dtype == 0 && d == 128 && a.T == 1 && !a.cu_seqlens && a.q_pre && !a.k_out &&
         a.q_scale == 1.0f &&
         8 * (a.H + 2 * a.G) <= kDecProThreads * kDecProItems;
}

// Up to this many tokens the per-part wavefronts are used, and up to the
// smaller bound they issue their loads before the angle arithmetic.
constexpr int64_t kRolesMaxRows = 2048;
constexpr int64_t kEarlyMaxRows = 512;

// Calls whose projected rows exceed this read them non-temporally: the rows
// are read once, and keeping them out of the 256 MiB last-level cache leaves
// it to the rotated rows and cache rows that the attention reads next (on
// the 7B layer shape, 192 MiB of rows: 15 % less prologue time).
constexpr int64_t kStreamInputBytes = (int64_t)128 << 20;

template <typename T, int D>
hipError_t launch_prologue_t(const PrologueArgs& a, const RopeTable& rope, hipStream_t s) {
  const int64_t rows = a.cu_seqlens ? a.n_rows : (int64_t)a.B * a.T;
  const int64_t in_bytes = rows * (int64_t)((a.q_pre ? a.H : 0) + 2 * a.G) * D * (int64_t)sizeof(T);
  if (rows <= kEarlyMaxRows) {
    qknorm_rope_append_kernel<T, D, true, true><<<(int)rows, kWave * 3, 0, s>>>(a, rope);
  } else if (rows <= kRolesMaxRows) {
    qknorm_rope_append_kernel<T, D, true, false><<<(int)rows, kWave * 3, 0, s>>>(a, rope);
  } else {
    const int blocks = (int)((rows + kTokensPerBlock - 1) / kTokensPerBlock);
    if (in_bytes > kStreamInputBytes)
      qknorm_rope_append_kernel<T, D, false, false, true>
          <<<blocks, kWave * kTokensPerBlock, 0, s>>>(a, rope);
    else
      qknorm_rope_append_kernel<T, D, false, false><<<blocks, kWave * kTokensPerBlock, 0, s>>>(a, rope);
  }
  return hipGetLastError();
}

// bf16 copy of the first n rows of each (sequence, head) of an e4m3 cache.
// One thread per 16 codes: one 16-byte load, two 16-byte stores; blockIdx.y
// picks keys (0) or values (1).
__global__ __launch_bounds__(256) void e4m3_rows_to_bf16_kernel(E4m3StageArgs a) {
  const bool val = blockIdx.y != 0;
  const uint8_t* src = (const uint8_t*)(val ? a.v_codes : a.k_codes);
  bf16* dst = (bf16*)(val ? a.v_out : a.k_out);
  const float scale = val ? a.v_scale : a.k_scale;
  const int per_row = a.d / 16;
  const int64_t per_head = a.n * per_row;
  const int64_t items = (int64_t)a.BG * per_head;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bg = i / per_head, rem = i - bg * per_head;
    const int64_t row = rem / per_row;
    const int c = (int)(rem - row * per_row) * 16;
    const u32x4 w = *(const u32x4*)(src + (bg * a.cap + row) * a.d + c);
    bf16x8 h[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float f[4];
      e4m3x4_to_f32(w[j], f);
#pragma unroll
      for (int e = 0; e < 4; ++e) h[j >> 1][4 * (j & 1) + e] = (bf16)(f[e] * scale);
    }
    bf16x8* o = (bf16x8*)(dst + (bg * a.rows + row) * a.d + c);
    o[0] = h[0];
    o[1] = h[1];
  }
}

}  // namespace

hipError_t launch_e4m3_rows_to_bf16(const E4m3StageArgs& a, hipStream_t s) {
  if (a.d % 16 || a.n < 0 || a.n > a.rows || a.n > a.cap) return hipErrorInvalidValue;
  const int64_t items = (int64_t)a.BG * a.n * (a.d / 16);
  if (items == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((items + 255) / 256, 8192);
  e4m3_rows_to_bf16_kernel<<<dim3(blocks, 2), 256, 0, s>>>(a);
  return hipGetLastError();
}

int prologue_max_heads(int dtype, int d) {
  const int vec = dtype == 0 ? 8 : 4;
  const int per_head = d / (2 * vec);
  return kMaxChunksPerLane * kWave / per_head;
}

hipError_t launch_prologue(const PrologueArgs& a, const RopeTable& rope, int dtype, int d,
                           hipStream_t s) {
  if (decode_prologue_fits(a, dtype, d)) {
    decode_prologue_kernel<<<a.B, kDecProThreads, 0, s>>>(a, rope);
    return hipGetLastError();
  }
#define OLMO3_PRO(T, DD) \
  if (d == DD) return launch_prologue_t<T, DD>(a, rope, s);
  if (dtype == 0) {
    OLMO3_PRO(bf16, 16) OLMO3_PRO(bf16, 32) OLMO3_PRO(bf16, 64) OLMO3_PRO(bf16, 128)
  } else {
    OLMO3_PRO(float, 16) OLMO3_PRO(float, 32) OLMO3_PRO(float, 64) OLMO3_PRO(float, 128)
  }
#undef OLMO3_PRO
  return hipErrorInvalidValue;
}

}  // namespace olmo3
