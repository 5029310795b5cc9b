// C ABI of libolmo3attn: argument validation, RoPE / YaRN rate tables,
// workspace layout and kernel dispatch.  Every check runs before the first
// launch, so a call that fails has no effect.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/olmo3_attn.h"
#include "kernels.h"
#include "tiles.h"

using namespace olmo3;

namespace {

constexpr double kLog2e = 1.4426950408889634;
constexpr size_t kAlign = 256;
constexpr int64_t kMaxPrefillPositions = (int64_t)1 << 30;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// bytes of an activation element (the e4m3 mode keeps bf16 activations)
size_t elem_size(int dtype) { return dtype == OLMO3_DTYPE_F32 ? 4 : 2; }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, size_t bytes) {
  return Span{(uintptr_t)p, (uintptr_t)p + bytes};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Sizes shared by all entry points.
int check_common(int B, int T, int H, int G, int d, int window, int layer_type, int dtype,
                 const olmo3_rope* rope, float eps, int64_t pos_offset) {
  if (B < 1 || T < 1 || H < 1 || G < 1 || d < 2 || window < 1) return OLMO3_ERR_INVALID_ARG;
  if (H % G) return OLMO3_ERR_INVALID_ARG;
  if (d % 2) return OLMO3_ERR_INVALID_ARG;
  if (layer_type != OLMO3_LAYER_SLIDING && layer_type != OLMO3_LAYER_FULL) return OLMO3_ERR_INVALID_ARG;
  if (dtype != OLMO3_DTYPE_BF16 && dtype != OLMO3_DTYPE_F32) return OLMO3_ERR_INVALID_ARG;
  if (!rope || !(rope->theta > 0.0) || !isfinite(rope->theta)) return OLMO3_ERR_INVALID_ARG;
  if (rope->yarn && (!(rope->factor >= 1.0) || rope->orig_ctx < 1 ||
                     !(rope->beta_fast > rope->beta_slow) || !(rope->beta_slow > 0.0) ||
                     !isfinite(rope->beta_fast) || !isfinite(rope->factor) ||
                     (rope->factor > 1.0 && !(rope->theta > 1.0))))
    return OLMO3_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !isfinite(eps)) return OLMO3_ERR_INVALID_ARG;
  if (pos_offset < 0) return OLMO3_ERR_INVALID_ARG;
  if (!supported_d(d)) return OLMO3_ERR_UNSUPPORTED;
  const int max_heads = prologue_max_heads(dtype, d);
  if (H > max_heads || G > max_heads) return OLMO3_ERR_UNSUPPORTED;
  if ((int64_t)B * T > INT32_MAX / 2 || (int64_t)B * H > 65535 * 64) return OLMO3_ERR_UNSUPPORTED;
  if (pos_offset + T > ((int64_t)1 << 40)) return OLMO3_ERR_UNSUPPORTED;
  return OLMO3_OK;
}

// A cache of more than 2^50 bytes cannot be allocated on any device; larger
// claimed capacities are refused before their byte sizes could overflow.
bool cache_size_ok(int64_t n_rows_blocks, int64_t cap, int d, size_t es) {
  const unsigned __int128 bytes = (unsigned __int128)n_rows_blocks * (unsigned __int128)cap *
                                  (unsigned __int128)d * es;
  return bytes <= ((unsigned __int128)1 << 50);
}

int check_capacity(int layer_type, int window, int64_t cap, int64_t last_pos) {
  if (cap < 1) return OLMO3_ERR_CAPACITY;
  if (layer_type == OLMO3_LAYER_SLIDING) return cap == window ? OLMO3_OK : OLMO3_ERR_CAPACITY;
  return cap >= last_pos + 1 ? OLMO3_OK : OLMO3_ERR_CAPACITY;
}

// Rates of a layer: theta^(-2i/d), or the YaRN interpolation of them on full
// layers (Peng et al., 2023: ramp over r = L / wavelength between beta_slow
// and beta_fast rotations), and the multiplier of rotated q and k.
void rope_table(const olmo3_rope* rope, int layer_type, int d, RopeTable* t) {
  memset(t, 0, sizeof(*t));
  const bool yarn = rope->yarn && layer_type == OLMO3_LAYER_FULL && rope->factor > 1.0;
  // YaRN in the form its authors' code computes it: pair i turns
  // orig_ctx * w_i / (2 pi) times over the original context, a count that
  // equals beta at the pair index c(beta) = d ln(orig_ctx / (2 pi beta)) /
  // (2 ln theta); the weight u of the interpolated rate w_i / factor ramps
  // linearly over the pair index from floor(c(beta_fast)) to
  // ceil(c(beta_slow)) (kept within [0, d - 1]).
  double lo = 0.0, hi = 1.0;
  if (yarn) {
    auto pair_index = [&](double beta) {
      return d * log((double)rope->orig_ctx / (2.0 * M_PI * beta)) / (2.0 * log(rope->theta));
    };
    lo = std::max(floor(pair_index(rope->beta_fast)), 0.0);
    hi = std::min(ceil(pair_index(rope->beta_slow)), (double)(d - 1));
    if (lo == hi) hi += 0.001;
  }
  for (int i = 0; i < d / 2; ++i) {
    const double w = pow(rope->theta, -2.0 * i / d);
    if (!yarn) {
      t->inv_freq[i] = w;
      continue;
    }
    double u = (i - lo) / (hi - lo);
    u = u < 0.0 ? 0.0 : (u > 1.0 ? 1.0 : u);
    t->inv_freq[i] = (1.0 - u) * w + u * (w / rope->factor);
  }
  double m = 1.0;
  if (rope->yarn && layer_type == OLMO3_LAYER_FULL) {
    if (rope->attn_factor > 0.0)
      m = rope->attn_factor;
    else if (rope->factor > 1.0)
      m = 0.1 * log(rope->factor) + 1.0;
  }
  t->mscale = (float)m;
}

float scale_log2(int d) { return (float)(kLog2e / sqrt((double)d)); }

bool use_mfma(int dtype, int d) { return dtype != OLMO3_DTYPE_F32 && d == 128; }

bool decode_uses_split(int dtype, int d, int H, int G) {
  return use_mfma(dtype, d) && H / G <= 8;
}

// Rotated queries, plus rotated keys where the attention cannot read them
// from the cache: a ring shorter than the call, or an e4m3 cache.
size_t prefill_ws_base(int B, int T, int H, int G, int d, int layer_type, int dtype) {
  const size_t es = elem_size(dtype);
  size_t bytes = align_up((size_t)B * T * H * d * es);
  if (layer_type == OLMO3_LAYER_SLIDING || dtype == OLMO3_DTYPE_BF16_E4M3)
    bytes += align_up((size_t)B * G * T * d * es);
  return bytes;
}

// Key splits of a uniform prefill without a prefix: two when the grid of
// query blocks x heads x sequences would not give every CU two workgroups.
// A sliding layer's blocks carry equal work, so there the split pays only
// while the doubled grid still runs in one round; a full layer's blocks
// differ in length, and halving the longest ones shortens the last round.
int prefill_kv_splits(int B, int T, int H, int d, int dtype, int layer_type) {
  const int64_t blocks = (int64_t)((T + pf::kBQ - 1) / pf::kBQ) * H * B;
  if (!use_mfma(dtype, d) || blocks >= pf::kSplitBelowBlocks) return 1;
  if (layer_type == OLMO3_LAYER_SLIDING && blocks * pf::kKvSplits > pf::kSplitBelowBlocks) return 1;
  return pf::kKvSplits;
}

// ... plus, for such grids, the partial states of the splits (after the rest).
// Workspace of a prefill call.  may_split: the call can split each query
// block's keys (uniform rows without a prefix source: not packed, not a
// sliding chunk after a ring prefix, not an e4m3 chunk after a staged
// prefix); only then are the split partial states reserved.
size_t prefill_ws(int B, int T, int H, int G, int d, int layer_type, int dtype,
                  bool may_split = true) {
  size_t bytes = prefill_ws_base(B, T, H, G, d, layer_type, dtype);
  const int splits = may_split ? prefill_kv_splits(B, T, H, d, dtype, layer_type) : 1;
  if (splits > 1) bytes += align_up((size_t)B * T * H * splits * (d + 2) * sizeof(float));
  return bytes;
}

// A later chunk of a prefill into e4m3 caches reads the cache's earlier rows
// through a bf16 copy of them (keys and values, `rows` per (sequence, head)).
size_t stage_ws(int B, int G, int d, int64_t rows) {
  return 2 * align_up((size_t)B * G * rows * d * sizeof(uint16_t));
}

// Rows of that copy: the whole ring (slot order kept) or positions
// 0 .. pos_offset-1 of a linear cache.
int64_t stage_rows(int layer_type, int window, int64_t pos_offset) {
  return layer_type == OLMO3_LAYER_SLIDING ? window : pos_offset;
}

size_t decode_ws(int B, int H, int G, int d, int layer_type, int window, int dtype, int64_t cap) {
  const size_t es = elem_size(dtype);
  size_t bytes = align_up((size_t)B * H * d * es);
  if (decode_uses_split(dtype, d, H, G)) {
    const int64_t n_max = layer_type == OLMO3_LAYER_SLIDING ? window : cap;
    const int splits = decode_splits(B, G, n_max);
    bytes += align_up((size_t)B * H * splits * (d + 2) * sizeof(float));
  }
  return bytes;
}

int hip_status(hipError_t e) { return e == hipSuccess ? OLMO3_OK : OLMO3_ERR_HIP; }

// Element format of the caches: bf16 (or fp32) rows, or e4m3 codes whose
// values are code * k_scale (keys) and code * v_scale (values).
struct CacheFormat {
  int e4m3;
  float k_scale, v_scale;
};
constexpr CacheFormat kPlainCache = {0, 1.f, 1.f};

void set_cache_format(PrologueArgs& p, const CacheFormat& cf) {
  p.cache_fp8 = cf.e4m3;
  p.k_inv_scale = (float)(1.0 / (double)cf.k_scale);
  p.v_inv_scale = (float)(1.0 / (double)cf.v_scale);
}

bool valid_scale(float x) { return x > 0.f && isfinite(x) && isfinite(1.0f / x); }

// QK-norm + RoPE + store of keys and values only (no attention).
int kv_append_impl(int B, int T, int G, int d, int window, int layer_type,
                   const olmo3_rope* rope, float eps, int64_t pos_offset, int dtype,
                   const void* k_pre, const void* v, const void* k_gain, void* k_cache,
                   void* v_cache, int64_t cache_capacity, hipStream_t stream,
                   const CacheFormat& cf) {
  int st = check_common(B, T, G, G, d, window, layer_type, dtype, rope, eps, pos_offset);
  if (st) return st;
  if (!k_pre || !v || !k_gain || !k_cache || !v_cache) return OLMO3_ERR_INVALID_ARG;
  if (!aligned16(k_pre) || !aligned16(v) || !aligned16(k_gain) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return OLMO3_ERR_INVALID_ARG;
  st = check_capacity(layer_type, window, cache_capacity, pos_offset + T - 1);
  if (st) return st;
  const size_t es = elem_size(dtype), ces = cf.e4m3 ? 1 : es;
  if (!cache_size_ok((int64_t)B * G, cache_capacity, d, ces)) return OLMO3_ERR_UNSUPPORTED;
  const Span kc = span(k_cache, (size_t)B * G * cache_capacity * d * ces);
  const Span vc = span(v_cache, (size_t)B * G * cache_capacity * d * ces);
  const Span in[] = {span(k_pre, (size_t)B * T * G * d * es), span(v, (size_t)B * T * G * d * es),
                     span(k_gain, (size_t)G * d * es)};
  if (overlap(kc, vc)) return OLMO3_ERR_INVALID_ARG;
  for (const Span& sp : in)
    if (overlap(sp, kc) || overlap(sp, vc)) return OLMO3_ERR_INVALID_ARG;

  RopeTable table;
  rope_table(rope, layer_type, d, &table);
  PrologueArgs a = {};
  a.k_pre = k_pre;
  a.v = v;
  a.k_gain = k_gain;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cap = cache_capacity;
  a.pos_offset = pos_offset;
  a.keep_last = layer_type == OLMO3_LAYER_SLIDING ? window : INT64_MAX;
  a.store = 1;
  a.B = B;
  a.T = T;
  a.H = G;
  a.G = G;
  a.window = window;
  a.sliding = layer_type == OLMO3_LAYER_SLIDING;
  a.eps = eps;
  set_cache_format(a, cf);
  return hip_status(launch_prologue(a, table, dtype, d, stream));
}

}  // namespace

extern "C" {

int olmo3_abi_version(void) { return OLMO3_ABI_VERSION; }

const char* olmo3_status_string(int status) {
  switch (status) {
    case OLMO3_OK: return "ok";
    case OLMO3_ERR_INVALID_ARG: return "invalid argument";
    case OLMO3_ERR_UNSUPPORTED: return "unsupported configuration";
    case OLMO3_ERR_CAPACITY: return "cache capacity does not fit the positions or the window";
    case OLMO3_ERR_HIP: return "HIP launch failed";
    case OLMO3_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int olmo3_layer_type(int layer, int n_layers) {
  if (n_layers < 1 || layer < 0 || layer >= n_layers) return -1;
  return (layer % 4 == 3 || layer == n_layers - 1) ? OLMO3_LAYER_FULL : OLMO3_LAYER_SLIDING;
}

size_t olmo3_workspace_bytes(int mode, int B, int T, int H, int G, int d, int layer_type,
                             int dtype, int64_t cache_capacity) {
  olmo3_rope plain = {10000.0, 0, 1.0, 1, 32.0, 1.0, 0.0};
  if (mode == OLMO3_MODE_DECODE) T = 1;
  const int act = dtype == OLMO3_DTYPE_BF16_E4M3 ? OLMO3_DTYPE_BF16 : dtype;
  if (check_common(B, T, H, G, d, 1, layer_type, act, &plain, 0.f, 0) != OLMO3_OK) return 0;
  if (mode == OLMO3_MODE_PREFILL) {
    size_t bytes = prefill_ws(B, T, H, G, d, layer_type, dtype);
    // e4m3: room for a bf16 copy of every cache row, for chunks after the first
    if (dtype == OLMO3_DTYPE_BF16_E4M3 && cache_capacity > 0) bytes += stage_ws(B, G, d, cache_capacity);
    return bytes;
  }
  if (mode == OLMO3_MODE_DECODE) {
    if (cache_capacity < 1) return 0;
    // a sliding layer's ring holds cache_capacity == window slots
    return decode_ws(B, H, G, d, layer_type, (int)std::min<int64_t>(cache_capacity, INT32_MAX),
                     dtype, cache_capacity);
  }
  return 0;
}

int olmo3_kv_append(int B, int T, int G, int d, int window, int layer_type,
                    const olmo3_rope* rope, float eps, int64_t pos_offset, int dtype,
                    const void* k_pre, const void* v, const void* k_gain, void* k_cache,
                    void* v_cache, int64_t cache_capacity, void* stream) {
  return kv_append_impl(B, T, G, d, window, layer_type, rope, eps, pos_offset, dtype, k_pre, v,
                        k_gain, k_cache, v_cache, cache_capacity, (hipStream_t)stream,
                        kPlainCache);
}

int olmo3_kv_append_e4m3(int B, int T, int G, int d, int window, int layer_type,
                         const olmo3_rope* rope, float eps, int64_t pos_offset, const void* k_pre,
                         const void* v, const void* k_gain, void* k_cache, void* v_cache,
                         float k_scale, float v_scale, int64_t cache_capacity, void* stream) {
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return OLMO3_ERR_INVALID_ARG;
  return kv_append_impl(B, T, G, d, window, layer_type, rope, eps, pos_offset, OLMO3_DTYPE_BF16,
                        k_pre, v, k_gain, k_cache, v_cache, cache_capacity, (hipStream_t)stream,
                        CacheFormat{1, k_scale, v_scale});
}

static int validate_attn(int B, int T, int H, int G, int d, int window, int layer_type,
                         const olmo3_rope* rope, float eps, int64_t pos_offset, int dtype,
                         const void* q_pre, const void* k_pre, const void* v, const void* q_gain,
                         const void* k_gain, void* k_cache, void* v_cache,
                         int64_t cache_capacity, void* out, void* workspace,
                         size_t workspace_bytes, size_t ws_needed, int cache_B,
                         int64_t last_pos, size_t cache_es = 0) {
  int st = check_common(B, T, H, G, d, window, layer_type, dtype, rope, eps, pos_offset);
  if (st) return st;
  const void* ptrs[] = {q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return OLMO3_ERR_INVALID_ARG;
  st = check_capacity(layer_type, window, cache_capacity, last_pos);
  if (st) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < ws_needed) return OLMO3_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  if (cache_B < 1 || (int64_t)cache_B * G > 65535 * 64) return OLMO3_ERR_INVALID_ARG;
  const size_t ces = cache_es ? cache_es : es;
  if (!cache_size_ok((int64_t)cache_B * G, cache_capacity, d, ces)) return OLMO3_ERR_UNSUPPORTED;
  const Span kc = span(k_cache, (size_t)cache_B * G * cache_capacity * d * ces);
  const Span vc = span(v_cache, (size_t)cache_B * G * cache_capacity * d * ces);
  const Span o = span(out, (size_t)B * T * H * d * es);
  const Span ws = span(workspace, ws_needed);
  const Span in[] = {span(q_pre, (size_t)B * T * H * d * es), span(k_pre, (size_t)B * T * G * d * es),
                     span(v, (size_t)B * T * G * d * es), span(q_gain, (size_t)H * d * es),
                     span(k_gain, (size_t)G * d * es)};
  if (overlap(kc, vc) || overlap(o, kc) || overlap(o, vc) || overlap(ws, kc) || overlap(ws, vc) ||
      overlap(ws, o))
    return OLMO3_ERR_INVALID_ARG;
  for (const Span& s : in)
    if (overlap(s, kc) || overlap(s, vc) || overlap(s, o) || overlap(s, ws)) return OLMO3_ERR_INVALID_ARG;
  return OLMO3_OK;
}

}  // extern "C"

namespace {

// The sequences of one prefill call.  Uniform: B sequences of T rows at
// positions pos_offset .. pos_offset+T-1.  Packed: B sequences in n_rows
// rows, sequence b at rows cu_seqlens[b] .. cu_seqlens[b+1]-1 and positions
// from pos_offsets[b] (device arrays), at most T = max_len rows each.
struct PrefillShape {
  int B, T;
  int64_t n_rows;
  int64_t pos_offset;
  const int32_t* cu_seqlens;
  const int32_t* pos_offsets;
};

int prefill_impl(int phases, const PrefillShape& sh, int H, int G, int d, int window,
                 int layer_type, const olmo3_rope* rope, float eps, int dtype, const void* q_pre,
                 const void* k_pre, const void* v, const void* q_gain, const void* k_gain,
                 void* k_cache, void* v_cache, int64_t cache_capacity, void* out,
                 void* workspace, hipStream_t s, const CacheFormat& cf = kPlainCache) {
  const bool packed = sh.cu_seqlens != nullptr;
  const bool sliding = layer_type == OLMO3_LAYER_SLIDING;
  const int B = sh.B, T = sh.T;
  const int64_t N = sh.n_rows;
  // A chunk on a sliding layer attends to the ring's earlier positions, and
  // its own keys would overwrite ring slots that its first queries still
  // read: such a chunk is stored in the ring only after the attention.  A
  // packed call may hold such chunks in any sequence.
  const bool ring_after = sliding && (packed || sh.pos_offset > 0);
  const size_t es = elem_size(dtype);
  char* ws = (char*)workspace;
  void* q_rot = ws;
  // the attention reads the new keys from the workspace and the new values
  // from the input, except on a full layer with a bf16 cache, which it reads
  // straight after the prologue has filled it
  const bool kv_from_ws = sliding || cf.e4m3;
  void* k_rot = kv_from_ws ? ws + align_up((size_t)N * H * d * es) : nullptr;
  // a later chunk with e4m3 caches reads the earlier positions from a bf16
  // copy of the cache rows that hold them, placed after the rotated keys
  const bool stage = cf.e4m3 && !packed && sh.pos_offset > 0;
  const int64_t st_rows = stage ? stage_rows(layer_type, window, sh.pos_offset) : 0;
  char* k_stage = stage ? (char*)k_rot + align_up((size_t)B * G * T * d * es) : nullptr;
  char* v_stage = stage ? k_stage + stage_ws(B, G, d, st_rows) / 2 : nullptr;

  RopeTable table;
  rope_table(rope, layer_type, d, &table);
  PrologueArgs p = {};
  p.q_pre = q_pre;
  p.k_pre = k_pre;
  p.v = v;
  p.q_gain = q_gain;
  p.k_gain = k_gain;
  p.q_out = q_rot;
  // rotated keys: [B][G][T][d], or [G][rows][d] when packed
  p.k_out = k_rot;
  p.k_sb = packed ? 0 : (int64_t)G * T * d;
  p.k_sg = (packed ? N : (int64_t)T) * d;
  p.k_st = d;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.cap = cache_capacity;
  p.pos_offset = sh.pos_offset;
  p.keep_last = sliding ? window : INT64_MAX;  // a ring keeps the last `window`
  p.store = !ring_after;
  // the MFMA kernel takes its queries times its base-2 softmax scale
  p.q_scale = use_mfma(dtype, d) ? scale_log2(d) : 1.0f;
  p.seq_pos = sh.pos_offsets;
  p.cu_seqlens = sh.cu_seqlens;
  p.n_rows = N;
  p.B = B;
  p.T = T;
  p.H = H;
  p.G = G;
  p.window = window;
  p.sliding = sliding;
  p.eps = eps;
  set_cache_format(p, cf);
  int st;
  if (phases & OLMO3_PHASE_PROLOGUE) {
    st = hip_status(launch_prologue(p, table, dtype, d, s));
    if (st) return st;
  }
  if (!(phases & OLMO3_PHASE_ATTENTION)) return OLMO3_OK;
  if (stage) {
    // before the chunk's own positions enter a ring (they are stored after
    // the attention); on a linear cache they lie past the copied rows
    E4m3StageArgs sa = {};
    sa.k_codes = k_cache;
    sa.v_codes = v_cache;
    sa.k_out = k_stage;
    sa.v_out = v_stage;
    sa.cap = cache_capacity;
    sa.rows = st_rows;
    sa.n = std::min<int64_t>(sh.pos_offset, st_rows);
    sa.BG = B * G;
    sa.d = d;
    sa.k_scale = cf.k_scale;
    sa.v_scale = cf.v_scale;
    st = hip_status(launch_e4m3_rows_to_bf16(sa, s));
    if (st) return st;
  }

  AttnArgs a = {};
  a.q = q_rot;
  if (kv_from_ws) {
    // the chunk: rotated keys from the workspace, values from the input;
    // earlier positions (if any) from the ring
    a.k = k_rot;
    a.k_sb = p.k_sb;
    a.k_sg = p.k_sg;
    a.k_sr = d;
    a.v = v;
    a.v_sb = packed ? 0 : (int64_t)T * G * d;
    a.v_sg = d;
    a.v_sr = (int64_t)G * d;
    a.main_pos0 = sh.pos_offset;
    a.main_packed = packed;
    if (stage) {
      // earlier positions from the bf16 copy: slot = position mod window on
      // a ring, row = position on a linear cache (all below st_rows)
      a.kp = k_stage;
      a.vp = v_stage;
      a.p_sb = (int64_t)G * st_rows * d;
      a.p_sg = st_rows * d;
      a.p_sr = d;
      a.ring = st_rows;
    } else if (ring_after && !cf.e4m3) {
      // (packed first chunks into e4m3 caches have no earlier positions)
      a.kp = k_cache;
      a.vp = v_cache;
      a.p_sb = (int64_t)G * cache_capacity * d;
      a.p_sg = cache_capacity * d;
      a.p_sr = d;
      a.ring = window;
    }
  } else {
    // the linear cache now holds every position up to the chunk's last
    a.k = k_cache;
    a.v = v_cache;
    a.k_sb = a.v_sb = (int64_t)G * cache_capacity * d;
    a.k_sg = a.v_sg = cache_capacity * d;
    a.k_sr = a.v_sr = d;
    a.main_pos0 = 0;
  }
  a.out = out;
  a.B = B;
  a.Tq = T;
  a.H = H;
  a.G = G;
  a.n_keys = sh.pos_offset + T;
  a.q_pos0 = sh.pos_offset;
  a.window = window;
  a.sliding = sliding;
  a.all_visible = 0;
  a.scale_log2 = scale_log2(d);
  a.cu_seqlens = sh.cu_seqlens;
  a.seq_pos = sh.pos_offsets;
  a.n_rows = N;
  a.key_limit = sliding ? kMaxPrefillPositions : cache_capacity;
  // split key ranges for small uniform grids; not with a prefix source or
  // packed rows (their instances keep one workgroup per query block)
  a.kv_splits = packed || a.kp ? 1 : prefill_kv_splits(B, T, H, d, dtype, layer_type);
  // partial states after the rotated queries and (if there) keys; calls that
  // split have neither a prefix nor packed rows, so no staged copy follows
  if (a.kv_splits > 1)
    a.part = (float*)(ws + align_up((size_t)N * H * d * es) +
                      (kv_from_ws ? align_up((size_t)B * G * T * d * es) : 0));
  st = hip_status(use_mfma(dtype, d) ? launch_prefill_mfma(a, s)
                                     : launch_attn_generic(a, dtype, d, s));
  if (!st && a.kv_splits > 1) {
    // one merge row per (query row, head)
    DecodeArgs m = {};
    m.part = a.part;
    m.out = out;
    m.B = (int)N;
    m.H = H;
    m.splits = a.kv_splits;
    st = hip_status(launch_decode_merge(m, s));
  }
  if (st || !ring_after) return st;
  // store the chunk's kept positions in the ring (keys normalised and rotated
  // again from k_pre: the same arithmetic, so the same bits)
  PrologueArgs r = p;
  r.q_pre = nullptr;
  r.q_out = nullptr;
  r.k_out = nullptr;
  r.store = 1;
  return hip_status(launch_prologue(r, table, dtype, d, s));
}

}  // namespace

extern "C" {

int olmo3_attn_prefill_phases(int phases, int B, int T, int H, int G, int d, int window,
                              int layer_type, const olmo3_rope* rope, float eps,
                              int64_t pos_offset, int dtype, const void* q_pre, const void* k_pre,
                              const void* v, const void* q_gain, const void* k_gain,
                              void* k_cache, void* v_cache, int64_t cache_capacity, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (phases <= 0 || (phases & ~(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION | OLMO3_PHASE_MERGE)))
    return OLMO3_ERR_INVALID_ARG;
  // a sliding chunk after a ring prefix keeps one workgroup per query block
  const bool may_split = !(layer_type == OLMO3_LAYER_SLIDING && pos_offset > 0);
  const size_t need = (B > 0 && T > 0 && H > 0 && G > 0 && d > 0)
                          ? prefill_ws(B, T, H, G, d, layer_type, dtype, may_split)
                          : 0;
  int st = validate_attn(B, T, H, G, d, window, layer_type, rope, eps, pos_offset, dtype, q_pre,
                         k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                         workspace, workspace_bytes, need, B, pos_offset + T - 1);
  if (st) return st;
  // positions are 32-bit inside the prefill kernels
  if (pos_offset + T > kMaxPrefillPositions) return OLMO3_ERR_UNSUPPORTED;
  const PrefillShape sh = {B, T, (int64_t)B * T, pos_offset, nullptr, nullptr};
  return prefill_impl(phases, sh, H, G, d, window, layer_type, rope, eps, dtype, q_pre, k_pre, v,
                      q_gain, k_gain, k_cache, v_cache, cache_capacity, out, workspace,
                      (hipStream_t)stream);
}

int olmo3_attn_prefill_ragged(int B, int n_tokens, int max_len, int64_t max_end, int H, int G,
                              int d, int window, int layer_type, const olmo3_rope* rope,
                              float eps, const int32_t* cu_seqlens, const int32_t* pos_offsets,
                              int dtype, const void* q_pre, const void* k_pre, const void* v,
                              const void* q_gain, const void* k_gain, void* k_cache,
                              void* v_cache, int64_t cache_capacity, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (B < 1 || n_tokens < 1 || max_len < 1 || max_len > n_tokens || max_end < max_len)
    return OLMO3_ERR_INVALID_ARG;
  if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3) || ((uintptr_t)pos_offsets & 3))
    return OLMO3_ERR_INVALID_ARG;
  const size_t need = (H > 0 && G > 0 && d > 0) ? prefill_ws(1, n_tokens, H, G, d, layer_type, dtype,
                                                             false)
                                                : 0;
  // the rows as one sequence for the input sizes; the caches hold B sequences
  int st = validate_attn(1, n_tokens, H, G, d, window, layer_type, rope, eps, 0, dtype, q_pre,
                         k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                         workspace, workspace_bytes, need, B, max_end - 1);
  if (st) return st;
  if (max_end > kMaxPrefillPositions) return OLMO3_ERR_UNSUPPORTED;
  const PrefillShape sh = {B, max_len, n_tokens, 0, cu_seqlens, pos_offsets};
  return prefill_impl(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION, sh, H, G, d, window,
                      layer_type, rope, eps, dtype, q_pre, k_pre, v, q_gain, k_gain, k_cache,
                      v_cache, cache_capacity, out, workspace, (hipStream_t)stream);
}

int olmo3_attn_prefill(int B, int T, int H, int G, int d, int window, int layer_type,
                       const olmo3_rope* rope, float eps, int64_t pos_offset, int dtype,
                       const void* q_pre, const void* k_pre, const void* v, const void* q_gain,
                       const void* k_gain, void* k_cache, void* v_cache, int64_t cache_capacity,
                       void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return olmo3_attn_prefill_phases(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION, B, T, H, G, d,
                                   window, layer_type, rope, eps, pos_offset, dtype, q_pre, k_pre,
                                   v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                                   workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Decode of one token per sequence: at position `pos` for every sequence, or
// at positions[b] (device array, each at most max_pos) when positions is set.
int decode_impl(int phases, int B, int H, int G, int d, int window, int layer_type,
                const olmo3_rope* rope, float eps, int64_t pos, const int32_t* positions,
                int64_t max_pos, int dtype, const void* q_pre, const void* k_pre, const void* v,
                const void* q_gain, const void* k_gain, void* k_cache, void* v_cache,
                int64_t cache_capacity, void* out, void* workspace, hipStream_t s,
                const CacheFormat& cf = kPlainCache) {
  const bool sliding = layer_type == OLMO3_LAYER_SLIDING;
  const size_t es = elem_size(dtype);
  char* ws = (char*)workspace;
  void* q_rot = ws;

  RopeTable table;
  rope_table(rope, layer_type, d, &table);
  PrologueArgs p = {};
  p.q_pre = q_pre;
  p.k_pre = k_pre;
  p.v = v;
  p.q_gain = q_gain;
  p.k_gain = k_gain;
  p.q_out = q_rot;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.cap = cache_capacity;
  p.pos_offset = pos;
  p.keep_last = INT64_MAX;
  p.store = 1;
  p.seq_pos = positions;
  p.B = B;
  p.T = 1;
  p.H = H;
  p.G = G;
  p.window = window;
  p.sliding = sliding;
  p.eps = eps;
  set_cache_format(p, cf);
  int st;
  if (phases & OLMO3_PHASE_PROLOGUE) {
    st = hip_status(launch_prologue(p, table, dtype, d, s));
    if (st) return st;
  }

  // rows read: the filled ring slots or slots 0 .. pos (the largest over the
  // batch when positions differ; each sequence then reads its own count)
  const int64_t n = sliding ? std::min<int64_t>(max_pos + 1, window) : max_pos + 1;
  if (decode_uses_split(dtype, d, H, G)) {
    DecodeArgs a = {};
    a.q = q_rot;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.cap = cache_capacity;
    a.n = n;
    a.splits = decode_splits(B, G, n);
    const int64_t per = (n + a.splits - 1) / a.splits;
    a.rows_per_split = (per + dec::kRowsPerIter - 1) / dec::kRowsPerIter * dec::kRowsPerIter;
    a.part = (float*)(ws + align_up((size_t)B * H * d * es));
    a.out = out;
    a.B = B;
    a.H = H;
    a.G = G;
    a.scale_log2 = scale_log2(d);
    a.seq_pos = positions;
    a.window = window;
    a.sliding = sliding;
    a.fp8 = cf.e4m3;
    a.k_scale = cf.k_scale;
    a.v_scale = cf.v_scale;
    if (phases & OLMO3_PHASE_ATTENTION) {
      st = hip_status(launch_decode_split(a, s));
      if (st) return st;
    }
    // one split: the split kernel has written the output rows
    if ((phases & OLMO3_PHASE_MERGE) && a.splits > 1) return hip_status(launch_decode_merge(a, s));
    return OLMO3_OK;
  }
  if (!(phases & OLMO3_PHASE_ATTENTION)) return OLMO3_OK;
  AttnArgs a = {};
  a.q = q_rot;
  a.k = k_cache;
  a.v = v_cache;
  a.k_sb = a.v_sb = (int64_t)G * cache_capacity * d;
  a.k_sg = a.v_sg = cache_capacity * d;
  a.k_sr = a.v_sr = d;
  a.out = out;
  a.B = B;
  a.Tq = 1;
  a.H = H;
  a.G = G;
  a.n_keys = n;
  a.q_pos0 = pos;
  a.window = window;
  a.sliding = sliding;
  a.all_visible = 1;
  a.scale_log2 = scale_log2(d);
  a.seq_pos = positions;
  a.key_limit = cache_capacity;
  return hip_status(launch_attn_generic(a, dtype, d, s));
}

}  // namespace

extern "C" {

int olmo3_attn_decode_phases(int phases, int B, int H, int G, int d, int window, int layer_type,
                             const olmo3_rope* rope, float eps, int64_t pos, int dtype,
                             const void* q_pre, const void* k_pre, const void* v,
                             const void* q_gain, const void* k_gain, void* k_cache,
                             void* v_cache, int64_t cache_capacity, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (phases <= 0 || (phases & ~(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION | OLMO3_PHASE_MERGE)))
    return OLMO3_ERR_INVALID_ARG;
  const size_t need = (B > 0 && H > 0 && G > 0 && d > 0 && G <= H && cache_capacity > 0)
                          ? decode_ws(B, H, G, d, layer_type, window, dtype, cache_capacity)
                          : 0;
  int st = validate_attn(B, 1, H, G, d, window, layer_type, rope, eps, pos, dtype, q_pre, k_pre,
                         v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out, workspace,
                         workspace_bytes, need, B, pos);
  if (st) return st;
  return decode_impl(phases, B, H, G, d, window, layer_type, rope, eps, pos, nullptr, pos, dtype,
                     q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                     workspace, (hipStream_t)stream);
}

int olmo3_attn_decode_ragged(int B, int H, int G, int d, int window, int layer_type,
                             const olmo3_rope* rope, float eps, const int32_t* positions,
                             int64_t max_pos, int dtype, const void* q_pre, const void* k_pre,
                             const void* v, const void* q_gain, const void* k_gain,
                             void* k_cache, void* v_cache, int64_t cache_capacity, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!positions || ((uintptr_t)positions & 3) || max_pos < 0 || max_pos > INT32_MAX)
    return OLMO3_ERR_INVALID_ARG;
  const size_t need = (B > 0 && H > 0 && G > 0 && d > 0 && G <= H && cache_capacity > 0)
                          ? decode_ws(B, H, G, d, layer_type, window, dtype, cache_capacity)
                          : 0;
  int st = validate_attn(B, 1, H, G, d, window, layer_type, rope, eps, max_pos, dtype, q_pre,
                         k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                         workspace, workspace_bytes, need, B, max_pos);
  if (st) return st;
  return decode_impl(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION | OLMO3_PHASE_MERGE, B, H, G,
                     d, window, layer_type, rope, eps, 0, positions, max_pos, dtype, q_pre, k_pre,
                     v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out, workspace,
                     (hipStream_t)stream);
}

int olmo3_attn_decode_ragged_e4m3(int B, int H, int G, int d, int window, int layer_type,
                                  const olmo3_rope* rope, float eps, const int32_t* positions,
                                  int64_t max_pos, const void* q_pre, const void* k_pre,
                                  const void* v, const void* q_gain, const void* k_gain,
                                  void* k_cache, void* v_cache, float k_scale, float v_scale,
                                  int64_t cache_capacity, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!positions || ((uintptr_t)positions & 3) || max_pos < 0 || max_pos > INT32_MAX)
    return OLMO3_ERR_INVALID_ARG;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return OLMO3_ERR_INVALID_ARG;
  const size_t need = (B > 0 && H > 0 && G > 0 && d > 0 && G <= H && cache_capacity > 0)
                          ? decode_ws(B, H, G, d, layer_type, window, OLMO3_DTYPE_BF16_E4M3,
                                      cache_capacity)
                          : 0;
  int st = validate_attn(B, 1, H, G, d, window, layer_type, rope, eps, max_pos, OLMO3_DTYPE_BF16,
                         q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                         workspace, workspace_bytes, need, B, max_pos, 1);
  if (st) return st;
  // the e4m3 cache is read by the split-KV kernels only
  if (!decode_uses_split(OLMO3_DTYPE_BF16_E4M3, d, H, G)) return OLMO3_ERR_UNSUPPORTED;
  return decode_impl(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION | OLMO3_PHASE_MERGE, B, H, G,
                     d, window, layer_type, rope, eps, 0, positions, max_pos, OLMO3_DTYPE_BF16,
                     q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                     workspace, (hipStream_t)stream, CacheFormat{1, k_scale, v_scale});
}

int olmo3_attn_decode(int B, int H, int G, int d, int window, int layer_type,
                      const olmo3_rope* rope, float eps, int64_t pos, int dtype,
                      const void* q_pre, const void* k_pre, const void* v, const void* q_gain,
                      const void* k_gain, void* k_cache, void* v_cache, int64_t cache_capacity,
                      void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return olmo3_attn_decode_phases(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION | OLMO3_PHASE_MERGE,
                                  B, H, G, d, window, layer_type, rope, eps, pos, dtype, q_pre,
                                  k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                                  workspace, workspace_bytes, stream);
}

int olmo3_attn_prefill_ragged_e4m3(int B, int n_tokens, int max_len, int H, int G, int d,
                                   int window, int layer_type, const olmo3_rope* rope, float eps,
                                   const int32_t* cu_seqlens, const void* q_pre,
                                   const void* k_pre, const void* v, const void* q_gain,
                                   const void* k_gain, void* k_cache, void* v_cache,
                                   float k_scale, float v_scale, int64_t cache_capacity, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || n_tokens < 1 || max_len < 1 || max_len > n_tokens) return OLMO3_ERR_INVALID_ARG;
  if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3)) return OLMO3_ERR_INVALID_ARG;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return OLMO3_ERR_INVALID_ARG;
  const size_t need = (H > 0 && G > 0 && d > 0)
                          ? prefill_ws(1, n_tokens, H, G, d, layer_type, OLMO3_DTYPE_BF16_E4M3,
                                       false)
                          : 0;
  // the rows as one sequence for the input sizes; the caches hold B sequences
  int st = validate_attn(1, n_tokens, H, G, d, window, layer_type, rope, eps, 0, OLMO3_DTYPE_BF16,
                         q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                         workspace, workspace_bytes, need, B, (int64_t)max_len - 1, 1);
  if (st) return st;
  if (max_len > kMaxPrefillPositions) return OLMO3_ERR_UNSUPPORTED;
  const PrefillShape sh = {B, max_len, n_tokens, 0, cu_seqlens, nullptr};
  return prefill_impl(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION, sh, H, G, d, window,
                      layer_type, rope, eps, OLMO3_DTYPE_BF16, q_pre, k_pre, v, q_gain, k_gain,
                      k_cache, v_cache, cache_capacity, out, workspace, (hipStream_t)stream,
                      CacheFormat{1, k_scale, v_scale});
}

int olmo3_attn_prefill_e4m3(int B, int T, int H, int G, int d, int window, int layer_type,
                            const olmo3_rope* rope, float eps, int64_t pos_offset,
                            const void* q_pre, const void* k_pre, const void* v,
                            const void* q_gain, const void* k_gain, void* k_cache,
                            void* v_cache, float k_scale, float v_scale, int64_t cache_capacity,
                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return OLMO3_ERR_INVALID_ARG;
  const bool sizes_ok = B > 0 && T > 0 && H > 0 && G > 0 && d > 0 && window > 0 && pos_offset >= 0;
  // a later chunk reads its prefix from a staged copy and does not split
  size_t need = sizes_ok ? prefill_ws(B, T, H, G, d, layer_type, OLMO3_DTYPE_BF16_E4M3,
                                      pos_offset == 0)
                         : 0;
  if (sizes_ok && pos_offset > 0) need += stage_ws(B, G, d, stage_rows(layer_type, window, pos_offset));
  int st = validate_attn(B, T, H, G, d, window, layer_type, rope, eps, pos_offset,
                         OLMO3_DTYPE_BF16, q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache,
                         cache_capacity, out, workspace, workspace_bytes, need, B,
                         pos_offset + T - 1, 1);
  if (st) return st;
  if (pos_offset + T > kMaxPrefillPositions) return OLMO3_ERR_UNSUPPORTED;
  const PrefillShape sh = {B, T, (int64_t)B * T, pos_offset, nullptr, nullptr};
  return prefill_impl(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION, sh, H, G, d, window,
                      layer_type, rope, eps, OLMO3_DTYPE_BF16, q_pre, k_pre, v, q_gain, k_gain,
                      k_cache, v_cache, cache_capacity, out, workspace, (hipStream_t)stream,
                      CacheFormat{1, k_scale, v_scale});
}

int olmo3_attn_decode_e4m3_phases(int phases, int B, int H, int G, int d, int window,
                                  int layer_type, const olmo3_rope* rope, float eps, int64_t pos,
                                  const void* q_pre, const void* k_pre, const void* v,
                                  const void* q_gain, const void* k_gain, void* k_cache,
                                  void* v_cache, float k_scale, float v_scale,
                                  int64_t cache_capacity, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (phases <= 0 || (phases & ~(OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION | OLMO3_PHASE_MERGE)))
    return OLMO3_ERR_INVALID_ARG;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return OLMO3_ERR_INVALID_ARG;
  const size_t need = (B > 0 && H > 0 && G > 0 && d > 0 && G <= H && cache_capacity > 0)
                          ? decode_ws(B, H, G, d, layer_type, window, OLMO3_DTYPE_BF16_E4M3,
                                      cache_capacity)
                          : 0;
  int st = validate_attn(B, 1, H, G, d, window, layer_type, rope, eps, pos, OLMO3_DTYPE_BF16,
                         q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, cache_capacity, out,
                         workspace, workspace_bytes, need, B, pos, 1);
  if (st) return st;
  // the e4m3 cache is read by the split-KV kernel only
  if (!decode_uses_split(OLMO3_DTYPE_BF16_E4M3, d, H, G)) return OLMO3_ERR_UNSUPPORTED;
  return decode_impl(phases, B, H, G, d, window, layer_type, rope, eps, pos, nullptr, pos,
                     OLMO3_DTYPE_BF16, q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache,
                     cache_capacity, out, workspace, (hipStream_t)stream,
                     CacheFormat{1, k_scale, v_scale});
}

int olmo3_attn_decode_e4m3(int B, int H, int G, int d, int window, int layer_type,
                           const olmo3_rope* rope, float eps, int64_t pos, const void* q_pre,
                           const void* k_pre, const void* v, const void* q_gain,
                           const void* k_gain, void* k_cache, void* v_cache, float k_scale,
                           float v_scale, int64_t cache_capacity, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return olmo3_attn_decode_e4m3_phases(
      OLMO3_PHASE_PROLOGUE | OLMO3_PHASE_ATTENTION | OLMO3_PHASE_MERGE, B, H, G, d, window,
      layer_type, rope, eps, pos, q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, k_scale,
      v_scale, cache_capacity, out, workspace, workspace_bytes, stream);
}

int olmo3_probe_prefill_visits(int T, int64_t pos_offset, int window, int layer_type,
                               int kv_splits, uint8_t* visit, void* stream) {
  if (T < 1 || pos_offset < 0 || window < 1 || !visit) return OLMO3_ERR_INVALID_ARG;
  if (kv_splits != 1 && kv_splits != pf::kKvSplits) return OLMO3_ERR_INVALID_ARG;
  if (T > 4096 || pos_offset + T > 8192) return OLMO3_ERR_UNSUPPORTED;
  if (layer_type != OLMO3_LAYER_SLIDING && layer_type != OLMO3_LAYER_FULL) return OLMO3_ERR_INVALID_ARG;
  return hip_status(launch_probe_prefill(T, pos_offset, window, layer_type == OLMO3_LAYER_SLIDING,
                                         kv_splits, visit, (hipStream_t)stream));
}

int olmo3_probe_prefill_order(int B, int T, int H, int G, int window, int layer_type,
                              int64_t pos_offset, int kv_splits, int32_t* work, int64_t work_len) {
  if (B < 1 || T < 1 || G < 1 || H < G || H % G || window < 1 || pos_offset < 0 || !work)
    return OLMO3_ERR_INVALID_ARG;
  if (kv_splits != 1 && kv_splits != pf::kKvSplits) return OLMO3_ERR_INVALID_ARG;
  if (layer_type != OLMO3_LAYER_SLIDING && layer_type != OLMO3_LAYER_FULL) return OLMO3_ERR_INVALID_ARG;
  if (pos_offset + T > kMaxPrefillPositions) return OLMO3_ERR_UNSUPPORTED;
  const int64_t n_qblk = (T + pf::kBQ - 1) / pf::kBQ;
  const int64_t n = n_qblk * H * B * kv_splits;
  if (n > ((int64_t)1 << 24)) return OLMO3_ERR_UNSUPPORTED;
  if (work_len < 4 * n) return OLMO3_ERR_INVALID_ARG;
  const int n_even = pf::even_blocks((int)n_qblk, H, G, layer_type == OLMO3_LAYER_SLIDING,
                                     window, (int)pos_offset);
  for (int bid = 0; bid < (int)n; ++bid) {
    int split = 0;
    const pf::Work w = kv_splits > 1
                           ? pf::work_of_split(bid, (int)n, (int)n_qblk, H, n_even, split)
                           : pf::work_of(bid, (int)n, (int)n_qblk, H, n_even);
    work[4 * bid] = w.b;
    work[4 * bid + 1] = w.h;
    work[4 * bid + 2] = w.qb;
    work[4 * bid + 3] = split;
  }
  return OLMO3_OK;
}

int olmo3_probe_decode_reads(int B, int H, int G, int d, int window, int layer_type, int dtype,
                             int64_t pos, int64_t cache_capacity, int32_t* count, void* stream) {
  if (B < 1 || G < 1 || H < G || H % G || d != 128 || window < 1 || pos < 0 || !count)
    return OLMO3_ERR_INVALID_ARG;
  if (dtype != OLMO3_DTYPE_BF16 && dtype != OLMO3_DTYPE_BF16_E4M3) return OLMO3_ERR_INVALID_ARG;
  if (layer_type != OLMO3_LAYER_SLIDING && layer_type != OLMO3_LAYER_FULL) return OLMO3_ERR_INVALID_ARG;
  int st = check_capacity(layer_type, window, cache_capacity, pos);
  if (st) return st;
  if (!cache_size_ok(1, cache_capacity, 1, sizeof(int32_t))) return OLMO3_ERR_UNSUPPORTED;
  const bool sliding = layer_type == OLMO3_LAYER_SLIDING;
  DecodeArgs a = {};
  a.cap = cache_capacity;
  a.n = sliding ? std::min<int64_t>(pos + 1, window) : pos + 1;
  a.splits = decode_splits(B, G, a.n);
  const int64_t per = (a.n + a.splits - 1) / a.splits;
  a.rows_per_split = (per + dec::kRowsPerIter - 1) / dec::kRowsPerIter * dec::kRowsPerIter;
  a.B = B;
  a.H = H;
  a.G = G;
  a.fp8 = dtype == OLMO3_DTYPE_BF16_E4M3;
  return hip_status(launch_probe_decode(a, count, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------- decode
// without allocation.  One scratch array per device, in the library's own
// device memory, stands in for the workspace argument.
namespace {

constexpr size_t kNoAllocScratchBytes = OLMO3_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Held by every device the library runs on until the process ends.  Host
// code never passes this name to a kernel or copy: it stands for a host-side
// shadow there.  The device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Address of the current device's scratch array, looked up once per device
// (with that device current) and kept; nullptr when the lookup fails.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int olmo3_attn_decode_noalloc(int B, int H, int G, int d, int window, int layer_type,
                              const olmo3_rope* rope, float eps, int64_t pos, int dtype,
                              const void* q_pre, const void* k_pre, const void* v,
                              const void* q_gain, const void* k_gain, void* k_cache,
                              void* v_cache, int64_t cache_capacity, void* out, void* stream) {
  // argument errors first, before anything touches the device
  int st = check_common(B, 1, H, G, d, window, layer_type, dtype, rope, eps, pos);
  if (st) return st;
  const void* ptrs[] = {q_pre, k_pre, v, q_gain, k_gain, k_cache, v_cache, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return OLMO3_ERR_INVALID_ARG;
  st = check_capacity(layer_type, window, cache_capacity, pos);
  if (st) return st;
  // the scratch takes the workspace's place, so the call must fit in it
  if (decode_ws(B, H, G, d, layer_type, window, dtype, cache_capacity) > kNoAllocScratchBytes)
    return OLMO3_ERR_WORKSPACE;
  // the rest (overlaps, cache size) as olmo3_attn_decode checks it
  void* ws = device_scratch();
  if (!ws) return OLMO3_ERR_HIP;
  return olmo3_attn_decode(B, H, G, d, window, layer_type, rope, eps, pos, dtype, q_pre, k_pre, v,
                           q_gain, k_gain, k_cache, v_cache, cache_capacity, out, ws,
                           kNoAllocScratchBytes, stream);
}

}  // extern "C"
