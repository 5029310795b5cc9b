/*
 * olmo3_attn.h -- C ABI of the OLMo 3 per-layer hybrid attention library
 * (libolmo3attn.so, HIP kernels for MI355X / gfx950).
 *
 * One call runs one attention layer of OLMo 3: QK-norm, RoPE at absolute
 * positions (YaRN-scaled on full layers), KV-cache append, and causal
 * attention that is either sliding-window or full.
 *
 * Sources of the operations (titles and sections of the pages they follow):
 *   - layer kinds: "OLMo 3's Sliding-Window Attention Pattern", "Which layers
 *     are full" (full iff layer mod 4 == 3, and always the last layer);
 *   - mask: same page, "The sliding-window mask" (key s visible from query t
 *     iff s <= t and, on sliding layers, t - s < window);
 *   - QK-norm: "Case Study: OLMo 3", architecture item 2, with gains of width
 *     H*d and G*d ("Count OLMo 3's Parameters", "What to count") and
 *     eps = 1e-6 ("Olmo-3 End-to-End Implementation", "Technical Details");
 *   - RoPE: "Case Study: OLMo 3", item 3 (rotate-half pairs i, i+d/2, base
 *     theta), with position offsets ("Olmo-3 End-to-End Implementation",
 *     "Inference Pipeline"); YaRN on full layers (item 7);
 *   - cache: "Olmo-3 End-to-End Implementation", "KV Cache Implementation"
 *     (per-layer [B, H_kv, T_total, D] tensors) and "Olmo 3 7B",
 *     "SERVICEABILITY JOIN" (a per-layer-type cache: windowed layers keep a
 *     bounded cache, and decode on them reads exactly `window` entries).
 *
 * Conventions common to every entry point
 *   Memory.  Every tensor pointer is a DEVICE pointer owned by the caller;
 *     `rope` is a HOST pointer.  The library never allocates or frees device
 *     memory and keeps no state between calls; calls are thread-safe.
 *   Layouts (row-major, contiguous, element type = `dtype`):
 *     q_pre  [B][T][H*d]      projected queries before QK-norm
 *     k_pre  [B][T][G*d]      projected keys before QK-norm
 *     v      [B][T][G*d]      projected values
 *     q_gain [H*d], k_gain [G*d]   QK-norm gains
 *     k_cache, v_cache [B][G][cache_capacity][d]
 *     out    [B][T][H*d]      attention output, heads concatenated in order
 *   Query head h reads key/value head h / (H/G).
 *   Cache slots.  Position p is stored at slot p on a full layer (linear
 *     cache, cache_capacity >= last position + 1) and at slot p mod window on
 *     a sliding layer (ring, cache_capacity == window).  When one call writes
 *     more than `window` positions to a ring, only the last `window` of them
 *     are stored.  Keys are stored after QK-norm and RoPE; values unchanged.
 *   Arithmetic.  bf16 inputs and outputs with fp32 accumulation (dtype 0),
 *     or fp32 throughout (dtype 1).  Softmax scale 1/sqrt(d).
 *   Streams.  `stream` is a hipStream_t cast to void* (NULL = the default
 *     stream).  Calls enqueue kernels and return without waiting.
 *   Errors.  Every entry point returns an olmo3_status.  All arguments are
 *     validated on the host before anything is enqueued, so a call that
 *     returns an error has no effect.  OLMO3_ERR_HIP reports a failed launch;
 *     faults inside a kernel surface at the caller's next synchronisation.
 */
#ifndef OLMO3_ATTN_H
#define OLMO3_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OLMO3_ABI_VERSION 11

typedef enum olmo3_status {
  OLMO3_OK = 0,
  OLMO3_ERR_INVALID_ARG = 1, /* bad size, null or overlapping pointer, bad enum   */
  OLMO3_ERR_UNSUPPORTED = 2, /* valid request the library does not implement      */
  OLMO3_ERR_CAPACITY = 3,    /* cache too small, or ring size != window            */
  OLMO3_ERR_HIP = 4,         /* a HIP call or kernel launch failed                 */
  OLMO3_ERR_WORKSPACE = 5    /* workspace null or smaller than olmo3_workspace_bytes */
} olmo3_status;

enum { OLMO3_LAYER_SLIDING = 0, OLMO3_LAYER_FULL = 1 };
/* Element types.  OLMO3_DTYPE_BF16_E4M3 (bf16 activations with e4m3 caches)
 * is accepted by olmo3_workspace_bytes only; the e4m3 entry points below
 * imply it. */
enum { OLMO3_DTYPE_BF16 = 0, OLMO3_DTYPE_F32 = 1, OLMO3_DTYPE_BF16_E4M3 = 2 };
enum { OLMO3_MODE_PREFILL = 0, OLMO3_MODE_DECODE = 1 };

/* RoPE / YaRN settings ("Case Study: OLMo 3", items 3 and 7).
 *   theta        RoPE base; rate of pair i is omega_i = theta^(-2i/d).
 *   yarn         nonzero: full layers use YaRN rates and temperature;
 *                sliding layers always use plain RoPE.
 *   factor       YaRN scale s (>= 1), e.g. 8 for 8192 -> 65536 positions.
 *   orig_ctx     original training context L, e.g. 8192.
 *   beta_fast    rotations over L above which rates are kept, e.g. 32.
 *   beta_slow    rotations over L below which rates are divided by s, e.g. 1.
 *   attn_factor  multiplier applied to rotated q and k; <= 0 selects
 *                0.1*ln(s) + 1 (Peng et al., 2023).  Logits scale by its square.
 * YaRN rate of pair i (Peng et al., 2023, as its authors' code and model
 * configurations compute it): pair i turns L*omega_i/(2*pi) times over L,
 * which equals beta at the pair index c(beta) = d*ln(L/(2*pi*beta)) /
 * (2*ln(theta)); with lo = max(floor(c(beta_fast)), 0), hi =
 * min(ceil(c(beta_slow)), d - 1) (hi = lo + 0.001 if they meet) and
 * u = clamp((i - lo)/(hi - lo), 0, 1): omega'_i = (1 - u)*omega_i + u*omega_i/s.
 * With yarn set: factor >= 1 and finite, orig_ctx >= 1, beta_fast >
 * beta_slow > 0, and theta > 1 when factor > 1; otherwise INVALID_ARG. */
typedef struct olmo3_rope {
  double theta;
  int32_t yarn;
  double factor;
  int64_t orig_ctx;
  double beta_fast;
  double beta_slow;
  double attn_factor;
} olmo3_rope;

/* Kind of layer `layer` (0-based) in a model of `n_layers` layers
 * ("OLMo 3's Sliding-Window Attention Pattern", "Which layers are full").
 * Returns OLMO3_LAYER_FULL (1) or OLMO3_LAYER_SLIDING (0); -1 when
 * n_layers < 1 or layer is outside [0, n_layers). */
int olmo3_layer_type(int layer, int n_layers);

/* Device workspace, in bytes, that olmo3_attn_prefill (mode 0, T tokens) or
 * olmo3_attn_decode (mode 1, T ignored) needs for these sizes; the decode
 * figure covers every position that fits `cache_capacity`.  With e4m3 caches
 * (dtype OLMO3_DTYPE_BF16_E4M3) the prefill figure includes a bf16 copy of
 * `cache_capacity` cache rows, which chunks at pos_offset > 0 need; a first
 * chunk may pass cache_capacity = 0.  For d = 128 bf16 calls whose query
 * blocks of 128 rows times H times B number fewer than 512 (full layers) or
 * at most 256 (sliding layers), the prefill figure also holds the partial
 * softmax states of a two-way split of every block's keys (B*T*H*2*(d+2)
 * floats), which such calls use unless they read a prefix (a sliding-layer
 * chunk at pos_offset > 0, an e4m3 chunk at pos_offset > 0) or come packed
 * (the ragged entry points); those calls accept the smaller workspace
 * without the split states.  The figure is therefore not monotone in T: a
 * workspace sized for the largest chunk of a prompt may be too small for a
 * shorter one that splits; size it per call, or for the largest figure over
 * the lengths used.  Returns 0 for invalid sizes. */
size_t olmo3_workspace_bytes(int mode, int B, int T, int H, int G, int d,
                             int layer_type, int dtype, int64_t cache_capacity);

/* Append T positions pos_offset .. pos_offset+T-1 of keys and values to one
 * layer's cache without attending: keys get QK-norm (gain k_gain, eps) and
 * RoPE at their absolute positions; values are copied unchanged.  k_pre, v:
 * [B][T][G*d].  Errors: INVALID_ARG (sizes <= 0, odd d, pos_offset < 0, bad
 * enum, null pointer, k_cache/v_cache overlapping each other or an input),
 * CAPACITY (ring size != window, or a linear cache shorter than
 * pos_offset + T), UNSUPPORTED (d not in {16, 32, 64, 128}, or a
 * cache_capacity that makes a cache larger than 2^50 bytes). */
int olmo3_kv_append(int B, int T, int G, int d, int window, int layer_type,
                    const olmo3_rope* rope, float eps, int64_t pos_offset,
                    int dtype, const void* k_pre, const void* v,
                    const void* k_gain, void* k_cache, void* v_cache,
                    int64_t cache_capacity, void* stream);

/* Prefill: attention of T new tokens at positions pos_offset .. +T-1, which
 * are also appended to the cache.  Query t attends to every key position
 * s <= t (and t - s < window on sliding layers): the new keys and, when
 * pos_offset > 0 (a later chunk of a prompt, or a multi-token step), the
 * positions the cache already holds, following "Olmo-3 End-to-End
 * Implementation", "Cache Operation Flow" (cached keys and values joined
 * with the new ones).  The caller must have filled the cache with positions
 * 0 .. pos_offset-1 (the ring with the last `window` of them).  out is
 * fully overwritten.  workspace must hold
 * olmo3_workspace_bytes(OLMO3_MODE_PREFILL, ...) bytes (device memory,
 * contents on entry ignored).  Errors: as olmo3_kv_append, plus H % G != 0
 * (INVALID_ARG), out overlapping any other buffer (INVALID_ARG), a short or
 * null workspace (WORKSPACE), and pos_offset + T > 2^30 (UNSUPPORTED). */
int olmo3_attn_prefill(int B, int T, int H, int G, int d, int window,
                       int layer_type, const olmo3_rope* rope, float eps,
                       int64_t pos_offset, int dtype, const void* q_pre,
                       const void* k_pre, const void* v, const void* q_gain,
                       const void* k_gain, void* k_cache, void* v_cache,
                       int64_t cache_capacity, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Decode: one new token per sequence at absolute position `pos` (the same
 * for every sequence of the batch).  Its key and value are appended at
 * slot(pos) first; the query then attends to the n = min(pos+1, window)
 * filled ring slots (sliding) or to slots 0..pos (full), i.e. positions
 * max(0, pos-window+1) .. pos or 0 .. pos, which the caller must have
 * filled earlier.  q_pre [B][H*d], k_pre and v [B][G*d], out [B][H*d].
 * The key range is split across workgroups and the partial softmax states
 * are merged by log-sum-exp.  Errors: as olmo3_attn_prefill with T = 1
 * (pos >= 0 required; CAPACITY if a linear cache has fewer than pos + 1
 * slots). */
int olmo3_attn_decode(int B, int H, int G, int d, int window, int layer_type,
                      const olmo3_rope* rope, float eps, int64_t pos,
                      int dtype, const void* q_pre, const void* k_pre,
                      const void* v, const void* q_gain, const void* k_gain,
                      void* k_cache, void* v_cache, int64_t cache_capacity,
                      void* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): olmo3_attn_decode
 * with the workspace replaced by a scratch array of
 * OLMO3_NOALLOC_SCRATCH_BYTES that the library holds in each device's memory
 * from load until the process ends.  Same arguments, layouts, results (bit
 * for bit) and errors as olmo3_attn_decode, without workspace and
 * workspace_bytes; the call makes no allocation.  A call whose
 * olmo3_workspace_bytes(OLMO3_MODE_DECODE, ...) exceeds
 * OLMO3_NOALLOC_SCRATCH_BYTES returns OLMO3_ERR_WORKSPACE and does nothing;
 * OLMO3_ERR_HIP if the scratch address of the current device cannot be
 * found.  Every call on one device uses that device's one array, and no
 * state carries from one call to the next: calls on one device that can
 * overlap in time (two streams, two host threads without ordering) race on
 * it and must be serialised by the caller. */
#define OLMO3_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int olmo3_attn_decode_noalloc(int B, int H, int G, int d, int window, int layer_type,
                              const olmo3_rope* rope, float eps, int64_t pos, int dtype,
                              const void* q_pre, const void* k_pre, const void* v,
                              const void* q_gain, const void* k_gain, void* k_cache,
                              void* v_cache, int64_t cache_capacity, void* out, void* stream);

/* Ragged batches: several prompts served together ("Olmo-3 End-to-End
 * Implementation", "Next Steps": batch processing), whose sequences differ in
 * length and position.  Per-sequence values live in DEVICE int32 arrays (they stay
 * on the GPU between steps); the host passes bounds that size the launch
 * and the checks.  Device values that break the stated bounds leave the
 * affected sequences' outputs and cache rows unspecified, but no kernel
 * reads or writes outside the buffers the host arguments describe. */

/* Ragged prefill: B sequences packed row after row.  Sequence b owns rows
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 of q_pre [n_tokens][H*d], k_pre and v
 * [n_tokens][G*d] and out [n_tokens][H*d]; its tokens sit at positions
 * pos_offsets[b] .. pos_offsets[b] + len_b - 1 (pos_offsets NULL: all 0) and
 * attend, as in olmo3_attn_prefill, to the positions its cache
 * k_cache[b] / v_cache[b] already holds and to each other.  Device arrays:
 * cu_seqlens [B+1] nondecreasing from 0 to n_tokens with every len_b <=
 * max_len; pos_offsets [B] >= 0 with pos_offsets[b] + len_b <= max_end.
 * workspace: olmo3_workspace_bytes(OLMO3_MODE_PREFILL, 1, n_tokens, ...).
 * Errors: as olmo3_attn_prefill with positions up to max_end - 1 (a linear
 * cache needs max_end slots), plus INVALID_ARG for B, n_tokens or max_len
 * < 1, max_len > n_tokens, max_end < max_len, a null or misaligned
 * cu_seqlens, a misaligned pos_offsets. */
int olmo3_attn_prefill_ragged(int B, int n_tokens, int max_len, int64_t max_end, int H, int G,
                              int d, int window, int layer_type, const olmo3_rope* rope,
                              float eps, const int32_t* cu_seqlens, const int32_t* pos_offsets,
                              int dtype, const void* q_pre, const void* k_pre, const void* v,
                              const void* q_gain, const void* k_gain, void* k_cache,
                              void* v_cache, int64_t cache_capacity, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Ragged decode: as olmo3_attn_decode, but sequence b's new token sits at
 * positions[b] (device int32 [B], each in [0, max_pos]); each sequence reads
 * its own min(positions[b]+1, window) ring slots or positions[b]+1 linear
 * slots.  Errors: as olmo3_attn_decode at pos = max_pos, plus INVALID_ARG for
 * a null or misaligned positions array or max_pos outside [0, 2^31). */
int olmo3_attn_decode_ragged(int B, int H, int G, int d, int window, int layer_type,
                             const olmo3_rope* rope, float eps, const int32_t* positions,
                             int64_t max_pos, int dtype, const void* q_pre, const void* k_pre,
                             const void* v, const void* q_gain, const void* k_gain,
                             void* k_cache, void* v_cache, int64_t cache_capacity, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- e4m3 key/value caches ----------------------------------------------
 * Half the cache bytes of bf16, for decode, which streams the cache ("Olmo-3
 * End-to-End Implementation", "Next Steps" lists quantization; "Olmo 3 7B",
 * "SERVICEABILITY JOIN" records that sliding-window layers with a quantized
 * cache break when the scales are applied twice or the window position is
 * mishandled).  A cache element is one byte, an OCP e4m3 code c (sign, 4
 * exponent bits with bias 7, 3 mantissa bits, largest finite 448, no
 * infinities); it stands for c * k_scale in k_cache and c * v_scale in
 * v_cache.  A key or value x is stored as the code nearest to the fp32
 * product x * fp32(1/scale) (ties to the even mantissa; magnitudes past 448,
 * infinities included, saturate to the code of +-448; a NaN is stored as a
 * NaN code, 0x7F or 0xFF), keys taken after QK-norm and RoPE in fp32.
 * Activations are bf16.  Layouts, slots and
 * errors as the bf16 entry points, with 1-byte cache elements; scales must
 * be finite and > 0 (INVALID_ARG). */

/* Append keys and values to e4m3 caches (as olmo3_kv_append). */
int olmo3_kv_append_e4m3(int B, int T, int G, int d, int window, int layer_type,
                         const olmo3_rope* rope, float eps, int64_t pos_offset, const void* k_pre,
                         const void* v, const void* k_gain, void* k_cache, void* v_cache,
                         float k_scale, float v_scale, int64_t cache_capacity, void* stream);

/* Prefill of positions pos_offset .. pos_offset+T-1 into e4m3 caches (as
 * olmo3_attn_prefill): the attention uses the chunk's own rotated keys and
 * values at bf16 precision and, when pos_offset > 0, the positions the cache
 * already holds as stored (code * scale, rounded to bf16: the library first
 * copies the ring, or rows 0 .. pos_offset-1 of a linear cache, into the
 * workspace); the cache then receives the chunk's codes.  workspace:
 * olmo3_workspace_bytes(OLMO3_MODE_PREFILL, ..., OLMO3_DTYPE_BF16_E4M3,
 * cache_capacity) bytes (with cache_capacity = 0 when pos_offset = 0). */
int olmo3_attn_prefill_e4m3(int B, int T, int H, int G, int d, int window, int layer_type,
                            const olmo3_rope* rope, float eps, int64_t pos_offset,
                            const void* q_pre, const void* k_pre, const void* v,
                            const void* q_gain, const void* k_gain, void* k_cache,
                            void* v_cache, float k_scale, float v_scale, int64_t cache_capacity,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Decode against e4m3 caches: the new token's key and value are stored as
 * codes first, then the query attends to the cache rows as stored (the new
 * token's included), as olmo3_attn_decode does.  Requires d = 128 and
 * H/G <= 8 (UNSUPPORTED otherwise).  The _phases form takes the phase bits
 * of olmo3_attn_decode_phases. */
int olmo3_attn_decode_e4m3(int B, int H, int G, int d, int window, int layer_type,
                           const olmo3_rope* rope, float eps, int64_t pos, const void* q_pre,
                           const void* k_pre, const void* v, const void* q_gain,
                           const void* k_gain, void* k_cache, void* v_cache, float k_scale,
                           float v_scale, int64_t cache_capacity, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);
int olmo3_attn_decode_e4m3_phases(int phases, int B, int H, int G, int d, int window,
                                  int layer_type, const olmo3_rope* rope, float eps, int64_t pos,
                                  const void* q_pre, const void* k_pre, const void* v,
                                  const void* q_gain, const void* k_gain, void* k_cache,
                                  void* v_cache, float k_scale, float v_scale,
                                  int64_t cache_capacity, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Ragged first chunks into e4m3 caches: B prompts packed row after row
 * (cu_seqlens as olmo3_attn_prefill_ragged, each sequence at positions
 * 0 .. len_b - 1, no earlier positions), attended at bf16 precision as
 * olmo3_attn_prefill_e4m3 does, their keys and values stored as codes.
 * Later chunks of one sequence: olmo3_attn_prefill_e4m3 with its offset.
 * workspace: olmo3_workspace_bytes(OLMO3_MODE_PREFILL, 1, n_tokens, ...,
 * OLMO3_DTYPE_BF16_E4M3, 0).  Errors: as olmo3_attn_prefill_ragged with
 * max_end = max_len, plus INVALID_ARG for scales as the e4m3 entry points. */
int olmo3_attn_prefill_ragged_e4m3(int B, int n_tokens, int max_len, int H, int G, int d,
                                   int window, int layer_type, const olmo3_rope* rope, float eps,
                                   const int32_t* cu_seqlens, const void* q_pre,
                                   const void* k_pre, const void* v, const void* q_gain,
                                   const void* k_gain, void* k_cache, void* v_cache,
                                   float k_scale, float v_scale, int64_t cache_capacity, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Ragged decode against e4m3 caches: olmo3_attn_decode_ragged's positions
 * (sequence b's new token at positions[b], each in [0, max_pos]) with
 * olmo3_attn_decode_e4m3's cache format and scales.  workspace:
 * olmo3_workspace_bytes(OLMO3_MODE_DECODE, ..., OLMO3_DTYPE_BF16_E4M3,
 * cache_capacity).  Errors: as those two. */
int olmo3_attn_decode_ragged_e4m3(int B, int H, int G, int d, int window, int layer_type,
                                  const olmo3_rope* rope, float eps, const int32_t* positions,
                                  int64_t max_pos, const void* q_pre, const void* k_pre,
                                  const void* v, const void* q_gain, const void* k_gain,
                                  void* k_cache, void* v_cache, float k_scale, float v_scale,
                                  int64_t cache_capacity, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Stage-by-stage variants, for callers that time or overlap the kernels of
 * one call.  `phases` is a bit set of:
 *   OLMO3_PHASE_PROLOGUE  (1)  QK-norm + RoPE of the new tokens, cache
 *                              append, rotated queries (and, on sliding
 *                              prefill, keys) written to the workspace;
 *   OLMO3_PHASE_ATTENTION (2)  attention reading the workspace and cache;
 *                              for decode, the split-KV partial states;
 *                              on a sliding-layer prefill with
 *                              pos_offset > 0, also the ring append, which
 *                              must follow the attention;
 *   OLMO3_PHASE_MERGE     (4)  decode only: log-sum-exp merge of the
 *                              partial states into out (a no-op when the
 *                              decode path needs no merge).
 * All phases together equal olmo3_attn_prefill / olmo3_attn_decode.  A later
 * phase must follow the earlier ones on the same stream with the same
 * arguments and workspace.  Arguments are validated as for the full call;
 * phases == 0 or unknown bits: INVALID_ARG. */
enum { OLMO3_PHASE_PROLOGUE = 1, OLMO3_PHASE_ATTENTION = 2, OLMO3_PHASE_MERGE = 4 };

int olmo3_attn_prefill_phases(int phases, int B, int T, int H, int G, int d, int window,
                              int layer_type, const olmo3_rope* rope, float eps,
                              int64_t pos_offset, int dtype, const void* q_pre,
                              const void* k_pre, const void* v, const void* q_gain,
                              const void* k_gain, void* k_cache, void* v_cache,
                              int64_t cache_capacity, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

int olmo3_attn_decode_phases(int phases, int B, int H, int G, int d, int window,
                             int layer_type, const olmo3_rope* rope, float eps, int64_t pos,
                             int dtype, const void* q_pre, const void* k_pre, const void* v,
                             const void* q_gain, const void* k_gain, void* k_cache,
                             void* v_cache, int64_t cache_capacity, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code; never NULL. */
const char* olmo3_status_string(int status);

/* OLMO3_ABI_VERSION of the built library. */
int olmo3_abi_version(void);

/* ---- Test probes (not part of the user API) ----------------------------
 * They run the prefill kernel's own tile enumeration and mask predicate, or
 * the decode kernel's own split / row enumeration, and record what those
 * visit, so that indexing can be compared bit for bit with the oracle.  */

/* visit [T][pos_offset + T] uint8 (device): entry (t, s) counts how many
 * times the d = 128 bf16 prefill kernel would accumulate the pair of query
 * position pos_offset + t and key position s (1 for every visible pair when
 * each is taken once; the probe clears the table first).  kv_splits 1: one
 * workgroup per query block; 2: the key-split instance (both workgroups of
 * a block counted together).  Any other kv_splits: INVALID_ARG.  T <= 4096, pos_offset + T <= 8192.
 * Errors: INVALID_ARG, UNSUPPORTED. */
int olmo3_probe_prefill_visits(int T, int64_t pos_offset, int window, int layer_type,
                               int kv_splits, uint8_t* visit, void* stream);

/* work [n][4] int32 (host memory; no device is touched): the (sequence,
 * head, query block, key split) that each workgroup of the d = 128 prefill
 * kernel over B uniform sequences of T queries at pos_offset takes, in
 * workgroup order, as the kernel computes it (same functions): n =
 * ceil(T / 128) * H * B workgroups with kv_splits 1, twice that with
 * kv_splits 2 (the key-split instance; split 0 or 1, else 0).  work_len: the
 * array's length in int32 (at least 4 n).  ABI version 11.
 * Errors: INVALID_ARG (shapes, layer type, kv_splits other than 1 or 2, a
 * null or short array), UNSUPPORTED (more than 2^24 workgroups). */
int olmo3_probe_prefill_order(int B, int T, int H, int G, int window, int layer_type,
                              int64_t pos_offset, int kv_splits, int32_t* work, int64_t work_len);

/* count [cache_capacity] int32 (device): number of times the decode kernel
 * at position `pos` reads each cache slot of one (sequence, KV head) into
 * its result, for the split count it would choose for batch B, H query and G
 * key/value heads, and cache element type `dtype` (OLMO3_DTYPE_BF16 or
 * OLMO3_DTYPE_BF16_E4M3): the row walk of the kernel those select (the
 * grouped MFMA kernel for bf16 caches with H/G >= 2, else the per-row one).
 * Errors: INVALID_ARG, CAPACITY.  */
int olmo3_probe_decode_reads(int B, int H, int G, int d, int window, int layer_type,
                             int dtype, int64_t pos, int64_t cache_capacity,
                             int32_t* count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OLMO3_ATTN_H */
