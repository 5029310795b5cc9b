// Host-side launchers of the attention kernels and their argument blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace olmo3 {

// QK-norm + RoPE + cache append over token rows.
//   uniform batch: B*T rows, row = b*T + t, position pos_offset + t (or
//     seq_pos[b] + t when seq_pos is set: per-sequence positions);
//   packed (cu_seqlens set): n_rows rows, sequence b owns rows
//     cu_seqlens[b] .. cu_seqlens[b+1]-1, t = row - cu_seqlens[b], position
//     (seq_pos ? seq_pos[b] : 0) + t.
// Row t of a sequence of `len` rows is stored in the cache when `store` is
// set and len - t <= keep_last (a ring keeps the last `window` rows), at slot
// pos (linear; skipped if pos >= cap) or pos mod window (ring).
struct PrologueArgs {
  const void* q_pre;   // [rows][H*d] or null (keys/values only)
  const void* k_pre;   // [rows][G*d]
  const void* v;       // [rows][G*d]
  const void* q_gain;  // [H*d]
  const void* k_gain;  // [G*d]
  void* q_out;         // [rows][H][d] rotated queries (when q_pre is set)
  void* k_out;         // rotated keys at b*k_sb + g*k_sg + t*k_st (packed:
                       // g*k_sg + row*k_st), or null
  int64_t k_sb, k_sg, k_st;
  void* k_cache;       // [B][G][cap][d]
  void* v_cache;
  int64_t cap;
  int64_t pos_offset;
  int64_t keep_last;
  const int32_t* seq_pos;     // [B] device, or null
  const int32_t* cu_seqlens;  // [B+1] device, or null
  int64_t n_rows;             // packed rows
  int B, T, H, G;
  int window;
  int sliding;
  int store;
  float eps;
  // e4m3 caches (bf16 rows only): code = e4m3(value * inv_scale)
  int cache_fp8;
  float k_inv_scale, v_inv_scale;
  // the rotated queries are written times this factor: the MFMA prefill
  // kernel takes them times its base-2 softmax scale, so that its scores
  // leave the MFMAs scaled; 1 everywhere else (a product by 1 is exact)
  float q_scale = 1.0f;
};

hipError_t launch_prologue(const PrologueArgs& a, const RopeTable& rope, int dtype, int d,
                           hipStream_t s);
int prologue_max_heads(int dtype, int d);

// bf16 image of e4m3 cache rows: rows 0 .. n-1 of each of the BG
// (sequence, head) pairs of k_codes / v_codes ([BG][cap][d] codes) become
// k_out / v_out [BG][rows][d] with value code * scale (fp32 product rounded
// to bf16).  d must be a multiple of 16 and n <= min(rows, cap).
struct E4m3StageArgs {
  const void* k_codes;
  const void* v_codes;
  void* k_out;
  void* v_out;
  int64_t cap, rows, n;
  int BG, d;
  float k_scale, v_scale;
};
hipError_t launch_e4m3_rows_to_bf16(const E4m3StageArgs& a, hipStream_t s);

// Attention over keys held in up to two strided buffers.
//   queries  q[(b*Tq + t)*H + h][d], absolute position q_pos0 + t
//   keys at positions 0 .. n_keys-1:
//     position p >= main_pos0: main row r = p - main_pos0,
//       k + b*k_sb + g*k_sg + r*k_sr (v likewise)
//     position p < main_pos0 (prefix, only when kp is set): ring slot
//       p mod ring, kp + b*p_sb + g*p_sg + slot*p_sr (vp likewise)
//   prefill: the mask decides which positions a query sees;
//   decode (all_visible): every main row r < n_keys is visible.
//   out[(b*Tq + t)*H*d + h*d + e]
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t k_sb, k_sg, k_sr;
  int64_t v_sb, v_sg, v_sr;
  const void* kp;  // prefix keys and values (a sliding layer's ring), or null
  const void* vp;
  int64_t p_sb, p_sg, p_sr;
  int64_t ring;
  int64_t main_pos0;
  void* out;
  int B, Tq, H, G;
  int64_t n_keys;
  int64_t q_pos0;
  int window;
  int sliding;
  int all_visible;
  float scale_log2;  // log2(e) / sqrt(d)
  // Packed batch (cu_seqlens set): sequence b's queries are rows
  // cu_seqlens[b] .. cu_seqlens[b+1]-1 (at most Tq of them, rows < n_rows)
  // of q and out, at positions seq_pos[b] + t (0 + t without seq_pos); its
  // keys are positions 0 .. seq_pos[b] + len - 1: with main_packed the
  // positions from seq_pos[b] on are its packed rows (k_sb, v_sb unused) and
  // earlier ones come from the prefix ring; otherwise main row = position in
  // sequence b's buffer.  A sequence whose keys would pass key_limit is
  // skipped.  Decode (all_visible) with seq_pos: sequence b
  // reads main rows 0 .. n_b - 1, n_b = min(seq_pos[b]+1, window) on a ring,
  // seq_pos[b]+1 on a linear cache, at most key_limit.
  const int32_t* cu_seqlens;
  const int32_t* seq_pos;
  int64_t n_rows;
  int64_t key_limit;
  int main_packed;  // packed batch: main rows are the sequence's packed rows
                    // (main_pos0 = its first position) instead of b*k_sb rows
  // kv_splits > 1 (uniform batches without a prefix only): each query block's
  // key tiles are split over kv_splits workgroups, which write unnormalised
  // partial states part[((row*H + h)*kv_splits + split)*(d+2) ..] = (m, l,
  // o[d]) instead of out; the decode merge kernel then combines them.
  float* part;
  int kv_splits;
};

// Flash-style prefill, d = 128, bf16, MFMA.  Requires n_keys == q_pos0 + Tq
// < 2^30, and main_pos0 == 0 unless a prefix is given.
hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t s);
// Plain per-query kernel for the other head sizes and for fp32.
hipError_t launch_attn_generic(const AttnArgs& a, int dtype, int d, hipStream_t s);

// Split-KV decode, d = 128, bf16 or e4m3 caches: one workgroup per
// (b, g, split) reads the split's cache rows once for all H/G query heads and
// writes a partial softmax state (m, l, o[d]) per head to
// part[((b*H + h)*splits + sp)*(d+2)]; with splits == 1 it writes the output
// rows out[(b*H + h)*d ..] instead and no merge is needed.
struct DecodeArgs {
  const void* q;       // [B][H][d] rotated queries
  const void* k_cache; // [B][G][cap][d]
  const void* v_cache;
  int64_t cap;
  int64_t n;           // rows read: slots 0 .. n-1
  int64_t rows_per_split;
  float* part;
  void* out;           // [B][H*d]
  int B, H, G, splits;
  float scale_log2;
  // per-sequence positions (device [B]) or null: sequence b reads
  // n_b = min(seq_pos[b]+1, window) (ring) or seq_pos[b]+1 (linear) rows,
  // at most cap, split evenly over the `splits` workgroups
  const int32_t* seq_pos;
  int window;
  int sliding;
  // e4m3 caches: a row holds codes c, values c * k_scale (keys) and
  // c * v_scale (values)
  int fp8;
  float k_scale, v_scale;
};
int decode_splits(int B, int G, int64_t n);
hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s);

// Probes: the prefill kernel's tile walk and the decode kernel's row walk.
hipError_t launch_probe_prefill(int T, int64_t pos_offset, int window, int sliding, int kv_splits,
                                uint8_t* visit, hipStream_t s);
hipError_t launch_probe_decode(const DecodeArgs& a, int32_t* count, hipStream_t s);

}  // namespace olmo3
