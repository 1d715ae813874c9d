// ra_internal.h -- parameters shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Everything one step launch needs.  Strides are in elements; the head dimension is
// contiguous.  All position logic is already folded into `diag` (see ra_pos.h).  A launch
// covers rows [0, n_q) and keys [0, n_k) of what q, k, v, o_acc, m and l point at, which may
// be a sub-range of the state (the zigzag layout runs one launch per pair of chunks).
struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  float* o_acc;        // O~ [B, Hq, n_q, D]
  float* m;            // [B, Hq, n_q], base-2 units
  float* l;            // [B, Hq, n_q]
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int32_t batch, q_heads, kv_heads, group;  // group = q_heads / kv_heads
  int32_t n_q, n_k;     // query rows and keys of this launch
  int32_t state_rows;   // rows per (batch, head) in the state (>= n_q; the state pointers
                        // and q already point at this launch's first row)
  int32_t diag;        // key t is visible to row i iff t <= i + diag
  float scale_log2;    // softmax scale * log2(e)
  int32_t fresh;       // 1: the state has never been written; start from the empty state
  unsigned long long* dbg;  // optional device counters [5]: unmasked tiles, masked tiles, pairs,
                            // (row, tile) events where a row holding keys moved its reference,
                            // and (wave, tile) events decided by the key-norm bound (bf16)
  // optional (bf16 only): an upper bound of the largest key norm |k| of every 32-key tile of
  // this launch's keys (tile t = keys 32t .. 32t+31 after p.k), [B * Hkv][knorm_stride]; null:
  // no bound, every tile takes the per-score guard
  const float* knorm;
  int32_t knorm_stride;
  // Where the write-back goes: O~ (o_out = o_acc), or, when the lap's last step finalizes as
  // it writes back (bf16 only; finalize = 1), O = O~ / l to o_out (laid out like O~) and lse to
  // fin_lse (may be null) instead of O~, m and l to the state.  A finalizing launch must be one
  // in which every row sees a key, so that no workgroup returns early.
  float* o_out;
  float* fin_lse;
  int32_t finalize;
};

struct FinalizeParams {
  const float* o_acc;
  const float* m;
  const float* l;
  float* o;
  float* lse;          // may be null
  int64_t rows;        // B * Hq * n_q
  int32_t d;
  int32_t fresh;       // 1: no step ever ran; write the empty result without reading
};

// The reduction of shard states: every part is a workspace laid out like the state (O~ at
// byte 0, m at m_off, l at l_off); the merged state goes to `merged` (same layout) and/or
// O and lse to o, lse.  Null outputs are skipped.
constexpr int kMergeMaxParts = 64;
struct MergeParams {
  const char* parts[kMergeMaxParts];
  int32_t n_parts;
  size_t m_off, l_off;
  char* merged;
  float* o;
  float* lse;
  int64_t rows;        // B * Hq * n
  int32_t d;
};

// Split-KV step for a few query rows: the keys [0, n_k) of the block are cut into n_parts
// chunks of `chunk` keys; chunk s's local state of every row goes to part_o / part_m /
// part_l at [s, row], rows = B * Hq * n_q in the state's order.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  float* part_o;       // [n_parts, rows, D]
  float* part_m;       // [n_parts, rows], base 2
  float* part_l;       // [n_parts, rows]
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int32_t batch, q_heads, kv_heads, group;
  int32_t n_q, n_k;
  int32_t n_parts, chunk;
  int32_t diag;
  float scale_log2;
  unsigned long long* dbg_moves;  // optional device counter: rows holding keys that moved their reference
};

// Folds the parts of a split-KV step (and the state itself unless fresh) into the state.
struct CombineParams {
  const float* part_o;
  const float* part_m;
  const float* part_l;
  int32_t n_parts;
  float* o_acc;
  float* m;
  float* l;
  int64_t rows;
  int32_t d;
  int32_t fresh;
};

// Backward: D = rowsum(dO * O) for every row of the state, and the dQ accumulator cleared.
struct BwdPrepParams {
  const void* d_out;   // [B, Hq, n, d] in the input dtype, Q's strides
  const float* out;    // O from the forward finalize, fp32 [B, Hq, n, d] contiguous
  float* D;            // [B, Hq, n]
  float* dq;           // [B, Hq, n, d]
  int64_t q_sb, q_sh, q_st;
  int32_t q_heads, n_q;
  int64_t rows;        // B * Hq * n
};

// One backward launch: rows [0, n_q) of q, d_out, lse, D, dq (a sub-range of the state, of
// state_rows rows per head) against keys [0, n_k) of k, v, dk, dv (of dkv_rows keys per head).
struct BwdParams {
  const void* q;
  const void* d_out;
  const void* k;
  const void* v;
  const float* lse;    // natural-log logsumexp of the forward, [.., state_rows]
  const float* D;
  float* dq;           // fp32 [.., state_rows, d]
  float* dk;           // fp32 [B, Hkv, dkv_rows, d]
  float* dv;
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int32_t batch, q_heads, kv_heads, group;
  int32_t n_q, n_k, state_rows, dkv_rows;
  int32_t diag;
  float scale;
};

// Tile sizes of each kernel (the planner reports and classifies with these).
constexpr int kBf16TileQ = 256;
constexpr int kBf16TileK = 32;
constexpr int kF32TileQ = 64;
constexpr int kF32TileK = 32;
constexpr int kDecodeRows = 32;   // packed (query head, token) rows per wave of the split-KV step
constexpr int kDecodeTileK = 32;

hipError_t launch_step_bf16(const StepParams& p, int head_dim, hipStream_t stream);
// Upper bounds of the largest key norm of every 32-key tile of a bf16 K block [B, Hkv, n_k, d]
// (strides in elements, multiples of 8), written as out[(b * Hkv + h) * n_tiles + t] with
// n_tiles = ceil(n_k / 32); keys past n_k count as zero.
hipError_t launch_key_tile_norms(const void* k, int64_t k_sb, int64_t k_sh, int64_t k_st, int batch,
                                 int kv_heads, int n_k, int head_dim, float* out, hipStream_t stream);
hipError_t launch_step_f32(const StepParams& p, int head_dim, hipStream_t stream);
hipError_t launch_finalize(const FinalizeParams& p, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
// Workgroup shape of the split-KV step.  decode_kernel: R = 1 or 2 row groups, one wave each,
// sharing V tiles in LDS (S = 1).  decode_ring_kernel (ring): R row groups x S tile subsets in
// four waves that share an LDS ring of K and V tiles, each (part, subset) leaving its own
// partial state.  Two row groups take the ring only on long blocks: below kDecodeRingMinKeys
// visible keys more, smaller workgroups stream a short block faster than a deep ring.
struct DecodeShape {
  int R, S;
  bool ring;
};
constexpr int64_t kDecodeRingMinKeys = 131072;
inline DecodeShape decode_shape(int64_t row_groups, int64_t n_keys) {
  if (row_groups <= 1) return {1, 1, false};
  if (row_groups == 2) return n_keys < kDecodeRingMinKeys ? DecodeShape{2, 1, false} : DecodeShape{2, 2, true};
  return {4, 1, true};
}
hipError_t launch_decode(const DecodeParams& p, int head_dim, DecodeShape shape, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_bwd_prep(const BwdPrepParams& p, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_bwd_step_f32(const BwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_bwd_step_bf16(const BwdParams& p, int head_dim, hipStream_t stream);

}  // namespace ra
