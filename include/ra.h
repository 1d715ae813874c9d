/*
 * ra.h -- C ABI of librocring: one rank's lap of ring attention on one MI355X (gfx950).
 *
 * The operation, as the pages state it ("Ring Attention：把超长序列沿设备环流动",
 * charlestar.github.io, section 环是怎样工作的, the forward loop):
 *
 *     state = empty online-softmax state for the local queries Q_r    -> ra_state_init
 *     for each of the P KV blocks of the lap:
 *         partial attention of Q_r against the block, merged into     -> ra_block_step
 *         the state by the online-softmax rescale
 *     local output = finalize(state)                                  -> ra_finalize
 *
 * The per-row state is the running maximum m, the running exponential sum l and the
 * unnormalised output O~ ("GPU ring attention", aicassindra.com, section "Why partial
 * results are allowed to merge"): when a block arrives both accumulators are rescaled by
 * exp(old max - new max) and the block's contribution is added; after the lap
 * O = O~ / l is exact softmax(scale * Q K^T) V over every allowed key.
 *
 * Masks are on global token positions.  Local query row i of this rank sits at global
 * position  q_offset + i * s  and key t of the arriving block at  k_offset + t * s,
 * where s = 1 for RA_MASK_NONE and RA_MASK_CAUSAL_CONTIGUOUS and s = ring_size for
 * RA_MASK_CAUSAL_STRIPED (token t lives on rank t mod P).  The causal rule is: query
 * position q may see key position k iff k <= q (same page, section Causal Attention
 * 让环不再完全对称; positions are global, section 位置编码必须使用全局位置).  For a contiguous
 * layout rank r passes q_offset = r * q_len and block j k_offset = j * kv_len; for the
 * striped layout q_offset = r and k_offset = j.  Offsets are ignored for RA_MASK_NONE.
 *
 * RA_MASK_CAUSAL_ZIGZAG is the paired layout of "GPU ring attention", section "Striping
 * the sequence to flatten the triangle": the sequence is cut into 2P chunks of c tokens
 * and rank r holds chunk r followed by chunk 2P-1-r, so local row i < c sits at position
 * r*c + i and row c + i at (2P-1-r)*c + i; a KV block from rank j is laid out the same
 * way.  Then q_len = kv_len = 2c, q_offset = r and k_offset = j (ranks in [0, P), P =
 * desc.ring_size).  A step runs as up to four contiguous causal sub-blocks (query chunk x
 * key chunk); a chunk pair wholly in the future is skipped like an empty block.
 *
 * Fully masked work is skipped at two granularities ("GPU ring attention", section
 * "Striping the sequence to flatten the triangle"; charlestar page, Causal section,
 * strictly-future / diagonal-crossing / unmasked rule): a block with no allowed pair
 * launches nothing, and inside a launch a (query tile, key tile) with no allowed pair is
 * never loaded or computed; only tiles that cross the diagonal apply the element mask.
 *
 * Conventions for every entry point
 *  - Tensors are row-major with the head dimension contiguous.  Q_r is addressed as
 *    Q[b*qs0 + h*qs1 + i*qs2 + c] (strides in elements, desc.q_strides), K_j and V_j as
 *    K[b*ks0 + g*ks1 + t*ks2 + c] (desc.kv_strides, shared by K and V).  Query head h
 *    reads KV head g = h / (q_heads / kv_heads) (contiguous GQA groups).
 *  - All device pointers are caller-owned device memory (e.g. allocated by torch);
 *    the library never allocates or frees device memory.  Host pointers are marked.
 *  - All device work is enqueued asynchronously on desc.stream (a hipStream_t; NULL is
 *    the null stream).  Device faults surface at the caller's next synchronisation.
 *  - The state, forward, decode, finalize, merge and backward calls only launch kernels on
 *    desc.stream: no allocation, memset, event or synchronisation.  A lap of them can be
 *    captured in a HIP graph once its buffers exist.  Host-side state (the fresh flag, the
 *    planner's counts) advances at capture, so a graph captured from a fresh state
 *    recomputes the whole lap on every replay.  ra_ring_lap_emulated uses events, a second
 *    stream and, with poison set, memsets.
 *  - Return value: RA_OK (0) or a negative RA_E_* code; nothing is enqueued on error.
 *    No C++ exception crosses the ABI.  ra_status_string() gives the text, including
 *    the HIP error for RA_E_HIP (kept per host thread).
 *  - One ra_state is driven by one host thread and one stream at a time.
 */
#ifndef RA_H_
#define RA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------- */
#define RA_OK 0
#define RA_E_INVALID (-1)     /* null pointer, bad dimension, q_heads % kv_heads != 0, bad stride or alignment */
#define RA_E_UNSUPPORTED (-2) /* head_dim or dtype without a compiled kernel, a form a call does not
                                 take, or more tiles than one launch holds (2^32 work-items) */
#define RA_E_STATE (-3)       /* step or finalize on a finalized state, double finalize */
#define RA_E_HIP (-4)         /* a HIP runtime call or kernel launch failed */

/* ---- enums ----------------------------------------------------------------------- */
typedef enum {
  RA_MASK_NONE = 0,               /* every key of every block is allowed */
  RA_MASK_CAUSAL_CONTIGUOUS = 1,  /* k <= q, positions offset + index (stride 1) */
  RA_MASK_CAUSAL_STRIPED = 2,     /* k <= q, positions offset + index * ring_size */
  RA_MASK_CAUSAL_ZIGZAG = 3       /* k <= q, rank r holds chunks r and 2P-1-r of 2P */
} ra_mask_kind;

typedef enum {
  RA_DTYPE_BF16 = 0,  /* Q, K, V in bfloat16; MFMA with fp32 accumulation */
  RA_DTYPE_F32 = 1    /* Q, K, V in float32; all arithmetic in fp32 (exactness path) */
} ra_dtype;

/* Tile classes reported by ra_tile_classes (same values as the oracle's enumeration). */
#define RA_TILE_EMPTY 0
#define RA_TILE_FULL 1
#define RA_TILE_PARTIAL 2

/* ---- descriptors ----------------------------------------------------------------- */
typedef struct ra_desc {
  int32_t batch;          /* B >= 1 */
  int32_t q_heads;        /* Hq >= 1 */
  int32_t kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t q_len;          /* local query rows n >= 0 (any length; a ragged tail is fine) */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t dtype;          /* ra_dtype of Q, K and V; the state is always fp32 */
  float softmax_scale;    /* 0 selects 1/sqrt(head_dim) */
  int32_t ring_size;      /* P >= 1: position stride of RA_MASK_CAUSAL_STRIPED */
  int64_t q_strides[3];   /* (batch, head, token) strides of Q_r in elements */
  int64_t kv_strides[3];  /* (batch, head, token) strides of K_j and V_j in elements */
  void* stream;           /* hipStream_t for all enqueued work */
} ra_desc;

/* Counts, summed over every (batch, query head) a launch covers.  live_pairs counts
 * allowed (query, key) pairs, so useful FLOPs = 4 * head_dim * live_pairs. */
typedef struct ra_stats {
  int64_t live_pairs;
  int64_t tiles_full;      /* (query tile, key tile) pairs computed without a mask */
  int64_t tiles_partial;   /* computed with the element mask (tile crosses the diagonal) */
  int64_t tiles_empty;     /* skipped: no allowed pair */
  int64_t blocks_run;      /* ra_block_step calls that launched the step kernel */
  int64_t blocks_skipped;  /* ra_block_step calls whose block held no allowed pair */
  int32_t tile_q;          /* query rows per tile of the kernel that runs this desc */
  int32_t tile_k;          /* keys per tile */
} ra_stats;

typedef struct ra_state ra_state; /* opaque, host-side, owned by the library */

/* ---- state buffer ---------------------------------------------------------------- */

/* Bytes of device workspace that holds the state (O~, m, l) for desc; 0 if desc is
 * invalid or q_len == 0.  Layout (all fp32, 256-byte aligned sections):
 *   O~ [B, Hq, n, d] at offset 0, m [B, Hq, n], l [B, Hq, n] at the offsets that
 *   ra_workspace_layout reports.  m is kept in base-2 units: with x = log2(e) * scale *
 *   <q, k> over the keys seen, m is a reference point and l = sum 2^(x - m),
 *   O~ = sum 2^(x - m) v.  The kernels keep max x - 32 <= m <= max x, so every term stays
 *   <= 2^32; a row that has seen no key holds m = -inf, l = 0, O~ = 0. */
size_t ra_workspace_bytes(const ra_desc* desc);

/* Byte offsets of O~, m and l inside the workspace (host out-pointers, any may be NULL). */
int ra_workspace_layout(const ra_desc* desc, size_t* o_off, size_t* m_off, size_t* l_off);

/* ---- the lap ----------------------------------------------------------------------- */

/* Bind the resident query slice Q_r (device, dtype desc.dtype) and a workspace of
 * ra_workspace_bytes(desc) device bytes to a new state with m = -inf, l = 0, O~ = 0.
 * Nothing is enqueued: the empty state is written by the first step that runs (or by
 * ra_finalize if none runs), so the workspace may hold garbage until then.
 * Q_r must stay valid and unchanged until ra_finalize's work has completed; the
 * workspace belongs to the state until ra_state_destroy.  *out receives a host
 * object to release with ra_state_destroy. */
int ra_state_init(const ra_desc* desc, const void* q, void* workspace, ra_state** out);

/* Like ra_state_init, but the workspace already holds a valid state (a checkpoint of a
 * partial lap, e.g. a copy of another state's workspace); the lap continues from it. */
int ra_state_resume(const ra_desc* desc, const void* q, void* workspace, ra_state** out);

/* Score Q_r against one KV block of kv_len >= 0 keys (device K_j, V_j of dtype
 * desc.dtype, strides desc.kv_strides) under mask_kind with the block's position
 * offsets, and merge the result into the state.  A block with no allowed pair returns
 * RA_OK without launching (counted in blocks_skipped).  K_j and V_j are read by work
 * enqueued on desc.stream: the caller must not overwrite them until that work has
 * completed (record an event after this call).  For bf16 blocks of at least 4096 keys a short
 * pass first bounds the largest key norm of every 32-key tile (Cauchy-Schwarz then lets the
 * step kernel skip its per-score guard on the reference): the state keeps those bounds in a
 * device buffer of its own, 4 bytes per 32 keys per (batch, KV head), allocated on the first
 * such call and grown when a longer block comes.  Under stream capture it is never grown; a
 * block it does not fit is then stepped without bounds, with the same result. */
int ra_block_step(ra_state* st, const void* k, const void* v, int32_t kv_len,
                  int32_t mask_kind, int64_t q_offset, int64_t k_offset);

/* O_r = O~ / l, written as fp32 [B, Hq, n, d] contiguous (device), and, if lse is not
 * NULL, lse = ln(sum over allowed keys of exp(scale * <q,k>)) as fp32 [B, Hq, n]
 * contiguous (device).  Rows that saw no allowed key give O = 0 and lse = -inf.
 * Afterwards the state accepts no more steps (RA_E_STATE); a second finalize is also
 * RA_E_STATE. */
int ra_finalize(ra_state* st, float* o, float* lse);

/* Release the host object and the state's key-tile norm buffer, if ra_block_step made one
 * (hipFree, which waits for the device first).  Enqueues nothing; the workspace is the
 * caller's. */
int ra_state_destroy(ra_state* st);

/* Host-side counts accumulated by the planner over this state's steps. */
int ra_get_stats(const ra_state* st, ra_stats* out);

/* Debug: when counters is a device pointer to 5 zeroed uint64 values, every later
 * ra_block_step of this state runs the counting variant of its kernel, which adds
 * (atomically, on the device) [0] the tiles it computed unmasked, [1] the tiles it computed
 * masked, [2] the allowed pairs it actually scored and [3] the (query row, key tile) events
 * in which a row that already held keys moved its reference m, rescaling l and O~ by
 * 2^(m_old - m_new) ("Ring attention" MCQ page, body: the running output is rescaled by
 * exp(old_max - new_max) when a new maximum appears), and [4] (bf16 only) the (wave of 64
 * query rows, key tile) events in which the tile's key-norm bound showed every score within
 * 2^32 of the reference, so that the scores' maximum was not taken.  ra_decode_step adds to
 * [3] only.
 * NULL switches counting off. */
int ra_state_set_debug_counters(ra_state* st, uint64_t* counters);

/* ---- reduction of shard states (split-KV decode) ---------------------------------- */

#define RA_MERGE_MAX_PARTS 64

/* Merge n_parts states of the same query rows, each over a disjoint set of keys, into one
 * ("Ring Attention：把超长序列沿设备环流动", section 训练与推理的适用方式不同: for decode the query is
 * sent to the KV shards, each computes a local attention state, and a global online-softmax
 * reduction combines them; the combination is the rescale-and-add of "GPU ring attention",
 * section "Why partial results are allowed to merge"):
 *     m = max_s m_s,   l = sum_s e^(m_s - m) l_s,   O~ = sum_s e^(m_s - m) O~_s.
 * parts: host array of n_parts (1 <= n_parts <= RA_MERGE_MAX_PARTS) device workspaces, each
 * laid out as ra_workspace_layout(desc) gives and holding a valid state of these rows: one
 * written by at least one launch of ra_block_step (ra_get_stats: blocks_run > 0); a state
 * whose blocks were all skipped holds nothing yet and must be left out.  Outputs (device,
 * each may be NULL but not both merged and o): merged, a workspace (256-byte aligned, it may
 * be one of the parts) that receives the merged state, and o / lse, which receive
 * O = O~ / l and lse exactly as ra_finalize would write them for the merged state (lse only
 * together with o).  Enqueued on desc.stream. */
int ra_merge_states(const ra_desc* desc, int32_t n_parts, void* const* parts, void* merged,
                    float* o, float* lse);

/* ---- the block step for a few query rows (split-KV) -------------------------------- */

/* Bytes of device workspace that ra_decode_step needs for a block of kv_len keys under desc
 * (0 if desc is invalid, q_len == 0 or kv_len == 0). */
size_t ra_decode_workspace_bytes(const ra_desc* desc, int32_t kv_len);

/* The same update of the state as ra_block_step (same arguments, same result up to the order
 * of fp32 rounding, same stats and skip rule), computed the way "Ring Attention：把超长序列沿设备
 * 环流动", section 训练与推理的适用方式不同, computes decode: the few query rows are sent to many
 * shards of the keys, each shard forms a local state (m, l, O~), and a global online-softmax
 * reduction combines the local states with the running state.  Here the shards are chunks of
 * K_j/V_j, one wave of the chip each (several waves of one workgroup share a chunk when a KV
 * head has more than 32 packed rows), so a block is streamed by the whole chip even when
 * B * Hq * q_len is far below one 128-row tile; the query heads of a GQA group are packed into
 * one wave.  Meant for short Q (decode, q_len up to a few tens); any q_len is accepted.
 * workspace: device, 256-byte aligned, at least ra_decode_workspace_bytes(desc, kv_len)
 * bytes (workspace_bytes says how many the caller passed); it holds the chunk states and is
 * free again once the enqueued work has completed.  fp32 inputs take the exactness path: the
 * call is ra_block_step's (the workspace is not used).  Errors: RA_E_UNSUPPORTED for
 * RA_MASK_CAUSAL_ZIGZAG; RA_E_INVALID for a missing or short workspace and everything
 * ra_block_step rejects. */
int ra_decode_step(ra_state* st, const void* k, const void* v, int32_t kv_len,
                   int32_t mask_kind, int64_t q_offset, int64_t k_offset, void* workspace,
                   size_t workspace_bytes);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ra_decode_step with the chunk states in
 * a scratch array the library holds per device (RA_DECODE_NOALLOC_MAX_BYTES, created with
 * the library's code object on each device it runs on and held until the process ends)
 * instead of a caller workspace.  Same arguments, result and errors as ra_decode_step,
 * plus RA_E_UNSUPPORTED when ra_decode_workspace_bytes(desc, kv_len) exceeds the array.
 * The device is desc.stream's.  The call allocates nothing; its first call on a device
 * looks up that device's array (hipGetSymbolAddress).  Every call on a device shares that
 * device's array, which keeps the last call's contents (nothing in it needs clearing: each
 * call writes every chunk state before reading it), so calls whose work overlaps on one
 * device (other streams, other host threads) race: serialise them. */
#define RA_DECODE_NOALLOC_MAX_BYTES (64u << 20)
int ra_decode_step_noalloc(ra_state* st, const void* k, const void* v, int32_t kv_len,
                           int32_t mask_kind, int64_t q_offset, int64_t k_offset);

/* ---- backward of the lap ------------------------------------------------------------ */

/* The backward pass runs the same lap with gradients travelling too ("Ring Attention：把超长序
 * 列沿设备环流动", section Backward 需要让梯度也沿环传播): the query owner accumulates dQ_r over every
 * KV block; the travelling block carries dK_j, dV_j, to which every query owner it passes
 * adds its contribution; the probabilities are recomputed per block from the forward's saved
 * per-row logsumexp.  With P = exp(scale * <q, k> - lse) on allowed pairs (the standard
 * gradient of softmax attention, not printed on the page):
 *     D = rowsum(dO * O),  dV_j += P^T dO,  dS = P * (dO V_j^T - D),
 *     dQ += scale * dS K_j,  dK_j += scale * dS^T Q.
 * Query head h adds to KV head h / (q_heads / kv_heads), as in the forward. */
typedef struct ra_bwd ra_bwd;   /* opaque host object */

/* Bytes of the backward workspace: the fp32 dQ accumulator [B, Hq, n, d] and D [B, Hq, n]. */
size_t ra_bwd_workspace_bytes(const ra_desc* desc);

/* Bind the backward of one rank's lap.  q: Q_r as for ra_state_init; d_out: dO_r, the
 * gradient of the forward output, in desc.dtype with Q_r's strides; out and lse: O_r and
 * lse_r as ra_finalize wrote them (fp32 contiguous, device); workspace: device,
 * 256-byte aligned, ra_bwd_workspace_bytes(desc) bytes.  Enqueues D = rowsum(dO * O) and
 * clears the dQ accumulator.  All of them must stay valid until ra_bwd_finalize. */
int ra_bwd_init(const ra_desc* desc, const void* q, const void* d_out, const float* out,
                const float* lse, void* workspace, ra_bwd** out_handle);

/* One backward ring step against KV block (k, v), with the block's travelling gradients dk,
 * dv (fp32 device [B, Hkv, kv_len, d] contiguous, accumulated into: they start at zero where
 * the block begins its lap).  kv_len, mask_kind and the offsets are those of the forward
 * ra_block_step for the same block; a block with no allowed pair launches nothing. */
int ra_bwd_block_step(ra_bwd* st, const void* k, const void* v, float* dk, float* dv,
                      int32_t kv_len, int32_t mask_kind, int64_t q_offset, int64_t k_offset);

/* dQ_r = the accumulated gradient, fp32 [B, Hq, n, d] contiguous (device).  Afterwards the
 * state takes no more steps (RA_E_STATE). */
int ra_bwd_finalize(ra_bwd* st, float* dq);

/* Host-side counts over this backward's steps (live pairs, blocks run and skipped). */
int ra_bwd_get_stats(const ra_bwd* st, ra_stats* out);

/* Release the host object. */
int ra_bwd_destroy(ra_bwd* st);

/* ---- host-only planner (no device work; safe without a GPU) ------------------------ */

/* What ra_block_step would do for this block, as counts for the whole launch. */
int ra_plan_block(const ra_desc* desc, int32_t kv_len, int32_t mask_kind,
                  int64_t q_offset, int64_t k_offset, ra_stats* out);

/* Class of every (query tile, key tile) of one head for this block, row-major
 * [ceil(q_len/tile_q)][ceil(kv_len/tile_k)] into host memory host_out of cap bytes,
 * using the kernel's own tile sizes (reported by ra_plan_block).  For
 * RA_MASK_CAUSAL_ZIGZAG the tiles follow the chunks: [2*ceil(c/tile_q)][2*ceil(c/tile_k)]
 * with c = q_len / 2, the first half of each axis covering the first chunk. */
int ra_tile_classes(const ra_desc* desc, int32_t kv_len, int32_t mask_kind,
                    int64_t q_offset, int64_t k_offset, uint8_t* host_out, size_t cap);

/* ---- emulated ring on one GPU ----------------------------------------------------- */

/* One whole lap for rank `rank` of a ring of desc.ring_size ranks, on one GPU.  The P
 * blocks sit in device memory (k_blocks[j], v_blocks[j]: host arrays of P device
 * pointers, each block kv_len keys in desc.kv_strides layout and block_bytes bytes
 * contiguous).  Step 0 uses the rank's own block in place; for every later step the
 * block (rank - s) mod P is copied into one of two receive buffers with hipMemcpyAsync
 * on side_stream while the previous step's kernel runs on desc.stream; events order
 * copy-after-consume and compute-after-arrival ("GPU ring attention", section "Hiding the
 * ring behind the GEMMs"; charlestar page, section 双缓冲是重叠成立的基础).  Every block is
 * received, as a ring rank forwards each one; a block that no query of the rank sees
 * launches nothing, and its buffer is free again as soon as it has landed.
 * recv_k[2], recv_v[2] are the receive buffers (block_bytes each).  Positions follow
 * mask_kind (contiguous: rank * q_len and j * kv_len; striped and zigzag: rank and j).
 * Writes O and lse as ra_finalize does; stats_out (host, may be NULL) receives the lap's
 * counts.  The workspace is used as the state.  Events are created and destroyed per
 * call. */
typedef struct ra_lap {
  const void* const* k_blocks;  /* host array [P] of device pointers */
  const void* const* v_blocks;  /* host array [P] of device pointers */
  void* recv_k[2];              /* device receive buffers */
  void* recv_v[2];
  size_t block_bytes;           /* bytes copied per K (and per V) block */
  int32_t rank;                 /* 0 <= rank < P */
  int32_t kv_len;               /* keys per block */
  int32_t mask_kind;
  int32_t poison;               /* nonzero: fill each receive buffer with NaN before its copy */
  void* side_stream;            /* hipStream_t for the emulated transfers */
  void* const* step_events;     /* NULL, or host array [2P] of hipEvent_t created by the caller:
                                   [2s] is recorded on desc.stream just before step s's kernel
                                   (after its wait for the block) and [2s+1] just after it */
  const int32_t* kv_valid;      /* NULL, or host array [P]: block j's first kv_valid[j] keys
                                   (0 <= kv_valid[j] <= kv_len) are real tokens and the rest of
                                   its kv_len slots are padding that no query sees: the shards
                                   of an N that P does not divide, each padded to kv_len =
                                   ceil(N/P) slots ("Ring Attention：把超长序列沿设备环流动", section
                                   正确性测试应覆盖哪些边界: tail-rank padding with a valid-length
                                   mask).  Positions keep the padded slots (contiguous: block j
                                   starts at j * kv_len), so Q_r is passed padded to the same
                                   q_len on every rank and the rows past a rank's real tokens
                                   are padding whose outputs mean nothing.  The whole block
                                   (block_bytes) still travels. */
} ra_lap;

int ra_ring_lap_emulated(const ra_desc* desc, const void* q, void* workspace,
                         const ra_lap* lap, float* o, float* lse, ra_stats* stats_out);

/* ---- misc ------------------------------------------------------------------------ */
const char* ra_status_string(int status);
int ra_version(void); /* ABI version, currently 1 */

#ifdef __cplusplus
}
#endif
#endif /* RA_H_ */
