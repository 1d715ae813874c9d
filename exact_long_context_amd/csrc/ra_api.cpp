// ra_api.cpp -- the C ABI (include/ra.h): argument validation, the block/tile planner
// and the launches of the step and finalize kernels.
//
// The planner is host-only arithmetic on the shared position algebra (ra_pos.h), so the
// same decisions the kernels take can be inspected without a GPU (ra_plan_block,
// ra_tile_classes).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/ra.h"
#include "ra_internal.h"
#include "ra_pos.h"

struct ra_state {
  ra_desc desc;
  const void* q;
  float* o_acc;
  float* m;
  float* l;
  int fresh;       // no step has written the workspace yet
  int finalized;
  ra_stats stats;
  unsigned long long* dbg;
  // bf16 blocks of at least kKeyNormMinKeys keys: bounds of the largest key norm per 32-key
  // tile, computed by a short pass before the step kernel so that it can skip its per-score
  // guard (device, owned by the state, grown on demand outside stream capture)
  float* knorm;
  size_t knorm_cap;   // floats
};

// The backward of one rank's lap: the resident Q_r and dO_r, the forward's lse_r, and the
// workspace holding the dQ accumulator and D = rowsum(dO * O).
struct ra_bwd {
  ra_desc desc;
  const void* q;
  const void* d_out;
  const float* lse;
  float* dq;
  float* D;
  int finalized;
  ra_stats stats;
};

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_bytes(int32_t dtype) { return dtype == RA_DTYPE_BF16 ? 2 : 4; }

int tile_q_of(const ra_desc* d) { return d->dtype == RA_DTYPE_BF16 ? ra::kBf16TileQ : ra::kF32TileQ; }
int tile_k_of(const ra_desc* d) { return d->dtype == RA_DTYPE_BF16 ? ra::kBf16TileK : ra::kF32TileK; }

// Checks a descriptor; the pointer checks are separate.
int check_desc(const ra_desc* d) {
  if (!d) return fail(RA_E_INVALID, "desc is NULL");
  if (d->batch < 1 || d->q_heads < 1 || d->kv_heads < 1)
    return fail(RA_E_INVALID, "batch, q_heads and kv_heads must be >= 1");
  if (d->q_heads % d->kv_heads)
    return fail(RA_E_INVALID, "q_heads (%d) is not a multiple of kv_heads (%d)", d->q_heads, d->kv_heads);
  if (d->q_len < 0) return fail(RA_E_INVALID, "q_len must be >= 0");
  if (d->ring_size < 1) return fail(RA_E_INVALID, "ring_size must be >= 1");
  if (d->dtype != RA_DTYPE_BF16 && d->dtype != RA_DTYPE_F32)
    return fail(RA_E_UNSUPPORTED, "dtype %d is not supported", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(RA_E_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (!(std::isfinite(d->softmax_scale) && d->softmax_scale >= 0.f))
    return fail(RA_E_INVALID, "softmax_scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  // vector loads need 16-byte aligned rows
  const int64_t vec = 16 / elem_bytes(d->dtype);
  for (int i = 0; i < 3; ++i) {
    if (d->q_strides[i] < 0 || d->kv_strides[i] < 0)
      return fail(RA_E_INVALID, "strides must be >= 0");
    if (d->q_strides[i] % vec || d->kv_strides[i] % vec)
      return fail(RA_E_INVALID, "strides must be multiples of %lld elements (16-byte rows)",
                  (long long)vec);
  }
  if (d->q_len > 1 && d->q_strides[2] < d->head_dim)
    return fail(RA_E_INVALID, "q token stride smaller than head_dim");
  // every launch over the query rows (64-row tiles at the smallest, 256 threads each) must
  // hold fewer than 2^32 work-items
  const int64_t q_tiles = ((int64_t)d->q_len + 63) / 64;
  if (q_tiles * d->q_heads * d->batch * 256 > 0xffffffffLL)
    return fail(RA_E_UNSUPPORTED, "%lld query tiles of 64 rows exceed one launch",
                (long long)(q_tiles * d->q_heads * d->batch));
  return RA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct Layout {
  size_t o_off, m_off, l_off, total;
};

Layout layout_of(const ra_desc* d) {
  const size_t rows = (size_t)d->batch * d->q_heads * d->q_len;
  Layout L;
  L.o_off = 0;
  L.m_off = align256(rows * d->head_dim * sizeof(float));
  L.l_off = L.m_off + align256(rows * sizeof(float));
  L.total = rows ? L.l_off + align256(rows * sizeof(float)) : 0;
  return L;
}

// A single token's stride never moves a pointer, but the kernels bound their buffer reads by
// tokens x stride bytes, so a lone row is reported with at least a full row's stride.
int64_t token_stride(int64_t stride, int32_t tokens, int32_t head_dim) {
  return tokens <= 1 && stride < head_dim ? head_dim : stride;
}

int32_t pos_stride(int32_t mask_kind, const ra_desc* d) {
  return mask_kind == RA_MASK_CAUSAL_STRIPED ? d->ring_size : 1;
}

// A block as launches see it: rows [row0, row0 + rows) of the state against keys
// [key0, key0 + keys) of the block, with every position fact folded into diag.  The
// single-range layouts give one sub-block.  The zigzag layout ("GPU ring attention",
// section "Striping the sequence to flatten the triangle": 2P chunks, rank r holds chunks
// r and 2P-1-r) gives four, one per (query chunk, key chunk): each is a contiguous causal
// block with its own diagonal, and a chunk pair wholly in the future is empty.
// Blocks shorter than this take the step kernel's full guard: they are bound by the state's
// HBM traffic, and the norm pass would add a launch for nothing.
constexpr int32_t kKeyNormMinKeys = 4096;

struct Sub {
  int32_t row0, rows, key0, keys, diag;
  int64_t pairs;   // allowed (row, key) pairs of one head
};

int64_t pairs_of(int32_t rows, int32_t keys, int32_t diag) {
  int64_t n = 0;
  for (int32_t i = 0; i < rows; ++i) n += ra::keys_visible(i, diag, keys);
  return n;
}

// Two sub-blocks of the same rows, b's keys right after a's, as one causal sub-block: possible
// when every row sees a prefix of the joined keys (b's keys only where all of a's are visible)
// and one diagonal gives every row's count.
bool merge_keys(const Sub& a, const Sub& b, Sub* m) {
  if (a.row0 != b.row0 || a.rows != b.rows || b.key0 != a.key0 + a.keys) return false;
  const int32_t diag = b.diag + a.keys;
  for (int32_t i = 0; i < a.rows; ++i) {
    const int32_t na = ra::keys_visible(i, a.diag, a.keys), nb = ra::keys_visible(i, b.diag, b.keys);
    if ((nb > 0 && na != a.keys) || ra::keys_visible(i, diag, a.keys + b.keys) != na + nb) return false;
  }
  *m = Sub{a.row0, a.rows, a.key0, a.keys + b.keys, diag, a.pairs + b.pairs};
  return true;
}

// A sub-block with the empty sub-block beside it (same rows, b's keys right after a's) taken
// in: possible when none of its rows sees b's keys under its own diagonal.
bool extend_keys(const Sub& a, const Sub& b, Sub* m) {
  if (a.row0 != b.row0 || a.rows != b.rows || b.key0 != a.key0 + a.keys || b.pairs != 0) return false;
  for (int32_t i = 0; i < a.rows; ++i)
    if (ra::keys_visible(i, a.diag, a.keys + b.keys) != ra::keys_visible(i, a.diag, a.keys)) return false;
  *m = Sub{a.row0, a.rows, a.key0, a.keys + b.keys, a.diag, a.pairs};
  return true;
}

// Two sub-blocks of the same keys, b's rows right after a's, as one: possible when a's
// diagonal, continued over b's rows, gives every one of them its own count.
bool merge_rows(const Sub& a, const Sub& b, Sub* m) {
  if (a.key0 != b.key0 || a.keys != b.keys || b.row0 != a.row0 + a.rows) return false;
  for (int32_t i = 0; i < b.rows; ++i)
    if (ra::keys_visible(a.rows + i, a.diag, a.keys) != ra::keys_visible(i, b.diag, b.keys)) return false;
  *m = Sub{a.row0, a.rows + b.rows, a.key0, a.keys, a.diag, a.pairs + b.pairs};
  return true;
}

int subs_of(const ra_desc* d, int32_t kv_len, int32_t mask_kind, int64_t q_off, int64_t k_off,
            Sub* out, int* n_out) {
  if (kv_len < 0) return fail(RA_E_INVALID, "kv_len must be >= 0");
  if (mask_kind < RA_MASK_NONE || mask_kind > RA_MASK_CAUSAL_ZIGZAG)
    return fail(RA_E_INVALID, "unknown mask_kind %d", mask_kind);
  if (mask_kind != RA_MASK_CAUSAL_ZIGZAG) {
    const int causal = mask_kind != RA_MASK_NONE;
    const int32_t diag = ra::diag_shift(causal, q_off, k_off, pos_stride(mask_kind, d), d->q_len, kv_len);
    out[0] = Sub{0, d->q_len, 0, kv_len, diag, pairs_of(d->q_len, kv_len, diag)};
    *n_out = 1;
    return RA_OK;
  }
  const int64_t P = d->ring_size;
  if (d->q_len % 2 != 0) return fail(RA_E_INVALID, "zigzag: q_len %d is not two chunks", d->q_len);
  if (kv_len != d->q_len)
    return fail(RA_E_INVALID, "zigzag: kv_len %d must equal q_len %d (one chunk length)", kv_len, d->q_len);
  if (q_off < 0 || q_off >= P || k_off < 0 || k_off >= P)
    return fail(RA_E_INVALID, "zigzag: q_offset and k_offset are ranks in [0, %lld)", (long long)P);
  const int32_t c = d->q_len / 2;
  const int64_t q_chunk[2] = {q_off, 2 * P - 1 - q_off};
  const int64_t k_chunk[2] = {k_off, 2 * P - 1 - k_off};
  for (int qa = 0; qa < 2; ++qa)
    for (int ka = 0; ka < 2; ++ka) {
      const int32_t diag = ra::diag_shift(1, q_chunk[qa] * c, k_chunk[ka] * c, 1, c, c);
      out[2 * qa + ka] = Sub{qa * c, c, ka * c, c, diag, pairs_of(c, c, diag)};
    }
  *n_out = 4;
  return RA_OK;
}

// Plan one block: counts for the whole launch (all batches and query heads).
int plan(const ra_desc* d, int32_t kv_len, int32_t mask_kind, int64_t q_off, int64_t k_off,
         ra_stats* out, Sub* subs, int* n_subs) {
  Sub local[4];
  int n_local = 0;
  if (!subs) subs = local;
  if (!n_subs) n_subs = &n_local;
  int rc = subs_of(d, kv_len, mask_kind, q_off, k_off, subs, n_subs);
  if (rc) return rc;
  const int tq = tile_q_of(d), tk = tile_k_of(d);
  std::memset(out, 0, sizeof *out);
  out->tile_q = tq;
  out->tile_k = tk;
  const int64_t heads = (int64_t)d->batch * d->q_heads;
  int64_t pairs = 0, full = 0, live = 0, tiles = 0;
  for (int u = 0; u < *n_subs; ++u) {
    const Sub& b = subs[u];
    pairs += b.pairs;
    const int32_t n_qt = (b.rows + tq - 1) / tq;
    const int32_t n_kt = (b.keys + tk - 1) / tk;
    tiles += (int64_t)n_qt * n_kt;
    for (int32_t a = 0; a < n_qt; ++a) {
      const int32_t i0 = a * tq, i1 = i0 + tq < b.rows ? i0 + tq : b.rows;
      full += ra::tiles_full(i0, i1, b.diag, b.keys, tk);
      live += ra::tiles_live(i0, i1, b.diag, b.keys, tk);
    }
  }
  out->live_pairs = pairs * heads;
  out->tiles_full = full * heads;
  out->tiles_partial = (live - full) * heads;
  out->tiles_empty = (tiles - live) * heads;
  if (pairs > 0) out->blocks_run = 1; else out->blocks_skipped = 1;
  return RA_OK;
}

void add_stats(ra_stats* acc, const ra_stats* s) {
  acc->live_pairs += s->live_pairs;
  acc->tiles_full += s->tiles_full;
  acc->tiles_partial += s->tiles_partial;
  acc->tiles_empty += s->tiles_empty;
  acc->blocks_run += s->blocks_run;
  acc->blocks_skipped += s->blocks_skipped;
  acc->tile_q = s->tile_q;
  acc->tile_k = s->tile_k;
}

int make_state(const ra_desc* d, const void* q, void* ws, int fresh, ra_state** out) {
  if (!out) return fail(RA_E_INVALID, "out is NULL");
  *out = nullptr;
  int rc = check_desc(d);
  if (rc) return rc;
  const Layout L = layout_of(d);
  if (d->q_len > 0) {
    if (!q) return fail(RA_E_INVALID, "Q_r is NULL");
    if (!ws) return fail(RA_E_INVALID, "workspace is NULL");
    if (!aligned16(q)) return fail(RA_E_INVALID, "Q_r must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
      return fail(RA_E_INVALID, "workspace must be 256-byte aligned");
  }
  ra_state* st = new (std::nothrow) ra_state;
  if (!st) return fail(RA_E_INVALID, "out of host memory");
  std::memset(st, 0, sizeof *st);
  st->desc = *d;
  if (st->desc.softmax_scale == 0.f) st->desc.softmax_scale = 1.0f / std::sqrt((float)d->head_dim);
  st->q = q;
  char* base = static_cast<char*>(ws);
  st->o_acc = reinterpret_cast<float*>(base + L.o_off);
  st->m = reinterpret_cast<float*>(base + L.m_off);
  st->l = reinterpret_cast<float*>(base + L.l_off);
  st->fresh = fresh;
  st->stats.tile_q = tile_q_of(d);
  st->stats.tile_k = tile_k_of(d);
  *out = st;
  return RA_OK;
}

// The split-KV step: enough key chunks that the whole chip streams the block, none so short
// that a wave's fixed cost or the chunk states outweigh its share of K and V.  Every chunk
// writes, and the combine reads back, 4 (d + 2) bytes per packed row, so the more rows a
// wave packs, the longer its chunks pay.  decode_kernel aims at 1024 waves (one per SIMD),
// or 2048 (two per SIMD) when a lone row group packs at most 8 rows (one token of an 8:1
// group) and its chunk states are cheap; chunks are at least kDecodeMinChunk keys per wave.
// decode_ring_kernel's four-wave workgroups hold an 80 KB LDS ring each and aim at 512 of
// them (two per CU), with chunks of at least kDecodeMinChunkRing keys per tile subset.
constexpr int64_t kDecodeTargetWaves = 1024;
constexpr int64_t kDecodeTargetWavesFewRows = 2048;
constexpr int64_t kDecodeFewRows = 8;
constexpr int64_t kDecodeTargetRings = 512;
constexpr int32_t kDecodeMinChunk = 256;
constexpr int32_t kDecodeMinChunkRing = 512;

struct DecodePlan {
  int32_t n_parts, chunk;
};

// query rows that share one KV head: (query head of the group, token) pairs
int64_t decode_packed_rows(const ra_desc* d) { return (int64_t)(d->q_heads / d->kv_heads) * d->q_len; }

int64_t decode_row_groups(const ra_desc* d) {
  return (decode_packed_rows(d) + ra::kDecodeRows - 1) / ra::kDecodeRows;
}

int32_t decode_min_chunk(ra::DecodeShape sh) { return sh.ring ? kDecodeMinChunkRing : kDecodeMinChunk; }

// key chunks wanted per (batch, KV head, workgroup of row groups)
int64_t decode_want(const ra_desc* d, ra::DecodeShape sh) {
  const int64_t n_wg = (decode_row_groups(d) + sh.R - 1) / sh.R;
  const int64_t base = (int64_t)d->batch * d->kv_heads * n_wg * (sh.ring ? 1 : sh.R);
  const int64_t target = sh.ring ? kDecodeTargetRings
                         : decode_packed_rows(d) <= kDecodeFewRows ? kDecodeTargetWavesFewRows
                                                                   : kDecodeTargetWaves;
  return base >= target ? 1 : (target + base - 1) / base;
}

DecodePlan decode_plan(const ra_desc* d, ra::DecodeShape sh, int32_t n_keys) {
  DecodePlan pl{0, 0};
  if (n_keys <= 0) return pl;
  const int64_t want = decode_want(d, sh);
  const int64_t step = (int64_t)ra::kDecodeTileK * sh.S;
  int64_t chunk = (n_keys + want - 1) / want;
  chunk = (chunk + step - 1) / step * step;
  const int64_t min_chunk = (int64_t)decode_min_chunk(sh) * sh.S;
  if (chunk < min_chunk) chunk = min_chunk;
  pl.chunk = (int32_t)chunk;
  pl.n_parts = (int32_t)((n_keys + chunk - 1) / chunk);
  return pl;
}

struct DecodeLayout {
  size_t o_off, m_off, l_off, total;
};

// Partial states of a block of kv_len keys.  A causal block plans over its visible keys
// n_keys <= kv_len, and the shape may change with n_keys (two row groups), so the bound is the
// larger over the shapes n_keys can take.  For one shape, n_parts <= want and
// n_parts <= ceil(n_keys / (S * its minimum chunk)), both non-decreasing in n_keys, and each
// part leaves S partial states.
DecodeLayout decode_layout(const ra_desc* d, int32_t kv_len) {
  const int64_t n_rg = decode_row_groups(d);
  auto bound = [&](ra::DecodeShape sh) {
    const int64_t per_part = (int64_t)sh.S * decode_min_chunk(sh);
    int64_t parts = ((int64_t)kv_len + per_part - 1) / per_part;
    const int64_t want = decode_want(d, sh);
    return (parts > want ? want : parts) * sh.S;
  };
  int64_t parts = bound(ra::decode_shape(n_rg, kv_len));
  if (n_rg == 2) {
    const int64_t p2 = bound(ra::decode_shape(n_rg, 0));
    if (p2 > parts) parts = p2;
  }
  const size_t rows = (size_t)d->batch * d->q_heads * d->q_len;
  DecodeLayout L;
  L.o_off = 0;
  L.m_off = align256((size_t)parts * rows * d->head_dim * sizeof(float));
  L.l_off = L.m_off + align256((size_t)parts * rows * sizeof(float));
  L.total = rows && parts && kv_len > 0 ? L.l_off + align256((size_t)parts * rows * sizeof(float)) : 0;
  return L;
}

}  // namespace

// Scratch of ra_decode_step_noalloc, for callers that cannot allocate: one copy of this
// array per device, created with the library's code object and held until the process ends.
// In host code its name is only a stand-in; the device address of the current device's copy
// comes from hipGetSymbolAddress, looked up once per device and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[RA_DECODE_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The device address of `scratch` on device dev (looked up with dev current, then kept).
int scratch_on_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_E_UNSUPPORTED, "device %d is out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (back != hipSuccess) return hip_fail(back, "hipSetDevice");
    if (!ptr) return fail(RA_E_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

size_t ra_workspace_bytes(const ra_desc* desc) {
  if (check_desc(desc)) return 0;
  return layout_of(desc).total;
}

int ra_workspace_layout(const ra_desc* desc, size_t* o_off, size_t* m_off, size_t* l_off) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const Layout L = layout_of(desc);
  if (o_off) *o_off = L.o_off;
  if (m_off) *m_off = L.m_off;
  if (l_off) *l_off = L.l_off;
  return RA_OK;
}

int ra_state_init(const ra_desc* desc, const void* q, void* workspace, ra_state** out) {
  return make_state(desc, q, workspace, 1, out);
}

int ra_state_resume(const ra_desc* desc, const void* q, void* workspace, ra_state** out) {
  return make_state(desc, q, workspace, 0, out);
}

namespace {
int block_step(ra_state* st, const void* k, const void* v, int32_t kv_len, int32_t mask_kind,
               int64_t q_offset, int64_t k_offset, float* fin_o, float* fin_lse, int* finalized);
}  // namespace

int ra_block_step(ra_state* st, const void* k, const void* v, int32_t kv_len, int32_t mask_kind,
                  int64_t q_offset, int64_t k_offset) {
  return block_step(st, k, v, kv_len, mask_kind, q_offset, k_offset, nullptr, nullptr, nullptr);
}

namespace {
// fin_o (optional): the block is the lap's last, and O and lse are wanted; when the step runs
// as one bf16 launch over all rows in which every row sees a key, that launch writes O = O~ / l
// and lse as it writes back (the arithmetic of the finalize pass), the state is finalized and
// *finalized is 1.  Otherwise the step keeps the state as usual and *finalized is 0.
int block_step(ra_state* st, const void* k, const void* v, int32_t kv_len, int32_t mask_kind,
               int64_t q_offset, int64_t k_offset, float* fin_o, float* fin_lse, int* finalized) {
  if (finalized) *finalized = 0;
  if (!st) return fail(RA_E_INVALID, "state is NULL");
  if (st->finalized) return fail(RA_E_STATE, "step after finalize");
  const ra_desc* d = &st->desc;
  ra_stats s;
  Sub subs[4];
  int n_subs = 0;
  int rc = plan(d, kv_len, mask_kind, q_offset, k_offset, &s, subs, &n_subs);
  if (rc) return rc;
  if (kv_len > 0) {
    if (!k || !v) return fail(RA_E_INVALID, "K_j or V_j is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(RA_E_INVALID, "K_j and V_j must be 16-byte aligned");
    if (kv_len > 1 && d->kv_strides[2] < d->head_dim)
      return fail(RA_E_INVALID, "kv token stride smaller than head_dim");
  }
  if (s.blocks_run == 0) {  // no allowed pair in the whole block: nothing to do
    add_stats(&st->stats, &s);
    return RA_OK;
  }
  const size_t elem = d->dtype == RA_DTYPE_BF16 ? 2 : 4;
  hipStream_t stream = static_cast<hipStream_t>(d->stream);
  // The key-tile norms of the whole block (tiles from its first key), when it is long enough
  // for the step kernel's guard to matter.  A buffer that must grow while the stream is being
  // captured is not grown: the launches then go without bounds (same result, full guard).
  const int32_t n_tiles = (kv_len + ra::kBf16TileK - 1) / ra::kBf16TileK;
  const float* knorm = nullptr;
  if (d->dtype == RA_DTYPE_BF16 && kv_len >= kKeyNormMinKeys) {
    const size_t need = (size_t)d->batch * d->kv_heads * n_tiles;
    if (need > st->knorm_cap) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      hipError_t e = hipStreamIsCapturing(stream, &cs);
      if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
      if (cs == hipStreamCaptureStatusNone) {
        if (st->knorm) {
          e = hipFree(st->knorm);
          st->knorm = nullptr;
          st->knorm_cap = 0;
          if (e != hipSuccess) return hip_fail(e, "hipFree (key-tile norms)");
        }
        void* buf = nullptr;
        e = hipMalloc(&buf, need * sizeof(float));
        if (e != hipSuccess) return hip_fail(e, "hipMalloc (key-tile norms)");
        st->knorm = static_cast<float*>(buf);
        st->knorm_cap = need;
      }
    }
    if (need <= st->knorm_cap) {
      hipError_t e = ra::launch_key_tile_norms(k, d->kv_strides[0], d->kv_strides[1],
                                               token_stride(d->kv_strides[2], kv_len, d->head_dim),
                                               d->batch, d->kv_heads, kv_len, d->head_dim, st->knorm, stream);
      if (e != hipSuccess) return hip_fail(e, "key-tile norm launch");
      knorm = st->knorm;
    }
  }
  bool fin = false;   // set once the launches are known
  auto launch = [&](const Sub& b, int fresh) -> int {
    ra::StepParams p;
    p.q = static_cast<const char*>(st->q) + (int64_t)b.row0 * d->q_strides[2] * elem;
    p.k = static_cast<const char*>(k) + (int64_t)b.key0 * d->kv_strides[2] * elem;
    p.v = static_cast<const char*>(v) + (int64_t)b.key0 * d->kv_strides[2] * elem;
    p.o_acc = st->o_acc + (int64_t)b.row0 * d->head_dim;
    p.m = st->m + b.row0;
    p.l = st->l + b.row0;
    p.q_sb = d->q_strides[0];
    p.q_sh = d->q_strides[1];
    p.q_st = token_stride(d->q_strides[2], d->q_len, d->head_dim);
    p.k_sb = d->kv_strides[0];
    p.k_sh = d->kv_strides[1];
    p.k_st = token_stride(d->kv_strides[2], kv_len, d->head_dim);
    p.batch = d->batch;
    p.q_heads = d->q_heads;
    p.kv_heads = d->kv_heads;
    p.group = d->q_heads / d->kv_heads;
    p.n_q = b.rows;
    p.n_k = b.keys;
    p.state_rows = d->q_len;
    p.diag = b.diag;
    p.scale_log2 = d->softmax_scale * 1.4426950408889634f;
    p.fresh = fresh;
    p.dbg = st->dbg;
    // tiles of a sub-block line up with the block's when it starts on a tile boundary
    p.knorm = knorm && b.key0 % ra::kBf16TileK == 0 ? knorm + b.key0 / ra::kBf16TileK : nullptr;
    p.knorm_stride = n_tiles;
    p.o_out = p.o_acc;
    p.fin_lse = nullptr;
    p.finalize = 0;
    if (fin) {
      p.o_out = fin_o + (int64_t)b.row0 * d->head_dim;
      p.fin_lse = fin_lse ? fin_lse + b.row0 : nullptr;
      p.finalize = 1;
    }
    hipError_t e = d->dtype == RA_DTYPE_BF16 ? ra::launch_step_bf16(p, d->head_dim, stream)
                                             : ra::launch_step_f32(p, d->head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "step kernel launch");
    return RA_OK;
  };
  // The launches: the sub-blocks with an allowed pair, in order (those that share query rows
  // run one after the other on the stream).  Zigzag chunk pairs that together form one causal
  // sub-block exactly (the two key chunks of one query chunk, or both query chunks against one
  // key chunk) run as one launch, which spares a launch's start and drain; only when the chunks
  // are whole tiles, so that every tile, and every count the kernels keep, is the one the
  // chunk pairs give.  covers[u]: the query chunks (bit per chunk) that launch u touches.
  const bool zz = n_subs == 4;
  Sub runs[4];
  unsigned covers[4];
  int n_runs = 0;
  for (int u = 0; u < n_subs; ++u)
    if (subs[u].pairs > 0) {
      runs[n_runs] = subs[u];
      covers[n_runs++] = zz ? 1u << (u >> 1) : 1u;
    }
  if (zz && subs[0].rows % tile_q_of(d) == 0 && subs[0].keys % tile_k_of(d) == 0) {
    Sub m;
    for (int a = 0; a + 1 < n_runs; ++a)
      if (covers[a] == covers[a + 1] && merge_keys(runs[a], runs[a + 1], &m)) {
        runs[a] = m;
        for (int u = a + 1; u + 1 < n_runs; ++u) {
          runs[u] = runs[u + 1];
          covers[u] = covers[u + 1];
        }
        --n_runs;
      }
    // both query chunks against one key chunk; or, on the rank's own block, the first query
    // chunk's diagonal pair with its empty neighbour and the second chunk's joined pairs: one
    // causal block over both chunks
    Sub ext;
    if (n_runs == 2 && covers[0] == 1u && covers[1] == 2u &&
        (merge_rows(runs[0], runs[1], &m) ||
         (extend_keys(runs[0], subs[1], &ext) && merge_rows(ext, runs[1], &m)))) {
      runs[0] = m;
      covers[0] |= covers[1];
      n_runs = 1;
    }
  }
  // The lap's last step finalizes in its launch when that launch is the whole step, covers
  // every row and every row sees a key (no workgroup then returns early).
  fin = fin_o && d->dtype == RA_DTYPE_BF16 && n_runs == 1 && runs[0].row0 == 0 && runs[0].rows == d->q_len &&
        ra::keys_visible(0, runs[0].diag, runs[0].keys) > 0 && aligned16(fin_o);
  // Only the first launch that touches a row range of a fresh state starts from the empty
  // state; a fresh row range with no allowed pair in this block still gets the empty state
  // written (with no keys), because the state stops being fresh as a whole.
  unsigned touched = 0;
  for (int u = 0; u < n_runs; ++u) {
    rc = launch(runs[u], st->fresh && (covers[u] & touched) == 0);
    if (rc) return rc;
    touched |= covers[u];
  }
  if (st->fresh)
    for (int c = 0; c < (zz ? 2 : 1); ++c)
      if (!((touched >> c) & 1u)) {
        Sub empty = subs[zz ? 2 * c : 0];
        empty.keys = 0;
        rc = launch(empty, 1);
        if (rc) return rc;
      }
  st->fresh = 0;
  add_stats(&st->stats, &s);
  if (fin) {
    st->finalized = 1;
    if (finalized) *finalized = 1;
  }
  return RA_OK;
}
}  // namespace

int ra_finalize(ra_state* st, float* o, float* lse) {
  if (!st) return fail(RA_E_INVALID, "state is NULL");
  if (st->finalized) return fail(RA_E_STATE, "state already finalized");
  const ra_desc* d = &st->desc;
  const int64_t rows = (int64_t)d->batch * d->q_heads * d->q_len;
  if (rows > 0 && !o) return fail(RA_E_INVALID, "O_r is NULL");
  if (rows > 0 && !aligned16(o)) return fail(RA_E_INVALID, "O_r must be 16-byte aligned");
  ra::FinalizeParams p;
  p.o_acc = st->o_acc;
  p.m = st->m;
  p.l = st->l;
  p.o = o;
  p.lse = lse;
  p.rows = rows;
  p.d = d->head_dim;
  p.fresh = st->fresh;
  hipError_t e = ra::launch_finalize(p, static_cast<hipStream_t>(d->stream));
  if (e != hipSuccess) return hip_fail(e, "finalize kernel launch");
  st->finalized = 1;
  return RA_OK;
}

int ra_merge_states(const ra_desc* desc, int32_t n_parts, void* const* parts, void* merged,
                    float* o, float* lse) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (n_parts < 1 || n_parts > RA_MERGE_MAX_PARTS)
    return fail(RA_E_INVALID, "n_parts %d is outside [1, %d]", n_parts, RA_MERGE_MAX_PARTS);
  if (!parts) return fail(RA_E_INVALID, "parts is NULL");
  if (!merged && !o) return fail(RA_E_INVALID, "neither a merged state nor O requested");
  if (lse && !o) return fail(RA_E_INVALID, "lse is written together with O only");
  const int64_t rows = (int64_t)desc->batch * desc->q_heads * desc->q_len;
  for (int s = 0; s < n_parts; ++s) {
    if (rows > 0 && !parts[s]) return fail(RA_E_INVALID, "parts[%d] is NULL", s);
    if ((reinterpret_cast<uintptr_t>(parts[s]) & 255) != 0)
      return fail(RA_E_INVALID, "parts[%d] must be 256-byte aligned", s);
  }
  if (merged && (reinterpret_cast<uintptr_t>(merged) & 255) != 0)
    return fail(RA_E_INVALID, "merged must be 256-byte aligned");
  if (o && !aligned16(o)) return fail(RA_E_INVALID, "O must be 16-byte aligned");
  const Layout L = layout_of(desc);
  ra::MergeParams p;
  std::memset(&p, 0, sizeof p);
  for (int s = 0; s < n_parts; ++s) p.parts[s] = static_cast<const char*>(parts[s]);
  p.n_parts = n_parts;
  p.m_off = L.m_off;
  p.l_off = L.l_off;
  p.merged = static_cast<char*>(merged);
  p.o = o;
  p.lse = lse;
  p.rows = rows;
  p.d = desc->head_dim;
  hipError_t e = ra::launch_merge(p, static_cast<hipStream_t>(desc->stream));
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return RA_OK;
}

size_t ra_decode_workspace_bytes(const ra_desc* desc, int32_t kv_len) {
  if (check_desc(desc) || kv_len < 0) return 0;
  return decode_layout(desc, kv_len).total;
}

int ra_decode_step(ra_state* st, const void* k, const void* v, int32_t kv_len, int32_t mask_kind,
                   int64_t q_offset, int64_t k_offset, void* workspace, size_t workspace_bytes) {
  if (!st) return fail(RA_E_INVALID, "state is NULL");
  if (st->finalized) return fail(RA_E_STATE, "step after finalize");
  const ra_desc* d = &st->desc;
  // fp32 inputs take the exactness path: the tiled fp32 step over the whole block
  if (d->dtype == RA_DTYPE_F32 && mask_kind != RA_MASK_CAUSAL_ZIGZAG)
    return ra_block_step(st, k, v, kv_len, mask_kind, q_offset, k_offset);
  if (mask_kind == RA_MASK_CAUSAL_ZIGZAG)
    return fail(RA_E_UNSUPPORTED, "the split-KV step takes single-range layouts (not zigzag)");
  ra_stats s;
  Sub subs[4];
  int n_subs = 0;
  int rc = plan(d, kv_len, mask_kind, q_offset, k_offset, &s, subs, &n_subs);
  if (rc) return rc;
  if (kv_len > 0) {
    if (!k || !v) return fail(RA_E_INVALID, "K_j or V_j is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(RA_E_INVALID, "K_j and V_j must be 16-byte aligned");
    if (kv_len > 1 && d->kv_strides[2] < d->head_dim)
      return fail(RA_E_INVALID, "kv token stride smaller than head_dim");
  }
  if (s.blocks_run == 0) {
    add_stats(&st->stats, &s);
    return RA_OK;
  }
  const DecodeLayout L = decode_layout(d, kv_len);
  if (!workspace) return fail(RA_E_INVALID, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(RA_E_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(RA_E_INVALID, "workspace holds %zu bytes, the block needs %zu", workspace_bytes, L.total);
  // keys past the last row's causal limit are seen by no row
  const Sub& b = subs[0];
  const int32_t n_keys = ra::keys_visible(d->q_len - 1, b.diag, kv_len);
  const int64_t n_rg = decode_row_groups(d);
  const ra::DecodeShape shape = ra::decode_shape(n_rg, n_keys);
  const DecodePlan pl = decode_plan(d, shape, n_keys);
  const int64_t waves = (int64_t)pl.n_parts * ((n_rg + shape.R - 1) / shape.R) * shape.R * shape.S *
                        d->kv_heads * d->batch;
  if (waves * 64 > 0xffffffffLL)   // a launch holds fewer than 2^32 work-items
    return fail(RA_E_UNSUPPORTED, "split-KV grid of %lld waves is too large", (long long)waves);
  char* ws = static_cast<char*>(workspace);
  ra::DecodeParams p;
  p.q = st->q;
  p.k = k;
  p.v = v;
  p.part_o = reinterpret_cast<float*>(ws + L.o_off);
  p.part_m = reinterpret_cast<float*>(ws + L.m_off);
  p.part_l = reinterpret_cast<float*>(ws + L.l_off);
  p.q_sb = d->q_strides[0];
  p.q_sh = d->q_strides[1];
  p.q_st = token_stride(d->q_strides[2], d->q_len, d->head_dim);
  p.k_sb = d->kv_strides[0];
  p.k_sh = d->kv_strides[1];
  p.k_st = token_stride(d->kv_strides[2], kv_len, d->head_dim);
  p.batch = d->batch;
  p.q_heads = d->q_heads;
  p.kv_heads = d->kv_heads;
  p.group = d->q_heads / d->kv_heads;
  p.n_q = d->q_len;
  p.n_k = n_keys;
  p.n_parts = pl.n_parts;
  p.chunk = pl.chunk;
  p.diag = b.diag;
  p.scale_log2 = d->softmax_scale * 1.4426950408889634f;
  p.dbg_moves = st->dbg ? st->dbg + 3 : nullptr;
  hipStream_t stream = static_cast<hipStream_t>(d->stream);
  // the row groups of one KV head share each chunk's tiles inside one workgroup
  hipError_t e = ra::launch_decode(p, d->head_dim, shape, stream);
  if (e != hipSuccess) return hip_fail(e, "split-KV step launch");
  ra::CombineParams c;
  c.part_o = p.part_o;
  c.part_m = p.part_m;
  c.part_l = p.part_l;
  c.n_parts = pl.n_parts * shape.S;
  c.o_acc = st->o_acc;
  c.m = st->m;
  c.l = st->l;
  c.rows = (int64_t)d->batch * d->q_heads * d->q_len;
  c.d = d->head_dim;
  c.fresh = st->fresh;
  e = ra::launch_combine(c, stream);
  if (e != hipSuccess) return hip_fail(e, "split-KV combine launch");
  st->fresh = 0;
  add_stats(&st->stats, &s);
  return RA_OK;
}

int ra_decode_step_noalloc(ra_state* st, const void* k, const void* v, int32_t kv_len,
                           int32_t mask_kind, int64_t q_offset, int64_t k_offset) {
  if (!st) return fail(RA_E_INVALID, "state is NULL");
  const ra_desc* d = &st->desc;
  // only bf16 forms chunk states (fp32 takes ra_block_step, zigzag is rejected)
  const bool chunked = d->dtype == RA_DTYPE_BF16 && mask_kind != RA_MASK_CAUSAL_ZIGZAG;
  const size_t need = chunked ? ra_decode_workspace_bytes(d, kv_len) : 0;
  if (need > RA_DECODE_NOALLOC_MAX_BYTES)
    return fail(RA_E_UNSUPPORTED,
                "the split-KV step needs %zu bytes of chunk states; the no-allocation entry point "
                "holds %zu (use ra_decode_step with a workspace)",
                need, (size_t)RA_DECODE_NOALLOC_MAX_BYTES);
  // the device the work goes to: the stream's
  int dev = 0;
  hipStream_t stream = static_cast<hipStream_t>(d->stream);
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of desc.stream");
  void* ws = nullptr;
  const int rc = scratch_on_device(dev, &ws);
  if (rc) return rc;
  return ra_decode_step(st, k, v, kv_len, mask_kind, q_offset, k_offset, ws, RA_DECODE_NOALLOC_MAX_BYTES);
}

size_t ra_bwd_workspace_bytes(const ra_desc* desc) {
  if (check_desc(desc)) return 0;
  const size_t rows = (size_t)desc->batch * desc->q_heads * desc->q_len;
  return rows ? align256(rows * desc->head_dim * sizeof(float)) + align256(rows * sizeof(float)) : 0;
}

int ra_bwd_init(const ra_desc* desc, const void* q, const void* d_out, const float* out,
                const float* lse, void* workspace, ra_bwd** handle) {
  if (!handle) return fail(RA_E_INVALID, "out is NULL");
  *handle = nullptr;
  int rc = check_desc(desc);
  if (rc) return rc;
  const int64_t rows = (int64_t)desc->batch * desc->q_heads * desc->q_len;
  if (rows > 0) {
    if (!q || !d_out || !out || !lse || !workspace)
      return fail(RA_E_INVALID, "Q_r, dO_r, O_r, lse_r and the workspace are required");
    if (!aligned16(q) || !aligned16(d_out) || !aligned16(out))
      return fail(RA_E_INVALID, "Q_r, dO_r and O_r must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
      return fail(RA_E_INVALID, "workspace must be 256-byte aligned");
  }
  ra_bwd* st = new (std::nothrow) ra_bwd;
  if (!st) return fail(RA_E_INVALID, "out of host memory");
  std::memset(st, 0, sizeof *st);
  st->desc = *desc;
  if (st->desc.softmax_scale == 0.f) st->desc.softmax_scale = 1.0f / std::sqrt((float)desc->head_dim);
  st->q = q;
  st->d_out = d_out;
  st->lse = lse;
  char* base = static_cast<char*>(workspace);
  st->dq = reinterpret_cast<float*>(base);
  st->D = reinterpret_cast<float*>(base + align256((size_t)rows * desc->head_dim * sizeof(float)));
  st->stats.tile_q = 64;
  st->stats.tile_k = 64;
  if (rows > 0) {
    ra::BwdPrepParams pp;
    pp.d_out = d_out;
    pp.out = out;
    pp.D = st->D;
    pp.dq = st->dq;
    pp.q_sb = desc->q_strides[0];
    pp.q_sh = desc->q_strides[1];
    pp.q_st = desc->q_strides[2];
    pp.q_heads = desc->q_heads;
    pp.n_q = desc->q_len;
    pp.rows = rows;
    hipError_t e = ra::launch_bwd_prep(pp, desc->head_dim, desc->dtype == RA_DTYPE_BF16,
                                       static_cast<hipStream_t>(desc->stream));
    if (e != hipSuccess) {
      delete st;
      return hip_fail(e, "backward prep launch");
    }
  }
  *handle = st;
  return RA_OK;
}

int ra_bwd_block_step(ra_bwd* st, const void* k, const void* v, float* dk, float* dv,
                      int32_t kv_len, int32_t mask_kind, int64_t q_offset, int64_t k_offset) {
  if (!st) return fail(RA_E_INVALID, "state is NULL");
  if (st->finalized) return fail(RA_E_STATE, "step after finalize");
  const ra_desc* d = &st->desc;
  ra_stats s;
  Sub subs[4];
  int n_subs = 0;
  int rc = plan(d, kv_len, mask_kind, q_offset, k_offset, &s, subs, &n_subs);
  if (rc) return rc;
  if (kv_len > 0) {
    if (!k || !v || !dk || !dv) return fail(RA_E_INVALID, "K_j, V_j, dK_j or dV_j is NULL");
    if (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv))
      return fail(RA_E_INVALID, "K_j, V_j, dK_j and dV_j must be 16-byte aligned");
    if (kv_len > 1 && d->kv_strides[2] < d->head_dim)
      return fail(RA_E_INVALID, "kv token stride smaller than head_dim");
    // the key-stationary launches: 32-key tiles at the smallest, 256 threads each
    const int64_t k_tiles = ((int64_t)kv_len + 31) / 32;
    if (k_tiles * d->kv_heads * d->batch * 256 > 0xffffffffLL)
      return fail(RA_E_UNSUPPORTED, "%lld key tiles exceed one launch", (long long)(k_tiles * d->kv_heads * d->batch));
  }
  s.tile_q = st->stats.tile_q;
  s.tile_k = st->stats.tile_k;
  s.tiles_full = s.tiles_partial = s.tiles_empty = 0;   // the backward kernels tile differently
  if (s.blocks_run == 0) {
    add_stats(&st->stats, &s);
    return RA_OK;
  }
  const size_t elem = d->dtype == RA_DTYPE_BF16 ? 2 : 4;
  for (int u = 0; u < n_subs; ++u) {
    const Sub& b = subs[u];
    if (b.pairs == 0) continue;
    ra::BwdParams p;
    p.q = static_cast<const char*>(st->q) + (int64_t)b.row0 * d->q_strides[2] * elem;
    p.d_out = static_cast<const char*>(st->d_out) + (int64_t)b.row0 * d->q_strides[2] * elem;
    p.k = static_cast<const char*>(k) + (int64_t)b.key0 * d->kv_strides[2] * elem;
    p.v = static_cast<const char*>(v) + (int64_t)b.key0 * d->kv_strides[2] * elem;
    p.lse = st->lse + b.row0;
    p.D = st->D + b.row0;
    p.dq = st->dq + (int64_t)b.row0 * d->head_dim;
    p.dk = dk + (int64_t)b.key0 * d->head_dim;
    p.dv = dv + (int64_t)b.key0 * d->head_dim;
    p.q_sb = d->q_strides[0];
    p.q_sh = d->q_strides[1];
    p.q_st = token_stride(d->q_strides[2], d->q_len, d->head_dim);
    p.k_sb = d->kv_strides[0];
    p.k_sh = d->kv_strides[1];
    p.k_st = token_stride(d->kv_strides[2], kv_len, d->head_dim);
    p.batch = d->batch;
    p.q_heads = d->q_heads;
    p.kv_heads = d->kv_heads;
    p.group = d->q_heads / d->kv_heads;
    p.n_q = b.rows;
    p.n_k = b.keys;
    p.state_rows = d->q_len;
    p.dkv_rows = kv_len;
    p.diag = b.diag;
    p.scale = d->softmax_scale;
    hipStream_t stream = static_cast<hipStream_t>(d->stream);
    hipError_t e = d->dtype == RA_DTYPE_BF16 ? ra::launch_bwd_step_bf16(p, d->head_dim, stream)
                                             : ra::launch_bwd_step_f32(p, d->head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "backward step launch");
  }
  add_stats(&st->stats, &s);
  return RA_OK;
}

int ra_bwd_finalize(ra_bwd* st, float* dq) {
  if (!st) return fail(RA_E_INVALID, "state is NULL");
  if (st->finalized) return fail(RA_E_STATE, "state already finalized");
  const ra_desc* d = &st->desc;
  const size_t bytes = (size_t)d->batch * d->q_heads * d->q_len * d->head_dim * sizeof(float);
  if (bytes > 0) {
    if (!dq) return fail(RA_E_INVALID, "dQ_r is NULL");
    hipError_t e = hipMemcpyAsync(dq, st->dq, bytes, hipMemcpyDeviceToDevice,
                                  static_cast<hipStream_t>(d->stream));
    if (e != hipSuccess) return hip_fail(e, "dQ copy");
  }
  st->finalized = 1;
  return RA_OK;
}

int ra_bwd_get_stats(const ra_bwd* st, ra_stats* out) {
  if (!st || !out) return fail(RA_E_INVALID, "state or out is NULL");
  *out = st->stats;
  return RA_OK;
}

int ra_bwd_destroy(ra_bwd* st) {
  delete st;
  return RA_OK;
}

int ra_state_destroy(ra_state* st) {
  // hipFree waits for the device, so work still reading the norms ends first
  if (st && st->knorm) hipFree(st->knorm);
  delete st;
  return RA_OK;
}

int ra_get_stats(const ra_state* st, ra_stats* out) {
  if (!st || !out) return fail(RA_E_INVALID, "state or out is NULL");
  *out = st->stats;
  return RA_OK;
}

int ra_state_set_debug_counters(ra_state* st, uint64_t* counters) {
  if (!st) return fail(RA_E_INVALID, "state is NULL");
  st->dbg = reinterpret_cast<unsigned long long*>(counters);
  return RA_OK;
}

int ra_plan_block(const ra_desc* desc, int32_t kv_len, int32_t mask_kind, int64_t q_offset,
                  int64_t k_offset, ra_stats* out) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!out) return fail(RA_E_INVALID, "out is NULL");
  return plan(desc, kv_len, mask_kind, q_offset, k_offset, out, nullptr, nullptr);
}

int ra_tile_classes(const ra_desc* desc, int32_t kv_len, int32_t mask_kind, int64_t q_offset,
                    int64_t k_offset, uint8_t* host_out, size_t cap) {
  int rc = check_desc(desc);
  if (rc) return rc;
  ra_stats s;
  Sub subs[4];
  int n_subs = 0;
  rc = plan(desc, kv_len, mask_kind, q_offset, k_offset, &s, subs, &n_subs);
  if (rc) return rc;
  const int tq = tile_q_of(desc), tk = tile_k_of(desc);
  // tile grid: per query chunk and key chunk (one of each for the single-range layouts)
  const int n_side = n_subs == 4 ? 2 : 1;
  const int32_t qt_c = (subs[0].rows + tq - 1) / tq;
  const int32_t kt_c = (subs[0].keys + tk - 1) / tk;
  const int64_t n_qt = (int64_t)n_side * qt_c, n_kt = (int64_t)n_side * kt_c;
  if ((size_t)(n_qt * n_kt) > cap)
    return fail(RA_E_INVALID, "host_out holds %zu bytes, need %lld", cap, (long long)(n_qt * n_kt));
  if (n_qt * n_kt > 0 && !host_out) return fail(RA_E_INVALID, "host_out is NULL");
  for (int qa = 0; qa < n_side; ++qa)
    for (int ka = 0; ka < n_side; ++ka) {
      const Sub& b = subs[qa * n_side + ka];
      for (int32_t a = 0; a < qt_c; ++a) {
        const int32_t i0 = a * tq, i1 = i0 + tq < b.rows ? i0 + tq : b.rows;
        for (int32_t c = 0; c < kt_c; ++c) {
          const int32_t t0 = c * tk, t1 = t0 + tk < b.keys ? t0 + tk : b.keys;
          host_out[(size_t)(qa * qt_c + a) * n_kt + ka * kt_c + c] =
              (uint8_t)ra::classify_tile(i0, i1, t0, t1, b.diag);
        }
      }
    }
  return RA_OK;
}

const char* ra_status_string(int status) {
  switch (status) {
    case RA_OK: return "ok";
    case RA_E_INVALID: return g_err[0] ? g_err : "invalid argument";
    case RA_E_UNSUPPORTED: return g_err[0] ? g_err : "unsupported";
    case RA_E_STATE: return g_err[0] ? g_err : "bad state";
    case RA_E_HIP: return g_err[0] ? g_err : "HIP error";
    default: return "unknown status";
  }
}

int ra_version(void) { return 1; }

}  // extern "C"

// ---------------------------------------------------------------------------------------
// internal helpers exported to the ring driver
// ---------------------------------------------------------------------------------------
namespace ra {
int set_error(int code, const char* msg) { return fail(code, "%s", msg); }
int set_hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }
int block_step_final(ra_state* st, const void* k, const void* v, int32_t kv_len, int32_t mask_kind,
                     int64_t q_offset, int64_t k_offset, float* o, float* lse, int* finalized) {
  return block_step(st, k, v, kv_len, mask_kind, q_offset, k_offset, o, lse, finalized);
}
}  // namespace ra
