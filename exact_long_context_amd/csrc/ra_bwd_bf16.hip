// ra_bwd_bf16.hip -- the backward ring step on the matrix cores (bf16 operands, fp32
// accumulation), for the step that "Ring Attention：把超长序列沿设备环流动", section
// Backward 需要让梯度也沿环传播 describes: dQ stays with the query owner, dK and dV accumulate
// on the travelling block, probabilities are recomputed from the forward's saved logsumexp.
// With P = exp(scale * <q, k> - lse) on allowed pairs:
//     dV += P^T dO,   dS = P * (dO V^T - D),   dQ += scale * dS K,   dK += scale * dS^T Q.
//
// v_mfma_f32_32x32x16_bf16 throughout, with the operand layouts of the forward kernel (lane l
// of operand A holds row l%32 and k = 8*(l/32)..+7; of B column l%32, same k; of the result
// column l%32 and rows 8*(j/4) + 4*(l/32) + j%4):
//  * bwd_dq_kernel (a workgroup of 4 waves owns 128 query rows of one head, 32 per wave):
//      S^T = K Q^T and dP^T = V dO^T (K and V rows from LDS as A, q and dO resident as B),
//      dS^T formed in registers and rounded to bf16, then dQ^T += K^T dS^T with K^T read by
//      ds_read_b64_tr_b16 from the same LDS tile: the forward's P V product with K for V.
//  * bwd_kv_kernel (a workgroup of 4 waves owns 128 keys of one KV head, 32 per wave, K
//      resident in registers and V parked in LDS as B operands): per streamed tile of query
//      rows it forms S = Q K^T and dP = dO V^T once, then P and dS in registers, and
//      accumulates both dV^T += dO^T P and dK^T += Q^T dS (Q and dO rows from LDS as A, their
//      transposes by ds_read_b64_tr_b16).  It walks the query rows of every query head that
//      reads its KV head.
// Streamed tiles are 32 or 64 rows, double-buffered, copied straight from HBM into LDS with
// buffer_load ... lds; one XOR swizzle per tile keeps both the 16-byte operand reads and the
// transposing reads free of bank conflicts.  Each output has one owner: no atomics.  Only
// tiles holding an allowed pair are visited, and the element mask runs only on tiles that
// cross the causal diagonal.  dS is rounded to bf16 without the softmax scale (the same
// relative precision), which dQ and dK take once, as they are written.  Both kernels issue
// their gradient products (dQ; dV and dK) at raised wave priority: of the two waves on a SIMD,
// the one with products to issue goes first while the other forms its probabilities.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_pos.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int NT = 256;     // 4 waves
constexpr int WR = 32;      // rows (dq) or keys (dkdv) per wave
constexpr int BO = 4 * WR;  // owned per workgroup
constexpr float kLog2e = 1.4426950408889634f;

// physical 16-byte chunk of logical chunk c of tile row t.  A tile here is read both ways:
// 16-byte operand reads (16 lanes at a time: 16 consecutive rows at one chunk) and
// transposing ds_read_b64_tr_b16 reads (32 lanes at a time: 4 consecutive rows, aligned,
// x 4 consecutive chunks, aligned).  The twist puts both on distinct banks of the 64: over 16
// consecutive rows it takes 16 distinct values (at d = 64, where a bank line holds two rows,
// 8 distinct values per row parity), and over 4 aligned rows it moves the 4-chunk group to 4
// disjoint groups.
template <int D>
__device__ __forceinline__ int phys(int t, int c) {
  if constexpr (D == 128) return c ^ (4 * (t & 3) + ((t >> 2) & 3));
  else return c ^ (4 * ((t >> 1) & 1) + ((t >> 2) & 3));
}

__device__ __forceinline__ void load_lds_b128_bwd(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bwd(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <int N>
using ic = std::integral_constant<int, N>;

// Per-lane pieces shared by both kernels: where this lane's 16-byte operand chunks sit in a
// tile (k_roff: row r32, chunk 2*ks + hi) and where its transposing reads go (t_roff: rows
// 4*(g>>1) + e (+8 for the second half, +16*kk as an immediate), columns 32*vb + 16*(g&1) +
// 4*a), and which global chunk it fetches for each direct load.
// x, through an empty asm statement the compiler cannot see into: what is computed from the
// result starts here, not earlier
__device__ __forceinline__ int opaque_copy(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int D, int BT>
struct TileMap {
  static constexpr int KS = D / 16, VB = D / 32, RB = D * 2, CPR = D / 8, RPL = 64 / CPR;
  static constexpr int LPW = BT * RB / 1024 / 4;
  int k_roff[KS];
  int t_roff[2][VB];
  int goff[LPW];
  __device__ void init(int lane, int wave, int row_bytes) {
    const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_roff[ks] = r32 * RB + (phys<D>(r32, 2 * ks + hi) << 4);
    const int g = lane >> 4, a = lane & 3, e = (lane >> 2) & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 4 * (g >> 1) + e + 8 * half;
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const int dv = 32 * vb + 16 * (g & 1) + 4 * a;
        t_roff[half][vb] = row * RB + (phys<D>(row, dv >> 3) << 4) + ((dv & 7) << 1);
      }
    }
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int t = (wave * LPW + u) * RPL + lane / CPR;
      goff[u] = (lane / CPR) * row_bytes + phys<D>(t, lane % CPR) * 16;
    }
  }
  // one tile of BT rows starting at global row r0 of base (row stride row_bytes, rows valid)
  __device__ void load(unsigned char* tile, const __bf16* base, int64_t r0, int64_t rows, int64_t st,
                       int wave, int row_bytes) const {
    const __amdgpu_buffer_rsrc_t r = rsrc_bwd(base + r0 * st, (rows - r0) * st * 2);
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int row0 = (wave * LPW + u) * RPL;
      load_lds_b128_bwd(r, tile + row0 * RB, goff[u], row0 * row_bytes);
    }
  }
  // operand chunk ks of tile row half * 32 + r32
  __device__ bf16x8 rd(const unsigned char* tile, int ks, int half = 0) const {
    return *reinterpret_cast<const bf16x8*>(tile + k_roff[ks] + half * 32 * RB);
  }
  __device__ bf16x8 rd_t(const unsigned char* tile, int kk, int vb) const {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + t_roff[0][vb] + kk * 16 * RB));
    const s16x4 hi8 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + t_roff[1][vb] + kk * 16 * RB));
    const s16x8 both = __builtin_shufflevector(lo, hi8, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 x;
    __builtin_memcpy(&x, &both, sizeof x);
    return x;
  }
};

__device__ __forceinline__ bf16x8 row_chunk(const __bf16* p, bool ok) {
  bf16x8 x;
  if (ok) {
    x = *reinterpret_cast<const bf16x8*>(p);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (__bf16)0.0f;
  }
  return x;
}

// ------------------------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
  using M = TileMap<D, BT>;
  constexpr int NH = BT / 32;   // 32-key halves of a streamed tile
  constexpr int KS = M::KS, VB = M::VB, RB = M::RB;
  __shared__ __attribute__((aligned(16))) unsigned char k_t0[BT * RB];
  __shared__ __attribute__((aligned(16))) unsigned char k_t1[BT * RB];
  __shared__ __attribute__((aligned(16))) unsigned char v_t0[BT * RB];
  __shared__ __attribute__((aligned(16))) unsigned char v_t1[BT * RB];
  unsigned char* const k_tiles[2] = {k_t0, k_t1};
  unsigned char* const v_tiles[2] = {v_t0, v_t1};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int n_qt = (p.n_q + BO - 1) / BO;
  const int total = gridDim.x;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int g_in = L % p.group;
  L /= p.group;
  const int qt = n_qt - 1 - (L % n_qt);
  L /= n_qt;
  const int g = L % p.kv_heads;
  const int b = L / p.kv_heads;
  const int h = g * p.group + g_in;
  const int i0 = qt * BO, i1 = min(i0 + BO, p.n_q);
  const int kt_live = tiles_live(i0, i1, p.diag, p.n_k, BT);
  if (kt_live == 0) return;   // no allowed pair: dQ gets nothing from this block

  const int row = i0 + wave * WR + r32;
  const bool row_ok = row < p.n_q;
  const int64_t srow = ((int64_t)b * p.q_heads + h) * p.state_rows + row;
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)row * p.q_st + hi * 8;
  const __bf16* dorow = static_cast<const __bf16*>(p.d_out) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)row * p.q_st + hi * 8;
  bf16x8 qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = row_chunk(qrow + ks * 16, row_ok);
    dof[ks] = row_chunk(dorow + ks * 16, row_ok);
  }
  // +inf for a row outside the launch or one that saw no key in the forward: 2^(x - lse) = 0
  float lse2 = row_ok ? p.lse[srow] * kLog2e : INFINITY;
  if (lse2 == -INFINITY) lse2 = INFINITY;
  const float Dr = row_ok ? p.D[srow] : 0.f;
  const float c2 = p.scale * kLog2e;

  M map;
  const int row_bytes = (int)(p.k_st * 2);
  map.init(lane, wave, row_bytes);
  const __bf16* kg = static_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const __bf16* vg = static_cast<const __bf16*>(p.v) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;

  f32x16 dq[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int j = 0; j < 16; ++j) dq[vb][j] = 0.f;

  auto step = [&](auto bufc, int kt) {
    constexpr int B = decltype(bufc)::value;
    // next tile into the other buffer (past the last live tile: zeros or unused keys)
    map.load(k_tiles[1 - B], kg, (int64_t)(kt + 1) * BT, p.n_k, p.k_st, wave, row_bytes);
    map.load(v_tiles[1 - B], vg, (int64_t)(kt + 1) * BT, p.n_k, p.k_st, wave, row_bytes);
    const unsigned char* kt_b = k_tiles[B];
    const unsigned char* vt_b = v_tiles[B];
    // the element mask only on tiles that cross the diagonal or the block's end for some row of
    // the wave
    const bool full = (kt + 1) * BT - 1 <= i0 + wave * WR + p.diag && (kt + 1) * BT <= p.n_k;
    const int lim = min(row + p.diag, p.n_k - 1) - kt * BT - 4 * hi;
    // The scores and dP of both 32-key halves first (four independent MFMA chains), then per
    // half the probabilities, dS and that half's share of dQ, so that the second half's softmax
    // can issue under the first half's dQ products.  From the first half's dQ products to the
    // end of the tile the wave runs at raised priority: of the two waves on a SIMD, the one with
    // products to issue goes first while the other forms its probabilities.
    f32x16 s[NH], dp[NH];
#pragma unroll
    for (int kh = 0; kh < NH; ++kh)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kh][j] = dp[kh][j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kh = 0; kh < NH; ++kh) {
        s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(map.rd(kt_b, ks, kh), qf[ks], s[kh], 0, 0, 0);
        dp[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(map.rd(vt_b, ks, kh), dof[ks], dp[kh], 0, 0, 0);
      }
    // lane holds keys 32*kh + 8*(j/4) + 4*hi + (j%4) of this row.  dS is left unscaled here
    // (bf16 keeps the same relative precision either way); dQ takes the softmax scale once, at
    // the end.
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kh][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kh][j], c2, -lse2));
      if (!full) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * kh + 8 * (j >> 2) + (j & 3) > lim) s[kh][j] = 0.f;
      }
      bf16x8 dsk[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) dsk[j >> 3][j & 7] = (__bf16)(s[kh][j] * (dp[kh][j] - Dr));
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
          dq[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(map.rd_t(kt_b, 2 * kh + k2, vb), dsk[k2], dq[vb], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of the next tile
    __syncthreads();
  };

  map.load(k_tiles[0], kg, 0, p.n_k, p.k_st, wave, row_bytes);
  map.load(v_tiles[0], vg, 0, p.n_k, p.k_st, wave, row_bytes);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int kt = 0; kt < kt_live; kt += 2) {
    step(ic<0>{}, kt);
    if (kt + 1 < kt_live) step(ic<1>{}, kt + 1);
  }

  if (row_ok) {
    float* op = p.dq + srow * D + 4 * hi;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float4* q4 = reinterpret_cast<float4*>(op + vb * 32 + 8 * a);
        float4 x = *q4;
        x.x += dq[vb][4 * a + 0] * p.scale;
        x.y += dq[vb][4 * a + 1] * p.scale;
        x.z += dq[vb][4 * a + 2] * p.scale;
        x.w += dq[vb][4 * a + 3] * p.scale;
        *q4 = x;
      }
  }
}

// ------------------------------------------------------------------------------------------
// Key-stationary kernel: a workgroup of 4 waves owns 128 keys of one KV head, 32 per wave, and
// walks the query rows of every query head that reads that KV head.  Per streamed tile of 32
// query rows it forms S = Q K^T and dP = dO V^T once, then P and dS in registers, and
// accumulates both dV^T += dO^T P and dK^T += Q^T dS (the transposed Q and dO operands from
// the same LDS tiles by ds_read_b64_tr_b16): 8 d flops per pair where separate dV and dK
// passes took 10 d.  K stays in registers as the score product's B operand; V, the dP
// product's B operand, is parked in LDS (one 1 KB fragment per wave and k-step, read back per
// tile), which frees the registers the second accumulator needs at two waves per SIMD.
constexpr int kBwdTileDq = 64, kBwdTileKv = 32;   // streamed tile rows of each kernel

template <int D, int BT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_kv_kernel(BwdParams p) {
  constexpr int KW = 32;        // keys per wave
  constexpr int KO = 4 * KW;    // keys per workgroup
  constexpr int NH = BT / 32;   // 32-row halves of a streamed tile
  using M = TileMap<D, BT>;
  constexpr int KS = M::KS, VB = M::VB, RB = M::RB;
  __shared__ __attribute__((aligned(16))) unsigned char q_t0[BT * RB];
  __shared__ __attribute__((aligned(16))) unsigned char q_t1[BT * RB];
  __shared__ __attribute__((aligned(16))) unsigned char o_t0[BT * RB];
  __shared__ __attribute__((aligned(16))) unsigned char o_t1[BT * RB];
  __shared__ __attribute__((aligned(16))) float lse_t[2][BT];
  __shared__ __attribute__((aligned(16))) float d_t[2][BT];
  __shared__ __attribute__((aligned(16))) unsigned char v_park[4 * KS * 1024];
  unsigned char* const q_tiles[2] = {q_t0, q_t1};
  unsigned char* const o_tiles[2] = {o_t0, o_t1};
  typedef __attribute__((address_space(3))) const volatile bf16x8 lds_cvbf16x8;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int n_kt = (p.n_k + KO - 1) / KO;
  const int total = gridDim.x;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int kt = L % n_kt;
  L /= n_kt;
  const int g = L % p.kv_heads;
  const int b = L / p.kv_heads;
  const int t0 = kt * KO;
  // query rows that can see some key of this workgroup: i >= t0 - diag
  const int i_first = max(0, t0 - p.diag);
  if (i_first >= p.n_q) return;
  const int r_start = (i_first / BT) * BT;
  const int n_rt = (p.n_q - r_start + BT - 1) / BT;   // query tiles per head
  const int n_it = n_rt * p.group;                     // over every head of the group

  const int key = t0 + wave * KW + r32;
  const bool key_ok = key < p.n_k;
  bf16x8 kf[KS];
  {
    const int64_t row = (int64_t)b * p.k_sb + (int64_t)g * p.k_sh + (int64_t)key * p.k_st + hi * 8;
    const __bf16* krow = static_cast<const __bf16*>(p.k) + row;
    const __bf16* vrow = static_cast<const __bf16*>(p.v) + row;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = row_chunk(krow + ks * 16, key_ok);
      *reinterpret_cast<bf16x8*>(v_park + (wave * KS + ks) * 1024 + lane * 16) = row_chunk(vrow + ks * 16, key_ok);
    }
  }
  const float c2 = p.scale * kLog2e;
  M map;
  const int row_bytes = (int)(p.q_st * 2);
  map.init(lane, wave, row_bytes);

  f32x16 acck[VB], accv[VB];   // dK^T and dV^T of the wave's 32 keys
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      acck[vb][j] = 0.f;
      accv[vb][j] = 0.f;
    }

  // iteration u: head g*group + u / n_rt, query rows r_start + (u % n_rt) * BT ..
  // The tile copies (the next tile past the last: a clamped head, never computed).
  auto stage = [&](int buf, int u) {
    const int hh = u / n_rt;
    const int r0 = r_start + (u % n_rt) * BT;
    const int h = g * p.group + (hh < p.group ? hh : p.group - 1);
    const __bf16* qb = static_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    const __bf16* ob = static_cast<const __bf16*>(p.d_out) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    map.load(q_tiles[buf], qb, r0, p.n_q, p.q_st, wave, row_bytes);
    map.load(o_tiles[buf], ob, r0, p.n_q, p.q_st, wave, row_bytes);
  };
  // The tile's lse and D rows (the first BT lanes of wave 0) go through registers: loaded
  // before the tile's copies are issued, written to LDS at the end of the step.  Loads complete
  // in order, so a wait for them that followed the copies would wait for the whole tile; the
  // loads are unconditional (a row past the launch reads nothing and returns 0), so that no
  // branch joins their results before the end of the step.
  auto fetch_rows = [&](int u, float& l, float& dd) {
    const int hh = u / n_rt;
    const int r0 = r_start + (u % n_rt) * BT;
    const int64_t row0 = ((int64_t)b * p.q_heads + g * p.group + min(hh, p.group - 1)) * p.state_rows + r0;
    const int64_t bytes = hh < p.group ? (int64_t)min(BT, p.n_q - r0) * 4 : 0;
    l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_bwd(p.lse + row0, bytes), tid * 4, 0, 0));
    dd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_bwd(p.D + row0, bytes), tid * 4, 0, 0));
  };
  auto put_rows = [&](int buf, int u, float l, float dd) {
    const bool ok = u / n_rt < p.group && r_start + (u % n_rt) * BT + tid < p.n_q;
    // +inf for a row outside the launch or one that saw no key in the forward: 2^(x - lse) = 0
    const float l2 = l * kLog2e;
    lse_t[buf][tid] = (!ok || l2 == -INFINITY) ? INFINITY : l2;
    d_t[buf][tid] = dd;   // 0 past the launch's rows
  };

  auto step = [&](auto bufc, int u) {
    constexpr int B = decltype(bufc)::value;
    float nl, nd;
    fetch_rows(u + 1, nl, nd);
    stage(1 - B, u + 1);
    const int r0 = r_start + (u % n_rt) * BT;
    const unsigned char* qt_b = q_tiles[B];
    const unsigned char* ot_b = o_tiles[B];
    f32x16 s[NH], dp[NH];
#pragma unroll
    for (int rh = 0; rh < NH; ++rh)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[rh][j] = 0.f;
        dp[rh][j] = 0.f;
      }
    // the scores first, then dP: the exponentials need only the scores and can issue under the
    // dP products
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int rh = 0; rh < NH; ++rh)
        s[rh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(map.rd(qt_b, ks, rh), kf[ks], s[rh], 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 vb8 = *(lds_cvbf16x8*)(v_park + (wave * KS + ks) * 1024 + lane * 16);
#pragma unroll
      for (int rh = 0; rh < NH; ++rh)
        dp[rh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(map.rd(ot_b, ks, rh), vb8, dp[rh], 0, 0, 0);
    }
    // lane holds key `key` against tile rows 32*rh + 8*(j/4) + 4*hi + (j%4); a tile whose
    // first row sees the wave's last key needs no element mask
    const bool full = t0 + wave * KW + KW - 1 <= r0 + p.diag;
    const float4* lse4 = reinterpret_cast<const float4*>(&lse_t[B][0]);
    const float4* d4 = reinterpret_cast<const float4*>(&d_t[B][0]);
    // Rows past the launch carry lse = +inf (p = 0) and keys past the block only feed their
    // own, unstored, column: only tiles on the causal diagonal need the element mask, which
    // sends a score to -inf (p = 0).
    if (!full) {
#pragma unroll
      for (int rh = 0; rh < NH; ++rh)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (key > r0 + 32 * rh + 8 * (j >> 2) + 4 * hi + (j & 3) + p.diag) s[rh][j] = -INFINITY;
    }
    bf16x8 wp[2 * NH], ws[2 * NH];   // P and dS in bf16, per 16-row step; dS unscaled
    auto probs = [&](int kk) {   // rows 16kk .. 16kk+15 of the tile
      const int rh = kk >> 1;
#pragma unroll
      for (int a = 2 * (kk & 1); a < 2 * (kk & 1) + 2; ++a) {
        const float4 l4 = lse4[8 * rh + 2 * a + hi];   // rows 32rh + 8a + 4hi .. +3
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float4 dd = d4[8 * rh + 2 * a + hi];
        const float dvv[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * a + c;
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rh][j], c2, -lv[c]));
          ws[kk][j & 7] = (__bf16)(pr * (dp[rh][j] - dvv[c]));
          wp[kk][j & 7] = (__bf16)pr;
        }
      }
    };
    auto grads = [&](int kk) {   // dV^T += dO^T P; dK^T += Q^T dS for those rows
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        accv[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(map.rd_t(ot_b, kk, vb), wp[kk], accv[vb], 0, 0, 0);
        acck[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(map.rd_t(qt_b, kk, vb), ws[kk], acck[vb], 0, 0, 0);
      }
    };
    // The first 16 rows' P and dS, then at raised wave priority each 16 rows' products with the
    // next 16 rows' P and dS formed between them: of the two waves on a SIMD, the one with
    // products to issue goes first, and this wave's softmax issues under its own products.
    probs(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 2 * NH; ++kk) {
      grads(kk);
      if (kk + 1 < 2 * NH) probs(kk + 1);
    }
    __builtin_amdgcn_s_setprio(0);
    if (tid < BT) put_rows(1 - B, u + 1, nl, nd);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };

  {
    float l0, d0;
    fetch_rows(0, l0, d0);
    stage(0, 0);
    if (tid < BT) put_rows(0, 0, l0, d0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int u = 0; u < n_it; u += 2) {
    step(ic<0>{}, u);
    if (u + 1 < n_it) step(ic<1>{}, u + 1);
  }

  // dK and dV of the wave's keys, added to the travelling block's accumulators.  The address
  // comes from a copy of the lane index made here, so that it is not held through the loop.
  const int el = opaque_copy(lane);
  const int ekey = t0 + wave * KW + (el & 31);
  if (ekey < p.n_k) {
    const int64_t kbase = (((int64_t)b * p.kv_heads + g) * p.dkv_rows + ekey) * D + 4 * (el >> 5);
    auto add = [&](float* out, const f32x16* acc, float f) {
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float4* o4 = reinterpret_cast<float4*>(out + kbase + vb * 32 + 8 * a);
          float4 x = *o4;
          x.x += acc[vb][4 * a + 0] * f;
          x.y += acc[vb][4 * a + 1] * f;
          x.z += acc[vb][4 * a + 2] * f;
          x.w += acc[vb][4 * a + 3] * f;
          *o4 = x;
        }
    };
    add(p.dk, acck, p.scale);
    add(p.dv, accv, 1.f);
  }
}

template <int D>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
  const int64_t gq = (int64_t)((p.n_q + BO - 1) / BO) * p.q_heads * p.batch;
  const int64_t gkv = (int64_t)((p.n_k + 127) / 128) * p.kv_heads * p.batch;
  if (gq > 0) hipLaunchKernelGGL((bwd_dq_kernel<D, kBwdTileDq>), dim3((unsigned)gq), dim3(NT), 0, stream, p);
  if (gkv > 0) hipLaunchKernelGGL((bwd_kv_kernel<D, kBwdTileKv>), dim3((unsigned)gkv), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_step_bf16(const BwdParams& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
