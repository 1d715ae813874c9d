// ra_step_bf16.hip -- the bf16 step kernel for gfx950: score a resident query slice
// against one KV block on the matrix cores and merge the result into the per-row
// online-softmax state, in registers.
//
// What it computes ("GPU ring attention", section "Why partial results are allowed to
// merge"; "Ring Attention：把超长序列沿设备环流动", sections 局部 Softmax 为什么不能直接相加 and
// 两层分块如何嵌套, the kernel updating the local accumulator directly): for every query row
// of the tile, with x = log2(e) * scale * <q, k> over the block's visible keys,
//     m'  = max(m, max x),   a = 2^(m - m'),
//     l'  = a * l + sum 2^(x - m'),   O~' = a * O~ + sum 2^(x - m') v.
//
// Design (gfx950, wave64, 160 KB LDS per CU):
//  * A workgroup of 4 waves owns a 128-row query tile of one head; each wave owns 32 rows
//    and keeps their q (as the MFMA B operand) and O~ (fp32 accumulators) in registers for
//    the whole block.  Grid order is XCD-aware: workgroups that read the same KV head are
//    dispatched to the same XCD, heaviest query tiles first.
//  * Keys stream through LDS in 64-key tiles, double-buffered: the next tile's global loads
//    (16-byte K rows, 8-byte V rows, all coalesced) are in flight while the current tile is
//    on the matrix cores; one barrier per tile.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as operand A, q from registers as operand B), so each lane ends up holding 16 keys of
//    one query row: the row max and row sum need only in-lane work plus one
//    v_permlane32_swap with the partner lane.
//  * The probabilities are rounded to bf16 in registers and reused directly as operand B of
//    O~^T += V^T P^T.  V^T operand A comes from an LDS copy of V that is transposed (by
//    v_perm_b32 in registers) on its way in, in the same permuted key order the score layout
//    produces, so no data moves between lanes.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that both the staging writes and the
//    operand reads hit distinct banks.
//  * Causal skipping: the workgroup visits only the key tiles that hold an allowed pair
//    and applies the element mask only on tiles that cross the diagonal or pass the
//    block's end (ra_pos.h).

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_pos.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int BQ = kBf16TileQ;  // 128 query rows per workgroup
constexpr int BK = kBf16TileK;  // 64 keys per LDS tile
constexpr int NT = 256;         // 4 waves
constexpr int WROWS = 32;       // query rows per wave

template <int D>
struct Lds {
  static constexpr int K_BYTES = BK * D * 2;  // K tile [BK][D], row = D*2 bytes
  static constexpr int V_BYTES = D * BK * 2;  // V^T tile [D][BK], row = 128 bytes
  static constexpr int BUF = K_BYTES + V_BYTES;
};

// byte offset of 16-byte chunk c (dims 8c..8c+7) of key row t in the K tile
template <int D>
__device__ __forceinline__ int k_off(int t, int c) {
  return t * (D * 2) + ((c ^ (t & 7)) << 4);
}
// byte offset of chunk ch (= 2*kk + h, eight keys) of value row dv in the V^T tile; the
// swizzle depends on dv mod 32 only, so the four 32-row blocks differ by a constant
__device__ __forceinline__ int v_off(int dv, int ch) {
  const int r = dv & 31;
  return dv * (BK * 2) + ((ch ^ ((r + (r >> 3)) & 7)) << 4);
}

// (value of this lane, value of lane ^ 32) in either order: enough for max and sum
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Buffer resource over [base, base + bytes): loads past the end return zero, which is how
// the tail of a block is padded without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// The running maximum may lag the true one by up to this much (base 2) before O~ and l are
// rescaled: every term 2^(x - m) then stays <= 2^8, and most tiles skip the rescale.
constexpr float kLagMax = 8.0f;

template <int D, bool DEBUG>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void step_bf16_kernel(StepParams p) {
  constexpr int KS = D / 16;           // k-steps of the score contraction
  constexpr int VB = D / 32;           // 32-wide blocks of the value dimension
  constexpr int KCH = D / 8;           // 16-byte chunks per K row
  constexpr int KPT = BK * KCH / NT;   // 16-byte K chunks staged per thread
  constexpr int KROWS = NT / KCH;      // K rows covered by one staging pass of the workgroup
  constexpr int BUF = Lds<D>::BUF;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * BUF];
  __shared__ unsigned long long dbg_acc;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  // ---- which (batch, head, query tile) this workgroup owns --------------------------
  const int n_qt = (p.n_q + BQ - 1) / BQ;
  const int total = gridDim.x;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);  // same XCD -> same KV head
  const int g_in = L % p.group;
  L /= p.group;
  const int qt = n_qt - 1 - (L % n_qt);                            // heaviest tiles first
  L /= n_qt;
  const int kvh = L % p.kv_heads;
  const int b = L / p.kv_heads;
  const int h = kvh * p.group + g_in;

  const int i0 = qt * BQ;
  const int i1 = min(i0 + BQ, p.n_q);
  const int kt_live = tiles_live(i0, i1, p.diag, p.n_k, BK);
  const int kt_full = tiles_full(i0, i1, p.diag, p.n_k, BK);
  if (!p.fresh && kt_live == 0) return;  // nothing visible: state unchanged

  const int qrow = i0 + wave * WROWS + r32;
  const bool row_ok = qrow < p.n_q;
  const int64_t srow = ((int64_t)b * p.q_heads + h) * p.n_q + qrow;

  if (DEBUG && tid == 0) dbg_acc = 0;

  // ---- resident operands and state ---------------------------------------------------
  bf16x8 qf[KS];
  {
    const __bf16* qp = static_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb +
                       (int64_t)h * p.q_sh + (int64_t)qrow * p.q_st + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row_ok) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.0f;
      }
    }
  }

  f32x16 oacc[VB];
  float m_run, l_run;
  if (p.fresh || !row_ok) {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[vb][j] = 0.f;
  } else {
    m_run = p.m[srow];
    l_run = p.l[srow];
    const float* op = p.o_acc + srow * D + 4 * hi;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 x = *reinterpret_cast<const float4*>(op + vb * 32 + 8 * a);
        oacc[vb][4 * a + 0] = x.x;
        oacc[vb][4 * a + 1] = x.y;
        oacc[vb][4 * a + 2] = x.z;
        oacc[vb][4 * a + 3] = x.w;
      }
  }

  // ---- staging: global -> registers -> LDS -------------------------------------------
  const __bf16* kg = static_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const __bf16* vg = static_cast<const __bf16*>(p.v) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const int row_bytes = (int)(p.k_st * 2);        // host guarantees BK rows fit in 31 bits
  // K: thread stages chunk (tid % KCH) of rows tid / KCH + u * KROWS
  const int k_goff = (tid / KCH) * row_bytes + (tid % KCH) * 16;
  const int k_woff = k_off<D>(tid / KCH, tid % KCH);   // + u * KROWS rows (a multiple of 8)
  // V: thread stages value dims 4*vdg..4*vdg+3 of the eight keys of group vkh (kk = vkh>>1,
  // half = vkh&1), in the permuted key order of the score layout; for D = 64 two threads
  // share each task and write identical data
  const int vdg = tid % (D / 4);
  const int vkh = (tid / (D / 4)) & 7;
  const int v_goff = (16 * (vkh >> 1) + 4 * (vkh & 1)) * row_bytes + vdg * 8;
  int v_woff[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v_woff[e] = Lds<D>::K_BYTES + v_off(vdg * 4 + e, vkh);
  // operand reads: loop-invariant per lane
  int k_roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_roff[ks] = k_off<D>(r32, 2 * ks + hi);
  int v_roff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) v_roff[kk] = Lds<D>::K_BYTES + v_off(r32, 2 * kk + hi);

  u32x4 kreg[KPT];
  u32x2 vreg[8];

  auto load_tile = [&](int kt) {
    const int64_t t0 = (int64_t)kt * BK;
    const int64_t bytes = ((int64_t)p.n_k - t0) * p.k_st * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + t0 * p.k_st, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + t0 * p.k_st, bytes);
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      kreg[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_goff, u * KROWS * row_bytes, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      vreg[q] = __builtin_amdgcn_raw_buffer_load_b64(rv, v_goff, ((q & 3) + 8 * (q >> 2)) * row_bytes, 0);
  };
  auto store_tile = [&](auto bufc) {
    constexpr int B = decltype(bufc)::value;
    unsigned char* base = lds + B * BUF;
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      *reinterpret_cast<u32x4*>(base + k_woff + u * KROWS * D * 2) = kreg[u];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x4 w;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        w[m] = __builtin_amdgcn_perm(vreg[2 * m + 1][e >> 1], vreg[2 * m][e >> 1], sel);
      *reinterpret_cast<u32x4*>(base + v_woff[e]) = w;
    }
  };

  const float c2 = p.scale_log2;
  unsigned long long my_pairs = 0;

  // one key tile from LDS buffer B: scores, mask, online softmax, value product
  auto compute_tile = [&](auto bufc, int kt) {
    constexpr int B = decltype(bufc)::value;
    const unsigned char* base = lds + B * BUF;

    // S^T = K Q^T: lane holds keys 8*(j/4) + 4*hi + (j%4) (+32*kh) of query row r32
    f32x16 sacc[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[kh][j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + k_roff[ks] + kh * 32 * D * 2);
        sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kh], 0, 0, 0);
      }
    }

    // element mask on tiles that cross the diagonal or run past the block's end
    if ((kt >= kt_full) || ((kt + 1) * BK > p.n_k)) {
      const int lim = min(qrow + p.diag, p.n_k - 1) - kt * BK - 4 * hi;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          sacc[kh][j] = (kh * 32 + 8 * (j >> 2) + (j & 3) > lim) ? -INFINITY : sacc[kh][j];
    }
    if (DEBUG && row_ok) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int j = 0; j < 16; ++j) my_pairs += (sacc[kh][j] != -INFINITY) ? 1 : 0;
    }

    // row max over the 64 keys: 32 in-lane values, then the partner lane
    float mx = sacc[0][0];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kh][j]);
    {
      float a, bb;
      pair32(mx, a, bb);
      mx = fmaxf(a, bb);
    }
    // move the reference maximum only when some row of the wave grew by more than kLagMax
    const float m_tile = mx * c2;
    const bool grow = m_tile > m_run + kLagMax;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // rows that do not grow keep their reference (alpha = 1; this also keeps a row that
      // has seen no key yet at -inf without forming -inf - -inf); a growing row from
      // -inf gets alpha = 0 on its empty accumulators
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int vb2 = 0; vb2 < VB; ++vb2)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[vb2][j] *= alpha;
      m_run = grow ? m_tile : m_run;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // probabilities, rounded to bf16: the B operand of the value product; the row sum
    // adds the same rounded values (v_dot2 with ones), so the weights used for O~ and for
    // l agree exactly and a row with a single visible key normalises to exactly 1
    bf16x8 pk[4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        pk[2 * kh + (j >> 3)][j & 7] =
            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kh][j], c2, -m_use));
    float rs = 0.f;
    {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 0, 1), ones, rs, false);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 2, 3), ones, rs, false);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 4, 5), ones, rs, false);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 6, 7), ones, rs, false);
      }
    }
    {
      float a, bb;
      pair32(rs, a, bb);
      rs = a + bb;
    }
    l_run += rs;

    // O~^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int vb2 = 0; vb2 < VB; ++vb2) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + v_roff[kk] + vb2 * 32 * BK * 2);
        oacc[vb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], oacc[vb2], 0, 0, 0);
      }
    }
  };

  // one pipeline step: prefetch tile kt+1 to registers, compute tile kt from buffer B,
  // stage tile kt+1 into the other buffer, barrier.  The prefetch and the staging are
  // unconditional (after the last live tile they fetch zeros or unused keys into the idle
  // buffer): with no branch around them the loads are waited for only at the LDS stores,
  // so the whole tile computation overlaps them.
  auto step = [&](auto bufc, int kt) {
    constexpr int B = decltype(bufc)::value;
    load_tile(kt + 1);
    compute_tile(bufc, kt);
    store_tile(std::integral_constant<int, 1 - B>{});
    __syncthreads();
  };

  load_tile(0);
  store_tile(std::integral_constant<int, 0>{});
  __syncthreads();
  for (int kt = 0; kt < kt_live; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < kt_live) step(std::integral_constant<int, 1>{}, kt + 1);
  }

  // ---- write the state back ----------------------------------------------------------
  if (row_ok) {
    if (hi == 0) {
      p.m[srow] = m_run;
      p.l[srow] = l_run;
    }
    float* op = p.o_acc + srow * D + 4 * hi;
#pragma unroll
    for (int vb2 = 0; vb2 < VB; ++vb2)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(op + vb2 * 32 + 8 * a) =
            make_float4(oacc[vb2][4 * a + 0], oacc[vb2][4 * a + 1], oacc[vb2][4 * a + 2],
                        oacc[vb2][4 * a + 3]);
  }

  if (DEBUG) {
    if (my_pairs) atomicAdd(&dbg_acc, my_pairs);
    __syncthreads();
    if (tid == 0) {
      atomicAdd(&p.dbg[0], (unsigned long long)kt_full);
      atomicAdd(&p.dbg[1], (unsigned long long)(kt_live - kt_full));
      atomicAdd(&p.dbg[2], dbg_acc);
    }
  }
}

template <int D>
hipError_t launch_d(const StepParams& p, hipStream_t stream) {
  const int n_qt = (p.n_q + BQ - 1) / BQ;
  const int64_t grid = (int64_t)n_qt * p.q_heads * p.batch;
  if (grid == 0) return hipSuccess;
  if (p.dbg)
    hipLaunchKernelGGL((step_bf16_kernel<D, true>), dim3((unsigned)grid), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((step_bf16_kernel<D, false>), dim3((unsigned)grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bf16(const StepParams& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
