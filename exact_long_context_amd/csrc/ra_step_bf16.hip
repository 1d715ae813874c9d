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
//  * Keys stream through LDS in 64-key tiles, double-buffered, copied straight from HBM
//    with buffer_load ... lds (no registers, no VALU): the next tiles' copies are in flight
//    while the current tile is on the matrix cores; one barrier per tile.  K runs one tile
//    ahead of V, so the scores of tile kt+1 overlap the probabilities of tile kt.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as operand A, q from registers as operand B), so each lane ends up holding 16 keys of
//    one query row per 32 keys: the row max and row sum need only in-lane work plus one
//    v_permlane32_swap with the partner lane.
//  * The probabilities are rounded to bf16 in registers and reused directly as operand B of
//    O~^T += V^T P^T.  V stays untransposed in LDS; operand A is read with
//    ds_read_b64_tr_b16, which transposes 16-bit elements within 16-lane groups and hands
//    each lane the keys in the permuted order the score layout produces, so no data moves
//    between lanes.
//  * LDS rows are XOR-swizzled in 16-byte chunks for gfx950's 64 banks, so that both the
//    direct copies and the operand reads hit distinct banks.
//  * The reference m of a row may lag its true maximum: a tile's terms 2^(x - m) are taken
//    as they come while their row sum stays <= 2^32.  The row maximum is computed, and O~
//    and l rescaled, only for a row past that bound or one setting its first reference,
//    which in practice is the first visible tile of each row.
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

constexpr int BQ = kBf16TileQ;
constexpr int BK = kBf16TileK;
constexpr int NT = 256;         // 4 waves
constexpr int WROWS = 32;       // query rows per wave


// LDS banking on gfx950: 64 banks of 4 bytes (a 256-byte bank line).  A 16-byte-per-lane
// access is served 16 lanes at a time and an 8-byte-per-lane access 32 lanes at a time, so
// those lanes must touch distinct banks.
//
// Tiles are written straight from global memory into LDS (buffer_load ... lds: lane i of a
// load writes bytes [16i, 16i+16) after the instruction's LDS base), so the swizzles below
// are realised by choosing which 16-byte global chunk each lane fetches.

// K tile [BK][D] bf16: physical 16-byte chunk of logical chunk c (dims 8c..8c+7) of key
// row t.  The score operand read (16 consecutive rows at one chunk) hits 16 groups.
template <int D>
__device__ __forceinline__ int k_phys(int t, int c) {
  if constexpr (D == 128) return c ^ (t & 15);
  else return c ^ ((t >> 1) & 7);
}
// V tile [BK][D] bf16, kept untransposed: the value operand is read with
// ds_read_b64_tr_b16, whose 16-lane groups fetch four consecutive keys x four 8-byte
// column pieces; the chunk twist below puts those 16 pieces (32 lanes: 256 bytes) on
// distinct banks.
template <int D>
__device__ __forceinline__ int v_phys(int t, int c) {
  if constexpr (D == 128) return c ^ (4 * (t & 3));
  else return c ^ (4 * ((t >> 1) & 1));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS at lds + 16 * lane (the LDS address is
// taken from the first lane).  Kept out of the kernel template: the builtin has no host
// form, and inside the template it would stop the host side from emitting the launch stub.
__device__ __forceinline__ void load_lds_b128_inl(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
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

// The reference m of a row may lag its true maximum: a tile's terms 2^(x - m) are used as
// they come as long as their row sum stays <= 2^32 (so every term does), which fp32 and bf16
// hold without loss; only a row past that, or one setting its first reference, takes the
// tile's maximum.  Most tiles compute no maximum at all.
constexpr float kSumMax = 4294967296.0f;   // 2^32


template <int D, bool DEBUG>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void step_bf16_kernel(StepParams p) {
  constexpr int KS = D / 16;             // k-steps of the score contraction
  constexpr int VB = D / 32;             // 32-wide blocks of the value dimension
  constexpr int RB = D * 2;              // bytes per key row in LDS
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int RPL = 64 / CPR;          // key rows per 1 KB direct load (one wave)
  constexpr int LPW = BK * RB / 1024 / 4;  // direct loads per wave per tile, per tensor
  // K tiles and V tiles, two of each, as separate objects so that the compiler can tell the
  // tile being read from the one a direct load is filling.  K runs one tile ahead of V:
  // while tile kt's probabilities are formed, tile kt+1's scores are on the matrix cores.
  __shared__ __attribute__((aligned(16))) unsigned char k_t0[BK * D * 2];
  __shared__ __attribute__((aligned(16))) unsigned char k_t1[BK * D * 2];
  __shared__ __attribute__((aligned(16))) unsigned char v_t0[BK * D * 2];
  __shared__ __attribute__((aligned(16))) unsigned char v_t1[BK * D * 2];
  __shared__ unsigned long long dbg_acc[2];
  unsigned char* const k_tiles[2] = {k_t0, k_t1};
  unsigned char* const v_tiles[2] = {v_t0, v_t1};
#define ktile(bufc) (k_tiles[decltype(bufc)::value])
#define vtile(bufc) (v_tiles[decltype(bufc)::value])

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS bases
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
  const int64_t srow = ((int64_t)b * p.q_heads + h) * p.state_rows + qrow;

  if (DEBUG && tid < 2) dbg_acc[tid] = 0;

  // ---- staging: global -> LDS directly ------------------------------------------------
  const __bf16* kg = static_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const __bf16* vg = static_cast<const __bf16*>(p.v) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const int row_bytes = (int)(p.k_st * 2);        // host guarantees BK rows fit in 31 bits
  // Load u of wave w covers key rows (w*LPW + u)*RPL .. +RPL-1; lane -> (row, physical
  // chunk) = (lane / CPR, lane % CPR) of that span; the global chunk is the inverse swizzle.
  int k_goff[LPW], v_goff[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int t = (wave * LPW + u) * RPL + lane / CPR;
    const int pc = lane % CPR;
    int ck = 0, cv = 0;   // logical chunks whose physical slot is pc (the swizzles are involutions)
    ck = k_phys<D>(t, pc);
    cv = v_phys<D>(t, pc);
    k_goff[u] = (lane / CPR) * row_bytes + ck * 16;
    v_goff[u] = (lane / CPR) * row_bytes + cv * 16;
  }
  auto rsrc_of = [&](const __bf16* base, int kt) {
    const int64_t t0 = (int64_t)kt * BK;
    return make_rsrc(base + t0 * p.k_st, ((int64_t)p.n_k - t0) * p.k_st * 2);
  };
  auto load_k = [&](auto bufc, int kt) {
    const __amdgpu_buffer_rsrc_t r = rsrc_of(kg, kt);
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int row0 = (wave * LPW + u) * RPL;
      load_lds_b128_inl(r, ktile(bufc) + row0 * RB, k_goff[u], row0 * row_bytes);
    }
  };
  auto load_v = [&](auto bufc, int kt) {
    const __amdgpu_buffer_rsrc_t r = rsrc_of(vg, kt);
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int row0 = (wave * LPW + u) * RPL;
      load_lds_b128_inl(r, vtile(bufc) + row0 * RB, v_goff[u], row0 * row_bytes);
    }
  };

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
  float m_run, l_run;   // m_run: the finite reference of l and O~ (0 before any key)
  if (p.fresh || !row_ok) {
    m_run = 0.f;
    l_run = 0.f;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[vb][j] = 0.f;
  } else {
    m_run = p.m[srow];
    l_run = p.l[srow];
    if (m_run == -INFINITY) m_run = 0.f;
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

  // operand reads: loop-invariant per-lane byte offsets inside one tile
  int k_roff[KS];   // score operand A: key row kh*32 + r32, chunk 2*ks + hi
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_roff[ks] = r32 * RB + (k_phys<D>(r32, 2 * ks + hi) << 4);
  // value operand A via ds_read_b64_tr_b16: in each 16-lane group, lane 4a+c receives
  // element c of the 8-byte pieces addressed by lanes a, a+4, a+8, a+12.  Lane j = 16g+a+4e
  // therefore addresses key 16*kk + 4*(g>>1) + 8*half + e, value dims
  // 32*vb + 16*(g&1) + 4*a .. +3, which hands lane l the transposed operand for value row
  // 32*vb + (l & 31), keys 16*kk + 4*(l>>5) + {0,1,2,3} (half 0) and +8 (half 1): the key
  // order of the score layout.
  int v_roff[VB];
  {
    const int g = lane >> 4, a = lane & 3, e = (lane >> 2) & 3;
    const int key = 4 * (g >> 1) + e;   // + 16*kk + 8*half: multiples of 4 (immediates)
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int dv = 32 * vb + 16 * (g & 1) + 4 * a;
      v_roff[vb] = key * RB + (v_phys<D>(key, dv >> 3) << 4) + ((dv & 7) << 1);
    }
  }

  // S^T = K Q^T for the K tile in buffer B: lane holds keys 8*(j/4) + 4*hi + (j%4) (+32*kh)
  // of query row r32
  auto scores = [&](auto bufc, f32x16 (&sacc)[2]) {
    const unsigned char* kt_base = ktile(bufc);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt_base + k_roff[ks] + kh * 32 * RB);
        sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? f32x16{} : sacc[kh], 0, 0, 0);
      }
    }
  };

  const float c2 = p.scale_log2;
  unsigned long long my_pairs = 0;
  unsigned my_moves = 0;   // tiles in which this lane's row, already holding keys, moved its reference

  // softmax of tile kt (scores in sacc) merged into the state, while the scores of tile
  // kt+1 (K buffer KN) go onto the matrix cores; then O~ += V^T P^T from V buffer VBF
  auto tile = [&](auto knext, auto vbuf, int kt, f32x16 (&sacc)[2], f32x16 (&snext)[2]) {
    const unsigned char* vt_base = vtile(vbuf);
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

    // the next tile's scores: independent of everything below, so the matrix cores work
    // on them while the vector unit forms this tile's probabilities
    scores(knext, snext);

    // probabilities 2^(x - m_run), rounded to bf16: the B operand of the value product; the
    // row sum adds the same rounded values (v_dot2 with ones), so the weights used for O~ and
    // for l agree exactly and a row with a single visible key normalises to exactly 1.  The
    // sum also guards the reference: a row whose sum exceeds kSumMax grew too far above
    // m_run, and a row that has seen nothing (l = 0) but has a visible key here must set its
    // reference first.  Only then is the tile's maximum taken.
    bf16x8 pk[4];
    auto probs = [&](float shift) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          pk[2 * kh + (j >> 3)][j & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kh][j], c2, -shift));
      float r = 0.f;
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 0, 1), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 2, 3), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 4, 5), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 6, 7), ones, r, false);
      }
      float a, bb;
      pair32(r, a, bb);
      return a + bb;
    };
    float rs = probs(m_run);
    const bool visible = kt * BK <= qrow + p.diag;
    const bool bad = !(rs <= kSumMax) || (l_run == 0.f && visible);
    if (__builtin_amdgcn_ballot_w64(bad)) {
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
      // a bad row moves its reference to the tile's maximum: l and O~ scale by 2^-shift
      // (a row that has seen nothing holds zeros and takes 0: 2^-shift may overflow there)
      // and this tile's probabilities are formed again
      const float shift = (bad && mx != -INFINITY) ? mx * c2 - m_run : 0.f;
      const float alpha = l_run == 0.f ? 0.f : __builtin_amdgcn_exp2f(-shift);
      if (DEBUG && row_ok && hi == 0 && bad && l_run != 0.f) ++my_moves;
      l_run *= alpha;
#pragma unroll
      for (int vb2 = 0; vb2 < VB; ++vb2)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[vb2][j] *= alpha;
      m_run += shift;
      rs = probs(m_run);
    }
    l_run += rs;

    // O~^T += V^T P^T; the transposed value operand comes from two transposing reads
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int vb2 = 0; vb2 < VB; ++vb2) {
        const unsigned char* base = vt_base + v_roff[vb2] + kk * 16 * RB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi8 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * RB));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 both = __builtin_shufflevector(lo, hi8, 0, 1, 2, 3, 4, 5, 6, 7);
        bf16x8 a;
        __builtin_memcpy(&a, &both, sizeof a);
        oacc[vb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], oacc[vb2], 0, 0, 0);
      }
    }
  };

  // One pipeline step for tile kt (B = kt & 1): K tile kt+1 is in K buffer 1-B, V tile kt
  // in V buffer B.  Start the direct loads of K tile kt+2 into K buffer B and V tile kt+1
  // into V buffer 1-B (both last read in the previous step), run the tile, wait for the
  // loads, barrier.  The loads are unconditional: past the last live tile they fetch
  // zeros or unused keys into buffers nobody reads.
  f32x16 sa[2], sb[2];
  auto step = [&](auto bufc, int kt, f32x16 (&scur)[2], f32x16 (&snext)[2]) {
    constexpr int B = decltype(bufc)::value;
    load_k(bufc, kt + 2);
    load_v(std::integral_constant<int, 1 - B>{}, kt + 1);
    tile(std::integral_constant<int, 1 - B>{}, bufc, kt, scur, snext);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's direct loads have landed
    __syncthreads();
  };

  load_k(std::integral_constant<int, 0>{}, 0);
  load_v(std::integral_constant<int, 0>{}, 0);
  load_k(std::integral_constant<int, 1>{}, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  scores(std::integral_constant<int, 0>{}, sa);
  // The first step's copy of K tile 2 goes into K buffer 0, which every wave has just read
  // for tile 0's scores: no wave may start it before all of them are done.  (Later steps
  // refill a buffer read in the step before, behind that step's barrier.)
  __syncthreads();
  for (int kt = 0; kt < kt_live; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt, sa, sb);
    if (kt + 1 < kt_live) step(std::integral_constant<int, 1>{}, kt + 1, sb, sa);
  }

  // ---- write the state back ----------------------------------------------------------
  if (row_ok) {
    if (hi == 0) {
      p.m[srow] = l_run == 0.f ? -INFINITY : m_run;
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
    if (my_pairs) atomicAdd(&dbg_acc[0], my_pairs);
    if (my_moves) atomicAdd(&dbg_acc[1], (unsigned long long)my_moves);
    __syncthreads();
    if (tid == 0) {
      atomicAdd(&p.dbg[0], (unsigned long long)kt_full);
      atomicAdd(&p.dbg[1], (unsigned long long)(kt_live - kt_full));
      atomicAdd(&p.dbg[2], dbg_acc[0]);
      atomicAdd(&p.dbg[3], dbg_acc[1]);
    }
  }
#undef ktile
#undef vtile
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
