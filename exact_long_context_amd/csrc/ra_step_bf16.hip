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
//  * A workgroup of 4 waves owns a 256-row query tile of one head; each wave owns 64 rows
//    as two 32-row sub-tiles and keeps their q (MFMA B operands) and O~ (fp32 accumulators)
//    in registers for the whole block.  Every K or V operand fragment a wave reads from LDS
//    feeds both sub-tiles' products, so LDS delivers 512 bytes per 32x32x16 MFMA.  Two
//    workgroups share a CU (two waves per SIMD): one wave's products run on the matrix core
//    while the other forms its probabilities.  Grid order is XCD-aware: workgroups that read
//    the same KV head are dispatched to the same XCD, heaviest query tiles first.
//  * Keys stream through LDS in 32-key tiles, three buffers per tensor, copied straight
//    from HBM with buffer_load ... lds (no registers, no VALU) two tiles ahead; one barrier
//    per tile.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as operand A, q from registers as operand B), so each lane holds 16 keys of one query
//    row per sub-tile: the row max and row sum need only in-lane work plus one
//    v_permlane32_swap with the partner lane.
//  * The probabilities are rounded to bf16 in registers and reused directly as operand B of
//    O~^T += V^T P^T.  V stays untransposed in LDS; operand A is read with
//    ds_read_b64_tr_b16, which transposes 16-bit elements within 16-lane groups and hands
//    each lane the keys in the permuted order the score layout produces, so no data moves
//    between lanes.
//  * LDS tiles are laid out fragment by fragment (below), so every operand read is a
//    per-lane base plus an immediate and every group of lanes served together reads 256
//    contiguous bytes: no bank conflicts and no address arithmetic per read.
//  * The reference m of a row may lag its true maximum: a tile's terms 2^(x - m) are taken
//    as they come while every one of them stays <= 2^32, which one comparison of each lane's
//    largest score per tile checks.  O~ and l are rescaled only for a row past that bound or
//    one setting its first reference, which in practice is the first visible tile of each
//    row; the common path is one branch-free run of probabilities and value products.
//  * Causal skipping: the workgroup visits only the key tiles that hold an allowed pair for
//    some of its rows, a wave computes only those that hold one for its own rows, and the
//    element mask runs only on tiles that cross the diagonal or pass the block's end
//    (ra_pos.h).

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_pos.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BQ = kBf16TileQ;  // 256 query rows per workgroup
constexpr int BK = kBf16TileK;  // 32 keys per tile
constexpr int NT = 256;         // 4 waves
constexpr int WROWS = 64;       // query rows per wave: two sub-tiles of 32
static_assert(BQ == 4 * WROWS && BK == 32, "tile shape");

// LDS layouts.  Tiles are written straight from global memory into LDS (buffer_load ... lds:
// lane i of a copy writes bytes [16i, 16i+16) after the instruction's LDS base), one 1 KB
// region per copy, and each tile is laid out fragment by fragment, in the order the operand
// reads want it:
//  * K tile: for each 16-dim slice ks of the head dimension, 1 KB holding the 32 keys' dims
//    16ks..16ks+7 (512 bytes, key-major) then dims 16ks+8..16ks+15.  The score operand
//    (lane (r32, hi): key r32, dims 16ks + 8hi ..) is one 16-byte read at ks*1024 + hi*512 +
//    r32*16: every 16 lanes read 256 contiguous bytes, all 64 banks.
//  * V tile: for each 32-wide block vb of the value dimension, 2 KB holding the 32 keys' 64
//    bytes of that block, key-major.  The transposing value-operand reads of a 32-lane half
//    cover four consecutive keys' 64 bytes: 256 contiguous bytes again.
// So every operand read is a per-lane base plus an immediate, with no swizzle; the copies in
// turn fetch 32 (K) or 64 (V) bytes of each key row per instruction.

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const volatile bf16x8 lds_cvbf16x8;

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

// The reference of a row that has seen no key yet: any visible key's score is then more than
// 32 (base 2) above it, so the guard sends the row to the slow path without a test of its
// own, while masked keys (x = -inf) never trip it.
constexpr float kNoRef = -1e30f;
// Relative margin on the norms behind the tile bound: covers the fp32 rounding of |q|^2, |k|^2,
// their square roots and the score products themselves (all far below 2^-9).
constexpr float kNormMargin = 1.001953125f;   // 1 + 2^-9

// Key-tile bounds are read through the constant address space, so that each tile's bound is one
// scalar load: a vector load would count against vmcnt, and waiting for it would wait for the
// tile copies in flight as well.  no_bound stands in when a launch has no bounds: its bits
// (a NaN) exceed every threshold's as signed integers, so every tile takes the full guard.
typedef __attribute__((address_space(4))) const unsigned const_u32;
__constant__ unsigned no_bound[1] = {0x7fffffffu};
// The stored maximum of a row that has seen no key: what a fresh state's rows read.
__constant__ float no_key_m[1] = {-INFINITY};

// max(a, b, c) in one instruction (the compiler splits fmaxf chains into two-input maxima)
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// x, through an empty asm statement the compiler cannot see into: what is computed from the
// result starts here, not earlier
__device__ __forceinline__ int opaque_copy(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s_waitcnt with vmcnt = N (six bits: [3:0] and [15:14]); expcnt and lgkmcnt not waited on
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The barrier between two tiles.  This wave's copies of the next tile have landed (vmcnt: all
// but the last N copy instructions, those of the tile after it, which stay in flight) and its
// reads of the current tile are done (lgkmcnt 0); s_barrier then publishes both to every wave.
// __syncthreads() would also wait for the copies still in flight.  The empty asm statements
// keep the compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));   // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, bool DEBUG>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void step_bf16_kernel(StepParams p) {
  constexpr int KS = D / 16;             // k-steps of the score contraction
  constexpr int VB = D / 32;             // 32-wide blocks of the value dimension
  constexpr int TB = BK * D * 2;          // bytes per K or V tile
  constexpr int KPW = KS / 4;             // K copies (1 KB each) per wave per tile
  constexpr int VPW = 2 * VB / 4;         // V copies per wave per tile
  constexpr int LPW = KPW + VPW;          // copies per wave per tile
  static_assert(KPW >= 1 && VPW >= 1, "every wave copies a share of each tile");
  // Three K and three V tile buffers, as separate objects so that the compiler can tell the
  // tile being read from the ones direct loads are filling.  Tile kt sits in buffer kt % 3;
  // the copies of tile kt+2 start while tile kt is computed.
  __shared__ __attribute__((aligned(16))) unsigned char k_t0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char k_t1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char k_t2[TB];
  __shared__ __attribute__((aligned(16))) unsigned char v_t0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char v_t1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char v_t2[TB];
  // q fragment 0 of both sub-tiles of every wave, parked in LDS: read back once per tile,
  // it frees 8 registers that the tile's probabilities need
  __shared__ __attribute__((aligned(16))) unsigned char q_park[4 * 2 * 1024];
  // |q| * |c2| of every row (with a margin), read only when the wave's threshold is rebuilt
  __shared__ float qn_park[4 * 2 * 64];
  __shared__ unsigned long long dbg_acc[3];
  unsigned char* const k_tiles[3] = {k_t0, k_t1, k_t2};
  unsigned char* const v_tiles[3] = {v_t0, v_t1, v_t2};
#define ktile(bufc) (k_tiles[decltype(bufc)::value])
#define vtile(bufc) (v_tiles[decltype(bufc)::value])
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

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

  // this wave's rows [w0, w1): the key tiles it computes, and those it needs no mask on
  const int w0 = i0 + wave * WROWS;
  const int w1 = min(w0 + WROWS, p.n_q);
  const int wt_live = tiles_live(w0, w1, p.diag, p.n_k, BK);
  const int wt_full = tiles_full(w0, w1, p.diag, p.n_k, BK);

  if (DEBUG && tid < 3) dbg_acc[tid] = 0;

  // ---- staging: global -> LDS directly ------------------------------------------------
  const __bf16* kg = static_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const __bf16* vg = static_cast<const __bf16*>(p.v) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
  const int row_bytes = (int)(p.k_st * 2);        // host guarantees BK rows fit in 31 bits
  // K copy ks: lane -> key lane & 31, dims 16ks + 8(lane >> 5) ..: global offset
  // k_goff + 32ks.  V copy (vb, h): lane -> key 16h + (lane >> 2), 16-byte piece lane & 3 of
  // block vb: v_goff + 64vb + 16h*row_bytes.  Wave w issues K copies ks = w*KPW .. and V
  // copies 2vb + h = w*VPW ...
  const int k_goff = (lane & 31) * row_bytes + (lane >> 5) * 16;
  const int v_goff = (lane >> 2) * row_bytes + (lane & 3) * 16;
  auto rsrc_of = [&](const __bf16* base, int kt) {
    const int64_t t0 = (int64_t)kt * BK;
    return make_rsrc(base + t0 * p.k_st, ((int64_t)p.n_k - t0) * p.k_st * 2);
  };
  auto load_kv = [&](auto bufc, int kt) {
    const __amdgpu_buffer_rsrc_t rk = rsrc_of(kg, kt);
    const __amdgpu_buffer_rsrc_t rv = rsrc_of(vg, kt);
    // the per-copy part of each offset is wave-uniform: it goes in the scalar offset, so one
    // VGPR per tensor serves every copy
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const int ks = wave * KPW + u;
      load_lds_b128_inl(rk, ktile(bufc) + ks * 1024, k_goff, ks * 32);
    }
#pragma unroll
    for (int u = 0; u < VPW; ++u) {
      const int c = wave * VPW + u, vb = c >> 1, h = c & 1;
      load_lds_b128_inl(rv, vtile(bufc) + vb * 2048 + h * 1024, v_goff, vb * 64 + h * 16 * row_bytes);
    }
  };

  // ---- resident operands and state ---------------------------------------------------
  // Every load the workgroup needs before its first tile is issued at once, with no branch
  // between them, so that their latencies overlap: tile 0's copies, q, the state rows, then
  // tile 1's copies.  Rows past the end read as zeros or are set aside below.
  int qrow[2];
  bool row_ok[2];
  int64_t srow[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    qrow[s] = w0 + 32 * s + r32;
    row_ok[s] = qrow[s] < p.n_q;
    srow[s] = ((int64_t)b * p.q_heads + h) * p.state_rows + qrow[s];
  }
  load_kv(I0{}, 0);
  bf16x8 qf[2][KS];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    // a row past the end reads the last row (always there) and is zeroed below
    const __bf16* qp = static_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh +
                       (int64_t)min(qrow[s], p.n_q - 1) * p.q_st + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[s][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }
  // The state rows of the workgroup through buffer resources over [i0, i1): rows past the
  // end, and every row of a fresh state (a resource of no bytes), read as zeros.
  f32x16 oacc[2][VB];
  // m_run: the row's finite reference (kNoRef before any key); l_run: this lane's share of
  // the row sum (its own keys' terms), the two lanes of a row added at the end
  float m_run[2], l_run[2];
  {
    const int64_t srow0 = ((int64_t)b * p.q_heads + h) * p.state_rows + i0;
    const int n_state = p.fresh ? 0 : i1 - i0;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o_acc + srow0 * D, (int64_t)n_state * D * 4);
    // a fresh state's rows all read the one stored -inf (no key seen): a select of address
    // and offset rather than a branch, which would hold the loads after it back
    const __amdgpu_buffer_rsrc_t rm =
        n_state ? make_rsrc(p.m + srow0, (int64_t)n_state * 4) : make_rsrc(no_key_m, 4);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.l + srow0, (int64_t)n_state * 4);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = qrow[s] - i0;
      const float m0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, n_state ? r * 4 : 0, 0, 0));
      const float l0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, r * 4, 0, 0));
      // a row that has seen no key (m = -inf), or is past the end, starts with no reference
      m_run[s] = (!row_ok[s] || m0 == -INFINITY) ? kNoRef : m0;
      l_run[s] = hi == 0 ? l0 : 0.f;
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 x = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (r * D + vb * 32 + 8 * a + 4 * hi) * 4, 0, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[s][vb][4 * a + e] = x[e];
        }
    }
  }
  load_kv(I1{}, 1);

  const float c2 = p.scale_log2;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (!row_ok[s]) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][ks][e] = (__bf16)0.0f;
    }
    *reinterpret_cast<bf16x8*>(q_park + (wave * 2 + s) * 1024 + lane * 16) = qf[s][0];
    // |q|^2 of the row: this lane's half of the dims, then the partner lane's
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 x = {qf[s][ks][e], qf[s][ks][e + 1]};
        ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
      }
    float a, bb;
    pair32(ss, a, bb);
    qn_park[(wave * 2 + s) * 64 + lane] = __builtin_sqrtf(a + bb) * __builtin_fabsf(c2) * kNormMargin;
  }

  // Operand reads: one per-lane base per tensor, everything else immediate.
  //  * score operand A, fragment ks (lane (r32, hi): key r32, dims 16ks + 8hi ..):
  //    ks*1024 + kb0;
  //  * value operand A via ds_read_b64_tr_b16: in each 16-lane group, lane 4a+c receives
  //    element c of the 8-byte pieces addressed by lanes a, a+4, a+8, a+12.  Lane
  //    j = 16g+a+4e therefore addresses key 16*kk + 4*(g>>1) + 8*half + e, value dims
  //    32*vb + 16*(g&1) + 4*a .. +3, which hands lane l the transposed operand for value row
  //    32*vb + (l & 31), keys 16*kk + 4*(l>>5) + {0,1,2,3} (half 0) and +8 (half 1): the key
  //    order of the score layout.  Address vb*2048 + (16kk + 8half)*64 + vb0.
  const int kb0 = hi * 512 + r32 * 16;
  const int vb0 = (4 * (lane >> 5) + ((lane >> 2) & 3)) * 64 + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  unsigned long long my_pairs = 0;
  unsigned my_moves = 0;   // reference moves of this lane's rows that already held keys
  unsigned my_bounded = 0; // tiles of this wave whose key-norm bound made the scores' maximum moot

  // The wave's threshold on the tile bound: T = min over its rows of (32 + m) / (|q| |c2|), so
  // that a tile whose largest key norm is <= T has every score x with x c2 - m <= 32
  // (Cauchy-Schwarz: |<q, k>| <= |q| |k|).  Returned as the bits of T, which order like T
  // against any norm (>= 0) as signed integers, so the per-tile test is one scalar compare.
  // Rebuilt only when a reference moves.
  auto threshold_bits = [&]() -> int {
    float t = INFINITY;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float qn = qn_park[(wave * 2 + s) * 64 + lane];
      const float num = 32.f + m_run[s];
      const float ts = qn > 0.f ? num / qn : (num >= 0.f ? INFINITY : -INFINITY);
      t = fminf(t, ts);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t = fminf(t, __shfl_xor(t, off));
    return __builtin_amdgcn_readfirstlane(__float_as_int(t));
  };
  int t_bits = threshold_bits();
  // this launch's key-tile bounds for the workgroup's KV head
  // Without bounds every tile reads the one entry of no_bound, which no threshold passes: a
  // select instead of a branch around the load.
  const_u32* knorm_row = p.knorm ? (const_u32*)(p.knorm + (int64_t)(b * p.kv_heads + kvh) * p.knorm_stride)
                                 : (const_u32*)no_bound;
  const int kn_step = p.knorm ? 1 : 0;

  // One 32-key tile from buffer B: S^T = K Q^T for both sub-tiles (each K fragment feeds
  // both), the guard on the reference, then per 16-key half the probabilities and
  // O~^T += V^T P^T (each V fragment feeds both sub-tiles).  Working in halves keeps about one
  // half's probabilities in registers at a time (the second half's are formed while the first
  // half's products issue).
  auto tile = [&](auto bufc, int kt) {
    const unsigned char* kt_base = ktile(bufc);
    const unsigned char* vt_base = vtile(bufc);
    // the tile's key-norm bound, loaded first so that the scores hide its latency
    const int kn_bits = (int)knorm_row[__builtin_amdgcn_readfirstlane(kt * kn_step)];
    f32x16 sacc[2];
    {
      // q fragment 0 comes back from LDS (a volatile read: the compiler may not keep it in a
      // register across tiles, which is the point)
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt_base + kb0);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 qb = *(lds_cvbf16x8*)(q_park + (wave * 2 + s) * 1024 + lane * 16);
        sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb, f32x16{}, 0, 0, 0);
      }
    }
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt_base + ks * 1024 + kb0);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s][ks], sacc[s], 0, 0, 0);
    }
    // element mask on tiles that cross the diagonal or run past the block's end
    if ((kt >= wt_full) || ((kt + 1) * BK > p.n_k)) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int lim = min(qrow[s] + p.diag, p.n_k - 1) - kt * BK - 4 * hi;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          sacc[s][j] = (8 * (j >> 2) + (j & 3) > lim) ? -INFINITY : sacc[s][j];
      }
    }
    if (DEBUG) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (row_ok[s])
#pragma unroll
          for (int j = 0; j < 16; ++j) my_pairs += (sacc[s][j] != -INFINITY) ? 1 : 0;
    }

    // The guard on the reference, once per tile and before any probability is formed: every
    // term 2^(x - m_run) must stay <= 2^32 (fp32 and bf16 hold it without loss).  First the
    // tile bound: if the tile's largest key norm is within the wave's threshold, every score
    // passes and nothing is looked at (one scalar compare).  Otherwise each lane's largest score
    // is checked (fma is monotonic in x, so the largest decides); a row whose lane fails (or
    // that has no reference yet: kNoRef makes any visible score fail) moves its reference to
    // the row's maximum here, rescaling l and O~.  That is rare (in practice the first visible
    // tile of a row), so the common path is one straight run of probabilities and value
    // products with no branch.
    if (DEBUG && kn_bits <= t_bits && lane == 0) ++my_bounded;
    if (kn_bits > t_bits) {
      float mx[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float a = max3(sacc[s][0], sacc[s][1], sacc[s][2]);
#pragma unroll
        for (int j = 3; j < 15; j += 2) a = max3(a, sacc[s][j], sacc[s][j + 1]);
        mx[s] = fmaxf(a, sacc[s][15]);
      }
      const unsigned long long bad0 = __builtin_amdgcn_ballot_w64(__builtin_fmaf(mx[0], c2, -m_run[0]) > 32.f);
      const unsigned long long bad1 = __builtin_amdgcn_ballot_w64(__builtin_fmaf(mx[1], c2, -m_run[1]) > 32.f);
      if (bad0 | bad1) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const unsigned long long bad = s == 0 ? bad0 : bad1;
          // the row is bad if either of its lanes is (lane r32 and lane r32 + 32)
          const unsigned rows = (unsigned)bad | (unsigned)(bad >> 32);
          const bool row_bad = (rows >> r32) & 1u;
          float a, bb;
          pair32(mx[s], a, bb);
          const float mrow = fmaxf(a, bb);
          // a bad row moves its reference to its maximum: l and O~ scale by 2^(m_old - m_new),
          // which is 0 for a row that had no reference (its O~ and l are 0 as well)
          const float m_new = row_bad ? mrow * c2 : m_run[s];
          const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);
          if (DEBUG && row_ok[s] && hi == 0 && row_bad && m_run[s] != kNoRef) ++my_moves;
          l_run[s] *= alpha;
#pragma unroll
          for (int vb = 0; vb < VB; ++vb)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[s][vb][j] *= alpha;
          m_run[s] = m_new;
        }
        t_bits = threshold_bits();
      }
    }

    // Per 16-key half kk: the probabilities 2^(x - m_run) of keys 16kk .. 16kk+15, rounded to
    // bf16, are the B operand of the value product; this lane's share of the row sum adds the
    // same rounded values (v_dot2 with ones), so the weights used for O~ and for l agree exactly
    // and a row with a single visible key normalises to exactly 1.
    auto probs = [&](int kk, bf16x8* pk) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pk[s][j] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s][8 * kk + j], c2, -m_run[s]));
        float r = l_run[s];
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 0, 1), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 2, 3), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 4, 5), ones, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[s], pk[s], 6, 7), ones, r, false);
        l_run[s] = r;
      }
    };
    // O~^T += V^T P^T for half kk; the transposed value operand comes from two transposing
    // reads.
    auto values = [&](int kk, const bf16x8* pk) {
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const unsigned char* base = vt_base + vb * 2048 + kk * 16 * 64 + vb0;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi8 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * 64));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 both = __builtin_shufflevector(lo, hi8, 0, 1, 2, 3, 4, 5, 6, 7);
        bf16x8 a;
        __builtin_memcpy(&a, &both, sizeof a);
#pragma unroll
        for (int s = 0; s < 2; ++s)
          oacc[s][vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[s], oacc[s][vb], 0, 0, 0);
      }
    };
    // The wave raises its priority once the first half's probabilities are formed and keeps it
    // through both halves' value products and the second half's probabilities.  Of the two waves
    // on a SIMD, the one in this stretch goes first and the other's softmax fills the matrix
    // core's shadow, which pulls the two into alternating phases; the second half's
    // probabilities, at raised priority, issue between the first half's products.
    bf16x8 pk0[2], pk1[2];
    probs(0, pk0);
    __builtin_amdgcn_s_setprio(1);
    values(0, pk0);
    probs(1, pk1);
    values(1, pk1);
    __builtin_amdgcn_s_setprio(0);
  };

  // One pipeline step for tile kt in buffer B = kt % 3: start the direct loads of tile kt+2
  // into buffer (kt+2) % 3 (last read at tile kt-1, behind that tile's barrier), compute tile
  // kt if any of this wave's rows sees it, wait for this wave's copies of tile kt+1 (issued a
  // step ago; those of kt+2 stay in flight), barrier.  The loads are unconditional: past the
  // block's end they fetch zeros into buffers nobody reads.
  auto step = [&](auto bufc, auto bufn, int kt) {
    load_kv(bufn, kt + 2);
    if (kt < wt_live) tile(bufc, kt);
    tile_barrier<LPW>();
  };

  tile_barrier<LPW>();   // tile 0 and the state have landed; tile 1 may still be in flight
  for (int kt = 0; kt < kt_live; kt += 3) {
    step(I0{}, I2{}, kt);
    if (kt + 1 < kt_live) step(I1{}, I0{}, kt + 1);
    if (kt + 2 < kt_live) step(I2{}, I1{}, kt + 2);
  }
  // ---- write the state back ----------------------------------------------------------
  // Every wave's copies have landed (the last ones, past the live tiles, fill buffers nobody
  // reads) and its tile reads are done: the tile buffers are free.  O~ goes out through them,
  // one 32-wide value block of a sub-tile at a time, so that each store instruction writes 8
  // rows x 128 contiguous bytes rather than 32 bytes of each of 32 rows.  Wave w stages in its
  // own tile buffer, in 4 KB regions (two used in turn where the buffer holds 8 KB, d = 128;
  // one at d = 64, where the wave's LDS order alone keeps a block's reads ahead of the next
  // block's writes): row R (0..31) of the block at R * 128, its
  // 16-byte chunk C at slot C ^ ((R >> 1) & 7).  With that swizzle neither the writes in the
  // accumulator layout (16 lanes: 16 rows, one chunk) nor the row-major reads (16 lanes: 2
  // rows, 8 chunks) meet a bank twice.
  __syncthreads();
  unsigned char* const stage = wave == 0 ? k_t0 : wave == 1 ? k_t1 : wave == 2 ? k_t2 : v_t0;
  // the staging addresses from a copy of the lane index made here, so that nothing of them is
  // computed before the loop and held through it
  const int el = opaque_copy(lane);
  const int e32 = el & 31, ehi = el >> 5;
  // The lap's last step may finalize here instead (p.finalize): O = O~ / l and lse in place of
  // O~, m and l, the arithmetic of the finalize pass.  A step that keeps the state scales by 1.
  const bool fin = p.finalize != 0;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float la, lb;
    pair32(l_run[s], la, lb);
    const float l_row = la + lb;
    if (row_ok[s] && hi == 0) {
      if (!fin) {
        p.m[srow[s]] = l_row == 0.f ? -INFINITY : m_run[s];
        p.l[srow[s]] = l_row;
      } else if (p.fin_lse) {
        p.fin_lse[srow[s]] = l_row > 0.f ? 0.69314718055994530942f * (m_run[s] + log2f(l_row)) : -INFINITY;
      }
    }
    const float f = !fin ? 1.0f : l_row > 0.f ? 1.0f / l_row : 0.f;
    // the sub-tile's rows through a resource that ends at the last row: stores past it are dropped
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(p.o_out + (((int64_t)b * p.q_heads + h) * p.state_rows + w0 + 32 * s) * D,
                  (int64_t)max(0, p.n_q - w0 - 32 * s) * D * 4);
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      static_assert(TB == 4096 || TB == 8192, "staging regions of 4 KB");
      unsigned char* const half = stage + (TB == 8192 ? ((s * VB + vb) & 1) * 4096 : 0);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(half + e32 * 128 + (((2 * a + ehi) ^ ((e32 >> 1) & 7)) * 16)) =
            f32x4{oacc[s][vb][4 * a + 0] * f, oacc[s][vb][4 * a + 1] * f, oacc[s][vb][4 * a + 2] * f,
                  oacc[s][vb][4 * a + 3] * f};
      f32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int R = 8 * j + (el >> 3), C = el & 7;
        x[j] = *reinterpret_cast<const f32x4*>(half + R * 128 + ((C ^ ((R >> 1) & 7)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int R = 8 * j + (el >> 3), C = el & 7;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x[j]), rs,
                                               (R * D + vb * 32 + C * 4) * 4, 0, 0);
      }
    }
  }

  if (DEBUG) {
    if (my_pairs) atomicAdd(&dbg_acc[0], my_pairs);
    if (my_moves) atomicAdd(&dbg_acc[1], (unsigned long long)my_moves);
    if (my_bounded) atomicAdd(&dbg_acc[2], (unsigned long long)my_bounded);
    __syncthreads();
    if (tid == 0) {
      atomicAdd(&p.dbg[0], (unsigned long long)kt_full);
      atomicAdd(&p.dbg[1], (unsigned long long)(kt_live - kt_full));
      atomicAdd(&p.dbg[2], dbg_acc[0]);
      atomicAdd(&p.dbg[3], dbg_acc[1]);
      atomicAdd(&p.dbg[4], dbg_acc[2]);
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

// Key-tile norms: one wave per (batch, KV head, 32-key tile).  Lanes 2j and 2j+1 take key j
// of the tile, half of its dims each, in 16-byte loads; the tile's largest |k| (times the
// margin) is written by lane 0.  Keys past the block's end contribute nothing.
template <int D>
__global__ __launch_bounds__(256) void key_tile_norm_kernel(const __bf16* k, int64_t k_sb, int64_t k_sh,
                                                            int64_t k_st, int kv_heads, int n_k,
                                                            int n_tiles, int64_t n_waves, float* out) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= n_waves) return;   // whole waves only
  const int lane = threadIdx.x & 63;
  const int t = (int)(w % n_tiles);
  const int64_t bh = w / n_tiles;
  const int64_t b = bh / kv_heads, h = bh % kv_heads;
  const int key = t * BK + (lane >> 1);
  float ss = 0.f;
  if (key < n_k) {
    const __bf16* row = k + b * k_sb + h * k_sh + (int64_t)key * k_st + (lane & 1) * (D / 2);
#pragma unroll
    for (int c = 0; c < D / 2; c += 8) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(row + c);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 y = {x[e], x[e + 1]};
        ss = __builtin_amdgcn_fdot2_f32_bf16(y, y, ss, false);
      }
    }
  }
  ss += __shfl_xor(ss, 1);
  float nrm = __builtin_sqrtf(ss);
#pragma unroll
  for (int off = 2; off < 64; off <<= 1) nrm = fmaxf(nrm, __shfl_xor(nrm, off));
  if (lane == 0) out[bh * n_tiles + t] = nrm * kNormMargin;
}

}  // namespace

hipError_t launch_key_tile_norms(const void* k, int64_t k_sb, int64_t k_sh, int64_t k_st, int batch,
                                 int kv_heads, int n_k, int head_dim, float* out, hipStream_t stream) {
  const int n_tiles = (n_k + BK - 1) / BK;
  const int64_t n_waves = (int64_t)batch * kv_heads * n_tiles;
  if (n_waves == 0) return hipSuccess;
  const int64_t grid = (n_waves + 3) / 4;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const __bf16* kb = static_cast<const __bf16*>(k);
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL(key_tile_norm_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, kb, k_sb, k_sh,
                         k_st, kv_heads, n_k, n_tiles, n_waves, out);
      break;
    case 128:
      hipLaunchKernelGGL(key_tile_norm_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, kb, k_sb, k_sh,
                         k_st, kv_heads, n_k, n_tiles, n_waves, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step_bf16(const StepParams& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
