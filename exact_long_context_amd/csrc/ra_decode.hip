// ra_decode.hip -- a KV block scored by a few query rows, split over the chip: the decode
// path of "Ring Attention：把超长序列沿设备环流动", section 训练与推理的适用方式不同.  There the
// query goes to every KV shard, each shard forms a local attention state and a global
// online-softmax reduction combines the states.  The same two stages run here inside one
// block: the keys are cut into chunks, one wave per chunk forms a local state, and
// combine_kernel folds the chunk states (and the running state of the lap) into the state.
// The shard states of different ranks are combined the same way by ra_merge.hip.
//
// A wave owns one (batch, KV head, group of 32 packed query rows, key chunk).  The packed rows
// are the (query head of the group, query token) pairs that read this KV head, so a GQA group
// of 8 heads decoding one token fills 8 of the matrix instruction's 32 columns, where the
// 128-row step tile would hold one head's single row.  Per 32-key tile: S^T = K Q^T (K rows
// straight from HBM into registers as operand A, q resident as operand B), the online-softmax
// update in base 2 (tile_update), and O~^T += V^T P^T with V staged in LDS by
// buffer_load ... lds and read back transposed by ds_read_b64_tr_b16.  The next tile's K and V
// are in flight while the current one is computed.  A chunk with no key, or a row that sees
// none of a chunk's keys, gives the empty state (m = -inf, l = 0, O~ = 0), which the
// reduction weighs by zero.  Reading K and V once is the bound: HBM.
//
// Several row groups per KV head (more tokens, or larger GQA groups) share each chunk inside
// one workgroup.  Two row groups on a short block: decode_kernel with two waves sharing V
// tiles.  Otherwise decode_ring_kernel: four waves (R row groups x S tile subsets) share a
// five-deep LDS ring of K and V tiles, so that enough bytes stay in flight per CU with only two
// such workgroups resident.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_pos.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = kDecodeTileK;   // keys per tile
constexpr int kDecodeRing = 5;     // LDS ring depth of decode_ring_kernel: 80 KB at d = 128, two workgroups per CU

// s_waitcnt with vmcnt = N (six bits: [3:0] and [15:14]); expcnt and lgkmcnt not waited on
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// V tile [BK][D] in LDS: a 16-lane group of ds_read_b64_tr_b16 fetches four consecutive keys
// x four 8-byte column pieces; this chunk twist puts a 32-lane half on distinct banks
template <int D>
__device__ __forceinline__ int v_swz(int t, int c) {
  if constexpr (D == 128) return c ^ (4 * (t & 3));
  else return c ^ (4 * ((t >> 1) & 1));
}

// V is read exactly once and each copy instruction covers whole 1 KB spans, so it goes with
// the nontemporal bit (cache policy 2): streamed past the L2 instead of filling it.  K keeps
// the default policy: its register loads touch each 128-byte line over several instructions.
__device__ __forceinline__ void load_lds_b128_dec(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_dec(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ void pair32_dec(float x, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// The online-softmax update of one 32-key tile for a wave's 32 packed rows, in base 2.  s holds
// S^T (lane: keys 8*(j/4) + 4*hi + (j%4) of its row, masked here past lim); visible says the
// row sees some key of the tile.  The reference m of a row may lag its true maximum: the tile's
// terms 2^(x - m) are taken as they come while their row sum stays <= 2^32, which fp32 and bf16
// hold without loss; only a row past that, or one meeting its first visible key, takes the
// tile's maximum and rescales l and O~, so that max x - 32 <= m <= max x holds throughout.
// Before any key m = 0 and l = 0.  The probabilities come back in bf16 (operand B of the value
// product), and the row sum adds the same rounded values.
constexpr float kDecodeSumMax = 4294967296.0f;   // 2^32

// moves (wave-uniform) counts, twice over (both lanes of a row), the rows that already held
// keys and moved their reference here: the debug count of the rescale by 2^(m_old - m_new).
template <int VB>
__device__ __forceinline__ void tile_update(f32x16& s, int lim, bool visible, float c2, float& m_run,
                                            float& l_run, f32x16 (&oacc)[VB], bf16x8 (&pk)[2],
                                            bool row_ok, unsigned& moves) {
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = (8 * (j >> 2) + (j & 3) > lim) ? -INFINITY : s[j];
  auto probs = [&](float ref) {
#pragma unroll
    for (int j = 0; j < 16; ++j) pk[j >> 3][j & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c2, -ref));
    float r = 0.f;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 0, 1), ones, r, false);
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 2, 3), ones, r, false);
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 4, 5), ones, r, false);
      r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[kk], pk[kk], 6, 7), ones, r, false);
    }
    float a, b;
    pair32_dec(r, a, b);
    return a + b;
  };
  float rs = probs(m_run);
  const bool bad = !(rs <= kDecodeSumMax) || (l_run == 0.f && visible);
  if (__builtin_amdgcn_ballot_w64(bad)) {
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
    {
      float a, b;
      pair32_dec(mx, a, b);
      mx = fmaxf(a, b);
    }
    // a bad row moves its reference to the tile's maximum: l and O~ scale by 2^-shift (a row
    // that has seen nothing holds zeros and takes 0: 2^-shift may overflow there)
    const float shift = (bad && mx != -INFINITY) ? mx * c2 - m_run : 0.f;
    const float alpha = l_run == 0.f ? 0.f : __builtin_amdgcn_exp2f(-shift);
    moves += (unsigned)__builtin_popcountll(__builtin_amdgcn_ballot_w64(row_ok && bad && l_run != 0.f));
    l_run *= alpha;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[vb][j] *= alpha;
    m_run += shift;
    rs = probs(m_run);
  }
  l_run += rs;
}

// W waves per workgroup: the W row groups of one (part, KV head) share the chunk's V tiles in
// LDS, each wave loading 1/W of every tile; their K loads are the same addresses at nearly the
// same time, served once from HBM.  With one wave, two V buffers and no barrier; with several,
// three buffers and one barrier per tile: a wave refills the buffer read two tiles earlier,
// which every wave has finished by the time any wave passes the barrier of the tile between.
template <int D, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecodeParams p) {
  constexpr int KS = D / 16, VB = D / 32, RB = D * 2, CPR = D / 8, RPL = 64 / CPR;
  constexpr int LPT = BK * RB / 1024;   // 1 KB direct loads per V tile
  static_assert(LPT % W == 0, "every wave loads the same share of a V tile");
  constexpr int LPW = LPT / W;          // this wave's share
  constexpr int NB = W == 1 ? 2 : 3;    // V buffers
  __shared__ __attribute__((aligned(16))) unsigned char v_t0[BK * RB];
  __shared__ __attribute__((aligned(16))) unsigned char v_t1[BK * RB];
  __shared__ __attribute__((aligned(16))) unsigned char v_t2[NB == 3 ? BK * RB : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  // grid: (part, group of W row groups, KV head, batch), part fastest
  int L = blockIdx.x;
  const int part = L % p.n_parts;
  L /= p.n_parts;
  const int n_rg = (p.group * p.n_q + 31) / 32;
  const int n_wg = (n_rg + W - 1) / W;
  const int rg = (L % n_wg) * W + wave;   // past the last row group: a wave with no rows
  L /= n_wg;
  const int g = L % p.kv_heads;
  const int b = L / p.kv_heads;

  // packed row -> (query head of the group, token)
  const int pr = rg * 32 + r32;
  const bool row_ok = pr < p.group * p.n_q;
  const int hh = row_ok ? pr / p.n_q : 0;
  const int i = row_ok ? pr - hh * p.n_q : 0;
  const int h = g * p.group + hh;
  const int64_t srow = ((int64_t)b * p.q_heads + h) * p.n_q + i;

  // this part's keys
  const int chunk = p.chunk;
  const int k0 = part * chunk;
  const int k1 = min(k0 + chunk, p.n_k);
  const int n_tiles = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;

  bf16x8 qf[KS];
  {
    const __bf16* qp = static_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)i * p.q_st + hi * 8;
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
  const float c2 = p.scale_log2;
  float m_run = 0.f, l_run = 0.f;   // m: the finite reference of l and O~ (0 before any key)
  unsigned moves = 0;
  f32x16 oacc[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[vb][j] = 0.f;

  const __bf16* kg = static_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const __bf16* vg = static_cast<const __bf16*>(p.v) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const int row_bytes = (int)(p.k_st * 2);
  // K operand A straight from HBM: lane reads key r32 of the tile, chunk 2*ks + hi
  auto load_k = [&](int t0, bf16x8 (&kr)[KS]) {
    const __amdgpu_buffer_rsrc_t r = rsrc_dec(kg + (int64_t)t0 * p.k_st, ((int64_t)k1 - t0) * p.k_st * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, r32 * row_bytes + (2 * ks + hi) * 16, 0, 0);
      __builtin_memcpy(&kr[ks], &x, sizeof x);
    }
  };
  // this wave's share of a V tile into LDS: 1 KB span w*LPW + u holds key rows
  // (w*LPW + u)*RPL + lane / CPR, lane at physical chunk lane % CPR
  auto load_v = [&](unsigned char* tile, int t0) {
    const __amdgpu_buffer_rsrc_t r = rsrc_dec(vg + (int64_t)t0 * p.k_st, ((int64_t)k1 - t0) * p.k_st * 2);
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int span = wave * LPW + u;
      const int row = span * RPL + lane / CPR;
      const int voff = (lane / CPR) * row_bytes + v_swz<D>(row, lane % CPR) * 16;
      load_lds_b128_dec(r, tile + span * RPL * RB, voff, span * RPL * row_bytes);
    }
  };
  auto vbuf = [&](auto bufc) -> unsigned char* {
    constexpr int B = decltype(bufc)::value;
    return B == 0 ? v_t0 : (B == 1 ? v_t1 : v_t2);
  };
  int v_roff[VB];
  {
    const int gg = lane >> 4, a = lane & 3, e = (lane >> 2) & 3;
    const int key = 4 * (gg >> 1) + e;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int dv = 32 * vb + 16 * (gg & 1) + 4 * a;
      v_roff[vb] = key * RB + (v_swz<D>(key, dv >> 3) << 4) + ((dv & 7) << 1);
    }
  }

  // One tile: the next tile's K (registers kn) and V (the other LDS buffer) are put in flight
  // first, then this tile (K in kc, V in buffer BUF) is computed.  The two V buffers are
  // distinct objects and BUF is a compile-time constant, so the compiler can tell the buffer
  // being read from the one a direct load is filling.
  auto tile = [&](auto bufc, int tt, bf16x8 (&kc)[KS], bf16x8 (&kn)[KS]) {
    constexpr int BUF = decltype(bufc)::value;
    const unsigned char* cur = vbuf(bufc);
    const int t0 = k0 + tt * BK;
    load_k(t0 + BK, kn);   // past the chunk's end: zeros, never used
    load_v(vbuf(std::integral_constant<int, (BUF + 1) % NB>{}), t0 + BK);
    wait_vmcnt<KS + LPW>();   // only the next tile's loads are outstanding: this tile's landed
    if constexpr (W > 1) {
      asm volatile("s_barrier" ::: "memory");   // every wave's share of this tile has landed
    } else {
      __builtin_amdgcn_wave_barrier();
    }
    // two independent accumulation chains over the contraction, added at the end
    f32x16 s, s1;
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = s1[j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[ks], qf[ks], s, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[ks + 1], qf[ks + 1], s1, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] += s1[j];
    // lane holds keys t0 + 8*(j/4) + 4*hi + (j%4) of packed row pr
    const int lim = min(i + p.diag, k1 - 1) - t0 - 4 * hi;
    bf16x8 pk[2];
    tile_update(s, lim, lim + 4 * hi >= 0, c2, m_run, l_run, oacc, pk, row_ok, moves);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const unsigned char* base = cur + v_roff[vb] + kk * 16 * RB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi8 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * RB));
        const s16x8 both = __builtin_shufflevector(lo, hi8, 0, 1, 2, 3, 4, 5, 6, 7);
        bf16x8 a;
        __builtin_memcpy(&a, &both, sizeof a);
        oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], oacc[vb], 0, 0, 0);
      }
    // every lane is done reading this V tile before a later copy overwrites it
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt not waited on
    __builtin_amdgcn_wave_barrier();
  };

  bf16x8 ka[KS], kb[KS];
  if (n_tiles > 0) {
    load_k(k0, ka);
    load_v(v_t0, k0);
  }
  // K alternates between two register sets, V between NB buffers: one period is 2 or 6 tiles
  // (n_tiles is the same for every wave of the workgroup, so all reach the same barriers)
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if constexpr (NB == 2) {
    for (int tt = 0; tt < n_tiles; tt += 2) {
      tile(I0{}, tt, ka, kb);
      if (tt + 1 < n_tiles) tile(I1{}, tt + 1, kb, ka);
    }
  } else {
    for (int tt = 0; tt < n_tiles; tt += 6) {
      tile(I0{}, tt, ka, kb);
      if (tt + 1 < n_tiles) tile(I1{}, tt + 1, kb, ka);
      if (tt + 2 < n_tiles) tile(I2{}, tt + 2, ka, kb);
      if (tt + 3 < n_tiles) tile(I0{}, tt + 3, kb, ka);
      if (tt + 4 < n_tiles) tile(I1{}, tt + 4, ka, kb);
      if (tt + 5 < n_tiles) tile(I2{}, tt + 5, kb, ka);
    }
  }
  wait_vmcnt<0>();   // the last prefetch (zeros past the chunk) is not left in flight
  if (p.dbg_moves && moves && lane == 0) atomicAdd(p.dbg_moves, (unsigned long long)(moves / 2));

  if (row_ok) {
    const int64_t rows = (int64_t)p.batch * p.q_heads * p.n_q;
    const int64_t prow = (int64_t)part * rows + srow;
    if (hi == 0) {
      p.part_m[prow] = l_run == 0.f ? -INFINITY : m_run;
      p.part_l[prow] = l_run;
    }
    float* op = p.part_o + prow * D + 4 * hi;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(op + vb * 32 + 8 * a) =
            make_float4(oacc[vb][4 * a + 0], oacc[vb][4 * a + 1], oacc[vb][4 * a + 2], oacc[vb][4 * a + 3]);
  }
}

// K tile [BK][D] in LDS: the score operand read (32 consecutive key rows at one chunk) hits
// distinct banks 16 lanes at a time
template <int D>
__device__ __forceinline__ int k_swz(int t, int c) {
  if constexpr (D == 128) return c ^ (t & 15);
  else return c ^ ((t >> 1) & 7);
}

// LDS operand reads of decode_ring_kernel, issued as inline asm.  Its copies stay in flight
// across tiles, and the compiler, which cannot follow which ring buffer they fill across the
// loop, would otherwise wait for all of them before reading any buffer.  The asm results are
// not ready until lgkm_wait() below, which takes them as operands so that nothing reads them
// earlier; the explicit vmcnt waits and the barrier order the copies against these reads.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ u32x4 ds_read_b128_asm(unsigned addr) {
  u32x4 x;
  asm volatile("ds_read_b128 %0, %1" : "=v"(x) : "v"(addr));
  return x;
}
__device__ __forceinline__ u32x2 ds_read_tr_b64_asm(unsigned addr) {
  u32x2 x;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(x) : "v"(addr));
  return x;
}
// the resident q rows, loaded ahead of the first copies so that the first tile's vmcnt wait
// (counts complete in issue order) also covers them; pass_through() after that wait hands the
// values on, so nothing reads them earlier
__device__ __forceinline__ u32x4 global_load_b128_asm(const void* p) {
  u32x4 x;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x) : "v"(p));
  return x;
}
template <int N, typename T>
__device__ __forceinline__ void pass_through(T (&x)[N]) {
#pragma unroll
  for (int n = 0; n < N; ++n) asm volatile("" : "+v"(x[n]));
}
template <int N, typename T>
__device__ __forceinline__ void lgkm_wait(T (&x)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int n = 0; n < N; ++n) asm volatile("" : "+v"(x[n]));
}

// Several row groups per KV head.  A workgroup of R * S = 4 waves takes R row groups of one
// (part, KV head); wave (r, s) computes row group r over the chunk's tiles t with t % S == s,
// so every SIMD still holds two waves when a KV head has only two row groups (R = 2, S = 2: the
// two tile parities are separate parts, folded by the combine).  K and V tiles both sit in an
// NB-deep LDS ring that all four waves fill, each copying its quarter of every tile with the
// nontemporal bit, so NB - 1 tiles are in flight per workgroup (two workgroups per CU) and each
// tile is read from HBM once.  Per tile: wait for this wave's copies of the tile, barrier (all
// copies landed, and every wave is done with the tile before, whose buffer is refilled next),
// copy tile t + NB - 1, compute.
template <int D, int R, int S, int NB>
__global__ __launch_bounds__(64 * R * S) __attribute__((amdgpu_waves_per_eu(2))) void decode_ring_kernel(DecodeParams p) {
  constexpr int W = R * S;
  constexpr int KS = D / 16, VB = D / 32, RB = D * 2, CPR = D / 8, RPL = 64 / CPR;
  constexpr int TB = BK * RB;           // bytes per tile and tensor
  constexpr int LPT = TB / 1024;        // 1 KB copies per tile and tensor
  static_assert(LPT % W == 0, "every wave copies the same share of a tile");
  constexpr int LPW = LPT / W;
  static_assert(NB >= 3 && NB <= 5, "ring depth");
  // K at [0, TB), V at [TB, 2 TB) of each buffer; distinct objects, selected at compile time
  __shared__ __attribute__((aligned(16))) unsigned char kv0[2 * TB];
  __shared__ __attribute__((aligned(16))) unsigned char kv1[2 * TB];
  __shared__ __attribute__((aligned(16))) unsigned char kv2[2 * TB];
  __shared__ __attribute__((aligned(16))) unsigned char kv3[NB > 3 ? 2 * TB : 16];
  __shared__ __attribute__((aligned(16))) unsigned char kv4[NB > 4 ? 2 * TB : 16];
  auto buf = [&](auto bc) -> unsigned char* {
    constexpr int B = decltype(bc)::value % NB;
    if constexpr (B == 0) return kv0;
    else if constexpr (B == 1) return kv1;
    else if constexpr (B == 2) return kv2;
    else if constexpr (B == 3) return kv3;
    else return kv4;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave % R, sub = wave / R;
  const int r32 = lane & 31, hi = lane >> 5;
  // grid: (part, group of R row groups, KV head, batch), part fastest
  int L = blockIdx.x;
  const int part = L % p.n_parts;
  L /= p.n_parts;
  const int n_rg = (p.group * p.n_q + 31) / 32;
  const int n_wg = (n_rg + R - 1) / R;
  const int rg = (L % n_wg) * R + wr;   // past the last row group: a wave with no rows
  L /= n_wg;
  const int g = L % p.kv_heads;
  const int b = L / p.kv_heads;

  const int pr = rg * 32 + r32;
  const bool row_ok = pr < p.group * p.n_q;
  const int hh = row_ok ? pr / p.n_q : 0;
  const int i = row_ok ? pr - hh * p.n_q : 0;
  const int h = g * p.group + hh;
  const int64_t srow = ((int64_t)b * p.q_heads + h) * p.n_q + i;

  const int k0 = part * p.chunk;
  const int k1 = min(k0 + p.chunk, p.n_k);
  const int n_tiles = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;

  u32x4 qf[KS];
  {
    const __bf16* qp = static_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)i * p.q_st + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? global_load_b128_asm(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  const float c2 = p.scale_log2;
  float m_run = 0.f, l_run = 0.f;   // m: the finite reference of l and O~ (0 before any key)
  unsigned moves = 0;
  f32x16 oacc[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[vb][j] = 0.f;

  const __bf16* kg = static_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const __bf16* vg = static_cast<const __bf16*>(p.v) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const int row_bytes = (int)(p.k_st * 2);
  // this wave's copies: 1 KB span wave*LPW + u of a tile holds key rows span*RPL + lane / CPR,
  // lane at physical chunk lane % CPR (the swizzles are involutions)
  int k_goff[LPW], v_goff[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int t = (wave * LPW + u) * RPL + lane / CPR;
    k_goff[u] = (lane / CPR) * row_bytes + k_swz<D>(t, lane % CPR) * 16;
    v_goff[u] = (lane / CPR) * row_bytes + v_swz<D>(t, lane % CPR) * 16;
  }
  auto copy_tile = [&](unsigned char* dst, int t0) {
    const int64_t bytes = ((int64_t)k1 - t0) * p.k_st * 2;   // past the chunk: none, zeros land
    const __amdgpu_buffer_rsrc_t rk = rsrc_dec(kg + (int64_t)t0 * p.k_st, bytes);
    const __amdgpu_buffer_rsrc_t rv = rsrc_dec(vg + (int64_t)t0 * p.k_st, bytes);
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int row0 = (wave * LPW + u) * RPL;
      load_lds_b128_dec(rk, dst + row0 * RB, k_goff[u], row0 * row_bytes);
      load_lds_b128_dec(rv, dst + TB + row0 * RB, v_goff[u], row0 * row_bytes);
    }
  };
  int k_roff[KS];   // score operand A: key row r32, chunk 2*ks + hi
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_roff[ks] = r32 * RB + (k_swz<D>(r32, 2 * ks + hi) << 4);
  int v_roff[VB];
  {
    const int gg = lane >> 4, a = lane & 3, e = (lane >> 2) & 3;
    const int key = 4 * (gg >> 1) + e;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int dv = 32 * vb + 16 * (gg & 1) + 4 * a;
      v_roff[vb] = TB + key * RB + (v_swz<D>(key, dv >> 3) << 4) + ((dv & 7) << 1);
    }
  }

  // this wave's rows against the tile at t0 in buffer cur
  auto compute = [&](const unsigned char* cur, int t0) {
    const unsigned cur_a = lds_addr(cur);
    u32x4 ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = ds_read_b128_asm(cur_a + k_roff[ks]);
    lgkm_wait(ka);
    f32x16 s, s1;   // two independent accumulation chains, added at the end
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = s1[j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      bf16x8 a0, b0, a1, b1;
      __builtin_memcpy(&a0, &ka[ks], sizeof a0);
      __builtin_memcpy(&b0, &qf[ks], sizeof b0);
      __builtin_memcpy(&a1, &ka[ks + 1], sizeof a1);
      __builtin_memcpy(&b1, &qf[ks + 1], sizeof b1);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, s, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, s1, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] += s1[j];
    // lane holds keys t0 + 8*(j/4) + 4*hi + (j%4) of packed row pr
    const int lim = min(i + p.diag, k1 - 1) - t0 - 4 * hi;
    bf16x8 pk[2];
    tile_update(s, lim, lim + 4 * hi >= 0, c2, m_run, l_run, oacc, pk, row_ok, moves);
    u32x2 va[2 * 2 * VB];   // (kk, vb, half)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const unsigned base = cur_a + v_roff[vb] + kk * 16 * RB;
        va[(kk * VB + vb) * 2 + 0] = ds_read_tr_b64_asm(base);
        va[(kk * VB + vb) * 2 + 1] = ds_read_tr_b64_asm(base + 8 * RB);
      }
    lgkm_wait(va);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const u32x4 both = __builtin_shufflevector(va[(kk * VB + vb) * 2], va[(kk * VB + vb) * 2 + 1], 0, 1, 2, 3);
        bf16x8 a;
        __builtin_memcpy(&a, &both, sizeof a);
        oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], oacc[vb], 0, 0, 0);
      }
  };

  // tile t in buffer B = t % NB: NB - 1 tiles are in flight on entry
  auto step = [&](auto bc, int t) {
    constexpr int B = decltype(bc)::value;
    wait_vmcnt<(NB - 2) * 2 * LPW>();   // this wave's copies of tile t (and its q) have landed
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): its reads of tile t - 1 are done
    asm volatile("s_barrier" ::: "memory");
    pass_through(qf);
    copy_tile(buf(std::integral_constant<int, B + NB - 1>{}), k0 + (t + NB - 1) * BK);
    if (S == 1 || (t % S) == sub) compute(buf(bc), k0 + t * BK);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  if (n_tiles > 0) {
    copy_tile(buf(I0{}), k0);
    copy_tile(buf(I1{}), k0 + BK);
    if constexpr (NB > 3) copy_tile(buf(I2{}), k0 + 2 * BK);
    if constexpr (NB > 4) copy_tile(buf(I3{}), k0 + 3 * BK);
  }
  // n_tiles is the same for every wave of the workgroup, so all reach the same barriers
  for (int tt = 0; tt < n_tiles; tt += NB) {
    step(I0{}, tt);
    if (tt + 1 < n_tiles) step(I1{}, tt + 1);
    if (tt + 2 < n_tiles) step(I2{}, tt + 2);
    if constexpr (NB > 3) if (tt + 3 < n_tiles) step(I3{}, tt + 3);
    if constexpr (NB > 4) if (tt + 4 < n_tiles) step(I4{}, tt + 4);
  }
  wait_vmcnt<0>();   // the copies past the chunk (zeros) land before the workgroup's LDS is freed
  if (p.dbg_moves && moves && lane == 0) atomicAdd(p.dbg_moves, (unsigned long long)(moves / 2));

  if (row_ok) {
    const int64_t rows = (int64_t)p.batch * p.q_heads * p.n_q;
    const int64_t prow = ((int64_t)part * S + sub) * rows + srow;
    if (hi == 0) {
      p.part_m[prow] = l_run == 0.f ? -INFINITY : m_run;
      p.part_l[prow] = l_run;
    }
    float* op = p.part_o + prow * D + 4 * hi;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(op + vb * 32 + 8 * a) =
            make_float4(oacc[vb][4 * a + 0], oacc[vb][4 * a + 1], oacc[vb][4 * a + 2], oacc[vb][4 * a + 3]);
  }
}

// One workgroup per state row, in one pass over the parts.  Thread (pl, c) folds float4
// column c of parts pl, pl + PL, ... into a running state of its own (m_t, l_t, O~_t): a batch
// of U parts is loaded, the reference moves to the batch maximum if that is larger (rescaling
// l_t and O~_t by 2^(m_t - m_new)), and each part is added with weight 2^(m_s - m_t).  The PL
// running states of a column then merge the same way through LDS, with the lap's running state
// folded in unless the state is fresh.  m_t is the same for every column of one pl, since the
// parts' m values are per row.  Empty parts (m = -inf) weigh nothing.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int C4 = D / 4;      // float4 columns of a row
  constexpr int PL = 256 / C4;   // parts summed side by side
  constexpr int U = 8;           // parts per batch, all loads issued before any is used
  __shared__ float4 acc_s[PL][C4];
  __shared__ float l_s[PL], m_s[PL];
  const int tid = threadIdx.x;
  const int c = tid % C4, pl = tid / C4;
  for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
    float mt = -INFINITY, lt = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto raise_to = [&](float m_new) {   // m_new >= mt, finite
      const float a = exp2f(mt - m_new);  // 0 while mt = -inf
      acc.x *= a;
      acc.y *= a;
      acc.z *= a;
      acc.w *= a;
      lt *= a;
      mt = m_new;
    };
    auto add = [&](float ms, float l, float4 x) {   // ms <= mt
      const float w = ms == -INFINITY ? 0.f : exp2f(ms - mt);
      acc.x += w * x.x;
      acc.y += w * x.y;
      acc.z += w * x.z;
      acc.w += w * x.w;
      lt += w * l;
    };
    int s = pl;
    for (; s + (U - 1) * PL < p.n_parts; s += U * PL) {
      float ms[U], lv[U];
      float4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t pr = (int64_t)(s + u * PL) * p.rows + row;
        ms[u] = p.part_m[pr];
        lv[u] = p.part_l[pr];
        x[u] = *reinterpret_cast<const float4*>(p.part_o + pr * D + 4 * c);
      }
      float bm = ms[0];
#pragma unroll
      for (int u = 1; u < U; ++u) bm = fmaxf(bm, ms[u]);
      if (bm > mt) raise_to(bm);
#pragma unroll
      for (int u = 0; u < U; ++u) add(ms[u], lv[u], x[u]);
    }
    for (; s < p.n_parts; s += PL) {
      const int64_t pr = (int64_t)s * p.rows + row;
      const float ms = p.part_m[pr];
      if (ms > mt) raise_to(ms);
      add(ms, p.part_l[pr], *reinterpret_cast<const float4*>(p.part_o + pr * D + 4 * c));
    }
    if (!p.fresh && pl == 0) {
      const float ms = p.m[row];
      if (ms > mt) raise_to(ms);
      add(ms, p.l[row], *reinterpret_cast<const float4*>(p.o_acc + row * D + 4 * c));
    }
    acc_s[pl][c] = acc;
    if (c == 0) {
      l_s[pl] = lt;
      m_s[pl] = mt;
    }
    __syncthreads();
    if (pl == 0) {
      float M = m_s[0];
      for (int u = 1; u < PL; ++u) M = fmaxf(M, m_s[u]);
      acc = make_float4(0.f, 0.f, 0.f, 0.f);
      float ls = 0.f;
      if (M != -INFINITY) {
        for (int u = 0; u < PL; ++u) {
          const float mu = m_s[u];
          const float w = mu == -INFINITY ? 0.f : exp2f(mu - M);
          const float4 x = acc_s[u][c];
          acc.x += w * x.x;
          acc.y += w * x.y;
          acc.z += w * x.z;
          acc.w += w * x.w;
          ls += w * l_s[u];
        }
      }
      *reinterpret_cast<float4*>(p.o_acc + row * D + 4 * c) = acc;
      if (c == 0) {
        p.m[row] = M;
        p.l[row] = ls;
      }
    }
    __syncthreads();   // acc_s, l_s and m_s are reused by the next row
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)(p.rows < 65536 ? p.rows : 65536);
  switch (p.d) {
    case 64:
      hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, DecodeShape shape, hipStream_t stream) {
  const int n_rg = (p.group * p.n_q + 31) / 32;
  const int n_wg = (n_rg + shape.R - 1) / shape.R;
  const int64_t grid = (int64_t)p.n_parts * n_wg * p.kv_heads * p.batch;
  if (grid == 0) return hipSuccess;
#define RA_DECODE_ONE(DD, WW) \
  hipLaunchKernelGGL((decode_kernel<DD, WW>), dim3((unsigned)grid), dim3(64 * WW), 0, stream, p)
#define RA_DECODE_RING(DD, RR, SS) \
  hipLaunchKernelGGL((decode_ring_kernel<DD, RR, SS, kDecodeRing>), dim3((unsigned)grid), dim3(64 * RR * SS), 0, stream, p)
  switch (head_dim * 64 + shape.ring * 32 + shape.R * 4 + shape.S) {
    case 64 * 64 + 0 + 1 * 4 + 1: RA_DECODE_ONE(64, 1); break;
    case 64 * 64 + 0 + 2 * 4 + 1: RA_DECODE_ONE(64, 2); break;
    case 64 * 64 + 32 + 2 * 4 + 2: RA_DECODE_RING(64, 2, 2); break;
    case 64 * 64 + 32 + 4 * 4 + 1: RA_DECODE_RING(64, 4, 1); break;
    case 128 * 64 + 0 + 1 * 4 + 1: RA_DECODE_ONE(128, 1); break;
    case 128 * 64 + 0 + 2 * 4 + 1: RA_DECODE_ONE(128, 2); break;
    case 128 * 64 + 32 + 2 * 4 + 2: RA_DECODE_RING(128, 2, 2); break;
    case 128 * 64 + 32 + 4 * 4 + 1: RA_DECODE_RING(128, 4, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef RA_DECODE_ONE
#undef RA_DECODE_RING
  return hipGetLastError();
}

}  // namespace ra
