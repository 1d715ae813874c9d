// ra_step_f32.hip -- fp32 step kernel: the exactness path (all arithmetic in fp32, no
// bf16 or reduced-precision conversion anywhere).
//
// One workgroup owns a 64-row query tile of one query head and streams the block's keys
// through LDS in 32-key tiles; four lanes share a query row, each holding a quarter of the
// head dimension of q and of the running output O~.  After each key tile the per-row state
// is rescaled by 2^(m_old - m_new) and the tile's terms are added ("GPU ring attention",
// section "Why partial results are allowed to merge"), in base-2 units
// (x = log2(e) * scale * <q, k>).  Tiles with no allowed pair are never visited and only
// tiles that cross the diagonal (or run past the block's end) apply the element mask
// (ra_pos.h).
//
// This path exists for exactness checks at small sizes, not for speed.

#include <hip/hip_runtime.h>

#include "ra_internal.h"
#include "ra_pos.h"

namespace ra {
namespace {

constexpr int TQ = kF32TileQ;   // 64 query rows per workgroup
constexpr int TK = kF32TileK;   // 32 keys per LDS tile
constexpr int NT = 256;         // 4 lanes per query row

template <int D, bool DEBUG>
__global__ __launch_bounds__(NT) void step_f32_kernel(StepParams p) {
  constexpr int DP = D / 4;     // dims per lane
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  __shared__ unsigned long long dbg_acc[4];

  const int tid = threadIdx.x;
  const int row = tid >> 2;     // 0..63
  const int part = tid & 3;     // which quarter of the head dimension

  const int n_qt = (p.n_q + TQ - 1) / TQ;
  int w = blockIdx.x;
  const int qt = w % n_qt;
  w /= n_qt;
  const int h = w % p.q_heads;
  const int b = w / p.q_heads;
  const int g = h / p.group;

  const int i0 = qt * TQ;
  const int i1 = min(i0 + TQ, p.n_q);
  const int i = i0 + row;
  const bool row_ok = i < p.n_q;
  const int64_t srow = ((int64_t)b * p.q_heads + h) * p.state_rows + i;   // state row index

  const int kt_live = tiles_live(i0, i1, p.diag, p.n_k, TK);
  const int kt_full = tiles_full(i0, i1, p.diag, p.n_k, TK);

  if (DEBUG && tid < 4) dbg_acc[tid] = 0;

  float m_run, l_run, o[DP];
  if (p.fresh) {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int c = 0; c < DP; ++c) o[c] = 0.f;
  } else {
    if (kt_live == 0) return;   // state unchanged
    m_run = row_ok ? p.m[srow] : -INFINITY;
    l_run = row_ok ? p.l[srow] : 0.f;
#pragma unroll
    for (int c = 0; c < DP; ++c) o[c] = row_ok ? p.o_acc[srow * D + part * DP + c] : 0.f;
  }

  float q[DP];
  {
    const float* qp = static_cast<const float*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh +
                      (int64_t)i * p.q_st + part * DP;
#pragma unroll
    for (int c = 0; c < DP; ++c) q[c] = row_ok ? qp[c] : 0.f;
  }

  const float* kbase = static_cast<const float*>(p.k) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const float* vbase = static_cast<const float*>(p.v) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  unsigned long long my_pairs = 0;
  unsigned long long my_moves = 0;   // tiles in which this row, already holding keys, raised its max

  for (int kt = 0; kt < kt_live; ++kt) {
    const int t0 = kt * TK;
    __syncthreads();
    // stage the key tile: TK * D floats of K and of V, zero past the block's end
    for (int e = tid; e < TK * D; e += NT) {
      const int t = e / D, c = e % D;
      const bool ok = t0 + t < p.n_k;
      ks[t][c] = ok ? kbase[(int64_t)(t0 + t) * p.k_st + c] : 0.f;
      vs[t][c] = ok ? vbase[(int64_t)(t0 + t) * p.k_st + c] : 0.f;
    }
    __syncthreads();

    const bool masked = (kt >= kt_full) || (t0 + TK > p.n_k);
    const int lim = min(i + p.diag, p.n_k - 1) - t0;   // key t visible iff t <= lim
    float s[TK];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TK; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) acc = fmaf(q[c], ks[t][part * DP + c], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      float x = acc * p.scale_log2;
      if (masked && t > lim) x = -INFINITY;
      if (DEBUG && row_ok && part == 0 && x != -INFINITY) ++my_pairs;
      s[t] = x;
      mx = fmaxf(mx, x);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    if (DEBUG && row_ok && part == 0 && l_run != 0.f && m_new > m_run) ++my_moves;
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < DP; ++c) o[c] *= alpha;
#pragma unroll
    for (int t = 0; t < TK; ++t) {
      const float pt = exp2f(s[t] - m_use);
      l_run += pt;
#pragma unroll
      for (int c = 0; c < DP; ++c) o[c] = fmaf(pt, vs[t][part * DP + c], o[c]);
    }
    m_run = m_new;
  }

  if (row_ok) {
    if (part == 0) {
      p.m[srow] = m_run;
      p.l[srow] = l_run;
    }
#pragma unroll
    for (int c = 0; c < DP; ++c) p.o_acc[srow * D + part * DP + c] = o[c];
  }

  if (DEBUG) {
    __syncthreads();
    if (my_pairs) atomicAdd(&dbg_acc[2], my_pairs);
    if (my_moves) atomicAdd(&dbg_acc[3], my_moves);
    __syncthreads();
    if (tid == 0) {
      atomicAdd(&p.dbg[0], (unsigned long long)kt_full);             // kt_full <= kt_live
      atomicAdd(&p.dbg[1], (unsigned long long)(kt_live - kt_full));
      atomicAdd(&p.dbg[2], dbg_acc[2]);
      atomicAdd(&p.dbg[3], dbg_acc[3]);
    }
  }
}

template <int D>
hipError_t launch_d(const StepParams& p, hipStream_t stream) {
  const int n_qt = (p.n_q + TQ - 1) / TQ;
  const int64_t grid = (int64_t)n_qt * p.q_heads * p.batch;
  if (grid == 0) return hipSuccess;
  if (p.dbg)
    hipLaunchKernelGGL((step_f32_kernel<D, true>), dim3((unsigned)grid), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((step_f32_kernel<D, false>), dim3((unsigned)grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_f32(const StepParams& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
