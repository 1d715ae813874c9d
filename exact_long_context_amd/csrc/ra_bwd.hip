// ra_bwd.hip -- the backward of one rank's lap, one ring step at a time ("Ring Attention：把超长
// 序列沿设备环流动", section Backward 需要让梯度也沿环传播): the query owner accumulates dQ over
// every KV block, the travelling block accumulates dK and dV over the query owners it
// passes, and the probabilities are recomputed per block from the saved per-row logsumexp
// rather than stored.  With P = exp(scale * <q, k> - lse) on allowed pairs (the standard
// gradient of softmax attention):
//     D   = rowsum(dO * O),   dV += P^T dO,   dS = P * (dO V^T - D),
//     dQ += scale * dS K,     dK += scale * dS^T Q.
//
// These are the fp32 kernels (vector-unit FMA, the exactness path; the bf16 path runs on the
// matrix cores, ra_bwd_bf16.hip), plus the D pass shared by both.  Each output has one owner,
// so nothing is accumulated with atomics:
//  * bwd_dq_kernel: a workgroup owns 64 query rows of one head (four lanes per row, each
//    with a quarter of the head dimension) and streams the block's keys through LDS;
//  * bwd_dkdv_kernel: a workgroup owns 64 keys of one KV head and streams the query rows
//    of every query head that reads that KV head through LDS.
// Both visit only the tiles that hold an allowed pair (ra_pos.h) and mask the rest per pair.

#include <hip/hip_runtime.h>

#include "ra_internal.h"
#include "ra_pos.h"

namespace ra {
namespace {

constexpr int NT = 256;
constexpr int TR = 64;   // rows (dq) or keys (dkdv) owned by a workgroup
constexpr int TS = 32;   // keys (dq) or rows (dkdv) streamed per LDS tile

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return (float)*p; }

// D = rowsum(dO * O) and dQ accumulator cleared, one row per 64 lanes' worth of d/4 lanes
template <typename T, int D>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(BwdPrepParams p) {
  constexpr int VPR = D / 4;
  constexpr int RPW = 64 / VPR;
  const int lane = threadIdx.x & 63;
  const int sub = lane / VPR, vec = lane % VPR;
  const int64_t wave = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * (NT / 64);
  for (int64_t r = wave * RPW + sub; r < p.rows; r += n_waves * RPW) {
    const int64_t bh = r / p.n_q;
    const int64_t i = r - bh * p.n_q;
    const int64_t b = bh / p.q_heads, h = bh - b * p.q_heads;
    const T* dop = static_cast<const T*>(p.d_out) + b * p.q_sb + h * p.q_sh + i * p.q_st + 4 * vec;
    const float* op = p.out + r * D + 4 * vec;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = __builtin_fmaf(ld(dop + c), op[c], acc);
    // sum over the row's VPR lanes (a contiguous power-of-two group of the wave)
#pragma unroll
    for (int w = VPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
    if (vec == 0) p.D[r] = acc;
    reinterpret_cast<float4*>(p.dq + r * D)[vec] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// dQ for 64 rows of one query head against one KV block
template <typename T, int D>
__global__ __launch_bounds__(NT) void bwd_dq_kernel(BwdParams p) {
  constexpr int DP = D / 4;
  __shared__ float ks[TS][D + 1];
  __shared__ float vs[TS][D + 1];
  const int tid = threadIdx.x;
  const int row = tid >> 2, part = tid & 3;
  const int n_qt = (p.n_q + TR - 1) / TR;
  int w = blockIdx.x;
  const int qt = w % n_qt;
  w /= n_qt;
  const int h = w % p.q_heads;
  const int b = w / p.q_heads;
  const int g = h / p.group;
  const int i0 = qt * TR, i1 = min(i0 + TR, p.n_q);
  const int i = i0 + row;
  const bool row_ok = i < p.n_q;
  const int kt_live = tiles_live(i0, i1, p.diag, p.n_k, TS);
  if (kt_live == 0) return;
  const int64_t srow = ((int64_t)b * p.q_heads + h) * p.state_rows + i;

  float q[DP], dov[DP], dq[DP];
  const T* qp = static_cast<const T*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)i * p.q_st + part * DP;
  const T* dop = static_cast<const T*>(p.d_out) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)i * p.q_st + part * DP;
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    q[c] = row_ok ? ld(qp + c) : 0.f;
    dov[c] = row_ok ? ld(dop + c) : 0.f;
    dq[c] = 0.f;
  }
  const float lse = row_ok ? p.lse[srow] : -INFINITY;
  const float Dr = row_ok ? p.D[srow] : 0.f;
  const bool seen = lse != -INFINITY;
  const T* kb = static_cast<const T*>(p.k) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  const T* vb = static_cast<const T*>(p.v) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh;
  for (int kt = 0; kt < kt_live; ++kt) {
    const int t0 = kt * TS;
    __syncthreads();
    for (int e = tid; e < TS * D; e += NT) {
      const int t = e / D, c = e % D;
      const bool ok = t0 + t < p.n_k;
      ks[t][c] = ok ? ld(kb + (int64_t)(t0 + t) * p.k_st + c) : 0.f;
      vs[t][c] = ok ? ld(vb + (int64_t)(t0 + t) * p.k_st + c) : 0.f;
    }
    __syncthreads();
    const int lim = min(i + p.diag, p.n_k - 1) - t0;   // key t visible iff t <= lim
    for (int t = 0; t < TS; ++t) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) {
        s = __builtin_fmaf(q[c], ks[t][part * DP + c], s);
        dp = __builtin_fmaf(dov[c], vs[t][part * DP + c], dp);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      dp += __shfl_xor(dp, 1);
      dp += __shfl_xor(dp, 2);
      const float pr = (seen && t <= lim) ? expf(s * p.scale - lse) : 0.f;
      const float ds = pr * (dp - Dr) * p.scale;
#pragma unroll
      for (int c = 0; c < DP; ++c) dq[c] = __builtin_fmaf(ds, ks[t][part * DP + c], dq[c]);
    }
  }
  if (row_ok) {
    float* out = p.dq + srow * D + part * DP;
#pragma unroll
    for (int c = 0; c < DP; ++c) out[c] += dq[c];
  }
}

// dK, dV for 64 keys of one KV head against the query rows of every head in its group
template <typename T, int D>
__global__ __launch_bounds__(NT) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int DP = D / 4;
  __shared__ float qs[TS][D + 1];
  __shared__ float dos[TS][D + 1];
  __shared__ float lses[TS], Ds[TS];
  const int tid = threadIdx.x;
  const int key = tid >> 2, part = tid & 3;
  const int n_kt = (p.n_k + TR - 1) / TR;
  int w = blockIdx.x;
  const int kt = w % n_kt;
  w /= n_kt;
  const int g = w % p.kv_heads;
  const int b = w / p.kv_heads;
  const int t0 = kt * TR;
  const int t = t0 + key;
  const bool key_ok = t < p.n_k;
  // rows that can see some key of this tile: i >= t0 - diag
  const int i_first = max(0, t0 - p.diag);
  if (i_first >= p.n_q) return;

  float k[DP], v[DP], dk[DP], dv[DP];
  const T* kp = static_cast<const T*>(p.k) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh + (int64_t)t * p.k_st + part * DP;
  const T* vp = static_cast<const T*>(p.v) + (int64_t)b * p.k_sb + (int64_t)g * p.k_sh + (int64_t)t * p.k_st + part * DP;
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    k[c] = key_ok ? ld(kp + c) : 0.f;
    v[c] = key_ok ? ld(vp + c) : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  for (int hh = 0; hh < p.group; ++hh) {
    const int h = g * p.group + hh;
    const T* qb = static_cast<const T*>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    const T* dob = static_cast<const T*>(p.d_out) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    const int64_t sbase = ((int64_t)b * p.q_heads + h) * p.state_rows;
    for (int r0 = (i_first / TS) * TS; r0 < p.n_q; r0 += TS) {
      __syncthreads();
      for (int e = tid; e < TS * D; e += NT) {
        const int r = e / D, c = e % D;
        const bool ok = r0 + r < p.n_q;
        qs[r][c] = ok ? ld(qb + (int64_t)(r0 + r) * p.q_st + c) : 0.f;
        dos[r][c] = ok ? ld(dob + (int64_t)(r0 + r) * p.q_st + c) : 0.f;
      }
      if (tid < TS) {
        const bool ok = r0 + tid < p.n_q;
        lses[tid] = ok ? p.lse[sbase + r0 + tid] : -INFINITY;
        Ds[tid] = ok ? p.D[sbase + r0 + tid] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < TS; ++r) {
        const int i = r0 + r;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < DP; ++c) {
          s = __builtin_fmaf(k[c], qs[r][part * DP + c], s);
          dp = __builtin_fmaf(v[c], dos[r][part * DP + c], dp);
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        dp += __shfl_xor(dp, 1);
        dp += __shfl_xor(dp, 2);
        const float lse = lses[r];
        const bool ok = key_ok && i < p.n_q && lse != -INFINITY && t <= i + p.diag;
        const float pr = ok ? expf(s * p.scale - lse) : 0.f;
        const float ds = pr * (dp - Ds[r]) * p.scale;
#pragma unroll
        for (int c = 0; c < DP; ++c) {
          dv[c] = __builtin_fmaf(pr, dos[r][part * DP + c], dv[c]);
          dk[c] = __builtin_fmaf(ds, qs[r][part * DP + c], dk[c]);
        }
      }
    }
  }
  if (key_ok) {
    float* dkp = p.dk + ((int64_t)b * p.kv_heads + g) * p.dkv_rows * D + (int64_t)t * D + part * DP;
    float* dvp = p.dv + ((int64_t)b * p.kv_heads + g) * p.dkv_rows * D + (int64_t)t * D + part * DP;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
      dkp[c] += dk[c];
      dvp[c] += dv[c];
    }
  }
}

template <typename T, int D>
hipError_t launch_all(const BwdParams& p, hipStream_t stream) {
  const int n_qt = (p.n_q + TR - 1) / TR;
  const int n_kt = (p.n_k + TR - 1) / TR;
  const int64_t gq = (int64_t)n_qt * p.q_heads * p.batch;
  const int64_t gk = (int64_t)n_kt * p.kv_heads * p.batch;
  if (gq > 0) hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3((unsigned)gq), dim3(NT), 0, stream, p);
  if (gk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<T, D>), dim3((unsigned)gk), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_prep_d(const BwdPrepParams& p, hipStream_t stream) {
  const int rows_per_block = (NT / 64) * (64 / (D / 4));
  int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 256 * 8) blocks = 256 * 8;
  if (blocks > 0) hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const BwdPrepParams& p, int head_dim, bool bf16, hipStream_t stream) {
  if (head_dim == 64) return bf16 ? launch_prep_d<__bf16, 64>(p, stream) : launch_prep_d<float, 64>(p, stream);
  if (head_dim == 128) return bf16 ? launch_prep_d<__bf16, 128>(p, stream) : launch_prep_d<float, 128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_step_f32(const BwdParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_all<float, 64>(p, stream);
  if (head_dim == 128) return launch_all<float, 128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra
