// ra_finalize.hip -- O = O~ / l and lse = ln(2) * (m + log2 l) after the last block
// ("Ring Attention：把超长序列沿设备环流动", section 环是怎样工作的: the local output is
// finalize(state); the normalisation is the one of "GPU ring attention", section "Why
// partial results are allowed to merge").
//
// A pure streaming pass (reads 4*d + 8 bytes and writes 4*d + 4 bytes per row), so it is
// bound by HBM bandwidth.  A row is d/4 lanes of 16-byte vectors, so one wave covers 64/(d/4)
// consecutive rows per pass with consecutive lanes on consecutive addresses; each wave
// takes four such groups per iteration (four loads in flight per lane) and the grid strides
// over the rows.  Rows that never saw an allowed key (l = 0) give O = 0 and lse = -inf.

#include <hip/hip_runtime.h>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int NT = 256;
constexpr int U = 4;   // row groups per wave per iteration
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(NT) void finalize_kernel(FinalizeParams p) {
  constexpr int VPR = D / 4;        // 16-byte vectors per row
  constexpr int RPW = 64 / VPR;     // rows per wave per group
  const int lane = threadIdx.x & 63;
  const int sub = lane / VPR, vec = lane % VPR;
  const int64_t wave = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * (NT / 64);
  const f32x4* src = reinterpret_cast<const f32x4*>(p.o_acc);
  f32x4* dst = reinterpret_cast<f32x4*>(p.o);
  for (int64_t r0 = wave * (RPW * U); r0 < p.rows; r0 += n_waves * (RPW * U)) {
    f32x4 x[U];
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u * RPW + sub;
      l[u] = 0.f;
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (r < p.rows && !p.fresh) {
        l[u] = p.l[r];
        x[u] = __builtin_nontemporal_load(&src[r * VPR + vec]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u * RPW + sub;
      if (r >= p.rows) continue;
      const f32x4 out = l[u] > 0.f ? x[u] * (1.0f / l[u]) : f32x4{0.f, 0.f, 0.f, 0.f};
      __builtin_nontemporal_store(out, &dst[r * VPR + vec]);
      if (p.lse && vec == 0)
        p.lse[r] = l[u] > 0.f ? 0.69314718055994530942f * (p.m[r] + log2f(l[u])) : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_finalize(const FinalizeParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const int rows_per_block = (NT / 64) * (64 / (p.d / 4)) * U;
  int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 8;   // 8 workgroups per CU is plenty for a streaming pass
  if (blocks > cap) blocks = cap;
  switch (p.d) {
    case 64:
      hipLaunchKernelGGL(finalize_kernel<64>, dim3((unsigned)blocks), dim3(NT), 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL(finalize_kernel<128>, dim3((unsigned)blocks), dim3(NT), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
