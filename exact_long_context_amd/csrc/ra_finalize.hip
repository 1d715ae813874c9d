// ra_finalize.hip -- O = O~ / l and lse = ln(2) * (m + log2 l) after the last block
// ("Ring Attention：把超长序列沿设备环流动", section 环是怎样工作的: the local output is
// finalize(state); the normalisation is the one of "GPU ring attention", section "Why
// partial results are allowed to merge").
//
// A pure streaming pass (reads 4*d + 8 bytes and writes 4*d + 4 bytes per row), so it is
// bound by HBM bandwidth.  A row is d/4 lanes of 16-byte vectors, so one wave covers 64/(d/4)
// consecutive rows per pass with consecutive lanes on consecutive addresses; each wave
// takes four such groups per iteration (four O~ loads in flight per lane, with their l and m)
// and the grid strides over the rows.  Rows that never saw an allowed key (l = 0) give O = 0 and lse = -inf.

#include <hip/hip_runtime.h>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int NT = 256;
constexpr int U = 4;   // row groups per wave per iteration
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fin_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 4))) void finalize_kernel(FinalizeParams p) {
  constexpr int VPR = D / 4;        // 16-byte vectors per row
  constexpr int RPW = 64 / VPR;     // rows per wave per group
  constexpr int RPI = RPW * U;      // rows per wave per iteration
  const int lane = threadIdx.x & 63;
  const int sub = lane / VPR, vec = lane % VPR;
  const int64_t wave = (int64_t)blockIdx.x * (NT / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * (NT / 64);
  for (int64_t r0 = wave * RPI; r0 < p.rows; r0 += n_waves * RPI) {
    // Every load of the iteration is issued before any is used: O~ (nontemporal, read once),
    // l and m, through resources that end at the last row (or hold nothing for a fresh state),
    // so a row past the end reads 0 with no branch around its load.
    const int64_t left = p.fresh ? 0 : p.rows - r0;
    const __amdgpu_buffer_rsrc_t ro = fin_rsrc(p.o_acc + r0 * D, left * D * 4);
    const __amdgpu_buffer_rsrc_t rl = fin_rsrc(p.l + r0, left * 4);
    const __amdgpu_buffer_rsrc_t rm = fin_rsrc(p.m + r0, left * 4);
    f32x4 x[U];
    float l[U], m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = u * RPW + sub;   // row within the iteration
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(ro, (rr * VPR + vec) * 16, 0, 2);
      __builtin_memcpy(&x[u], &v, sizeof x[u]);
      l[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, rr * 4, 0, 0));
      m[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, rr * 4, 0, 0));
    }
    // The stores go through resources that end at the last row as well: the hardware drops a
    // store past the end, so no branch holds a load back to its use.  One lane per row (vec 0)
    // writes lse; the others aim past the end.
    const int64_t rows_left = p.rows - r0;
    const __amdgpu_buffer_rsrc_t wo = fin_rsrc(p.o + r0 * D, rows_left * D * 4);
    const __amdgpu_buffer_rsrc_t wl = fin_rsrc(p.lse ? p.lse + r0 : nullptr, p.lse ? rows_left * 4 : 0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = u * RPW + sub;
      const bool seen = l[u] > 0.f;
      const float inv = 1.0f / l[u];
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = seen ? x[u][e] * inv : 0.f;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, out), wo, (rr * VPR + vec) * 16, 0, 2);
      const float lse = seen ? 0.69314718055994530942f * (m[u] + log2f(l[u])) : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), wl, vec == 0 ? rr * 4 : 0x7fffffff, 0, 0);
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
