// ra_finalize.hip -- O = O~ / l and lse = ln(2) * (m + log2 l) after the last block
// ("Ring Attention：把超长序列沿设备环流动", section 环是怎样工作的: the local output is
// finalize(state); the normalisation is the one of "GPU ring attention", section "Why
// partial results are allowed to merge").
//
// A pure streaming pass (reads 4*d + 8 bytes and writes 4*d + 4 bytes per row), so it is
// bound by HBM bandwidth: each lane moves 16-byte vectors, consecutive lanes cover
// consecutive addresses, and the grid is sized to keep every CU busy with a grid-stride
// loop.  Rows that never saw an allowed key (l = 0) give O = 0 and lse = -inf.

#include <hip/hip_runtime.h>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int NT = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(NT) void finalize_kernel(FinalizeParams p) {
  const int vec_per_row = p.d / 4;
  const int64_t n_vec = p.rows * vec_per_row;
  const int64_t stride = (int64_t)gridDim.x * NT;
  const f32x4* src = reinterpret_cast<const f32x4*>(p.o_acc);
  f32x4* dst = reinterpret_cast<f32x4*>(p.o);
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < n_vec; e += stride) {
    const int64_t r = e / vec_per_row;
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    if (!p.fresh) {
      const float l = p.l[r];
      if (l > 0.f) {
        const float inv = 1.0f / l;
        out = __builtin_nontemporal_load(&src[e]) * inv;
      }
    }
    __builtin_nontemporal_store(out, &dst[e]);
    if (p.lse && (e - r * vec_per_row) == 0) {
      float lse = -INFINITY;
      if (!p.fresh) {
        const float l = p.l[r];
        if (l > 0.f) lse = 0.69314718055994530942f * (p.m[r] + log2f(l));
      }
      p.lse[r] = lse;
    }
  }
}

}  // namespace

hipError_t launch_finalize(const FinalizeParams& p, hipStream_t stream) {
  const int64_t n_vec = p.rows * (p.d / 4);
  if (n_vec == 0) return hipSuccess;
  int64_t blocks = (n_vec + NT - 1) / NT;
  const int64_t cap = 256 * 16;   // 16 workgroups per CU is plenty for a streaming pass
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
