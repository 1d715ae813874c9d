// ra_merge.hip -- the global online-softmax reduction of shard states: several states of the
// same query rows, each over a disjoint set of keys, combined into one
// ("Ring Attention：把超长序列沿设备环流动", section 训练与推理的适用方式不同: for decode the query goes to
// the KV shards, each computes a local attention state, and one reduction combines them; the
// combination is the rescale-and-add of "GPU ring attention", section "Why partial results are
// allowed to merge").  With the states' reference maxima m_s in base 2 and m = max_s m_s:
//     l = sum_s 2^(m_s - m) l_s,     O~ = sum_s 2^(m_s - m) O~_s,
// optionally followed by the finalize O = O~ / l, lse = ln 2 * (m + log2 l).
//
// A streaming pass like finalize: it reads every part's state once (n_parts * (4d + 8) bytes
// per row) and writes the merged state and/or O and lse, so it is bound by HBM bandwidth.  A
// row is d/4 lanes of 16-byte vectors; a wave covers 64/(d/4) rows per group and two groups
// per iteration; the parts loop keeps one O~ load per part and group in flight.

#include <hip/hip_runtime.h>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int NT = 256;
constexpr int U = 2;   // row groups per wave per iteration
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(NT) void merge_kernel(MergeParams p) {
  constexpr int VPR = D / 4;        // 16-byte vectors per row
  constexpr int RPW = 64 / VPR;     // rows per wave per group
  const int lane = threadIdx.x & 63;
  const int sub = lane / VPR, vec = lane % VPR;
  const int64_t wave = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * (NT / 64);
  for (int64_t r0 = wave * (RPW * U); r0 < p.rows; r0 += n_waves * (RPW * U)) {
    int64_t r[U];
    bool ok[U];
    float mx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      r[u] = r0 + u * RPW + sub;
      ok[u] = r[u] < p.rows;
      mx[u] = -INFINITY;
    }
    // the common reference: the largest of the parts' references
    for (int s = 0; s < p.n_parts; ++s) {
      const float* m_s = reinterpret_cast<const float*>(p.parts[s] + p.m_off);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ok[u]) mx[u] = fmaxf(mx[u], m_s[r[u]]);
    }
    float l[U];
    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      l[u] = 0.f;
      acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s = 0; s < p.n_parts; ++s) {
      const float* o_s = reinterpret_cast<const float*>(p.parts[s]);
      const float* m_s = reinterpret_cast<const float*>(p.parts[s] + p.m_off);
      const float* l_s = reinterpret_cast<const float*>(p.parts[s] + p.l_off);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const float ms = m_s[r[u]];
        // a part that has seen no key of this row (m_s = -inf) adds nothing; when no part
        // has (mx = -inf) the row stays empty
        const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mx[u]);
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o_s) + r[u] * VPR + vec);
        l[u] = __builtin_fmaf(w, l_s[r[u]], l[u]);
        acc[u] += w * x;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      if (p.merged) {
        if (vec == 0) {
          reinterpret_cast<float*>(p.merged + p.m_off)[r[u]] = mx[u];
          reinterpret_cast<float*>(p.merged + p.l_off)[r[u]] = l[u];
        }
        reinterpret_cast<f32x4*>(p.merged)[r[u] * VPR + vec] = acc[u];
      }
      if (p.o) {
        const f32x4 out = l[u] > 0.f ? acc[u] * (1.0f / l[u]) : f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_nontemporal_store(out, reinterpret_cast<f32x4*>(p.o) + r[u] * VPR + vec);
        if (p.lse && vec == 0)
          p.lse[r[u]] = l[u] > 0.f ? 0.69314718055994530942f * (mx[u] + log2f(l[u])) : -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const int rows_per_block = (NT / 64) * (64 / (p.d / 4)) * U;
  int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 8;
  if (blocks > cap) blocks = cap;
  switch (p.d) {
    case 64:
      hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(NT), 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(NT), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
