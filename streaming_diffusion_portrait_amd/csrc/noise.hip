// The pile's device-side roll: window noise, staircase prefill and the first
// frames' motion interpolation.
//
// PersonaLive write-up, section 流式金字塔去噪: a new window of noise enters
// the pile every round; section 首帧怎么办: the queue starts with 12 frames
// (three windows) of staircase noise, and the pose / expression inputs of
// those frames are linear interpolations, 12 + 1 points from the reference's
// to the first driving frame's with the last point dropped.  The noise recipe
// is in philox.h.  All three are elementwise and memory-light (a window is
// 256 KiB at 512x512), so each is one plain launch.
#include "philox.h"
#include "pl_internal.h"

namespace pl {
namespace {

constexpr int kThreads = 256;

// out[w][i] = ca[w] * ref[i] + cb[w] * noise(seed, id0 + w)[i] (ref may be
// null: then out = cb * noise).  One thread per 4-element noise block.
__global__ void __launch_bounds__(kThreads)
noise_affine_kernel(const float* ref, float* out, int64_t n, int64_t out_stride, uint64_t seed, uint64_t id0,
                    NoiseLaunch cf) {
  const int w = blockIdx.y;
  const int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t i0 = 4 * blk;
  if (i0 >= n) return;
  const f4n z = normal4(seed, id0 + (uint64_t)w, (uint64_t)blk);
  float* o = out + (int64_t)w * out_stride;
  const float ca = cf.ca[w], cb = cf.cb[w];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t i = i0 + e;
    if (i < n) o[i] = ref ? fmaf(ca, ref[i], cb * z[e]) : cb * z[e];
  }
}

// out[k][i] = a[i] + (b[i] - a[i]) * k / n for k < n.
__global__ void __launch_bounds__(kThreads)
lerp_points_kernel(const float* a, const float* b, int64_t D, int n, float* out) {
  const int k = blockIdx.y;
  const float t = (float)k / (float)n;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < D; i += (int64_t)gridDim.x * kThreads) {
    const float av = a[i];
    out[(int64_t)k * D + i] = fmaf(b[i] - av, t, av);
  }
}

}  // namespace

hipError_t launch_noise_affine(const NoiseLaunch& a, hipStream_t stream) {
  const int64_t blocks = (a.n + 4 * kThreads - 1) / (4 * kThreads);
  hipLaunchKernelGGL(noise_affine_kernel, dim3((unsigned)blocks, (unsigned)a.nw), dim3(kThreads), 0, stream, a.ref,
                     a.out, a.n, a.out_stride, a.seed, a.id0, a);
  return hipGetLastError();
}

hipError_t launch_lerp_points(const float* a, const float* b, int64_t D, int n, float* out, hipStream_t stream) {
  int64_t bx = (D + kThreads - 1) / kThreads;
  if (bx > 4096) bx = 4096;
  hipLaunchKernelGGL(lerp_points_kernel, dim3((unsigned)bx, (unsigned)n), dim3(kThreads), 0, stream, a, b, D, n, out);
  return hipGetLastError();
}

}  // namespace pl
