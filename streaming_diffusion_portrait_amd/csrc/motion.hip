// Motion-bank minimum-L2 drift check (latency bound: <= 10 KiB of input).
//
// PersonaLive write-up, section 抗身份漂移的补丁: the current expression
// embedding is compared with every motion-bank entry; the smallest Euclidean
// distance decides whether an anchor is appended (distance above 17).
//
// One wavefront per query.  Lane l accumulates the squared differences of
// elements l, l+64, l+128, ... in fp32 for every bank entry, then the wave
// reduces the 64 partial sums with a fixed xor-butterfly, so the result is
// the same on every run.  Lane 0 takes sqrt, the minimum (lowest index on
// ties) and the strict comparison with the threshold.
#include "pl_internal.h"

namespace pl {
namespace {

constexpr int kWave = 64;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__global__ void __launch_bounds__(kWave)
motion_min_l2_kernel(const float* __restrict__ query, const float* __restrict__ bank, int n, int D,
                     float threshold, float* __restrict__ min_dist, int32_t* __restrict__ argmin,
                     uint8_t* __restrict__ exceeds) {
  const int qi = blockIdx.x;
  const int lane = threadIdx.x;
  const float* q = query + (int64_t)qi * D;
  float part[PL_MAX_MOTION_BANK];
#pragma unroll
  for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) part[j] = 0.f;
  // Every entry slot is read without a branch (slots past n re-read the last
  // entry; their sums are ignored) and the loop is unrolled, so the loads of 8
  // strides (all of a 512-d embedding) are in flight together instead of one
  // memory round trip per load.
  const float* brow[PL_MAX_MOTION_BANK];
#pragma unroll
  for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) brow[j] = bank + (int64_t)min(j, n - 1) * D;
#pragma unroll 8
  for (int k = lane; k < D; k += kWave) {
    const float qv = q[k];
#pragma unroll
    for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) {
      const float diff = qv - brow[j][k];
      part[j] = fmaf(diff, diff, part[j]);
    }
  }
  float best = 0.f;
  int best_j = 0;
#pragma unroll
  for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) {
    if (j < n) {
      const float dist = sqrtf(wave_sum(part[j]));
      if (j == 0 || dist < best) {
        best = dist;
        best_j = j;
      }
    }
  }
  if (lane == 0) {
    min_dist[qi] = best;
    argmin[qi] = best_j;
    exceeds[qi] = best > threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_motion_min_l2(const MotionLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(motion_min_l2_kernel, dim3(a.nq), dim3(kWave), 0, stream, a.query, a.bank, a.n, a.D,
                     a.threshold, a.min_dist, a.argmin, a.exceeds);
  return hipGetLastError();
}

}  // namespace pl
