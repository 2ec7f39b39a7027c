// Motion-bank minimum-L2 drift check (latency bound: <= 10 KiB of input).
//
// PersonaLive write-up, section 抗身份漂移的补丁: the current expression
// embedding is compared with every motion-bank entry; the smallest Euclidean
// distance decides whether an anchor is appended (distance above 17).
//
// One wavefront per query.  The inputs are fp32; each difference and its
// square are exact in fp64, and lane l sums the squares of elements l, l+64,
// l+128, ... in fp64 for every bank entry; the wave then reduces the 64
// partial sums with a fixed xor-butterfly, so the result is the same on every
// run and within a few fp64 ulps of the exact distance.  The minimum (lowest
// index on ties) and the strict comparison with the threshold are taken on
// the fp64 distances, so the decision only differs from an exact evaluation
// when a distance lies within about 1e-15 relative of the threshold; the
// reported minimum is that distance rounded to fp32.
#include "pl_internal.h"

namespace pl {
namespace {

constexpr int kWave = 64;

__device__ inline double wave_sum(double v) {
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
  double part[PL_MAX_MOTION_BANK];
#pragma unroll
  for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) part[j] = 0.0;
  // Every entry slot and element is read without a branch (slots past n
  // re-read the last entry, whose sums are ignored).  The elements are taken
  // in batches of 8 strides (all of a 512-d embedding): a batch's fp32 loads
  // all go out before any of them is used, so they share one memory round
  // trip, and only then are they widened and accumulated in fp64.
  const float* brow[PL_MAX_MOTION_BANK];
#pragma unroll
  for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) brow[j] = bank + (int64_t)min(j, n - 1) * D;
  constexpr int kStrides = 8;
  for (int k0 = 0; k0 < D; k0 += kWave * kStrides) {
    float qf[kStrides], bf[PL_MAX_MOTION_BANK][kStrides];
    // (elements beyond D are read at D-1 and their differences set to zero)
#pragma unroll
    for (int s = 0; s < kStrides; ++s) {
      const int k = min(k0 + s * kWave + lane, D - 1);
      qf[s] = q[k];
#pragma unroll
      for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) bf[j][s] = brow[j][k];
    }
#pragma unroll
    for (int s = 0; s < kStrides; ++s) {
      const bool in = k0 + s * kWave + lane < D;
#pragma unroll
      for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) {
        const double diff = in ? (double)qf[s] - (double)bf[j][s] : 0.0;
        part[j] = fma(diff, diff, part[j]);
      }
    }
  }
  double best = 0.0;
  int best_j = 0;
#pragma unroll
  for (int j = 0; j < PL_MAX_MOTION_BANK; ++j) {
    if (j < n) {
      const double dist = sqrt(wave_sum(part[j]));
      if (j == 0 || dist < best) {
        best = dist;
        best_j = j;
      }
    }
  }
  if (lane == 0) {
    min_dist[qi] = (float)best;
    argmin[qi] = best_j;
    exceeds[qi] = best > (double)threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_motion_min_l2(const MotionLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(motion_min_l2_kernel, dim3(a.nq), dim3(kWave), 0, stream, a.query, a.bank, a.n, a.D,
                     a.threshold, a.min_dist, a.argmin, a.exceeds);
  return hipGetLastError();
}

}  // namespace pl
