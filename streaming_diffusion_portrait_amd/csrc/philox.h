// Counter-based normal noise for the latents pile (device side).
//
// PersonaLive write-up, section 流式金字塔去噪: every round a new window of
// pure noise enters the pile at the top timestep; the TensorRT section feeds
// it as the new_noise input and keeps the rolling state on the device.  Here
// the noise of window `id` under `seed` is a pure function of (seed, id,
// element), so any window can be drawn on the device, in place, at any time.
//
// Generator: Philox-4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011): key (seed, id),
// counter (element / 4, 0, 0, 0), word element % 4.  A word x gives the
// uniform u = ((x >> 40) + 1) * 2^-24 in (0, 1] (exact in fp32); words (0, 1)
// and (2, 3) give two normals each by Box-Muller: r = sqrt(-2 ln u_even),
// z = r cos(2 pi u_odd), r sin(2 pi u_odd).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pl {

typedef float f4n __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;  // round multipliers
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;  // key increments
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t hi0 = __umul64hi(kM0, c[0]), lo0 = kM0 * c[0];
    const uint64_t hi1 = __umul64hi(kM1, c[2]), lo1 = kM1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

__device__ __forceinline__ float uniform24(uint64_t x) {
  return (float)((uint32_t)(x >> 40) + 1u) * (1.0f / 16777216.0f);
}

// The four normals of block `blk` (elements 4*blk .. 4*blk+3) of window `id`.
__device__ __forceinline__ f4n normal4(uint64_t seed, uint64_t id, uint64_t blk) {
  uint64_t c[4] = {blk, 0, 0, 0};
  philox4x64_10(c, seed, id);
  f4n z;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float r = sqrtf(-2.0f * logf(uniform24(c[2 * p])));
    float s, co;
    sincospif(2.0f * uniform24(c[2 * p + 1]), &s, &co);  // sin, cos of 2 pi u
    z[2 * p] = r * co;
    z[2 * p + 1] = r * s;
  }
  return z;
}

}  // namespace pl
