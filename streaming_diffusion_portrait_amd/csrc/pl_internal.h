// Internal interface between the C-ABI host layer (pl_api.hip) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pl.h"

namespace pl {

// ---- reference-bank attention ---------------------------------------------
struct AttnSegment {
  const _Float16* k;
  const _Float16* v;
  int64_t len;
  int64_t ld;
  int64_t frame_stride;
};

struct AttnLaunch {
  const _Float16* q;
  _Float16* o;
  int64_t q_ld, q_frame_stride;
  int64_t o_ld, o_frame_stride;
  int32_t F, Lq, H, d;
  int32_t nseg;
  AttnSegment seg[PL_MAX_SEGMENTS];
  float scale;
  void* workspace;  // >= refbank_attn_workspace_bytes(...) bytes, 16-byte aligned, or nullptr (no key split)
};

// Bytes of workspace the launch below uses for these sizes (0: it splits nothing).
size_t refbank_attn_workspace_bytes(int32_t F, int32_t Lq, int32_t H, int32_t d, const int64_t* seg_len,
                                    int32_t nseg);

// Launch the flash-style MFMA attention for one layer on `stream`.
hipError_t launch_refbank_attn(const AttnLaunch& a, hipStream_t stream);

// Bounds-checking builds: read (and optionally clear) the mask of access sites
// that failed their check; hipErrorNotSupported in other builds.
hipError_t debug_bounds_mask(unsigned long long* mask, bool reset);

// ---- pyramid DDIM -------------------------------------------------------------
struct DdimLaunch {
  const float* x_t;
  const float* eps;
  float* x_prev;
  float* x0_out;      // nullptr when no window is emitted
  int32_t W;
  int64_t elems_per_window;
  int32_t emit_window;  // -1 = none
  // per-window coefficients: x_prev = a*x_t + b*eps, x0 = c*x_t + d*eps
  float a[PL_MAX_WINDOWS], b[PL_MAX_WINDOWS], c[PL_MAX_WINDOWS], d[PL_MAX_WINDOWS];
  // roll: the emitted window's x_prev slot receives noise(seed, new_id)
  int32_t roll;
  uint64_t seed, new_id;
};

hipError_t launch_pyramid_ddim(const DdimLaunch& a, hipStream_t stream);

// The rolling step driven by a device-resident pile state, then the state's
// advance (two launches).  Requires 16-byte aligned buffers and
// elems_per_window % 4 == 0.
struct DeviceRoundLaunch {
  const float* x_t;
  const float* eps;
  float* x_prev;
  float* x0_out;
  int32_t W;
  int64_t elems_per_window;
  pl_pile* pile;                 // device
  const double* alphas_cumprod;  // device [T]
  int32_t T;
  double final_alpha_cumprod;
  uint64_t seed;
};

hipError_t launch_pyramid_round_device(const DeviceRoundLaunch& a, hipStream_t stream);

// ---- pile roll: window noise, staircase prefill, interpolation -----------------
struct NoiseLaunch {
  const float* ref;    // nullptr: pure noise
  float* out;          // nw windows of n elements, out_stride apart
  int64_t n, out_stride;
  int32_t nw;
  uint64_t seed, id0;  // window w draws noise(seed, id0 + w)
  float ca[PL_MAX_WINDOWS], cb[PL_MAX_WINDOWS];
};

hipError_t launch_noise_affine(const NoiseLaunch& a, hipStream_t stream);
hipError_t launch_lerp_points(const float* a, const float* b, int64_t D, int n, float* out, hipStream_t stream);

// ---- projections: y = x W^T (+ b) ----------------------------------------------
struct LinearLaunch {
  const _Float16* x;  // [M][x_ld]
  const _Float16* w;  // [N][w_ld] (out features x in features)
  const float* bias;  // [N] or nullptr
  _Float16* y;        // [M][y_ld]
  int64_t x_ld, w_ld, y_ld;
  int64_t M;
  int32_t N, K;       // N % 64 == 0, K % 16 == 0
};

hipError_t launch_linear(const LinearLaunch& a, hipStream_t stream);

// ---- motion-bank min-L2 -------------------------------------------------------
struct MotionLaunch {
  const float* query;
  const float* bank;
  int32_t nq, n, D;
  float threshold;
  float* min_dist;
  int32_t* argmin;
  uint8_t* exceeds;
};

hipError_t launch_motion_min_l2(const MotionLaunch& a, hipStream_t stream);

}  // namespace pl
