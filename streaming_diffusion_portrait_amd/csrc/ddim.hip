// Fused per-window DDIM step over the latents pile (HBM-bandwidth bound).
//
// PersonaLive write-up, section 流式金字塔去噪: one forward gives every window
// of the pile its epsilon estimate, every window steps from its own t to
// t - 333, and the window leaving the queue hands its x0 estimate
// (pred_original_sample) to the VAE.  The host folds alpha_bar[t] and
// alpha_bar[t - step] into four fp64 coefficients per window, rounded to fp32:
//   x_prev = a_w * x_t + b_w * eps,   x0 = c_w * x_t + d_w * eps.
//
// One pass: each element of x_t and eps is read once; x_prev is written for
// every window and x0 only for the emitted one (12 B/element + 4 B per
// emitted element).  The grid is 2-D: blockIdx.y selects the window, so the
// coefficients are wave-uniform (scalar registers) and no per-element
// division is needed.  Loads and stores are 16 B per lane.
#include "philox.h"
#include "pl_internal.h"

namespace pl {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kDdimThreads = 256;
constexpr int kDdimUnroll = 4;  // float4 per thread per grid-stride step

// ROLL: the emitted window's x_prev slot takes the next window's noise (a
// separate instantiation, so the plain step carries none of that code).
template <bool ROLL>
__global__ void __launch_bounds__(kDdimThreads)
ddim_vec4_kernel(const f4v* x_t, const f4v* eps, f4v* x_prev,
                 f4v* __restrict__ x0_out, int64_t n4_per_window, int emit_window, DdimLaunch cf) {
  const int w = blockIdx.y;
  const float a = cf.a[w], b = cf.b[w], c = cf.c[w], d = cf.d[w];
  const bool emit = (w == emit_window);
  const f4v* xw = x_t + (int64_t)w * n4_per_window;
  const f4v* ew = eps + (int64_t)w * n4_per_window;
  f4v* pw = x_prev + (int64_t)w * n4_per_window;
  const int64_t stride = (int64_t)gridDim.x * kDdimThreads * kDdimUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kDdimThreads * kDdimUnroll + threadIdx.x; base < n4_per_window;
       base += stride) {
    f4v xv[kDdimUnroll], ev[kDdimUnroll];
#pragma unroll
    for (int u = 0; u < kDdimUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kDdimThreads;
      if (i < n4_per_window) {
        xv[u] = __builtin_nontemporal_load(xw + i);
        ev[u] = __builtin_nontemporal_load(ew + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kDdimUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kDdimThreads;
      if (i < n4_per_window) {
        f4v pv;
        if (ROLL && emit) {
          // the leaving window's slot becomes next round's new window: its own
          // x_prev is never used, so the slot takes the new window's noise
          // (float4 i of the window is noise block i)
          pv = normal4(cf.seed, cf.new_id, (uint64_t)i);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) pv[k] = fmaf(a, xv[u][k], b * ev[u][k]);
        }
        __builtin_nontemporal_store(pv, pw + i);
        if (emit) {
          f4v z;
#pragma unroll
          for (int k = 0; k < 4; ++k) z[k] = fmaf(c, xv[u][k], d * ev[u][k]);
          __builtin_nontemporal_store(z, x0_out + i);
        }
      }
    }
  }
}

// Scalar variant for sizes or pointers that do not allow 16 B accesses.
template <bool ROLL>
__global__ void __launch_bounds__(kDdimThreads)
ddim_scalar_kernel(const float* x_t, const float* eps, float* x_prev,
                   float* __restrict__ x0_out, int64_t n_per_window, int emit_window, DdimLaunch cf) {
  const int w = blockIdx.y;
  const float a = cf.a[w], b = cf.b[w], c = cf.c[w], d = cf.d[w];
  const bool emit = (w == emit_window);
  const int64_t off = (int64_t)w * n_per_window;
  for (int64_t i = (int64_t)blockIdx.x * kDdimThreads + threadIdx.x; i < n_per_window;
       i += (int64_t)gridDim.x * kDdimThreads) {
    const float xv = x_t[off + i], ev = eps[off + i];
    if (emit) x0_out[i] = fmaf(c, xv, d * ev);
    if (ROLL && emit)
      x_prev[off + i] = normal4(cf.seed, cf.new_id, (uint64_t)(i >> 2))[i & 3];
    else
      x_prev[off + i] = fmaf(a, xv, b * ev);
  }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- device-resident round -----------------------------------------------------
//
// The round's integer state (the pl_pile struct) lives in device memory, so a
// round is a fixed sequence of launches that one captured graph can replay
// every round: the step reads each slot's timestep, the leaving slot and the
// next window's id from the state, takes its coefficients from an fp64
// alpha_bar table in device memory, and a one-thread kernel then advances the
// state.  Every index read from the state is clamped into range, so a
// corrupted state gives wrong values but no access out of bounds.

struct RoundView {
  int t[PL_MAX_WINDOWS];
  int emit;        // slot of the window at t = 0 after the new window enters, or -1
  uint64_t roll_id;  // id of the window that enters next round (its noise fills the leaving slot)
};

__device__ inline int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// The state as pl_pile_begin_round would leave it, without writing it.
__device__ inline RoundView round_view(const pl_pile* st, int W) {
  RoundView v;
  const int head = clampi(st->head, 0, W - 1);
  const int count = clampi(st->count, 0, W);
  const int fresh = count < W ? (head + count) % W : -1;  // slot of the window entering now
  for (int s = 0; s < W; ++s) v.t[s] = (st->id[s] >= 0 && s != fresh) ? st->t[s] : st->t_top;
  v.emit = (count > 0 && st->id[head] >= 0 && st->t[head] == 0) ? head : -1;
  v.roll_id = (uint64_t)(st->next_id + (fresh >= 0 ? 1 : 0));
  return v;
}

// Per-window coefficients in fp64, rounded to fp32 (as the host path does).
__device__ inline void window_coefficients(const double* ab, int T, int t, int step_len, double fin, float& a,
                                           float& b, float& c, float& d) {
  t = clampi(t, 0, T - 1);
  const double at = ab[t];
  const int prev = t - step_len;
  const double ap = prev >= 0 ? ab[prev] : fin;
  const double cc = 1.0 / sqrt(at);
  const double dd = -sqrt(1.0 - at) / sqrt(at);
  a = (float)(sqrt(ap) * cc);
  b = (float)(sqrt(ap) * dd + sqrt(1.0 - ap));
  c = (float)cc;
  d = (float)dd;
}

__global__ void __launch_bounds__(kDdimThreads)
ddim_device_state_kernel(const f4v* x_t, const f4v* eps, f4v* x_prev, f4v* __restrict__ x0_out,
                         int64_t n4_per_window, int W, const pl_pile* __restrict__ st, const double* __restrict__ ab,
                         int T, double fin, uint64_t seed) {
  const int w = blockIdx.y;
  const RoundView v = round_view(st, W);
  const int step_len = max(st->step_len, 1);
  float a, b, c, d;
  window_coefficients(ab, T, v.t[w], step_len, fin < 0.0 ? ab[0] : fin, a, b, c, d);
  const bool emit = (w == v.emit);
  const f4v* xw = x_t + (int64_t)w * n4_per_window;
  const f4v* ew = eps + (int64_t)w * n4_per_window;
  f4v* pw = x_prev + (int64_t)w * n4_per_window;
  const int64_t stride = (int64_t)gridDim.x * kDdimThreads * kDdimUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kDdimThreads * kDdimUnroll + threadIdx.x; base < n4_per_window;
       base += stride) {
    f4v xv[kDdimUnroll], ev[kDdimUnroll];
#pragma unroll
    for (int u = 0; u < kDdimUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kDdimThreads;
      if (i < n4_per_window) {
        xv[u] = __builtin_nontemporal_load(xw + i);
        ev[u] = __builtin_nontemporal_load(ew + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kDdimUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kDdimThreads;
      if (i < n4_per_window) {
        f4v pv;
        if (emit) {
          pv = normal4(seed, v.roll_id, (uint64_t)i);
          f4v z;
#pragma unroll
          for (int k = 0; k < 4; ++k) z[k] = fmaf(c, xv[u][k], d * ev[u][k]);
          __builtin_nontemporal_store(z, x0_out + i);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) pv[k] = fmaf(a, xv[u][k], b * ev[u][k]);
        }
        __builtin_nontemporal_store(pv, pw + i);
      }
    }
  }
}

// begin_round + end_round of the pile's state machine, on the device (one thread).
__global__ void pile_advance_kernel(pl_pile* st, int W) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int head = clampi(st->head, 0, W - 1);
  int count = clampi(st->count, 0, W);
  if (count < W) {  // the new window enters at the top
    const int s = (head + count) % W;
    st->id[s] = st->next_id;
    st->next_id += 1;
    st->t[s] = st->t_top;
    count += 1;
  }
  if (count > 0 && st->id[head] >= 0 && st->t[head] == 0) {  // the window at t = 0 leaves
    st->id[head] = -1;
    st->t[head] = st->t_top;
    head = (head + 1) % W;
    count -= 1;
  }
  for (int k = 0; k < count; ++k) st->t[(head + k) % W] -= st->step_len;
  st->head = head;
  st->count = count;
  st->in_round = 0;
}

}  // namespace

hipError_t launch_pyramid_round_device(const DeviceRoundLaunch& a, hipStream_t stream) {
  const int64_t per_block = (int64_t)kDdimThreads * kDdimUnroll * 4;
  int64_t bx = (a.elems_per_window + per_block - 1) / per_block;
  const int64_t cap = (256 * 64 + a.W - 1) / a.W;
  if (bx > cap) bx = cap;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL(ddim_device_state_kernel, dim3((unsigned)bx, (unsigned)a.W), dim3(kDdimThreads), 0, stream,
                     reinterpret_cast<const f4v*>(a.x_t), reinterpret_cast<const f4v*>(a.eps),
                     reinterpret_cast<f4v*>(a.x_prev), reinterpret_cast<f4v*>(a.x0_out), a.elems_per_window / 4,
                     a.W, a.pile, a.alphas_cumprod, a.T, a.final_alpha_cumprod, a.seed);
  if (hipError_t e = hipGetLastError()) return e;
  hipLaunchKernelGGL(pile_advance_kernel, dim3(1), dim3(64), 0, stream, a.pile, a.W);
  return hipGetLastError();
}

hipError_t launch_pyramid_ddim(const DdimLaunch& a, hipStream_t stream) {
  const bool vec = (a.elems_per_window % 4 == 0) && aligned16(a.x_t) && aligned16(a.eps) &&
                   aligned16(a.x_prev) && (a.x0_out == nullptr || aligned16(a.x0_out));
  // Enough blocks to cover the window in one grid-stride step, capped at 64
  // blocks per CU in total (measured on 832 MiB piles: 16 per CU reached 77%
  // of 8 TB/s, 64 or more 80%).
  const int64_t per_block = vec ? (int64_t)kDdimThreads * kDdimUnroll * 4 : (int64_t)kDdimThreads;
  int64_t bx = (a.elems_per_window + per_block - 1) / per_block;
  const int64_t cap = (256 * 64 + a.W - 1) / a.W;
  if (bx > cap) bx = cap;
  if (bx < 1) bx = 1;
  dim3 grid((unsigned)bx, (unsigned)a.W);
  if (vec) {
    hipLaunchKernelGGL(a.roll ? ddim_vec4_kernel<true> : ddim_vec4_kernel<false>, grid, dim3(kDdimThreads), 0, stream,
                       reinterpret_cast<const f4v*>(a.x_t), reinterpret_cast<const f4v*>(a.eps),
                       reinterpret_cast<f4v*>(a.x_prev), reinterpret_cast<f4v*>(a.x0_out),
                       a.elems_per_window / 4, a.emit_window, a);
  } else {
    hipLaunchKernelGGL(a.roll ? ddim_scalar_kernel<true> : ddim_scalar_kernel<false>, grid, dim3(kDdimThreads), 0,
                       stream, a.x_t, a.eps, a.x_prev,
                       a.x0_out, a.elems_per_window, a.emit_window, a);
  }
  return hipGetLastError();
}

}  // namespace pl
