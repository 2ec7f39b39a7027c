// C-ABI host layer: argument validation, per-window DDIM coefficients, the
// pile state machine and kernel dispatch.  Every check runs before any HIP
// call, so an invalid call returns without touching the device.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "pl_internal.h"

namespace {

thread_local char g_last_error[512] = "";

pl_status fail(pl_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

pl_status ok() {
  g_last_error[0] = '\0';
  return PL_OK;
}

pl_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PL_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A strided fp16 view: rows of `width` elements, `ld` apart, in `frames`
// frames `fs` apart (fs = 0: one set of rows shared by every frame).
struct View {
  const void* p;
  int64_t ld, fs, rows, frames, width;
};

// May two views share an element?  Their byte ranges are compared first;
// when those meet, two views with the same row stride whose frame strides are
// whole rows are still disjoint if their column ranges within a row (taken
// modulo the row stride) do not meet -- the case of column slices of one
// fused buffer.  Anything else that meets is reported as overlapping.
bool views_may_overlap(const View& a, const View& b) {
  auto span = [](const View& v) {
    const int64_t nf = v.fs == 0 ? 1 : v.frames;
    return ((nf - 1) * v.fs + (v.rows - 1) * v.ld + v.width) * (int64_t)sizeof(uint16_t);
  };
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  const uintptr_t a1 = a0 + (uintptr_t)span(a), b1 = b0 + (uintptr_t)span(b);
  if (a1 <= b0 || b1 <= a0) return false;
  if (a.ld == b.ld && a.fs % a.ld == 0 && b.fs % b.ld == 0) {
    const int64_t diff = (int64_t)(a0 - b0);  // bytes; both views are 16-byte aligned
    const int64_t c = ((diff / 2) % a.ld + a.ld) % a.ld;  // a's first column relative to b's, modulo a row
    if (c >= b.width && c + a.width <= a.ld) return false;
  }
  return true;
}

// Stable Diffusion's scaled_linear schedule: beta_i = (s0 + i*(s1-s0)/(T-1))^2
// with s0 = sqrt(0.00085), s1 = sqrt(0.012), alpha_bar_t = prod_{i<=t}(1 - beta_i).
struct SdSchedule {
  double ab[1000];
  SdSchedule() {
    const int T = 1000;
    const double s0 = std::sqrt(0.00085), s1 = std::sqrt(0.012);
    double prod = 1.0;
    for (int i = 0; i < T; ++i) {
      const double r = (i == T - 1) ? s1 : s0 + (s1 - s0) * (double)i / (double)(T - 1);
      prod *= 1.0 - r * r;
      ab[i] = prod;
    }
  }
};

const SdSchedule& sd_schedule() {
  static const SdSchedule s;
  return s;
}

}  // namespace

namespace {

// The resolved noise schedule of a call (user table or the built-in one).
pl_status resolve_schedule(const char* fn, const double* alphas_cumprod_host, int32_t T, const double** ab) {
  if (alphas_cumprod_host) {
    if (T < 1) return fail(PL_EINVAL, "%s: T must be >= 1", fn);
    for (int i = 0; i < T; ++i)
      if (!(alphas_cumprod_host[i] > 0.0 && alphas_cumprod_host[i] <= 1.0))
        return fail(PL_EINVAL, "%s: alphas_cumprod[%d] not in (0, 1]", fn, i);
    *ab = alphas_cumprod_host;
  } else {
    if (T != 1000) return fail(PL_EINVAL, "%s: the built-in schedule has T = 1000 (got %d)", fn, T);
    *ab = sd_schedule().ab;
  }
  return PL_OK;
}

pl_status ddim_step_impl(const float* x_t, const float* eps, float* x_prev, float* x0_out, int32_t W,
                         int64_t elems_per_window, const int32_t* t_host, int32_t step_len,
                         const double* alphas_cumprod_host, int32_t T, double final_alpha_cumprod,
                         int32_t emit_window, int32_t roll, uint64_t seed, uint64_t new_id, void* stream) {
  if (!x_t || !eps || !x_prev) return fail(PL_EINVAL, "pl_pyramid_ddim_step: x_t, eps, x_prev must be non-null");
  if (!t_host) return fail(PL_EINVAL, "pl_pyramid_ddim_step: t_host must be non-null");
  if (W < 1 || W > PL_MAX_WINDOWS)
    return fail(PL_EINVAL, "pl_pyramid_ddim_step: W must be in [1, %d] (got %d)", PL_MAX_WINDOWS, W);
  if (elems_per_window < 1) return fail(PL_EINVAL, "pl_pyramid_ddim_step: elems_per_window must be >= 1");
  if (elems_per_window > (int64_t(1) << 40)) return fail(PL_EINVAL, "pl_pyramid_ddim_step: elems_per_window too large");
  if (step_len < 1) return fail(PL_EINVAL, "pl_pyramid_ddim_step: step_len must be >= 1");
  if (emit_window < -1 || emit_window >= W)
    return fail(PL_EINVAL, "pl_pyramid_ddim_step: emit_window must be -1 or in [0, W) (got %d)", emit_window);
  if (emit_window >= 0 && !x0_out) return fail(PL_EINVAL, "pl_pyramid_ddim_step: x0_out is required when emitting");
  const double* ab = nullptr;
  if (pl_status st = resolve_schedule("pl_pyramid_ddim_step", alphas_cumprod_host, T, &ab)) return st;
  double fin = final_alpha_cumprod;
  if (fin < 0.0) fin = ab[0];
  if (!(fin > 0.0 && fin <= 1.0)) return fail(PL_EINVAL, "pl_pyramid_ddim_step: final_alpha_cumprod not in (0, 1]");
  pl::DdimLaunch a;
  std::memset(&a, 0, sizeof(a));
  for (int w = 0; w < W; ++w) {
    const int t = t_host[w];
    if (t < 0 || t >= T) return fail(PL_EINVAL, "pl_pyramid_ddim_step: t[%d] = %d not in [0, %d)", w, t, T);
    const double at = ab[t];
    const int prev = t - step_len;
    const double ap = prev >= 0 ? ab[prev] : fin;
    // x0 = (x_t - sqrt(1-at) eps)/sqrt(at); x_prev = sqrt(ap) x0 + sqrt(1-ap) eps
    const double c = 1.0 / std::sqrt(at);
    const double d = -std::sqrt(1.0 - at) / std::sqrt(at);
    a.a[w] = (float)(std::sqrt(ap) * c);
    a.b[w] = (float)(std::sqrt(ap) * d + std::sqrt(1.0 - ap));
    a.c[w] = (float)c;
    a.d[w] = (float)d;
  }
  a.x_t = x_t;
  a.eps = eps;
  a.x_prev = x_prev;
  a.x0_out = emit_window >= 0 ? x0_out : nullptr;
  a.W = W;
  a.elems_per_window = elems_per_window;
  a.emit_window = emit_window;
  a.roll = roll;
  a.seed = seed;
  a.new_id = new_id;
  return device_status(pl::launch_pyramid_ddim(a, static_cast<hipStream_t>(stream)), "pl_pyramid_ddim_step launch");
}

}  // namespace

extern "C" {

int32_t pl_abi_version(void) { return PL_ABI_VERSION; }

const char* pl_status_string(pl_status s) {
  switch (s) {
    case PL_OK: return "PL_OK";
    case PL_EINVAL: return "PL_EINVAL";
    case PL_EUNSUPPORTED: return "PL_EUNSUPPORTED";
    case PL_EDEVICE: return "PL_EDEVICE";
    default: return "PL_UNKNOWN";
  }
}

const char* pl_last_error(void) { return g_last_error; }

// ---------------------------------------------------------------------------
size_t pl_refbank_attn_workspace_size(int32_t F, int32_t Lq, int32_t H, int32_t d, const int64_t* seg_len,
                                      int32_t nseg) {
  if (!seg_len || F < 1 || Lq < 1 || H < 1 || nseg < 1 || nseg > PL_MAX_SEGMENTS) return 0;
  if (d != 32 && d != 40 && d != 80 && d != 160) return 0;
  for (int i = 0; i < nseg; ++i)
    if (seg_len[i] < 1) return 0;
  return pl::refbank_attn_workspace_bytes(F, Lq, H, d, seg_len, nseg);
}

}  // extern "C"

namespace {

// Scratch of the allocation-free attention call: the key-split partials go to
// this device array instead of a caller workspace.  Each GPU holds its own
// copy for the life of the process.  Host code never uses the array's name
// as an address (on the host it is a stand-in): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pl_status scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PL_EDEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PL_EUNSUPPORTED, "%s: device index %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(PL_EDEVICE, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    if (!ptr) return fail(PL_EDEVICE, "%s: hipGetSymbolAddress(scratch) returned NULL", fn);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PL_OK;
}

// The checks of pl_refbank_attn and its variants; fills the launch
// description (noalloc: the key-split partials go to the library's scratch;
// workspace arguments are unused).
pl_status validate_attn(const char* fn, const void* q, int64_t q_ld, int64_t q_frame_stride, void* o, int64_t o_ld,
                        int64_t o_frame_stride, int32_t F, int32_t Lq, int32_t H, int32_t d,
                        const pl_kv_segment* segs, int32_t nseg, float scale, void* workspace,
                        size_t workspace_bytes, bool noalloc, pl::AttnLaunch* out) {
  pl::AttnLaunch& a = *out;
  if (!q || !o) return fail(PL_EINVAL, "pl_refbank_attn: q and o must be non-null");
  if (!segs) return fail(PL_EINVAL, "pl_refbank_attn: segs must be non-null");
  if (F < 1 || Lq < 1 || H < 1) return fail(PL_EINVAL, "pl_refbank_attn: F, Lq, H must be >= 1 (got %d, %d, %d)", F, Lq, H);
  if (nseg < 1 || nseg > PL_MAX_SEGMENTS)
    return fail(PL_EINVAL, "pl_refbank_attn: nseg must be in [1, %d] (got %d)", PL_MAX_SEGMENTS, nseg);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PL_EINVAL, "pl_refbank_attn: scale must be finite and > 0");
  if (d != 32 && d != 40 && d != 80 && d != 160)
    return fail(PL_EUNSUPPORTED, "pl_refbank_attn: head dim %d not supported (32, 40, 80, 160)", d);
  const int64_t width = (int64_t)H * d;
  if (q_ld < width || o_ld < width)
    return fail(PL_EINVAL, "pl_refbank_attn: q_ld/o_ld must be >= H*d = %lld", (long long)width);
  if (q_frame_stride < 0 || o_frame_stride < 0) return fail(PL_EINVAL, "pl_refbank_attn: frame strides must be >= 0");
  if (F > 1 && o_frame_stride < (int64_t)Lq * o_ld)
    return fail(PL_EINVAL, "pl_refbank_attn: o_frame_stride must be >= Lq*o_ld so frames do not overlap");
  if (q_ld % 8 || o_ld % 8 || q_frame_stride % 8 || o_frame_stride % 8)
    return fail(PL_EUNSUPPORTED, "pl_refbank_attn: strides must be multiples of 8 elements");
  if (!aligned16(q) || !aligned16(o)) return fail(PL_EUNSUPPORTED, "pl_refbank_attn: q and o must be 16-byte aligned");
  int64_t total = 0;
  std::memset(&a, 0, sizeof(a));
  for (int i = 0; i < nseg; ++i) {
    const pl_kv_segment& s = segs[i];
    if (!s.k || !s.v) return fail(PL_EINVAL, "pl_refbank_attn: segment %d has a null k or v", i);
    if (s.len < 1) return fail(PL_EINVAL, "pl_refbank_attn: segment %d has len %lld < 1", i, (long long)s.len);
    if (s.ld < width) return fail(PL_EINVAL, "pl_refbank_attn: segment %d ld < H*d", i);
    if (s.frame_stride < 0) return fail(PL_EINVAL, "pl_refbank_attn: segment %d frame_stride < 0", i);
    if (s.ld % 8 || s.frame_stride % 8)
      return fail(PL_EUNSUPPORTED, "pl_refbank_attn: segment %d strides must be multiples of 8 elements", i);
    if (!aligned16(s.k) || !aligned16(s.v))
      return fail(PL_EUNSUPPORTED, "pl_refbank_attn: segment %d pointers must be 16-byte aligned", i);
    total += s.len;
    a.seg[i].k = static_cast<const _Float16*>(s.k);
    a.seg[i].v = static_cast<const _Float16*>(s.v);
    a.seg[i].len = s.len;
    a.seg[i].ld = s.ld;
    a.seg[i].frame_stride = s.frame_stride;
  }
  // o is written while q and every K/V row are still being read
  const View vo{o, o_ld, o_frame_stride, Lq, F, width};
  if (views_may_overlap(vo, View{q, q_ld, q_frame_stride, Lq, F, width}))
    return fail(PL_EINVAL, "pl_refbank_attn: o overlaps q");
  for (int i = 0; i < nseg; ++i) {
    const pl_kv_segment& s = segs[i];
    if (views_may_overlap(vo, View{s.k, s.ld, s.frame_stride, s.len, F, width}) ||
        views_may_overlap(vo, View{s.v, s.ld, s.frame_stride, s.len, F, width}))
      return fail(PL_EINVAL, "pl_refbank_attn: o overlaps the keys or values of segment %d", i);
  }
  if (total > (int64_t(1) << 24)) return fail(PL_EINVAL, "pl_refbank_attn: total key length exceeds 2^24");
  // workspace: the key-split partials where the launch splits the key axis;
  // NULL with 0 bytes runs the single-pass kernels
  int64_t lens[PL_MAX_SEGMENTS];
  for (int i = 0; i < nseg; ++i) lens[i] = segs[i].len;
  const size_t need = pl::refbank_attn_workspace_bytes(F, Lq, H, d, lens, nseg);
  a.workspace = nullptr;
  if (noalloc) {
    if (need > kScratchBytes)
      return fail(PL_EINVAL, "%s: the key split of these sizes needs %zu bytes of scratch; the library holds %zu", fn,
                  need, kScratchBytes);
    if (need > 0) {
      if (pl_status st = scratch_for_current_device(fn, &a.workspace)) return st;
    }
  } else if (workspace || workspace_bytes) {
    if (!workspace) return fail(PL_EINVAL, "pl_refbank_attn: workspace_bytes is %zu but workspace is NULL", workspace_bytes);
    if (workspace_bytes < need)
      return fail(PL_EINVAL, "pl_refbank_attn: workspace of %zu bytes is too small (%zu needed)", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PL_EUNSUPPORTED, "pl_refbank_attn: workspace must be 16-byte aligned");
    if (need > 0) a.workspace = workspace;
  }
  a.q = static_cast<const _Float16*>(q);
  a.o = static_cast<_Float16*>(o);
  a.q_ld = q_ld;
  a.q_frame_stride = q_frame_stride;
  a.o_ld = o_ld;
  a.o_frame_stride = o_frame_stride;
  a.F = F;
  a.Lq = Lq;
  a.H = H;
  a.d = d;
  a.nseg = nseg;
  a.scale = scale;
  return PL_OK;
}

pl_status refbank_attn_impl(const char* fn, const void* q, int64_t q_ld, int64_t q_frame_stride, void* o,
                            int64_t o_ld, int64_t o_frame_stride, int32_t F, int32_t Lq, int32_t H, int32_t d,
                            const pl_kv_segment* segs, int32_t nseg, float scale, void* workspace,
                            size_t workspace_bytes, bool noalloc, void* stream) {
  pl::AttnLaunch a;
  if (pl_status st = validate_attn(fn, q, q_ld, q_frame_stride, o, o_ld, o_frame_stride, F, Lq, H, d, segs, nseg,
                                   scale, workspace, workspace_bytes, noalloc, &a))
    return st;
  return device_status(pl::launch_refbank_attn(a, static_cast<hipStream_t>(stream)), "pl_refbank_attn launch");
}

}  // namespace

extern "C" {

pl_status pl_refbank_attn(const void* q, int64_t q_ld, int64_t q_frame_stride, void* o, int64_t o_ld,
                          int64_t o_frame_stride, int32_t F, int32_t Lq, int32_t H, int32_t d,
                          const pl_kv_segment* segs, int32_t nseg, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return refbank_attn_impl("pl_refbank_attn", q, q_ld, q_frame_stride, o, o_ld, o_frame_stride, F, Lq, H, d, segs,
                           nseg, scale, workspace, workspace_bytes, false, stream);
}

pl_status pl_refbank_attn_chunked(const void* q, int64_t q_ld, int64_t q_frame_stride, void* o, int64_t o_ld,
                                  int64_t o_frame_stride, int32_t F, int32_t Lq, int32_t H, int32_t d,
                                  const pl_kv_segment* segs, int32_t nseg, int32_t causal_seg, int32_t chunk_len,
                                  int32_t max_history, float scale, void* stream) {
  const char* fn = "pl_refbank_attn_chunked";
  if (!segs) return fail(PL_EINVAL, "%s: segs must be non-null", fn);
  if (nseg < 1 || nseg > PL_MAX_SEGMENTS)
    return fail(PL_EINVAL, "%s: nseg must be in [1, %d] (got %d)", fn, PL_MAX_SEGMENTS, nseg);
  if (causal_seg < 0 || causal_seg >= nseg)
    return fail(PL_EINVAL, "%s: causal_seg must be in [0, nseg) (got %d)", fn, causal_seg);
  if (Lq < 1 || chunk_len < 1) return fail(PL_EINVAL, "%s: Lq and chunk_len must be >= 1 (got %d, %d)", fn, Lq, chunk_len);
  if (segs[causal_seg].len != Lq)
    return fail(PL_EINVAL, "%s: the causal segment must hold the Lq = %d rows of the queries' sequence (got %lld)", fn,
                Lq, (long long)segs[causal_seg].len);
  const int nchunks = (Lq + chunk_len - 1) / chunk_len;
  if (nchunks > 65536) return fail(PL_EINVAL, "%s: more than 65536 chunks (one launch each)", fn);
  // the whole call first (every view at its full extent), then each chunk's
  // launch: all checks run before anything is launched
  pl::AttnLaunch whole;
  if (pl_status st = validate_attn(fn, q, q_ld, q_frame_stride, o, o_ld, o_frame_stride, F, Lq, H, d, segs, nseg,
                                   scale, nullptr, 0, false, &whole))
    return st;
  std::vector<pl::AttnLaunch> launches((size_t)nchunks);
  for (int c = 0; c < nchunks; ++c) {
    const int64_t r0 = (int64_t)c * chunk_len;
    const int rows = (int)std::min<int64_t>(chunk_len, Lq - r0);
    const int64_t lo = max_history < 0 ? 0 : std::max<int64_t>(0, c - (int64_t)max_history);
    const int64_t k0 = lo * chunk_len, k1 = std::min<int64_t>(Lq, r0 + chunk_len);
    pl_kv_segment cs[PL_MAX_SEGMENTS];
    for (int i = 0; i < nseg; ++i) cs[i] = segs[i];
    pl_kv_segment& sc = cs[causal_seg];
    sc.k = static_cast<const char*>(sc.k) + k0 * sc.ld * 2;
    sc.v = static_cast<const char*>(sc.v) + k0 * sc.ld * 2;
    sc.len = k1 - k0;
    const void* qc = static_cast<const char*>(q) + r0 * q_ld * 2;
    void* oc = static_cast<char*>(o) + r0 * o_ld * 2;
    if (pl_status st = validate_attn(fn, qc, q_ld, q_frame_stride, oc, o_ld, o_frame_stride, F, rows, H, d, cs, nseg,
                                     scale, nullptr, 0, false, &launches[(size_t)c])) {
      char msg[512];
      std::snprintf(msg, sizeof(msg), "%s", g_last_error);
      return fail(st, "%s (chunk %d)", msg, c);
    }
  }
  for (int c = 0; c < nchunks; ++c) {
    const hipError_t e = pl::launch_refbank_attn(launches[(size_t)c], static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PL_EDEVICE, "%s: launch of chunk %d: %s", fn, c, hipGetErrorString(e));
  }
  return ok();
}

pl_status pl_debug_bounds(uint64_t* mask, int32_t reset) {
  if (!mask) return fail(PL_EINVAL, "pl_debug_bounds: mask must be non-null");
  unsigned long long m = 0;
  const hipError_t e = pl::debug_bounds_mask(&m, reset != 0);
  *mask = m;
  if (e == hipErrorNotSupported)
    return fail(PL_EUNSUPPORTED, "pl_debug_bounds: this library was built without PL_DEBUG_BOUNDS");
  return device_status(e, "pl_debug_bounds");
}

pl_status pl_refbank_attn_noalloc(const void* q, int64_t q_ld, int64_t q_frame_stride, void* o, int64_t o_ld,
                                  int64_t o_frame_stride, int32_t F, int32_t Lq, int32_t H, int32_t d,
                                  const pl_kv_segment* segs, int32_t nseg, float scale, void* stream) {
  return refbank_attn_impl("pl_refbank_attn_noalloc", q, q_ld, q_frame_stride, o, o_ld, o_frame_stride, F, Lq, H, d,
                           segs, nseg, scale, nullptr, 0, true, stream);
}

// ---------------------------------------------------------------------------
pl_status pl_pyramid_ddim_step(const float* x_t, const float* eps, float* x_prev, float* x0_out, int32_t W,
                               int64_t elems_per_window, const int32_t* t_host, int32_t step_len,
                               const double* alphas_cumprod_host, int32_t T, double final_alpha_cumprod,
                               int32_t emit_window, void* stream) {
  return ddim_step_impl(x_t, eps, x_prev, x0_out, W, elems_per_window, t_host, step_len, alphas_cumprod_host, T,
                        final_alpha_cumprod, emit_window, 0, 0, 0, stream);
}

pl_status pl_pyramid_ddim_step_roll(const float* x_t, const float* eps, float* x_prev, float* x0_out, int32_t W,
                                    int64_t elems_per_window, const int32_t* t_host, int32_t step_len,
                                    const double* alphas_cumprod_host, int32_t T, double final_alpha_cumprod,
                                    int32_t emit_window, uint64_t seed, uint64_t new_window_id, void* stream) {
  return ddim_step_impl(x_t, eps, x_prev, x0_out, W, elems_per_window, t_host, step_len, alphas_cumprod_host, T,
                        final_alpha_cumprod, emit_window, 1, seed, new_window_id, stream);
}

pl_status pl_sd_alphas_cumprod(double* out, int32_t T) {
  if (!out) return fail(PL_EINVAL, "pl_sd_alphas_cumprod: out must be non-null");
  if (T != 1000) return fail(PL_EINVAL, "pl_sd_alphas_cumprod: the built-in schedule has T = 1000 (got %d)", T);
  std::memcpy(out, sd_schedule().ab, sizeof(double) * 1000);
  return ok();
}

pl_status pl_pyramid_ddim_step_device(const float* x_t, const float* eps, float* x_prev, float* x0_out, int32_t W,
                                      int64_t elems_per_window, pl_pile* pile, const double* alphas_cumprod, int32_t T,
                                      double final_alpha_cumprod, uint64_t seed, void* stream) {
  const char* fn = "pl_pyramid_ddim_step_device";
  if (!x_t || !eps || !x_prev || !x0_out) return fail(PL_EINVAL, "%s: x_t, eps, x_prev and x0_out must be non-null", fn);
  if (!pile || !alphas_cumprod) return fail(PL_EINVAL, "%s: pile and alphas_cumprod must be non-null", fn);
  if (W < 2 || W > PL_MAX_WINDOWS) return fail(PL_EINVAL, "%s: W must be in [2, %d] (got %d)", fn, PL_MAX_WINDOWS, W);
  if (elems_per_window < 1 || elems_per_window > (int64_t(1) << 40))
    return fail(PL_EINVAL, "%s: elems_per_window must be in [1, 2^40]", fn);
  if (T < 1) return fail(PL_EINVAL, "%s: T must be >= 1", fn);
  if (!(final_alpha_cumprod < 0.0 || (final_alpha_cumprod > 0.0 && final_alpha_cumprod <= 1.0)))
    return fail(PL_EINVAL, "%s: final_alpha_cumprod must be negative (alpha_bar[0]) or in (0, 1]", fn);
  if (elems_per_window % 4 || !aligned16(x_t) || !aligned16(eps) || !aligned16(x_prev) || !aligned16(x0_out))
    return fail(PL_EUNSUPPORTED, "%s: buffers must be 16-byte aligned and elems_per_window a multiple of 4", fn);
  if ((reinterpret_cast<uintptr_t>(pile) & 7) || (reinterpret_cast<uintptr_t>(alphas_cumprod) & 7))
    return fail(PL_EUNSUPPORTED, "%s: pile and alphas_cumprod must be 8-byte aligned", fn);
  pl::DeviceRoundLaunch a;
  a.x_t = x_t;
  a.eps = eps;
  a.x_prev = x_prev;
  a.x0_out = x0_out;
  a.W = W;
  a.elems_per_window = elems_per_window;
  a.pile = pile;
  a.alphas_cumprod = alphas_cumprod;
  a.T = T;
  a.final_alpha_cumprod = final_alpha_cumprod;
  a.seed = seed;
  return device_status(pl::launch_pyramid_round_device(a, static_cast<hipStream_t>(stream)), "pl_pyramid_ddim_step_device launch");
}

// ---------------------------------------------------------------------------
pl_status pl_window_noise(float* out, int64_t n, uint64_t seed, uint64_t window_id, void* stream) {
  if (!out) return fail(PL_EINVAL, "pl_window_noise: out must be non-null");
  if (n < 1 || n > (int64_t(1) << 40)) return fail(PL_EINVAL, "pl_window_noise: n must be in [1, 2^40]");
  pl::NoiseLaunch a;
  std::memset(&a, 0, sizeof(a));
  a.ref = nullptr;
  a.out = out;
  a.n = n;
  a.out_stride = n;
  a.nw = 1;
  a.seed = seed;
  a.id0 = window_id;
  a.ca[0] = 0.f;
  a.cb[0] = 1.f;
  return device_status(pl::launch_noise_affine(a, static_cast<hipStream_t>(stream)), "pl_window_noise launch");
}

pl_status pl_pile_prefill(const float* ref, float* pile, int32_t n_windows, int64_t elems_per_window,
                          int32_t step_len, const double* alphas_cumprod_host, int32_t T, uint64_t seed,
                          void* stream) {
  if (!ref || !pile) return fail(PL_EINVAL, "pl_pile_prefill: ref and pile must be non-null");
  if (n_windows < 1 || n_windows > PL_MAX_WINDOWS)
    return fail(PL_EINVAL, "pl_pile_prefill: n_windows must be in [1, %d] (got %d)", PL_MAX_WINDOWS, n_windows);
  if (elems_per_window < 1 || elems_per_window > (int64_t(1) << 40))
    return fail(PL_EINVAL, "pl_pile_prefill: elems_per_window must be in [1, 2^40]");
  if (step_len < 1) return fail(PL_EINVAL, "pl_pile_prefill: step_len must be >= 1");
  const double* ab = nullptr;
  if (pl_status st = resolve_schedule("pl_pile_prefill", alphas_cumprod_host, T, &ab)) return st;
  if ((int64_t)(n_windows - 1) * step_len >= T)
    return fail(PL_EINVAL, "pl_pile_prefill: window %d would sit at t = %lld >= T", n_windows - 1,
                (long long)(n_windows - 1) * step_len);
  const int64_t bytes = elems_per_window * (int64_t)sizeof(float);
  const char* r0 = reinterpret_cast<const char*>(ref);
  const char* p0 = reinterpret_cast<const char*>(pile);
  if (r0 < p0 + bytes * n_windows && p0 < r0 + bytes)
    return fail(PL_EINVAL, "pl_pile_prefill: ref must not overlap the pile");
  pl::NoiseLaunch a;
  std::memset(&a, 0, sizeof(a));
  a.ref = ref;
  a.out = pile;
  a.n = elems_per_window;
  a.out_stride = elems_per_window;
  a.nw = n_windows;
  a.seed = seed;
  a.id0 = 0;
  for (int w = 0; w < n_windows; ++w) {
    const double at = ab[w * step_len];
    a.ca[w] = (float)std::sqrt(at);
    a.cb[w] = (float)std::sqrt(1.0 - at);
  }
  return device_status(pl::launch_noise_affine(a, static_cast<hipStream_t>(stream)), "pl_pile_prefill launch");
}

pl_status pl_linear(const void* x, int64_t x_ld, const void* w, int64_t w_ld, const float* bias, void* y,
                    int64_t y_ld, int64_t M, int32_t N, int32_t K, void* stream) {
  if (!x || !w || !y) return fail(PL_EINVAL, "pl_linear: x, w and y must be non-null");
  if (M < 1 || N < 1 || K < 1) return fail(PL_EINVAL, "pl_linear: M, N and K must be >= 1");
  if (M > (int64_t(1) << 31)) return fail(PL_EINVAL, "pl_linear: M must be <= 2^31");
  if (N % 64) return fail(PL_EUNSUPPORTED, "pl_linear: N must be a multiple of 64 (got %d)", N);
  if (K % 16) return fail(PL_EUNSUPPORTED, "pl_linear: K must be a multiple of 16 (got %d)", K);
  if (x_ld < K || w_ld < K || y_ld < N) return fail(PL_EINVAL, "pl_linear: x_ld, w_ld >= K and y_ld >= N required");
  if (x_ld % 8 || w_ld % 8 || y_ld % 4)
    return fail(PL_EUNSUPPORTED, "pl_linear: x_ld and w_ld must be multiples of 8 elements, y_ld of 4");
  if (!aligned16(x) || !aligned16(w) || (reinterpret_cast<uintptr_t>(y) & 7))
    return fail(PL_EUNSUPPORTED, "pl_linear: x and w must be 16-byte aligned, y 8-byte aligned");
  if (bias && !aligned16(bias)) return fail(PL_EUNSUPPORTED, "pl_linear: bias must be 16-byte aligned");
  // y must not overlap x or w (the rows of y are written while others are read)
  const char* y0 = static_cast<const char*>(y);
  const char* y1 = y0 + ((M - 1) * y_ld + N) * 2;
  const char* x0 = static_cast<const char*>(x);
  const char* x1 = x0 + ((M - 1) * x_ld + K) * 2;
  const char* w0 = static_cast<const char*>(w);
  const char* w1 = w0 + ((int64_t)(N - 1) * w_ld + K) * 2;
  if ((y0 < x1 && x0 < y1) || (y0 < w1 && w0 < y1)) return fail(PL_EINVAL, "pl_linear: y overlaps x or w");
  pl::LinearLaunch a;
  a.x = static_cast<const _Float16*>(x);
  a.w = static_cast<const _Float16*>(w);
  a.bias = bias;
  a.y = static_cast<_Float16*>(y);
  a.x_ld = x_ld;
  a.w_ld = w_ld;
  a.y_ld = y_ld;
  a.M = M;
  a.N = N;
  a.K = K;
  return device_status(pl::launch_linear(a, static_cast<hipStream_t>(stream)), "pl_linear launch");
}

pl_status pl_lerp_points(const float* a, const float* b, int64_t D, int32_t n, float* out, void* stream) {
  if (!a || !b || !out) return fail(PL_EINVAL, "pl_lerp_points: pointers must be non-null");
  if (D < 1 || D > (int64_t(1) << 40)) return fail(PL_EINVAL, "pl_lerp_points: D must be in [1, 2^40]");
  if (n < 1 || n > 65535) return fail(PL_EINVAL, "pl_lerp_points: n must be in [1, 65535] (got %d)", n);
  const int64_t bytes = D * (int64_t)sizeof(float);
  const char* o0 = reinterpret_cast<const char*>(out);
  for (const float* src : {a, b}) {
    const char* s0 = reinterpret_cast<const char*>(src);
    if (s0 < o0 + bytes * n && o0 < s0 + bytes) return fail(PL_EINVAL, "pl_lerp_points: out must not overlap a or b");
  }
  return device_status(pl::launch_lerp_points(a, b, D, n, out, static_cast<hipStream_t>(stream)),
                       "pl_lerp_points launch");
}

// ---------------------------------------------------------------------------
pl_status pl_motion_bank_min_l2(const float* query, int32_t nq, const float* bank, int32_t n, int32_t D,
                                float threshold, float* min_dist, int32_t* argmin, uint8_t* exceeds,
                                void* stream) {
  if (!query || !bank || !min_dist || !argmin || !exceeds)
    return fail(PL_EINVAL, "pl_motion_bank_min_l2: pointers must be non-null");
  if (nq < 1) return fail(PL_EINVAL, "pl_motion_bank_min_l2: nq must be >= 1 (got %d)", nq);
  if (n < 1 || n > PL_MAX_MOTION_BANK)
    return fail(PL_EINVAL, "pl_motion_bank_min_l2: n must be in [1, %d] (got %d)", PL_MAX_MOTION_BANK, n);
  if (D < 1 || D > 65536) return fail(PL_EINVAL, "pl_motion_bank_min_l2: D must be in [1, 65536] (got %d)", D);
  if (std::isnan(threshold)) return fail(PL_EINVAL, "pl_motion_bank_min_l2: threshold is NaN");
  pl::MotionLaunch a{query, bank, nq, n, D, threshold, min_dist, argmin, exceeds};
  return device_status(pl::launch_motion_min_l2(a, static_cast<hipStream_t>(stream)), "pl_motion_bank_min_l2 launch");
}

// ---------------------------------------------------------------------------
pl_status pl_pile_init(pl_pile* p, int32_t W, int32_t step_len, int32_t t_top, int32_t prefill) {
  if (!p) return fail(PL_EINVAL, "pl_pile_init: p must be non-null");
  if (W < 2 || W > PL_MAX_WINDOWS) return fail(PL_EINVAL, "pl_pile_init: W must be in [2, %d]", PL_MAX_WINDOWS);
  if (step_len < 1) return fail(PL_EINVAL, "pl_pile_init: step_len must be >= 1");
  if (t_top != (W - 1) * step_len)
    return fail(PL_EINVAL, "pl_pile_init: t_top must equal (W-1)*step_len so a window leaves after W evaluations");
  std::memset(p, 0, sizeof(*p));
  p->W = W;
  p->step_len = step_len;
  p->t_top = t_top;
  for (int s = 0; s < PL_MAX_WINDOWS; ++s) {
    p->id[s] = -1;
    p->t[s] = t_top;
  }
  if (prefill) {
    // staircase: slot s holds the s-th oldest window at t = s * step_len
    for (int s = 0; s < W - 1; ++s) {
      p->id[s] = p->next_id++;
      p->t[s] = s * step_len;
    }
    p->count = W - 1;
  }
  return ok();
}

pl_status pl_pile_begin_round(pl_pile* p, int32_t* new_slot, int32_t* t_slot, int32_t* emit_slot) {
  if (!p || !new_slot || !t_slot || !emit_slot) return fail(PL_EINVAL, "pl_pile_begin_round: null argument");
  if (p->in_round) return fail(PL_EINVAL, "pl_pile_begin_round: a round is already open");
  if (p->count >= p->W) return fail(PL_EINVAL, "pl_pile_begin_round: pile is full");
  const int slot = (p->head + p->count) % p->W;
  p->id[slot] = p->next_id++;
  p->t[slot] = p->t_top;
  p->count += 1;
  p->in_round = 1;
  *new_slot = slot;
  *emit_slot = -1;
  for (int s = 0; s < p->W; ++s) t_slot[s] = p->id[s] >= 0 ? p->t[s] : p->t_top;
  if (p->t[p->head] == 0 && p->id[p->head] >= 0) *emit_slot = p->head;
  return ok();
}

pl_status pl_pile_end_round(pl_pile* p, int64_t* emitted_id) {
  if (!p || !emitted_id) return fail(PL_EINVAL, "pl_pile_end_round: null argument");
  if (!p->in_round) return fail(PL_EINVAL, "pl_pile_end_round: no round is open");
  *emitted_id = -1;
  if (p->count > 0 && p->t[p->head] == 0) {
    *emitted_id = p->id[p->head];
    p->id[p->head] = -1;
    p->t[p->head] = p->t_top;
    p->head = (p->head + 1) % p->W;
    p->count -= 1;
  }
  for (int k = 0; k < p->count; ++k) p->t[(p->head + k) % p->W] -= p->step_len;
  p->in_round = 0;
  return ok();
}

}  // extern "C"
