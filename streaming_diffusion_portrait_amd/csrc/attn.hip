// Reference-bank spatial self-attention: flash-style fp16 MFMA kernel for gfx950.
//
// PersonaLive write-up, section 三条条件通路: the denoiser concatenates the
// reference bank's features of a layer with its own keys/values and runs
// spatial self-attention; section 抗身份漂移的补丁: anchors add more bank
// entries.  Here the concatenation is virtual: the kernel walks a table of
// key/value segments (the frame's own tokens, then the shared bank entries)
// and never materialises the concatenated keys in HBM.
//
// Work decomposition
//   * one workgroup = 4 wavefronts = one (head, frame, query tile); each wave
//     owns NT tiles of 16 query rows, so a workgroup covers 64*NT rows;
//   * K and V tiles of BN keys are staged in LDS, double buffered: the loads
//     of tile i+1 are issued before tile i is consumed and written to the
//     other buffer afterwards, one barrier per tile;
//   * workgroup ids are remapped so that each of the 8 XCDs (ids are dealt
//     round-robin to them) works on a contiguous range of (head, frame, tile),
//     i.e. mostly on one head, whose shared bank keys then stay in that XCD's L2.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_f16; lane l = 16*g + c):
//   S^T = K Q^T   A = K rows (16 keys x 32 d) from LDS, B = Q^T held in
//                 registers for the whole kernel; lane (g, c) receives the
//                 scores of query c for keys 4g..4g+3 of each 16-key block.
//   O^T = V^T P^T A = V^T (16 d x 32 keys) from LDS, B = P^T built in
//                 registers from two 16-key blocks of S^T, so probabilities
//                 never leave the lane that computed them.  V is therefore
//                 stored transposed in LDS, with keys permuted inside each
//                 32-key group to match the order in which P^T holds them.
//   Every per-query quantity (running max, rescale factor, row sum) lives in
//   the lanes of its query column, so no cross-lane traffic is needed except
//   two xor-shuffles per tile for the row maximum.
//
// Softmax (fp32): scores are compared in log2 units, p = exp2(s*scale*log2e - m).
// The running max m is raised only when a tile's max exceeds it by more than
// 8 (then p <= 2^8 always, safe in fp16), so the accumulator rescale is rare.
// The row sum comes out of the PV product itself: V^T carries a row of ones at
// row d (inside the zero padding when d is not a multiple of 16), so
// sum_j p_j is accumulated by the matrix core from the same fp16 values that
// weight V.  For d = 160 the sum is accumulated on the vector unit instead.
#include "pl_internal.h"

namespace pl {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a tile max may exceed the running max by

template <int D_, int NT_, int BN_>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int NT = NT_;                  // 16-row query tiles per wave
  static constexpr int BN = BN_;                  // keys per LDS tile
  static constexpr int KSTEPS = (D + 31) / 32;    // 32-wide contraction steps for S^T
  static constexpr int DK = KSTEPS * 32;          // zero-padded head dim in the K tile
  static constexpr bool ONES = (D != 160);        // row sum through the matrix core
  static constexpr int NDV = ONES ? D / 16 + 1 : D / 16;  // 16-row tiles of O^T
  static constexpr int KROW = DK + 8;             // K tile row stride (halves); +16 B avoids bank conflicts
  static constexpr int VROW = BN + 8;             // V^T tile row stride (halves)
  static constexpr int K_ELEMS = BN * KROW;
  static constexpr int V_ELEMS = NDV * 16 * VROW;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int CPR = D / 8;               // 16-byte chunks per key row
  static constexpr int CHUNKS = BN * CPR;         // chunks per tile (K or V)
  static constexpr int CPT = (CHUNKS + kThreads - 1) / kThreads;  // chunks per thread
  static constexpr int QROWS = 64 * NT;           // query rows per workgroup
  static_assert(D % 16 == 0 || D % 16 == 8, "head dim must be a multiple of 8");
  static_assert(BN % 32 == 0, "BN must be a multiple of 32");
};

struct KParams {
  const _Float16* q;
  _Float16* o;
  int64_t q_ld, q_fs, o_ld, o_fs;
  int F, Lq, H, nqt, nseg;
  float c2;  // scale * log2(e)
  AttnSegment seg[PL_MAX_SEGMENTS];
};

// Position of key kk (0..31) of a 32-key group inside the permuted V^T row:
// keys 4g..4g+3 -> 8g..8g+3 and keys 16+4g..16+4g+3 -> 8g+4..8g+7.
__device__ __forceinline__ int vt_pos(int key) {
  const int grp = key & ~31, kk = key & 31;
  const int hi = kk >> 4, lo = kk & 15;
  return grp + ((lo >> 2) << 3) + (hi << 2) + (lo & 3);
}

template <class C>
__device__ __forceinline__ void load_tile(const KParams& p, int s, int64_t off, int f, int h, int tid,
                                          uint4 (&kr)[C::CPT], uint4 (&vr)[C::CPT]) {
  const AttnSegment& sg = p.seg[s];
  const int64_t base = (int64_t)f * sg.frame_stride + (int64_t)h * C::D;
  const int64_t len = sg.len;
#pragma unroll
  for (int u = 0; u < C::CPT; ++u) {
    const int idx = tid + u * kThreads;
    const int row = idx / C::CPR, ch = idx - row * C::CPR;
    const int64_t key = off + row;
    uint4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
    if (idx < C::CHUNKS && key < len) {
      const int64_t e = base + key * sg.ld + ch * 8;
      zk = *reinterpret_cast<const uint4*>(sg.k + e);
      zv = *reinterpret_cast<const uint4*>(sg.v + e);
    }
    kr[u] = zk;
    vr[u] = zv;
  }
}

template <class C>
__device__ __forceinline__ void store_tile(_Float16* buf, int tid, const uint4 (&kr)[C::CPT],
                                           const uint4 (&vr)[C::CPT]) {
  _Float16* ks = buf;
  _Float16* vt = buf + C::K_ELEMS;
#pragma unroll
  for (int u = 0; u < C::CPT; ++u) {
    const int idx = tid + u * kThreads;
    if (idx < C::CHUNKS) {
      const int row = idx / C::CPR, ch = idx - row * C::CPR;
      *reinterpret_cast<uint4*>(ks + row * C::KROW + ch * 8) = kr[u];
      const int pos = vt_pos(row);
      const _Float16* hv = reinterpret_cast<const _Float16*>(&vr[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(ch * 8 + e) * C::VROW + pos] = hv[e];
    }
  }
}

template <class C>
__global__ void __launch_bounds__(kThreads, 2) refbank_attn_kernel(KParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * C::BUF_ELEMS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;

  // XCD-aware remap of the workgroup id onto (head, frame, query tile).
  const int total = p.nqt * p.F * p.H;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int h = lid / (p.F * p.nqt);
  const int rem = lid - h * (p.F * p.nqt);
  const int f = rem / p.nqt;
  const int qt = rem - f * p.nqt;
  const int qrow0 = qt * C::QROWS + wave * 16 * C::NT;

  // Constant padding of both buffers: K columns [D, DK) = 0, V^T rows >= D = 0
  // except the ones row at D.  Tile stores never touch these.
  for (int b = 0; b < 2; ++b) {
    _Float16* ks = smem + b * C::BUF_ELEMS;
    _Float16* vt = ks + C::K_ELEMS;
    if (C::DK > C::D)
      for (int i = tid; i < C::BN * (C::DK - C::D); i += kThreads) {
        const int r = i / (C::DK - C::D), col = C::D + i % (C::DK - C::D);
        ks[r * C::KROW + col] = (_Float16)0.0f;
      }
    for (int i = tid; i < (C::NDV * 16 - C::D) * C::BN; i += kThreads) {
      const int r = C::D + i / C::BN, col = i % C::BN;
      vt[r * C::VROW + col] = (_Float16)((C::ONES && r == C::D) ? 1.0f : 0.0f);
    }
  }

  // Q^T operands, resident for the whole kernel (zero beyond d and beyond Lq).
  h8 qf[C::NT][C::KSTEPS];
  {
    const _Float16* qb = p.q + (int64_t)f * p.q_fs + (int64_t)h * C::D;
#pragma unroll
    for (int n = 0; n < C::NT; ++n) {
      const int row = qrow0 + 16 * n + c;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const int col = 32 * s + 8 * g;
        h8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (row < p.Lq && col < C::D) v = *reinterpret_cast<const h8*>(qb + (int64_t)row * p.q_ld + col);
        qf[n][s] = v;
      }
    }
  }

  f4 oacc[C::NT][C::NDV];
  float mrun[C::NT], lsum[C::NT];
#pragma unroll
  for (int n = 0; n < C::NT; ++n) {
    mrun[n] = -1e30f;
    lsum[n] = 0.f;
#pragma unroll
    for (int t = 0; t < C::NDV; ++t) oacc[n][t] = (f4){0.f, 0.f, 0.f, 0.f};
  }

  // Tile cursor over the segment table.
  int s = 0;
  int64_t off = 0;
  uint4 kr[C::CPT], vr[C::CPT];
  load_tile<C>(p, 0, 0, f, h, tid, kr, vr);
  store_tile<C>(smem, tid, kr, vr);

  for (int buf = 0;; buf ^= 1) {
    // next tile
    int s_n = s;
    int64_t off_n = off + C::BN;
    if (off_n >= p.seg[s].len) { s_n = s + 1; off_n = 0; }
    const bool has_next = s_n < p.nseg;
    const int valid = (int)min((int64_t)C::BN, p.seg[s].len - off);

    __syncthreads();
    if (has_next) load_tile<C>(p, s_n, off_n, f, h, tid, kr, vr);

    const _Float16* ks = smem + buf * C::BUF_ELEMS;
    const _Float16* vt = ks + C::K_ELEMS;

    // ---- S^T = K Q^T for BN keys ----
    f4 sacc[C::NT][C::BN / 16];
#pragma unroll
    for (int b = 0; b < C::BN / 16; ++b) {
      const _Float16* krow = ks + (16 * b + c) * C::KROW + 8 * g;
      h8 ka[C::KSTEPS];
#pragma unroll
      for (int st = 0; st < C::KSTEPS; ++st) ka[st] = *reinterpret_cast<const h8*>(krow + 32 * st);
#pragma unroll
      for (int n = 0; n < C::NT; ++n) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[st], qf[n][st], acc, 0, 0, 0);
        sacc[n][b] = acc;
      }
    }
    if (valid < C::BN) {
#pragma unroll
      for (int b = 0; b < C::BN / 16; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * b + 4 * g + r >= valid)
#pragma unroll
            for (int n = 0; n < C::NT; ++n) sacc[n][b][r] = -INFINITY;
    }

    // ---- tile row max (raw units), lazy rescale ----
    float mnew[C::NT];
    bool need = false;
#pragma unroll
    for (int n = 0; n < C::NT; ++n) {
      float mx = sacc[n][0][0];
#pragma unroll
      for (int b = 0; b < C::BN / 16; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[n][b][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mt = mx * p.c2;
      mnew[n] = fmaxf(mrun[n], mt);
      need |= (mt > mrun[n] + kRescaleSlack);
    }
    if (__any(need)) {
#pragma unroll
      for (int n = 0; n < C::NT; ++n) {
        const float alpha = __builtin_amdgcn_exp2f(mrun[n] - mnew[n]);
        mrun[n] = mnew[n];
        lsum[n] *= alpha;
#pragma unroll
        for (int t = 0; t < C::NDV; ++t) oacc[n][t] *= alpha;
      }
    }

    // ---- P^T and O^T += V^T P^T ----
#pragma unroll
    for (int j = 0; j < C::BN / 32; ++j) {
      h8 pb[C::NT];
#pragma unroll
      for (int n = 0; n < C::NT; ++n) {
        const float mneg = -mrun[n];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[n][2 * j][e], p.c2, mneg));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[n][2 * j + 1][e], p.c2, mneg));
          pb[n][e] = (_Float16)p0;
          pb[n][4 + e] = (_Float16)p1;
          if (!C::ONES) lsum[n] += p0 + p1;
        }
      }
#pragma unroll
      for (int t = 0; t < C::NDV; ++t) {
        const h8 va = *reinterpret_cast<const h8*>(vt + (16 * t + c) * C::VROW + 32 * j + 8 * g);
#pragma unroll
        for (int n = 0; n < C::NT; ++n) oacc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[n], oacc[n][t], 0, 0, 0);
      }
    }

    if (!has_next) break;
    store_tile<C>(smem + (buf ^ 1) * C::BUF_ELEMS, tid, kr, vr);
    s = s_n;
    off = off_n;
  }

  // ---- normalise and write O (fp16, round to nearest even) ----
  _Float16* ob = p.o + (int64_t)f * p.o_fs + (int64_t)h * C::D;
#pragma unroll
  for (int n = 0; n < C::NT; ++n) {
    float l;
    if (C::ONES) {
      constexpr int tl = C::D / 16, lr = C::D % 16;
      l = __shfl(oacc[n][tl][lr & 3], 16 * (lr >> 2) + c, 64);
    } else {
      l = lsum[n];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
    }
    const float inv = 1.0f / l;
    const int row = qrow0 + 16 * n + c;
    if (row < p.Lq) {
#pragma unroll
      for (int t = 0; t < C::NDV; ++t) {
        const int col = 16 * t + 4 * g;
        if (col < C::D) {
          h4 out;
#pragma unroll
          for (int r = 0; r < 4; ++r) out[r] = (_Float16)(oacc[n][t][r] * inv);
          *reinterpret_cast<h4*>(ob + (int64_t)row * p.o_ld + col) = out;
        }
      }
    }
  }
}

template <int D, int NT, int BN>
hipError_t launch_cfg(const KParams& kp, hipStream_t stream) {
  using C = Cfg<D, NT, BN>;
  KParams p = kp;
  p.nqt = (p.Lq + C::QROWS - 1) / C::QROWS;
  const int64_t blocks = (int64_t)p.nqt * p.F * p.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(refbank_attn_kernel<C>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_refbank_attn(const AttnLaunch& a, hipStream_t stream) {
  KParams p;
  p.q = a.q;
  p.o = a.o;
  p.q_ld = a.q_ld;
  p.q_fs = a.q_frame_stride;
  p.o_ld = a.o_ld;
  p.o_fs = a.o_frame_stride;
  p.F = a.F;
  p.Lq = a.Lq;
  p.H = a.H;
  p.nqt = 0;
  p.nseg = a.nseg;
  p.c2 = a.scale * kLog2e;
  for (int i = 0; i < PL_MAX_SEGMENTS; ++i) p.seg[i] = a.seg[i];
  const bool big = a.Lq >= 1024;
  switch (a.d) {
    case 32: return big ? launch_cfg<32, 4, 64>(p, stream) : launch_cfg<32, 1, 64>(p, stream);
    case 40: return big ? launch_cfg<40, 4, 64>(p, stream) : launch_cfg<40, 1, 64>(p, stream);
    case 80: return big ? launch_cfg<80, 2, 64>(p, stream) : launch_cfg<80, 1, 64>(p, stream);
    case 160: return big ? launch_cfg<160, 2, 32>(p, stream) : launch_cfg<160, 1, 32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pl
