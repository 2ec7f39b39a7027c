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
//     owns NQB blocks of 32 query rows;
//   * K and V tiles of BN keys are copied HBM -> LDS by the direct-to-LDS
//     loads (global_load_lds_dwordx4), row-major exactly as they sit in HBM
//     (2*d bytes per key), double buffered: the copy of tile i+1 is in flight
//     while tile i is consumed; one barrier per tile;
//   * workgroup ids are remapped so that each of the 8 XCDs (ids are dealt
//     round-robin to them) works on a contiguous range of (head, frame, tile),
//     i.e. mostly on one head, whose shared bank keys then stay in its L2.
//
// Matrix-core mapping
//   S^T = K Q^T   v_mfma_f32_32x32x16_f16: A = 32 keys x 16 d from LDS,
//                 B = Q^T for 32 queries held in registers for the whole
//                 kernel.  Lane l ends up with the scores of query l%32 for
//                 16 of the 32 keys (4 runs of 4 consecutive keys).
//   O^T = V^T P^T v_mfma_f32_16x16x32_f16: B = P^T is assembled from the S^T
//                 registers of two query halves with v_permlane16_swap, so
//                 probabilities never touch LDS; A = V^T is read from the
//                 row-major V tile with ds_read_b64_tr_b16 (transposing read),
//                 two reads per operand.  The order in which the swapped P^T
//                 lists the keys fixes which V rows each transposing read
//                 fetches (vrow() below).
//
// Softmax (fp32, log2 units).  Q is pre-scaled by scale*log2(e) and rounded
// to fp16 once, so the matrix core yields s = scale*log2(e)*q.k directly.
//   * Exact tiles: the row maximum of the tile is taken, and the running
//     offset m is raised when the tile maximum exceeds it by more than 8
//     (then p <= 2^8 always, safe in fp16); the accumulator is rescaled then.
//   * Fast tiles: after the first tile the offset is frozen at that tile's
//     maximum and no per-element maximum is taken at all.  For a head dim
//     that leaves a zero-padded column (d = 40), the padding carries the
//     offset into the matrix core: K gets a column of ones and Q the value -m,
//     so s - m comes out of the MFMA and p = exp2 of the accumulator.
//     A fast tile would only go wrong if a later score exceeded the frozen
//     offset by 16 or more (p beyond the fp16 range): the row sum then turns
//     inf/NaN, which is checked once at the end; the workgroup then recomputes
//     everything with exact tiles.
//   * Row sums come from the same fp16 values that weight V: through the
//     matrix core (a row of ones in the V^T padding, d = 40) or with
//     v_dot2_f32_f16 on the packed probabilities (other head dims).
#include "pl_internal.h"

namespace pl {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));


constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units a tile max may exceed the running offset by
constexpr float kFastMaxOffset = 1024.0f;  // |m| bound for freezing the offset in fp16

// Key rows (within a 32-key block) fetched by the two transposing reads of
// lane group g (lanes 16g..16g+15) for the V^T operand.  They follow from the
// S^T accumulator layout (lane half h holds keys 8i + 4h + j) and the
// permlane16 swaps of key runs i = {0,1} and {2,3}: contraction index
// k = 8g + e maps to key vrow(g) + e for e < 4 and to vrow(g) + 16 + e - 4
// for e >= 4, with vrow(g) = 0, 8, 4, 12 for g = 0..3.
__device__ __forceinline__ int vrow(int g) { return 8 * (g & 1) + 4 * (g >> 1); }

template <int D_, int NQB_, int NKB_, int MINB_>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int MINB = MINB_;          // workgroups per CU the register budget is sized for
  static constexpr int NQB = NQB_;            // 32-query blocks per wave
  static constexpr int NKB = NKB_;            // 32-key blocks per tile
  static constexpr int BN = 32 * NKB;         // keys per tile
  static constexpr int QWG = 32 * NQB * kWaves;  // query rows per workgroup
  static constexpr int KST = (D + 15) / 16;   // 16-wide contraction steps of S^T
  static constexpr int NDT = (D + 15) / 16;   // 16-row tiles of O^T
  static constexpr bool ONES = (D % 16) != 0; // padding column D carries ones / -m
  static constexpr int ROWB = 2 * D;          // bytes per staged key row
  static constexpr int TILEB = BN * ROWB;     // bytes of one K (or V) tile
  static constexpr int CPR = D / 8;           // 16-byte chunks per key row
  static constexpr int LI = BN * CPR / 64;    // wave-wide 16-byte load instructions per tile (K or V)
  static constexpr int NI = (2 * LI + kWaves - 1) / kWaves;  // load instructions per wave per tile
  static constexpr int BUFB = 2 * TILEB;      // K tile + V tile
  static constexpr int LDSB = 2 * BUFB + 128; // two buffers + slack read past the last row
  static_assert(D % 8 == 0, "head dim must be a multiple of 8");
  static_assert(!ONES || D % 16 == 8, "the ones column must start the upper half of the last step");
  static_assert((BN * CPR) % 64 == 0, "a tile must be whole wave-wide load instructions");
};

struct KParams {
  const _Float16* q;
  _Float16* o;
  int64_t q_ld, q_fs, o_ld, o_fs;
  int F, Lq, H, nqt, nseg;
  float c2;  // scale * log2(e)
  AttnSegment seg[PL_MAX_SEGMENTS];
};

__device__ __forceinline__ unsigned pack_h2(float a, float b) {
  h2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Round x up to an fp16-representable value (m must not be exceeded by the
// scores of the tile that defined it).
__device__ __forceinline__ float round_up_half(float x) {
  _Float16 hx = (_Float16)(x + fabsf(x) * 0.0009765625f);
  float r = (float)hx;
  return r < x ? x : r;  // never below x (guard; unreachable for |x| <= 1024)
}

// Issue this wave's share of the direct-to-LDS copies of one K/V tile.
// (M0 is named as clobbered by the asm below; nothing else in this kernel
// keeps a value in it.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <class C>
__device__ __forceinline__ void issue_tile(const KParams& p, char* buf, int s, int64_t off, int f, int h, int wave,
                                           int lane) {
  const AttnSegment& sg = p.seg[s];
  const int64_t valid = sg.len - off;  // >= 1
  const int64_t base = (int64_t)f * sg.frame_stride + off * sg.ld + (int64_t)h * C::D;
  const _Float16* kbase = sg.k + base;
  const _Float16* vbase = sg.v + base;
  const int64_t ld = sg.ld;
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int u = wave + kWaves * j;  // wave-uniform
    if (u < 2 * C::LI) {
      const bool isv = u >= C::LI;
      const int uu = isv ? u - C::LI : u;
      const int c = uu * 64 + lane;
      int row = c / C::CPR;
      const int ch = c - row * C::CPR;
      if (row >= valid) row = (int)valid - 1;  // ragged tail: duplicate a valid row (masked later)
      const _Float16* src = (isv ? vbase : kbase) + (int64_t)row * ld + ch * 8;
      const char* dst = buf + (isv ? C::TILEB : 0) + uu * 1024;
      // Lane i's 16 bytes land at M0 + 16*i.  Written as asm so the compiler
      // does not serialise the LDS reads of the other buffer behind this
      // copy; completion is awaited explicitly (vmcnt) before the barrier
      // that publishes the tile.  The instruction has no register result.
      const unsigned m0 = __builtin_amdgcn_readfirstlane(
          (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)dst);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(m0), "v"(src)
                   : "memory", "m0");
    }
  }
}
#pragma clang diagnostic pop

// One K/V tile for one wave.  FAST: offset frozen (no tile maximum).
// FIRST: the first tile of a pass (sets the offset from its own maximum).
template <class C, bool FAST>
__device__ __forceinline__ void tile_step(const char* kt, const h8 (&qf)[C::NQB][C::KST], f4 (&oacc)[C::NQB][2][C::NDT],
                                          float (&mrun)[C::NQB], float (&lsum)[C::NQB], bool first, int valid,
                                          int lane, int h, int c16, int g, const u4& kones, const u4& vsel_const,
                                          bool vsel_data, int krow_off, const int (&vrow_off)[2]) {
  const char* vt = kt + C::TILEB;

  // ---- S^T = K Q^T for the tile ----
  f16v sacc[C::NQB][C::NKB];
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb) {
    h8 ka[C::KST];
#pragma unroll
    for (int st = 0; st < C::KST; ++st)
      ka[st] = *reinterpret_cast<const h8*>(kt + krow_off + kb * 32 * C::ROWB + 32 * st);
    if (C::ONES) {
      u4 t = __builtin_bit_cast(u4, ka[C::KST - 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = h ? kones[e] : t[e];
      ka[C::KST - 1] = __builtin_bit_cast(h8, t);
    }
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      f16v a = {};
#pragma unroll
      for (int st = 0; st < C::KST; ++st) a = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[st], qf[qb][st], a, 0, 0, 0);
      sacc[qb][kb] = a;
    }
  }

  // ---- ragged tail: keys at or beyond `valid` get no weight ----
  if (valid < C::BN) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key >= valid)
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) sacc[qb][kb][r] = -INFINITY;
      }
  }

  // ---- exact tiles: tile maximum and lazy rescale of the running offset ----
  if (!FAST) {
    float mnew[C::NQB], alpha[C::NQB];
    bool need = first;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (first) {
        mnew[qb] = (C::ONES && fabsf(mx) <= kFastMaxOffset) ? round_up_half(mx) : mx;
        alpha[qb] = 0.f;  // accumulators are still zero
      } else {
        need |= (mx > mrun[qb] + kRescaleSlack);
        mnew[qb] = fmaxf(mrun[qb], mx);
        alpha[qb] = __builtin_amdgcn_exp2f(mrun[qb] - mnew[qb]);
      }
    }
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        mrun[qb] = mnew[qb];
        lsum[qb] *= alpha[qb];
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
          const float a = __shfl(alpha[qb], 16 * grp + c16, 64);
#pragma unroll
          for (int t = 0; t < C::NDT; ++t) oacc[qb][grp][t] *= a;
        }
      }
    }
  }
  if (!FAST || !C::ONES) {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][kb][r] -= mrun[qb];
  }

  // ---- P = exp2(S - m), P^T operands, O^T += V^T P^T ----
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb) {
    h8 va[C::NDT];
#pragma unroll
    for (int t = 0; t < C::NDT; ++t) {
      const char* vb = vt + kb * 32 * C::ROWB + 32 * t;
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(vb + vrow_off[0]));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(vb + vrow_off[1]));
      u4 w;
      w[0] = __builtin_bit_cast(unsigned, (short __attribute__((ext_vector_type(2)))){lo[0], lo[1]});
      w[1] = __builtin_bit_cast(unsigned, (short __attribute__((ext_vector_type(2)))){lo[2], lo[3]});
      w[2] = __builtin_bit_cast(unsigned, (short __attribute__((ext_vector_type(2)))){hi[0], hi[1]});
      w[3] = __builtin_bit_cast(unsigned, (short __attribute__((ext_vector_type(2)))){hi[2], hi[3]});
      if (C::ONES && t == C::NDT - 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = vsel_data ? w[e] : vsel_const[e];
      }
      va[t] = __builtin_bit_cast(h8, w);
    }
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      unsigned pk[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int x = 0; x < 2; ++x)
          pk[i][x] = pack_h2(__builtin_amdgcn_exp2f(sacc[qb][kb][4 * i + 2 * x]),
                             __builtin_amdgcn_exp2f(sacc[qb][kb][4 * i + 2 * x + 1]));
      if (!C::ONES) {
        const h2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int x = 0; x < 2; ++x)
            lsum[qb] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pk[i][x]), one2, lsum[qb], false);
      }
      u4 b0, b1;  // P^T for queries 0..15 and 16..31 of the block
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const auto s01 = __builtin_amdgcn_permlane16_swap(pk[0][x], pk[1][x], false, false);
        const auto s23 = __builtin_amdgcn_permlane16_swap(pk[2][x], pk[3][x], false, false);
        b0[x] = s01[0];
        b1[x] = s01[1];
        b0[2 + x] = s23[0];
        b1[2 + x] = s23[1];
      }
      const h8 bq0 = __builtin_bit_cast(h8, b0), bq1 = __builtin_bit_cast(h8, b1);
#pragma unroll
      for (int t = 0; t < C::NDT; ++t) {
        oacc[qb][0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[t], bq0, oacc[qb][0][t], 0, 0, 0);
        oacc[qb][1][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[t], bq1, oacc[qb][1][t], 0, 0, 0);
      }
    }
  }
}

template <class C>
__global__ void __launch_bounds__(kThreads, C::MINB) refbank_attn_kernel(KParams p) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDSB];
  __shared__ int flags[kWaves];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, c32 = lane & 31;   // 32x32 layout: lane half, query column
  const int g = lane >> 4, c16 = lane & 15;   // 16x16 layout: row group, column

  // XCD-aware remap of the workgroup id onto (head, frame, query tile).
  const int total = p.nqt * p.F * p.H;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int hd = lid / (p.F * p.nqt);
  const int rem = lid - hd * (p.F * p.nqt);
  const int f = rem / p.nqt;
  const int qt = rem - f * p.nqt;
  const int qrow0 = qt * C::QWG + wave * 32 * C::NQB;

  // Q^T operands: Q * scale * log2(e) rounded to fp16, zero beyond d and beyond Lq.
  h8 qf[C::NQB][C::KST];
  {
    const _Float16* qb_ = p.q + (int64_t)f * p.q_fs + (int64_t)hd * C::D;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const int row = qrow0 + 32 * qb + c32;
#pragma unroll
      for (int st = 0; st < C::KST; ++st) {
        const int col = 16 * st + 8 * h;
        h8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (row < p.Lq && col < C::D) {
          const h8 x = *reinterpret_cast<const h8*>(qb_ + (int64_t)row * p.q_ld + col);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (_Float16)((float)x[e] * p.c2);
        }
        qf[qb][st] = v;
      }
    }
  }

  // Constant operand parts for the padding column D (used when C::ONES):
  // K columns D..D+7 = (1, 0, ..., 0); V^T rows D.. = ones at row D, zeros below.
  u4 kones = {0u, 0u, 0u, 0u}, vsel_const = {0u, 0u, 0u, 0u};
  kones[0] = pack_h2(1.0f, 0.0f);
  const int vrow_in_tile = C::ONES ? (16 * (C::NDT - 1) + c16) : 0;  // d row of this lane in the last V^T tile
  const bool vsel_data = vrow_in_tile < C::D;
  if (vrow_in_tile == C::D) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vsel_const[e] = pack_h2(1.0f, 1.0f);
  }
  // Per-lane LDS byte offsets of the operand reads.
  const int krow_off = c32 * C::ROWB + 16 * h;
  int vrow_off[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) vrow_off[r] = (vrow(g) + 16 * r + (c16 >> 2)) * C::ROWB + 8 * (c16 & 3);

  f4 oacc[C::NQB][2][C::NDT];
  float mrun[C::NQB], lsum[C::NQB];

  for (int attempt = 0;; ++attempt) {
    const bool exact_all = attempt > 0;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      mrun[qb] = 0.f;
      lsum[qb] = 0.f;
#pragma unroll
      for (int grp = 0; grp < 2; ++grp)
#pragma unroll
        for (int t = 0; t < C::NDT; ++t) oacc[qb][grp][t] = (f4){0.f, 0.f, 0.f, 0.f};
      if (C::ONES && h) qf[qb][C::KST - 1][0] = (_Float16)0.0f;  // offset column: none yet
    }
    bool fast = false;

    int s = 0;
    int64_t off = 0;
    issue_tile<C>(p, smem, 0, 0, f, hd, wave, lane);
    for (int it = 0;; ++it) {
      char* cur = smem + (it & 1) * C::BUFB;
      const int valid = (int)min((int64_t)C::BN, p.seg[s].len - off);
      int s_n = s;
      int64_t off_n = off + C::BN;
      if (off_n >= p.seg[s].len) {
        s_n = s + 1;
        off_n = 0;
      }
      const bool has_next = s_n < p.nseg;

      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (has_next) issue_tile<C>(p, smem + ((it + 1) & 1) * C::BUFB, s_n, off_n, f, hd, wave, lane);

      if (fast)
        tile_step<C, true>(cur, qf, oacc, mrun, lsum, false, valid, lane, h, c16, g, kones, vsel_const, vsel_data,
                           krow_off, vrow_off);
      else
        tile_step<C, false>(cur, qf, oacc, mrun, lsum, it == 0, valid, lane, h, c16, g, kones, vsel_const,
                            vsel_data, krow_off, vrow_off);

      if (it == 0 && !exact_all) {
        // freeze the offset: from now on no tile maximum is taken
        bool ok = true;
        if (C::ONES) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) ok &= fabsf(mrun[qb]) <= kFastMaxOffset;
          ok = __all(ok);
          if (ok && h) {
#pragma unroll
            for (int qb = 0; qb < C::NQB; ++qb) qf[qb][C::KST - 1][0] = (_Float16)(-mrun[qb]);
          }
        }
        fast = ok;
      }
      if (!has_next) break;
      s = s_n;
      off = off_n;
    }

    if (exact_all) break;
    // A frozen offset is only unsafe if some probability left the fp16 range:
    // then a row sum is inf or NaN.  Decide for the whole workgroup.
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      if (C::ONES) {
        constexpr int tl = C::D / 16, gl = (C::D % 16) / 4, rl = C::D % 4;
        if (g == gl) {
#pragma unroll
          for (int grp = 0; grp < 2; ++grp) bad |= !(fabsf(oacc[qb][grp][tl][rl]) <= 3.0e38f);
        }
      } else {
        bad |= !(fabsf(lsum[qb]) <= 3.0e38f);
      }
    }
    bad = __any(bad);
    if (lane == 0) flags[wave] = bad ? 1 : 0;
    __syncthreads();
    const bool any_bad = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
    if (!any_bad) break;
    __syncthreads();  // every wave has read the flags and left the tile buffers
  }

  // ---- normalise and write O (fp16, round to nearest even) ----
  _Float16* ob = p.o + (int64_t)f * p.o_fs + (int64_t)hd * C::D;
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    float tot = 0.f;
    if (!C::ONES) tot = lsum[qb] + __shfl_xor(lsum[qb], 32, 64);
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      float l;
      if (C::ONES) {
        constexpr int tl = C::D / 16, gl = (C::D % 16) / 4, rl = C::D % 4;
        l = __shfl(oacc[qb][grp][tl][rl], 16 * gl + c16, 64);
      } else {
        l = __shfl(tot, 16 * grp + c16, 64);
      }
      const float inv = 1.0f / l;
      const int row = qrow0 + 32 * qb + 16 * grp + c16;
      if (row < p.Lq) {
#pragma unroll
        for (int t = 0; t < C::NDT; ++t) {
          const int col = 16 * t + 4 * g;
          if (col < C::D) {
            h4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = (_Float16)(oacc[qb][grp][t][r] * inv);
            *reinterpret_cast<h4*>(ob + (int64_t)row * p.o_ld + col) = out;
          }
        }
      }
    }
  }
}

template <int D, int NQB, int NKB, int MINB>
hipError_t launch_cfg(const KParams& kp, hipStream_t stream) {
  using C = Cfg<D, NQB, NKB, MINB>;
  KParams p = kp;
  p.nqt = (p.Lq + C::QWG - 1) / C::QWG;
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
  switch (a.d) {
    case 32: return launch_cfg<32, 2, 2, 2>(p, stream);
    case 40: return launch_cfg<40, 2, 2, 2>(p, stream);
    case 80: return launch_cfg<80, 1, 2, 2>(p, stream);
    case 160: return launch_cfg<160, 1, 1, 1>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pl
