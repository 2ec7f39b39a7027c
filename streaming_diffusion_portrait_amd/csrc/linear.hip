// The projections either side of the attention: y = x W^T (+ b), fp16 in and
// out, fp32 accumulation on the matrix cores.
//
// PersonaLive write-up, section 三条条件通路: the bank holds each reference
// layer's hidden states, which the layer projects into keys and values; the
// denoiser's own queries, keys and values and its output projection are the
// same kind of linear layer.  W is stored [out features][in features], as
// such layers keep it.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_f16): the product is taken as
// Y^T = W X^T, so both operands are rows read straight from memory, 16 bytes
// per lane per step -- A = 32 rows of W, B = 32 rows of X -- and the
// accumulator gives each lane one output row (row m = l % 32 of the tile) and
// runs of 4 consecutive output features, stored as 8-byte chunks.  A wave owns
// 64 features x 64 rows (2 x 2 products per 16-wide step, the operands of the
// next kPrefetch steps in flight); a workgroup of 4 waves owns 64 features x
// 256 rows.
// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2; the
// ids are remapped so that each XCD works through a compact block of output
// tiles (tile_of below), which it reads x and W for through that L2.
#include <cmath>

#include "pl_internal.h"

namespace pl {
namespace {

// Workgroup -> output tile (row tile mt, feature tile nt).  blockIdx.x goes to
// XCD blockIdx.x % 8, so the ids are first remapped to one contiguous range
// per XCD (XCD x holds total / 8 of them, one more for the first total % 8).
// In that order the tiles run in groups of gm row tiles, row tiles fastest:
// the tiles one XCD holds form a block of about gm row tiles by share / gm
// feature tiles, whose x rows and W rows are what its L2 has to fetch.
__device__ __forceinline__ void tile_of(int total, int m_tiles, int n_tiles, int gm, int64_t& mt, int& nt) {
  const int b = blockIdx.x, x = b & 7, q = total >> 3, rem = total & 7;
  const int lid = (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + (b >> 3);
  const int gsz = gm * n_tiles;
  const int g = lid / gsz, r = lid - g * gsz;
  const int first = g * gm, ge = min(gm, m_tiles - first);
  mt = first + r % ge;
  nt = r / ge;
}

// The group height that makes an XCD's block cheapest to fetch: with P tiles
// per XCD as a x (P / a) tiles of bm rows and bn features, the bytes are
// proportional to a bm + (P / a) bn, least at a = sqrt(P bn / bm).
int group_rows(int64_t m_tiles, int n_tiles, int bm, int bn) {
  const double share = (double)(m_tiles * n_tiles + 7) / 8.0;
  int a = (int)std::lround(std::sqrt(share * bn / bm));
  if (a < 1) a = 1;
  if (a > m_tiles) a = (int)m_tiles;
  return a;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kTileN = 64;                 // features per wave (and per workgroup)
constexpr int kTileMW = 64;                // rows per wave
constexpr int kTileM = kTileMW * kWaves;   // rows per workgroup
#ifndef PL_LINEAR_PREFETCH
#define PL_LINEAR_PREFETCH 4
#endif
constexpr int kPrefetch = PL_LINEAR_PREFETCH;  // 16-wide steps loaded ahead

struct Operands {
  h8 a[2];  // W rows n0 + 32i + l%32, k0 + 8h .. +7
  h8 b[2];  // X rows m0 + 32j + l%32, same k
};

__device__ __forceinline__ void load_step(const LinearLaunch& p, int64_t nrow0, const int64_t (&mrow)[2], int k0,
                                          int h, Operands& o) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    o.a[i] = *reinterpret_cast<const h8*>(p.w + (nrow0 + 32 * i) * p.w_ld + k0 + 8 * h);
#pragma unroll
  for (int j = 0; j < 2; ++j) o.b[j] = *reinterpret_cast<const h8*>(p.x + mrow[j] * p.x_ld + k0 + 8 * h);
}

template <int PF>
__global__ void __launch_bounds__(64 * kWaves, 2)
    linear_kernel(LinearLaunch p, int m_tiles, int n_tiles, int total, int gm) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
  int64_t mt;
  int nt;
  tile_of(total, m_tiles, n_tiles, gm, mt, nt);
  const int64_t n0 = (int64_t)nt * kTileN;
  const int64_t m0 = mt * kTileM + (int64_t)wave * kTileMW;

  // rows this lane loads as B operands (clamped to the last row: their
  // results land in rows that are not stored)
  int64_t mrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) mrow[j] = min(m0 + 32 * j + c32, p.M - 1);
  const int64_t nrow0 = n0 + c32;

  f16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f16v){};

  // a ring of PF operand sets: step s's loads are issued PF steps before its
  // products, so PF memory round trips are in flight.  K is a multiple of
  // 16 * PF, so the loop has no conditions and the waits stay precise.
  Operands ring[PF];
  const int ksteps = p.K / 16;
#pragma unroll
  for (int q = 0; q < PF; ++q) load_step(p, nrow0, mrow, 16 * q, h, ring[q]);
  for (int s0 = 0; s0 + PF < ksteps; s0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[q].a[i], ring[q].b[j], acc[i][j], 0, 0, 0);
      load_step(p, nrow0, mrow, 16 * (s0 + PF + q), h, ring[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < PF; ++q)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[q].a[i], ring[q].b[j], acc[i][j], 0, 0, 0);

  // acc[i][j][4r + q]: feature n0 + 32i + 8r + 4h + q of row m0 + 32j + l%32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t m = m0 + 32 * j + c32;
    if (m >= p.M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + 32 * i + 8 * r + 4 * h;
        float bq[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.bias) {
          const float4 b4 = *reinterpret_cast<const float4*>(p.bias + n);
          bq[0] = b4.x;
          bq[1] = b4.y;
          bq[2] = b4.z;
          bq[3] = b4.w;
        }
        h4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = (_Float16)(acc[i][j][4 * r + q] + bq[q]);
        *reinterpret_cast<h4*>(p.y + m * p.y_ld + n) = out;
      }
  }
}

// ---- staged variant (K a multiple of 64) ---------------------------------------
// The direct loads above touch 32 rows of 32 bytes per instruction, so the
// memory pipeline, not the matrix core, sets the pace.  Here 64-wide K chunks
// of the workgroup's x rows and W rows are copied to LDS with direct-to-LDS
// loads that read whole 128-byte row segments (8 lanes per row), through a
// ring of STAGES buffers so that the next chunks stream in while one is
// multiplied; the operands are then read from LDS in matrix-core layout.  The
// 16-byte chunk c of staged row r sits at slot c ^ ((r / 2) % 8), which puts
// the 16 rows one read serves on 16 different bank groups.
//
// The W waves of a workgroup form a WR x (W / WR) grid; each owns 32 IM rows
// x 32 IN features, so per 16-wide step it reads IM + IN operands from LDS for
// IM x IN products.  Larger wave tiles cut the LDS bytes per product (the LDS,
// not the matrix core, is what small tiles run out of).
template <int WR_, int IM_, int IN_, int STAGES_, int W_ = 4>
struct GemmCfg {
  static constexpr int W = W_, THREADS = 64 * W_;  // waves per workgroup
  static constexpr int WR = WR_, WF = W_ / WR_, IM = IM_, IN = IN_, STAGES = STAGES_;
  static constexpr int BM = WR * 32 * IM;          // rows per workgroup
  static constexpr int BN = WF * 32 * IN;          // features per workgroup
  static constexpr int kChunkK = 64;               // K per stage
  static constexpr int kRowB = kChunkK * 2;        // bytes per staged row
  static constexpr int STAGE_X = BM * kRowB;       // x rows of a stage
  static constexpr int STAGE_B = STAGE_X + BN * kRowB;
  static constexpr int NCOPY = STAGE_B / 1024;     // wave-wide 16-byte copies per stage (8 rows each)
  static constexpr int CPW = NCOPY / W;            // per wave
  static constexpr int LDS = STAGES * STAGE_B;
  static constexpr int MINW = LDS <= 80 * 1024 ? 2 : 1;  // workgroups per CU the registers are sized for
  static_assert(W % WR == 0, "2D grid of waves");
  static_assert(NCOPY % W == 0, "copies split evenly over the waves");
  static_assert(STAGES >= 2 && CPW * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(unsigned m0, const _Float16* src) {
  // lane i's 16 bytes land at M0 + 16 i; completion is awaited with vmcnt
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(src)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Output tile staged in LDS for the row-contiguous stores: the 16-byte chunk
// c of tile row r sits at slot so(r, c), so that the accumulator's writes (one
// row per lane, 8 bytes each) and the row reads (16 bytes per lane) both hit 16
// different bank groups (256 bytes = 16 slots) for 16 consecutive rows.  With
// CR = 8 (mod 16) chunks per row, row parity picks the half and (r / 2) % 8 the
// slot within it; with CR = 0 (mod 16), r % 16 picks the slot.  XOR with a
// value below 8 (or 16) keeps the slot inside the row.
template <int CR>
__device__ __forceinline__ int so(int row, int c) {
  static_assert(CR % 8 == 0, "rows of whole 128-byte lines");
  return CR % 16 == 8 ? c ^ ((row >> 1) & 7) : c ^ (row & 15);
}

template <class G, bool LDS_OUT>
__global__ void __launch_bounds__(G::THREADS, G::MINW)
    linear_staged_kernel(LinearLaunch p, int m_tiles, int n_tiles, int total, int gm) {
  __shared__ __attribute__((aligned(16))) char smem[G::LDS];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / G::WF, wf = wave % G::WF;
  const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
  int64_t mt;
  int nt;
  tile_of(total, m_tiles, n_tiles, gm, mt, nt);
  const int64_t n0 = (int64_t)nt * G::BN;
  const int64_t mw0 = mt * G::BM;  // workgroup's first row

  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)smem;
  // copy instruction t (this wave issues t = wave, wave + W, ...) fills staged
  // rows 8t .. 8t+7 (x rows first, then W rows); lane i takes row 8t + i/8 and
  // the chunk whose swizzled slot is i % 8
  auto issue = [&](int stage) {
    const int k0 = stage * G::kChunkK;
    const unsigned buf = lds0 + (unsigned)((stage % G::STAGES) * G::STAGE_B);
#pragma unroll
    for (int u = 0; u < G::CPW; ++u) {
      const int t = wave + G::W * u;
      const int r = 8 * t + (lane >> 3);
      const int chunk = (lane & 7) ^ ((r >> 1) & 7);
      const _Float16* src;
      if (r < G::BM) {
        const int64_t m = min(mw0 + r, p.M - 1);
        src = p.x + m * p.x_ld + k0 + 8 * chunk;
      } else {
        src = p.w + (n0 + (r - G::BM)) * p.w_ld + k0 + 8 * chunk;
      }
      dma16(buf + t * 1024, src);
    }
  };

  f16v acc[G::IN][G::IM];
#pragma unroll
  for (int i = 0; i < G::IN; ++i)
#pragma unroll
    for (int j = 0; j < G::IM; ++j) acc[i][j] = (f16v){};

  const int nst = p.K / G::kChunkK;
#pragma unroll
  for (int q = 0; q < G::STAGES - 1; ++q)
    if (q < nst) issue(q);
  for (int st = 0; st < nst; ++st) {
    // chunk st has landed (the copies of the STAGES-2 chunks after it may still fly)
    if (st + G::STAGES - 2 < nst)
      wait_vmcnt<G::CPW * (G::STAGES - 2)>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // ... everywhere; the buffer of chunk st-1 is free
    if (st + G::STAGES - 1 < nst) issue(st + G::STAGES - 1);
    const char* xb = smem + (st % G::STAGES) * G::STAGE_B;
    const char* wb = xb + G::STAGE_X;
    // all operands of the chunk's 4 steps are read up front; the schedule
    // below issues the reads of step ks + 2 right after the products of step
    // ks, so two steps of reads overlap the matrix core instead of waiting in
    // front of it
    constexpr int KS = G::kChunkK / 16;
    h8 a[KS][G::IN], b[KS][G::IM];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int chunk = 2 * ks + h;
#pragma unroll
      for (int i = 0; i < G::IN; ++i) {
        const int nl = (wf * G::IN + i) * 32 + c32;
        a[ks][i] = *reinterpret_cast<const h8*>(wb + nl * G::kRowB + 16 * swz(nl, chunk));
      }
#pragma unroll
      for (int j = 0; j < G::IM; ++j) {
        const int ml = (wr * G::IM + j) * 32 + c32;
        b[ks][j] = *reinterpret_cast<const h8*>(xb + ml * G::kRowB + 16 * swz(ml, chunk));
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < G::IN; ++i)
#pragma unroll
        for (int j = 0; j < G::IM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (G::IN + G::IM), 0);  // reads of steps 0, 1
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, G::IN * G::IM, 0);  // products of step ks
      if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, G::IN + G::IM, 0);  // reads of step ks + 2
    }
  }

  // acc[i][j][4r + q]: feature (wf IN + i) 32 + 8r + 4h + q of row (wr IM + j) 32 + l%32
  if constexpr (LDS_OUT) {
    // y tile -> LDS (bias added, rounded to fp16), then whole 16-byte chunks of
    // row segments -> y: a wave's store covers 64 / CR rows of BN features
    constexpr int CR = G::BN / 8;  // 16-byte chunks per tile row
    constexpr int RB = G::BN * 2;  // bytes per tile row
    // the bias of this lane's features, all loads issued before the first use
    float4 bias4[G::IN][4];
#pragma unroll
    for (int i = 0; i < G::IN; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) bias4[i][r] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.bias) {
#pragma unroll
      for (int i = 0; i < G::IN; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bias4[i][r] = *reinterpret_cast<const float4*>(p.bias + n0 + 8 * ((wf * G::IN + i) * 4 + r) + 4 * h);
    }
    __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
    for (int i = 0; i < G::IN; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = (wf * G::IN + i) * 4 + r;
        const float bq[4] = {bias4[i][r].x, bias4[i][r].y, bias4[i][r].z, bias4[i][r].w};
#pragma unroll
        for (int j = 0; j < G::IM; ++j) {
          const int row = (wr * G::IM + j) * 32 + c32;
          h4 out;
#pragma unroll
          for (int q = 0; q < 4; ++q) out[q] = (_Float16)(acc[i][j][4 * r + q] + bq[q]);
          *reinterpret_cast<h4*>(smem + row * RB + 16 * so<CR>(row, c) + 8 * h) = out;
        }
      }
    __syncthreads();
    // read the thread's chunks in groups of up to 8, then store them
    constexpr int U = G::BM * CR / G::THREADS;
    constexpr int UG = U % 8 == 0 ? 8 : U % 4 == 0 ? 4 : U % 2 == 0 ? 2 : 1;
#pragma unroll
    for (int u0 = 0; u0 < U; u0 += UG) {
      h8 v[UG];
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        const int e = tid + G::THREADS * (u0 + u), row = e / CR, c = e % CR;
        v[u] = *reinterpret_cast<const h8*>(smem + row * RB + 16 * so<CR>(row, c));
      }
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        const int e = tid + G::THREADS * (u0 + u), row = e / CR, c = e % CR;
        const int64_t m = mw0 + row;
        if (m < p.M) *reinterpret_cast<h8*>(p.y + m * p.y_ld + n0 + 8 * c) = v[u];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < G::IM; ++j) {
      const int64_t m = mw0 + (wr * G::IM + j) * 32 + c32;
      if (m >= p.M) continue;
#pragma unroll
      for (int i = 0; i < G::IN; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t n = n0 + (wf * G::IN + i) * 32 + 8 * r + 4 * h;
          float bq[4] = {0.f, 0.f, 0.f, 0.f};
          if (p.bias) {
            const float4 b4 = *reinterpret_cast<const float4*>(p.bias + n);
            bq[0] = b4.x;
            bq[1] = b4.y;
            bq[2] = b4.z;
            bq[3] = b4.w;
          }
          h4 out;
#pragma unroll
          for (int q = 0; q < 4; ++q) out[q] = (_Float16)(acc[i][j][4 * r + q] + bq[q]);
          *reinterpret_cast<h4*>(p.y + m * p.y_ld + n) = out;
        }
    }
  }
}

// gm = 0 picks the group height by group_rows
template <class G>
hipError_t launch_staged(const LinearLaunch& a, hipStream_t stream, int gm = 0) {
  static_assert(G::BM * G::BN * 2 <= G::LDS, "the output tile fits in the stage buffers");
  const int n_tiles = a.N / G::BN;
  const int64_t m_tiles = (a.M + G::BM - 1) / G::BM;
  const int64_t total = m_tiles * n_tiles;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  if (gm <= 0) gm = group_rows(m_tiles, n_tiles, G::BM, G::BN);
  if (gm > m_tiles) gm = (int)m_tiles;
  // 16-byte row stores need y 16-byte aligned with a row pitch of 8 elements
  if ((reinterpret_cast<uintptr_t>(a.y) & 15) == 0 && a.y_ld % 8 == 0)
    hipLaunchKernelGGL((linear_staged_kernel<G, true>), dim3((unsigned)total), dim3(G::THREADS), 0, stream, a,
                       (int)m_tiles, n_tiles, (int)total, gm);
  else
    hipLaunchKernelGGL((linear_staged_kernel<G, false>), dim3((unsigned)total), dim3(G::THREADS), 0, stream, a,
                       (int)m_tiles, n_tiles, (int)total, gm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinearLaunch& a, hipStream_t stream) {
  if (a.K % 64 == 0) {
    // Tile shape by problem shape (measured at the projections of the four
    // UNet levels): 256 x 256 tiles where K is long and they still give about
    // one workgroup per CU (the contraction-bound case; 8 waves of 64 x 128,
    // two per SIMD, hide the operand reads that one wave per SIMD could not);
    // 128 x 128 with three stages in flight where K is long and those give
    // one workgroup per CU (the rows are few, so each workgroup streams a
    // long slice of W: the deeper pipeline covers its fetch latency);
    // 128 x 192 where N allows and M is large enough for 1024+ of them (the
    // fused q/k/v weights: x is read through L2 a third as often as with
    // 64-wide tiles, and 5 operand reads feed 6 products); 256 x 64 where M
    // is large enough for 1024+ of those; 128 x 64 otherwise.
    using Square = GemmCfg<4, 2, 4, 2, 8>;
    using Deep = GemmCfg<2, 2, 2, 3, 4>;
    using Wide = GemmCfg<2, 2, 3, 2>;
    using Tall = GemmCfg<4, 2, 2, 2>;
    using Base = GemmCfg<4, 1, 2, 2>;
    auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * (a.N / bn); };
    if (a.K >= 1024 && a.N % Square::BN == 0 && tiles(Square::BM, Square::BN) >= 224)
      return launch_staged<Square>(a, stream);
    if (a.K >= 1024 && a.N % Deep::BN == 0 && tiles(Deep::BM, Deep::BN) >= 192 && tiles(Deep::BM, Deep::BN) <= 256)
      return launch_staged<Deep>(a, stream);
    if (a.N % Wide::BN == 0 && tiles(Wide::BM, Wide::BN) >= 1024) return launch_staged<Wide>(a, stream);
    if (tiles(Tall::BM, Tall::BN) >= 1024) return launch_staged<Tall>(a, stream);
    return launch_staged<Base>(a, stream);
  }
  const int n_tiles = a.N / kTileN;
  const int64_t m_tiles = (a.M + kTileM - 1) / kTileM;
  const int64_t total = m_tiles * n_tiles;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  const int gm = group_rows(m_tiles, n_tiles, kTileM, kTileN);
  if (a.K % (16 * kPrefetch) == 0)
    hipLaunchKernelGGL(linear_kernel<kPrefetch>, dim3((unsigned)total), dim3(64 * kWaves), 0, stream, a, (int)m_tiles,
                       n_tiles, (int)total, gm);
  else
    hipLaunchKernelGGL(linear_kernel<1>, dim3((unsigned)total), dim3(64 * kWaves), 0, stream, a, (int)m_tiles, n_tiles,
                       (int)total, gm);
  return hipGetLastError();
}

}  // namespace pl
