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
// Workgroups run feature tiles fastest and the ids dealt round-robin to the 8
// XCDs are remapped to contiguous ranges, so the feature tiles of the same
// rows share one L2 and x is read from HBM once.
#include "pl_internal.h"

namespace pl {
namespace {

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
__global__ void __launch_bounds__(64 * kWaves, 2) linear_kernel(LinearLaunch p, int n_tiles, int total) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int nt = lid % n_tiles;
  const int64_t mt = lid / n_tiles;
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
// of the workgroup's x rows and 64 W rows are copied to LDS with
// direct-to-LDS loads that read whole 128-byte row segments (8 lanes per
// row), through a ring of kStages buffers so that the next chunks stream in
// while one is multiplied; the operands are then read from LDS in
// matrix-core layout.  The 16-byte chunk c of staged row r sits at slot
// c ^ ((r / 2) % 8), which puts the 16 rows one read serves on 16 different
// bank groups.
#ifndef PL_LINEAR_MW
#define PL_LINEAR_MW 32
#endif
#ifndef PL_LINEAR_STAGES
#define PL_LINEAR_STAGES 2
#endif
constexpr int kSMW = PL_LINEAR_MW;                // rows per wave (32 or 64)
constexpr int kSJ = kSMW / 32;                    // 32-row products per wave
constexpr int kSTileM = kSMW * kWaves;            // rows per workgroup
constexpr int kStages = PL_LINEAR_STAGES;         // ring depth
constexpr int kChunkK = 64;                       // K per stage
constexpr int kRowB = kChunkK * 2;                // bytes per staged row
constexpr int kStageX = kSTileM * kRowB;          // x rows of a stage
constexpr int kStageB = kStageX + kTileN * kRowB; // + 8 KB of W rows
constexpr int kDmaPerStage = kStageB / 1024;      // wave-wide 16-byte copies per stage
constexpr int kDmaPerWave = kDmaPerStage / kWaves;
static_assert(kDmaPerStage % kWaves == 0, "copies split evenly over the waves");
static_assert(kDmaPerWave * (kStages - 2) <= 63, "vmcnt range");

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

__global__ void __launch_bounds__(64 * kWaves, 2) linear_staged_kernel(LinearLaunch p, int n_tiles, int total) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kStageB];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h = lane >> 5, c32 = lane & 31;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int nt = lid % n_tiles;
  const int64_t mt = lid / n_tiles;
  const int64_t n0 = (int64_t)nt * kTileN;
  const int64_t mw0 = mt * kSTileM;  // workgroup's first row

  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)smem;
  // copy instruction t (this wave issues t = wave, wave + 4, ...) fills staged
  // rows 8t .. 8t+7 (x rows first, then W rows); lane i takes row 8t + i/8 and
  // the chunk whose swizzled slot is i % 8
  auto issue = [&](int stage) {
    const int k0 = stage * kChunkK;
    const unsigned buf = lds0 + (unsigned)((stage % kStages) * kStageB);
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
      const int t = wave + kWaves * u;
      const int r = 8 * t + (lane >> 3);
      const int chunk = (lane & 7) ^ ((r >> 1) & 7);
      const _Float16* src;
      if (r < kSTileM) {
        const int64_t m = min(mw0 + r, p.M - 1);
        src = p.x + m * p.x_ld + k0 + 8 * chunk;
      } else {
        src = p.w + (n0 + (r - kSTileM)) * p.w_ld + k0 + 8 * chunk;
      }
      dma16(buf + t * 1024, src);
    }
  };

  f16v acc[2][kSJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < kSJ; ++j) acc[i][j] = (f16v){};

  const int nst = p.K / kChunkK;
#pragma unroll
  for (int q = 0; q < kStages - 1; ++q)
    if (q < nst) issue(q);
  for (int st = 0; st < nst; ++st) {
    // chunk st has landed (the copies of the kStages-2 chunks after it may still fly)
    if (st + kStages - 2 < nst)
      wait_vmcnt<kDmaPerWave * (kStages - 2)>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // ... everywhere; the buffer of chunk st-1 is free
    if (st + kStages - 1 < nst) issue(st + kStages - 1);
    const char* xb = smem + (st % kStages) * kStageB;
    const char* wb = xb + kStageX;
#pragma unroll
    for (int ks = 0; ks < kChunkK / 16; ++ks) {
      const int chunk = 2 * ks + h;
      h8 a[2], b[kSJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int nl = 32 * i + c32;
        a[i] = *reinterpret_cast<const h8*>(wb + nl * kRowB + 16 * swz(nl, chunk));
      }
#pragma unroll
      for (int j = 0; j < kSJ; ++j) {
        const int ml = wave * kSMW + 32 * j + c32;
        b[j] = *reinterpret_cast<const h8*>(xb + ml * kRowB + 16 * swz(ml, chunk));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kSJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  const int64_t m0 = mw0 + (int64_t)wave * kSMW;
#pragma unroll
  for (int j = 0; j < kSJ; ++j) {
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

}  // namespace

hipError_t launch_linear(const LinearLaunch& a, hipStream_t stream) {
  const int n_tiles = a.N / kTileN;
  const int64_t m_tiles = (a.M + kTileM - 1) / kTileM;
  const int64_t total = m_tiles * n_tiles;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  if (a.K % kChunkK == 0) {
    const int64_t st_total = ((a.M + kSTileM - 1) / kSTileM) * n_tiles;
    if (st_total > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(linear_staged_kernel, dim3((unsigned)st_total), dim3(64 * kWaves), 0, stream, a, n_tiles,
                       (int)st_total);
  } else if (a.K % (16 * kPrefetch) == 0)
    hipLaunchKernelGGL(linear_kernel<kPrefetch>, dim3((unsigned)total), dim3(64 * kWaves), 0, stream, a, n_tiles,
                       (int)total);
  else
    hipLaunchKernelGGL(linear_kernel<1>, dim3((unsigned)total), dim3(64 * kWaves), 0, stream, a, n_tiles, (int)total);
  return hipGetLastError();
}

}  // namespace pl
