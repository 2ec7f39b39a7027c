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
// 64 features x 64 rows (2 x 2 products per 16-wide step, both operands loaded
// one step ahead); a workgroup of 4 waves owns 64 features x 256 rows.
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

  Operands cur, nxt;
  load_step(p, nrow0, mrow, 0, h, cur);
  const int ksteps = p.K / 16;
  for (int s = 0; s < ksteps; ++s) {
    if (s + 1 < ksteps) load_step(p, nrow0, mrow, 16 * (s + 1), h, nxt);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
    cur = nxt;
  }

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
        h4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = acc[i][j][4 * r + q];
          if (p.bias) v += p.bias[n + q];
          out[q] = (_Float16)v;
        }
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
  hipLaunchKernelGGL(linear_kernel, dim3((unsigned)total), dim3(64 * kWaves), 0, stream, a, n_tiles, (int)total);
  return hipGetLastError();
}

}  // namespace pl
