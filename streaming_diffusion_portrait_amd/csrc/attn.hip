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
//   * one workgroup = W wavefronts (4; 8 at d = 80) = one (head, frame,
//     query tile); each wave owns NQB blocks of 32 query rows (the K/V
//     operands read from LDS serve all of them, which keeps LDS traffic per
//     score low);
//   * K and V tiles of BN = 64 keys are copied HBM -> LDS by direct-to-LDS
//     loads (global_load_lds_dwordx4) into a ring of NBUF buffers that runs
//     up to NBUF-1 tiles ahead of the tile being consumed; one barrier per
//     tile.  A staged tile is plane-major: plane c holds the 16-byte chunk c
//     (dims 8c..8c+7) of all 64 keys, so one wave-wide copy fills one plane,
//     every lane keeps a single byte offset (its key row) and the operand
//     reads below hit consecutive LDS addresses;
//   * workgroup ids are remapped so that each of the 8 XCDs (ids are dealt
//     round-robin to them) works on a contiguous range of (head, frame, tile),
//     i.e. mostly on one head, whose shared bank keys then stay in its L2.
//
// Matrix-core mapping
//   S^T = K Q^T   v_mfma_f32_32x32x16_f16: A = 32 keys x 16 d from LDS,
//                 B = Q^T for 32 queries, held in registers for the whole
//                 kernel.  Lane l ends up with the scores of query l%32
//                 for 16 of the 32 keys (4 runs of 4 consecutive keys).
//   O^T = V^T P^T v_mfma_f32_16x16x32_f16: B = P^T is assembled from the S^T
//                 registers of two query halves with v_permlane16_swap, so
//                 probabilities never touch LDS; A = V^T is read from the
//                 staged V tile with ds_read_b64_tr_b16 (transposing read),
//                 two reads per operand.  The order in which the swapped P^T
//                 lists the keys fixes which V rows each transposing read
//                 fetches (vrow() below).
//
// Software pipeline (fast tiles, per wave, 32-key blocks b): iteration b
// evaluates softmax(b+1) on the vector ALU, O^T += V^T(b) P^T(b) and
// S^T(b+2) = K(b+2) Q^T on the matrix core, and reads the K operands of
// block b+3 and V of block b from LDS -- independent streams that are
// interleaved instruction by instruction in a fixed order, so the
// exponentials and conversions issue while the matrix products execute and
// no product waits for an LDS read issued in the same iteration except PV(b)
// for V(b).  Two waves share each SIMD; the one in its PV part runs at raised
// issue priority, which settles the pair into alternating phases.
//
// Softmax (fp32, log2 units).  Q is pre-scaled by scale*log2(e) and rounded
// to fp16 once, so the matrix core yields s = scale*log2(e)*q.k directly.
//   * Exact tiles (the first tile; every tile of an exact pass): the block's
//     row maximum is taken; the running offset m is raised when the maximum
//     exceeds it by more than 8 (so p <= 2^8, safe in fp16) and the
//     accumulator is rescaled then.
//   * Fast tiles: after the first tile the offset is frozen and no maximum is
//     taken.  For a head dim that leaves a zero-padded column (d = 40), the
//     padding carries the offset into the matrix core: K gets a column of
//     ones and Q the value -m, so s - m comes out of the MFMA and p = exp2 of
//     the accumulator; for the other head dims the S^T products start from an
//     accumulator seeded with -m, to the same effect.  A frozen offset only
//     fails if a later score exceeds it by 16 or more (p beyond the fp16
//     range): a row sum then turns inf/NaN, which is checked once at the end;
//     the workgroup then recomputes everything with exact tiles.
//   * Row sums come from the same fp16 values that weight V, through the
//     matrix core: a row of ones in the V^T padding (d = 40), or two more PV
//     products per query block whose A is a constant with a first row of ones
//     (other head dims).
#include "pl_internal.h"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace pl {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef short s2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;      // log2 units a block max may exceed the running offset by
constexpr float kFastMaxOffset = 1024.0f;  // |m| bound for freezing the offset in fp16

// sched_group_barrier instruction classes
constexpr int kSchedMfma = 0x008, kSchedValu = 0x002, kSchedDsRead = 0x100;

// Key rows (within a 32-key block) fetched by the two transposing reads of
// lane group g (lanes 16g..16g+15) for the V^T operand.  They follow from the
// S^T accumulator layout (lane half h holds keys 8i + 4h + j) and the
// permlane16 swaps of key runs i = {0,1} and {2,3}: contraction index
// k = 8g + e maps to key vrow(g) + e for e < 4 and to vrow(g) + 16 + e - 4
// for e >= 4, with vrow(g) = 0, 8, 4, 12 for g = 0..3.
__device__ __forceinline__ int vrow(int g) { return 8 * (g & 1) + 4 * (g >> 1); }

// Bytes of padding after each 1 KB plane of a staged tile; it moves the two
// planes one transposing read touches onto different LDS banks.
#ifndef PL_PLANE_PAD
#define PL_PLANE_PAD 64
#endif

template <int D_, int NQB_, int NKB_, int NBUF_, int MINB_, bool PIPE_, int W_, int DSPLIT_ = 1>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int W = W_;                // wavefronts per workgroup
  static constexpr int THREADS = 64 * W;
  static constexpr int NQB = NQB_;            // 32-query blocks per wave
  static constexpr bool PIPE = PIPE_;         // software-pipelined fast tiles
  static constexpr int NKB = NKB_;            // 32-key blocks per tile
  static constexpr int NBUF = NBUF_;          // LDS tile buffers in the ring
  static constexpr int MINB = MINB_;          // workgroups per CU the register budget is sized for
  static constexpr int BN = 32 * NKB;         // keys per tile
  // DSPLIT waves share each query block, each holding NDT / DSPLIT of the
  // O^T d tiles (all of them compute the block's S^T and softmax): fewer
  // registers per wave, so more waves per SIMD
  static constexpr int DSPLIT = DSPLIT_;
  static constexpr int WQ = W / DSPLIT;        // waves with distinct query blocks
  static constexpr int QWG = 32 * NQB * WQ;    // query rows per workgroup
  static constexpr int KST = (D + 15) / 16;   // 16-wide contraction steps of S^T
  static constexpr int NDT = (D + 15) / 16;   // 16-row tiles of O^T
  static constexpr int NDW = NDT / DSPLIT_;   // ... held by one wave
  static constexpr bool ONES = (D % 16) != 0; // padding column D carries ones / -m
  // no ones column (d = 32, 80, 160): the row sums come from two more PV
  // products per query block with a constant A whose first row is ones (with
  // a ones column, from the ones row of the V^T padding)
  static constexpr bool RSUM = !ONES;
  static constexpr int CPR = D / 8;           // 16-byte chunks per key row (dims 8c..8c+7)
  static constexpr int NPL = 2 * KST;         // planes per tile: the chunks, then the (1, 0, ..., 0) plane if any
  static constexpr int PLB = 64 * 16 + PL_PLANE_PAD;  // bytes per plane (64 keys x 16 bytes + padding)
  static constexpr int KBLK = 32 * 16;        // byte step of a 32-key block within a plane
  static constexpr int TILEB = NPL * PLB;     // bytes of one K (or V) tile
  static constexpr int LI = CPR;              // wave-wide 16-byte load instructions per tile (K or V): one per plane
  static constexpr int NI = (2 * LI + W - 1) / W;  // load instructions per wave per tile (max)
  static constexpr int BUFB = 2 * TILEB;      // K tile + V tile
  static constexpr int LDSB = NBUF * BUFB;
  static_assert(D % 8 == 0, "head dim must be a multiple of 8");
  static_assert(!ONES || D % 16 == 8, "the ones column must start the upper half of the last step");
  static_assert(NPL - CPR == (ONES ? 1 : 0), "one constant plane exactly when d leaves a padding column");
  static_assert(BN == 64, "one plane per load instruction: 64 keys of 16 bytes");
  static_assert(PLB % 16 == 0, "planes hold 16-byte chunks");
  static_assert(NBUF >= 2 && NBUF <= 6, "ring of 2 to 6 buffers");
  static_assert(W % DSPLIT == 0 && NDT % DSPLIT == 0, "waves and d tiles split evenly");
  static_assert(DSPLIT == 1 || RSUM, "with a d split every wave needs the row sums: no ones column");
  static_assert(NI * (NBUF - 1) <= 48, "vmcnt wait table range");
  // the pass-end flags: their own bytes when the first tile's fast-path
  // decision needs them while the ring is in use (ones column), else the last
  // ring slot, which a following pass fills only after its first barrier
  static constexpr int FLAGS_AT = ONES ? LDSB : (NBUF - 1) * BUFB;
  static constexpr int SMEM = ONES ? LDSB + 4 * W : LDSB;
  static_assert(ONES || 4 * W <= BUFB, "flags fit in a ring slot");
};

struct KParams {
  const _Float16* q;
  _Float16* o;
  int64_t q_ld, q_fs, o_ld, o_fs;
  int F, Lq, H, nqt, nseg;
  float c2;  // scale * log2(e)
  AttnSegment seg[PL_MAX_SEGMENTS];
  // key-axis split: nsplit workgroups per (head, frame, query tile), split s
  // taking key tiles [s*tps, (s+1)*tps); with nsplit > 1 the kernel writes
  // per-split partials (unnormalised O, offset, row sum) instead of O
  int nsplit, tps;
  float* part_o;  // [F*H*nsplit][Lq][D] fp32
  float* part_ml; // [F*H*nsplit][Lq][2] fp32: offset (log2 units), row sum
#ifdef PL_DEBUG_BOUNDS
  // elements from q, o and each segment's k (and v) to one past the last one
  // the call may touch; floats of part_o
  int64_t q_ext, o_ext, seg_ext[PL_MAX_SEGMENTS], part_ext;
#endif
};

// ---- bounds-checking build ------------------------------------------------------
// Built with PL_DEBUG_BOUNDS, every global and LDS access of the attention
// kernels is first checked against the extent of the buffer it belongs to; a
// failed check sets bit `site` of a device-wide mask (read back by
// pl_debug_bounds) and the access is skipped, so a wrong index is reported
// instead of touching memory the call does not own.  Other builds compile the
// checks away (the condition is not even evaluated).
enum BoundsSite {
  kSiteKvSrc = 0,   // K/V tile copy: global source
  kSiteKvDst,       // K/V tile copy: LDS destination
  kSiteQLoad,       // Q operands
  kSiteOStore,      // O rows
  kSitePartO,       // key split: partial O
  kSitePartMl,      // key split: offset and row sum
  kSiteLdsK,        // K operand reads from LDS
  kSiteLdsV,        // V^T operand reads from LDS
  kSiteShortQSrc,   // short context: Q block copy, global source
  kSiteShortQDst,   // short context: Q block copy, LDS destination
  kSiteShortO,      // short context: O rows
  kSiteShortBuf,    // short context: block buffer in LDS
  kSiteCombineIn,   // key split merge: partials read
  kSiteCombineOut,  // key split merge: O rows
};
#ifdef PL_DEBUG_BOUNDS
__device__ unsigned long long g_bounds_mask;
__device__ __forceinline__ bool bounds_ok(bool ok, int site) {
  if (!ok) atomicOr(&g_bounds_mask, 1ull << site);
  return ok;
}
#define PL_BOUNDS(ok, site) bounds_ok((ok), (site))
#else
#define PL_BOUNDS(ok, site) true
#endif
// [off, off + n) inside [0, ext)
#define PL_IN(off, n, ext) ((int64_t)(off) >= 0 && (int64_t)(off) + (int64_t)(n) <= (int64_t)(ext))

__device__ __forceinline__ unsigned pack_h2(float a, float b) {
  h2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Round x up to an fp16-representable value (the offset must not be exceeded
// by the scores of the block that defined it).
__device__ __forceinline__ float round_up_half(float x) {
  _Float16 hx = (_Float16)(x + fabsf(x) * 0.0009765625f);
  float r = (float)hx;
  return r < x ? x : r;
}

// Wait until at most n of this wave's vector-memory operations are in flight
// (n <= 0: all of them; n above the table waits for more than asked, which is safe).
#define PL_VMCNT_CASE(k) \
  case k:                \
    asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    PL_VMCNT_CASE(1) PL_VMCNT_CASE(2) PL_VMCNT_CASE(3) PL_VMCNT_CASE(4) PL_VMCNT_CASE(5) PL_VMCNT_CASE(6)
    PL_VMCNT_CASE(7) PL_VMCNT_CASE(8) PL_VMCNT_CASE(9) PL_VMCNT_CASE(10) PL_VMCNT_CASE(11) PL_VMCNT_CASE(12)
    PL_VMCNT_CASE(13) PL_VMCNT_CASE(14) PL_VMCNT_CASE(15) PL_VMCNT_CASE(16) PL_VMCNT_CASE(17) PL_VMCNT_CASE(18)
    PL_VMCNT_CASE(19) PL_VMCNT_CASE(20) PL_VMCNT_CASE(21) PL_VMCNT_CASE(22) PL_VMCNT_CASE(23) PL_VMCNT_CASE(24)
    PL_VMCNT_CASE(25) PL_VMCNT_CASE(26) PL_VMCNT_CASE(27) PL_VMCNT_CASE(28) PL_VMCNT_CASE(29) PL_VMCNT_CASE(30)
    PL_VMCNT_CASE(31) PL_VMCNT_CASE(32) PL_VMCNT_CASE(33) PL_VMCNT_CASE(34) PL_VMCNT_CASE(35) PL_VMCNT_CASE(36)
    PL_VMCNT_CASE(37) PL_VMCNT_CASE(38) PL_VMCNT_CASE(39) PL_VMCNT_CASE(40) PL_VMCNT_CASE(41) PL_VMCNT_CASE(42)
    PL_VMCNT_CASE(43) PL_VMCNT_CASE(44) PL_VMCNT_CASE(45) PL_VMCNT_CASE(46) PL_VMCNT_CASE(47) PL_VMCNT_CASE(48)
    default:
      if (n > 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      break;
  }
}
#undef PL_VMCNT_CASE

// Wave-uniform copies of values the compiler cannot prove uniform (they live
// in scalar registers from here on).  readfirstlane yields a signed int:
// widen through unsigned so a low word never sign-extends into the high one.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((uint64_t)x >> 32));
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(uint64_t)x);
  return (int64_t)((hi << 32) | lo);
}
__device__ __forceinline__ const char* uniform_ptr(const char* x) {
  return reinterpret_cast<const char*>(uniform64((int64_t)(uintptr_t)x));
}

// The copy side of the ring.  A staged tile is plane-major: plane c holds the
// 16-byte chunk c (dims 8c..8c+7) of each of the 64 keys, so one wave-wide
// direct-to-LDS load (lane i's 16 bytes land at M0 + 16*i) fills one plane,
// lane i copying key i.  Copy instruction u of a tile (u < LI: K plane u,
// else V plane u - LI) belongs to wave u % W.
template <class C>
struct Copier {
  int s;        // segment of the next tile to copy
  int64_t off;  // its first key within the segment
  int issued;   // tiles copied so far
  int ni;       // copy instructions this wave issues per tile
#ifdef PL_DEBUG_BOUNDS
  unsigned lds_end;  // LDS byte address one past the kernel's shared memory
#endif
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One wave-wide direct-to-LDS copy: 16 bytes from gbase + voff (per lane)
// to LDS address m0 + 16*lane.  Written as asm so the compiler does not
// serialise the LDS reads of the other buffers behind it; completion is
// awaited explicitly (vmcnt) before the barrier that publishes the tile.  The
// instruction has no register result.  (M0 is named as clobbered; nothing
// else in this kernel keeps a value in it.)
__device__ __forceinline__ void lds_dma16(unsigned m0, unsigned voff, const char* gbase) {
  const uint64_t sbase = (uint64_t)(uintptr_t)uniform_ptr(gbase);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ unsigned lds_addr(const char* x) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)x;
}

// Issue this wave's share of the copies of the next tile and advance.  A
// ragged last tile of a segment repeats its last real key in the lanes beyond
// it (those keys are masked in the softmax).
template <class C>
__device__ __forceinline__ void issue_tile(const KParams& p, char* smem, Copier<C>& cp, int f, int h, int wave,
                                           int lane) {
  const AttnSegment& sg = p.seg[cp.s];
  const int valid = (int)min((int64_t)C::BN, sg.len - cp.off);  // >= 1
  const int64_t base = (int64_t)f * sg.frame_stride + cp.off * sg.ld + (int64_t)h * C::D;
  const char* kbase = reinterpret_cast<const char*>(sg.k + base);
  const char* vbase = reinterpret_cast<const char*>(sg.v + base);
  const unsigned voff = (unsigned)min(lane, valid - 1) * (unsigned)(sg.ld * 2);
  const unsigned buf = lds_addr(smem) + (unsigned)((cp.issued % C::NBUF) * C::BUFB);
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int u = wave + C::W * j;  // wave-uniform
    if (u < 2 * C::LI) {
      const bool isv = u >= C::LI;
      const int pl = isv ? u - C::LI : u;
      const unsigned dst = buf + (isv ? C::TILEB : 0) + pl * C::PLB;
      if (PL_BOUNDS(!__any(!PL_IN(base + voff / 2 + 8 * pl, 8, p.seg_ext[cp.s])), kSiteKvSrc) &&
          PL_BOUNDS(dst + 1024u <= cp.lds_end, kSiteKvDst))
        lds_dma16(dst, voff, (isv ? vbase : kbase) + 16 * pl);
    }
  }
  cp.off += C::BN;
  if (cp.off >= sg.len) {
    cp.s += 1;
    cp.off = 0;
  }
  cp.issued += 1;
}

// Copy side for key sequences made of full tiles only: the (frame, head)
// base addresses live in scalar registers and each lane's byte offset (its
// key row) is fixed per segment, so issuing a tile costs no vector arithmetic.
template <class C>
struct FastCopier {
  const char* kp;  // next tile's K rows for this (frame, head)
  const char* vp;  // ... and V rows
  int64_t step;    // bytes from one tile to the next (BN rows)
  int rem;         // tiles left in the current segment
  int s;           // current segment
  unsigned voff;   // per lane: byte offset of its key row
};

template <class C>
__device__ __forceinline__ void fast_seek(const KParams& p, FastCopier<C>& fc, int s, int64_t off, int f, int h,
                                          int lane) {
  fc.s = __builtin_amdgcn_readfirstlane(s);
  if (fc.s >= p.nseg) return;
  const AttnSegment& sg = p.seg[fc.s];
  off = uniform64(off);
  const int64_t base = (int64_t)f * sg.frame_stride + off * sg.ld + (int64_t)h * C::D;
  fc.kp = uniform_ptr(reinterpret_cast<const char*>(sg.k + base));
  fc.vp = uniform_ptr(reinterpret_cast<const char*>(sg.v + base));
  fc.step = uniform64(sg.ld * 2 * C::BN);
  fc.rem = __builtin_amdgcn_readfirstlane((int)((sg.len - off) / C::BN));
  // the lane id is recomputed here rather than kept live across the pipeline
  // (a spilled copy would be reloaded, and that load's wait would also wait
  // for every copy in flight)
  // (volatile, so that it is not hoisted out of the loop either)
  (void)lane;
  unsigned ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  fc.voff = ln * (unsigned)(sg.ld * 2);
}

template <class C>
__device__ __forceinline__ void fast_issue(const KParams& p, char* smem, FastCopier<C>& fc, Copier<C>& cp, int f,
                                           int h, int wave, int lane) {
  const unsigned buf = lds_addr(smem) + (unsigned)((cp.issued % C::NBUF) * C::BUFB);
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int u = wave + C::W * j;  // wave-uniform
    if (u < 2 * C::LI) {
      const bool isv = u >= C::LI;
      const int pl = isv ? u - C::LI : u;
      const unsigned dst = buf + (isv ? C::TILEB : 0) + pl * C::PLB;
      if (PL_BOUNDS(!__any(!PL_IN(((isv ? fc.vp : fc.kp) - reinterpret_cast<const char*>(isv ? p.seg[fc.s].v : p.seg[fc.s].k)) / 2 +
                                      fc.voff / 2 + 8 * pl,
                                  8, p.seg_ext[fc.s])),
                    kSiteKvSrc) &&
          PL_BOUNDS(dst + 1024u <= cp.lds_end, kSiteKvDst))
        lds_dma16(dst, fc.voff, (isv ? fc.vp : fc.kp) + 16 * pl);
    }
  }
  fc.kp += fc.step;
  fc.vp += fc.step;
  cp.issued += 1;
  if (--fc.rem == 0) fast_seek<C>(p, fc, fc.s + 1, 0, f, h, lane);
}

// Per-wave register state.
template <class C>
struct WaveState {
  h8 qf[C::NQB][C::KST];       // Q^T operands (scaled, fp16)
  f4 oacc[C::NQB][2][C::NDW];  // O^T accumulators: [query block][16-query half][16-row d tile, from dt0]
  int dt0;                     // first O^T d tile of this wave
  float mrun[C::NQB];          // running offset of query l%32 of each block
  f16v negm[C::NQB];           // -mrun in every accumulator slot: the seed of fast S^T products (no ones column)
  f4 osum[C::NQB][2];          // RSUM: row 0 holds the row sums of the half's 16 queries
  h8 onesA;                    // RSUM: the constant A (row 0 ones: lanes with l % 16 == 0)
};

// Lane constants.
struct LaneCtx {
  int lane, h, c16, g;
  int krow_off;     // K operand LDS byte offset within a 32-key block (plane 0)
  int vrow_off[2];  // V^T operand LDS byte offsets of the two transposing reads (planes 0, 1)
#ifdef PL_DEBUG_BOUNDS
  int lds_bytes;    // the kernel's shared memory
#endif
};

// K step st: lane half h reads plane 2st+h at key c32.  V^T read r of lane
// (g, c16): key vrow(g) + 16r + c16/4, dims 4(c16%4)..+3 of the 16-dim tile,
// i.e. plane 2t + (c16%4)/2, byte 8*(c16%2) of the key's chunk.
template <class C>
__device__ __forceinline__ void lane_offsets(LaneCtx& lc) {
  lc.krow_off = (lc.lane & 31) * 16 + lc.h * C::PLB;
#pragma unroll
  for (int r = 0; r < 2; ++r)
    lc.vrow_off[r] = (vrow(lc.g) + 16 * r + (lc.c16 >> 2)) * 16 + ((lc.c16 & 3) >> 1) * C::PLB + 8 * (lc.c16 & 1);
}

// K operands of one 32-key block: step st reads planes 2st (lanes 0..31)
// and 2st+1 (lanes 32..63); the padding column D, if any, lies in the
// constant plane.
template <class C>
__device__ __forceinline__ void load_k(const char* smem, int kblk, const LaneCtx& lc, h8 (&ka)[C::KST]) {
#pragma unroll
  for (int st = 0; st < C::KST; ++st) {
    const int a = kblk + lc.krow_off + 2 * st * C::PLB;
    ka[st] = PL_BOUNDS(PL_IN(a, 16, lc.lds_bytes), kSiteLdsK) ? *reinterpret_cast<const h8*>(smem + a) : (h8){};
  }
}

// S^T = K Q^T for every query block of the wave, from K operands in registers.
// (Steps outermost: consecutive products accumulate into different query
// blocks, so none waits for the one just issued.)  SEED: the accumulation
// starts from -offset instead of 0, so the scores come out with the frozen
// offset already subtracted (fast blocks when d leaves no ones column).
template <class C, bool SEED>
__device__ __forceinline__ void qk_regs(const h8 (&ka)[C::KST], const WaveState<C>& ws, f16v (&sacc)[C::NQB]) {
#pragma unroll
  for (int st = 0; st < C::KST; ++st)
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
      sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[st], ws.qf[qb][st],
                                                        st > 0 ? sacc[qb] : SEED ? ws.negm[qb] : (f16v){}, 0, 0, 0);
}

// S^T(block) = K(block) Q^T for every query block of the wave.
template <class C, bool SEED>
__device__ __forceinline__ void qk_block(const char* smem, int kblk, const WaveState<C>& ws, const LaneCtx& lc,
                                         f16v (&sacc)[C::NQB]) {
  h8 ka[C::KST];
  load_k<C>(smem, kblk, lc, ka);
  qk_regs<C, SEED>(ka, ws, sacc);
}

// V^T operands of one 32-key block.
template <class C>
__device__ __forceinline__ void load_vt(const char* smem, int vblk, const LaneCtx& lc, int dt0, h8 (&va)[C::NDW]) {
#pragma unroll
  for (int t = 0; t < C::NDW; ++t) {
    int a0 = vblk + 2 * (dt0 + t) * C::PLB + lc.vrow_off[0];
    int a1 = vblk + 2 * (dt0 + t) * C::PLB + lc.vrow_off[1];
    if (!PL_BOUNDS(!__any(!(PL_IN(a0, 8, lc.lds_bytes) && PL_IN(a1, 8, lc.lds_bytes))), kSiteLdsV)) a0 = a1 = 0;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(smem + a0));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(smem + a1));
    u4 w;
    w[0] = __builtin_bit_cast(unsigned, (s2){lo[0], lo[1]});
    w[1] = __builtin_bit_cast(unsigned, (s2){lo[2], lo[3]});
    w[2] = __builtin_bit_cast(unsigned, (s2){hi[0], hi[1]});
    w[3] = __builtin_bit_cast(unsigned, (s2){hi[2], hi[3]});
    va[t] = __builtin_bit_cast(h8, w);
  }
}

// O^T += V^T P^T for one 32-key block.
template <class C>
__device__ __forceinline__ void pv_block(const h8 (&va)[C::NDW], const h8 (&pb)[C::NQB][2], WaveState<C>& ws) {
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
    for (int t = 0; t < C::NDW; ++t)
#pragma unroll
      for (int grp = 0; grp < 2; ++grp)
        ws.oacc[qb][grp][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[t], pb[qb][grp], ws.oacc[qb][grp][t], 0, 0, 0);
  if constexpr (C::RSUM) {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int grp = 0; grp < 2; ++grp)
        ws.osum[qb][grp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ws.onesA, pb[qb][grp], ws.osum[qb][grp], 0, 0, 0);
  }
}

// Softmax of one 32-key block: S^T -> P^T operands; keys at or beyond
// `valid` get no weight.  EXACT: take the block maximum and update the
// offsets (FIRST: set them from this block).  When an offset moves,
// `rescale` is set and alpha (S layout) holds the factors the accumulated
// products of earlier blocks must be multiplied by (the caller applies
// them, the row sums included).
template <class C, bool EXACT>
__device__ __forceinline__ void softmax_block(f16v (&sacc)[C::NQB], WaveState<C>& ws, const LaneCtx& lc, int valid,
                                              bool first, h8 (&pb)[C::NQB][2], float (&alpha)[C::NQB], bool& rescale) {
  if (valid < 32) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * lc.h + (r & 3);
      if (key >= valid)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) sacc[qb][r] = -INFINITY;
    }
  }
  rescale = false;
  if (EXACT) {
    float mx[C::NQB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      float v = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, sacc[qb][r]);
      mx[qb] = fmaxf(v, __shfl_xor(v, 32, 64));
      need |= mx[qb] > ws.mrun[qb] + kRescaleSlack;
    }
    if (first) {
      rescale = true;
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        ws.mrun[qb] = (C::ONES && fabsf(mx[qb]) <= kFastMaxOffset) ? round_up_half(mx[qb]) : mx[qb];
        alpha[qb] = 0.f;  // nothing accumulated yet
      }
    } else if (__any(need)) {
      rescale = true;
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        const float mnew = fmaxf(ws.mrun[qb], mx[qb]);
        alpha[qb] = __builtin_amdgcn_exp2f(ws.mrun[qb] - mnew);
        ws.mrun[qb] = mnew;
      }
    }
  }
  if (EXACT) {  // fast blocks carry the frozen offset inside the scores already
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[qb][r] -= ws.mrun[qb];
  }
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    unsigned pk[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        pk[i][x] = pack_h2(__builtin_amdgcn_exp2f(sacc[qb][4 * i + 2 * x]),
                           __builtin_amdgcn_exp2f(sacc[qb][4 * i + 2 * x + 1]));
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
    pb[qb][0] = __builtin_bit_cast(h8, b0);
    pb[qb][1] = __builtin_bit_cast(h8, b1);
  }
}

// O^T *= alpha (alpha given in S layout, moved to the O^T layout).
template <class C>
__device__ __forceinline__ void rescale_acc(WaveState<C>& ws, const LaneCtx& lc, const float (&alpha)[C::NQB]) {
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const float a = __shfl(alpha[qb], 16 * grp + lc.c16, 64);
#pragma unroll
      for (int t = 0; t < C::NDW; ++t) ws.oacc[qb][grp][t] *= a;
      if constexpr (C::RSUM) ws.osum[qb][grp] *= a;
    }
}

// One tile, blocks in sequence (exact tiles, and fast tiles outside the pipeline).
template <class C, bool FAST>
__device__ __forceinline__ void tile_step(const char* smem, int kt, int valid, bool first, WaveState<C>& ws,
                                          const LaneCtx& lc) {
#pragma unroll
  for (int kb = 0; kb < C::NKB; ++kb) {
    if (kb > 0 && valid <= 32 * kb) break;  // a tile's last block holds no key (short segments)
    f16v s[C::NQB];
    qk_block<C, FAST && !C::ONES>(smem, kt + kb * C::KBLK, ws, lc, s);
    h8 va[C::NDW];
    load_vt<C>(smem, kt + C::TILEB + kb * C::KBLK, lc, ws.dt0, va);
    h8 pb[C::NQB][2];
    float alpha[C::NQB];
    bool resc;
    softmax_block<C, !FAST>(s, ws, lc, valid - 32 * kb, first && kb == 0, pb, alpha, resc);
    if (!FAST && resc) rescale_acc<C>(ws, lc, alpha);  // O^T holds only earlier blocks here
    pv_block<C>(va, pb, ws);
  }
}

// Interleave hint for one pipelined iteration: LDS operand reads first, then
// the softmax's vector work threaded between the matrix products.
#ifndef PL_SCHED_PER
#define PL_SCHED_PER 3
#endif
template <class C>
__device__ __forceinline__ void sched_iteration() {
  // V^T reads first (used last); the S^T products (operands already in
  // registers) threaded with the softmax's vector work; then the reads of the
  // next K operands (into the registers those products just read) and the PV
  // products with the rest of the vector work
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * C::NDW, 0);
#pragma unroll
  for (int i = 0; i < C::NQB * C::KST; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, PL_SCHED_PER, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::KST, 0);
#pragma unroll
  for (int i = 0; i < C::NQB * 2 * C::NDW; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, PL_SCHED_PER, 0);
  }
}

// The softmax of one fast block (offset already inside the scores) as a
// stream of single vector instructions, so that a schedule can place each of
// them: per query block, 16 exponentials, 8 packs to fp16 (each issued two
// exponentials after its inputs, so it never waits for them) and 4
// permlane16 swaps that assemble P^T.  sm_ops<C>() instructions per query
// block.
template <class C>
constexpr int sm_ops() {
  return 28;
}
template <class C>
struct FastSoftmax {
  static constexpr int kSmOps = sm_ops<C>();
  f16v* s;          // [NQB] scores -> exponentials, in place
  unsigned pk[C::NQB][8];
  h8* pb;           // [NQB][2] P^T operands out
  __device__ __forceinline__ void op(int v) {
    const int qb = v / kSmOps, r = v % kSmOps;
    if (r < 4) {  // exponentials 0..3
      s[qb][r] = __builtin_amdgcn_exp2f(s[qb][r]);
    } else if (r < 4 + 3 * 6) {  // (pack i, exponentials 2i+4, 2i+5) for i = 0..5
      const int i = (r - 4) / 3, k = (r - 4) % 3;
      if (k == 0) pk[qb][i] = pack_h2(s[qb][2 * i], s[qb][2 * i + 1]);
      else s[qb][2 * i + 4 + (k - 1)] = __builtin_amdgcn_exp2f(s[qb][2 * i + 4 + (k - 1)]);
    } else if (r < 24) {  // packs 6, 7
      const int i = r - 16;
      pk[qb][i] = pack_h2(s[qb][2 * i], s[qb][2 * i + 1]);
    } else {  // swaps: pack (2j+x) with pack (2j+2+x) for j = 0, 2 and x = 0, 1
      const int k = r - 24, x = k & 1, j = (k >> 1) * 4;
      const auto sw = __builtin_amdgcn_permlane16_swap(pk[qb][j + x], pk[qb][j + 2 + x], false, false);
      u4 b0 = __builtin_bit_cast(u4, pb[2 * qb]), b1 = __builtin_bit_cast(u4, pb[2 * qb + 1]);
      b0[(k >> 1) * 2 + x] = sw[0];
      b1[(k >> 1) * 2 + x] = sw[1];
      pb[2 * qb] = __builtin_bit_cast(h8, b0);
      pb[2 * qb + 1] = __builtin_bit_cast(h8, b1);
    }
  }
};

// Vector instructions placed after each S^T product and each PV product of a
// steady pipelined iteration (the rest follow the last product).
#ifndef PL_FIXED_ORDER
#define PL_FIXED_ORDER 1
#endif
#ifndef PL_SLOT_QK
#define PL_SLOT_QK 4
#endif
#ifndef PL_SLOT_PV
#define PL_SLOT_PV 3
#endif
// Steady pipelined iteration with a fixed instruction order: the LDS reads,
// then slots of one matrix product and a share of the softmax's vector
// instructions, fenced so that the compiler keeps the interleave.  Computes
// the same as pipe_iteration<C, true, true, true>.
template <class C>
__device__ __forceinline__ void pipe_iteration_fixed(const char* smem, int vblk, int kblk3, f16v (&s_in)[C::NQB],
                                                     f16v (&s_out)[C::NQB], const h8 (&p_in)[C::NQB][2],
                                                     h8 (&p_out)[C::NQB][2], const h8 (&ka_cur)[C::KST],
                                                     h8 (&ka_next)[C::KST], WaveState<C>& ws, const LaneCtx& lc) {
  constexpr int NQK = C::KST * C::NQB, NPV = (C::NDW + (C::RSUM ? 1 : 0)) * C::NQB * 2, NM = NQK + NPV;
  constexpr int NV = sm_ops<C>() * C::NQB;
  // vector instructions after each S^T / PV product (d = 40: tuned; otherwise
  // 4 after each S^T product and the rest spread over the PV products)
  constexpr int SQK = C::ONES ? PL_SLOT_QK : 4;
  constexpr int SPV = C::ONES ? PL_SLOT_PV : (NV - NQK * SQK + NPV - 1) / NPV;
  h8 va[C::NDW];
  load_vt<C>(smem, vblk, lc, ws.dt0, va);
  load_k<C>(smem, kblk3, lc, ka_next);
  __builtin_amdgcn_sched_barrier(0);
  FastSoftmax<C> sm;
  sm.s = s_in;
  sm.pb = &p_out[0][0];
  int v = 0;
  // Two waves share each SIMD.  The wave in its PV phase (16x16 products, the
  // packs and swaps) runs at raised issue priority, so while one wave streams
  // its PV products the other fills the gaps with its S^T products and
  // exponentials, and the two drift into alternating phases.
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m == NQK) __builtin_amdgcn_s_setprio(1);
    if (m < NQK) {  // S^T(b+2): steps outermost, query blocks alternate
      const int st = m / C::NQB, qb = m % C::NQB;
      s_out[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          ka_cur[st], ws.qf[qb][st], st > 0 ? s_out[qb] : C::ONES ? (f16v){} : ws.negm[qb], 0, 0, 0);
    } else {  // O^T += V^T(b) P^T(b): d tiles outermost (the V reads land in that order), then the row sums
      const int i = m - NQK, t = i / (2 * C::NQB), qb = (i / 2) % C::NQB, grp = i % 2;
      if (t < C::NDW)
        ws.oacc[qb][grp][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[t], p_in[qb][grp], ws.oacc[qb][grp][t], 0, 0, 0);
      else
        ws.osum[qb][grp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ws.onesA, p_in[qb][grp], ws.osum[qb][grp], 0, 0, 0);
    }
    const int nv = m < NQK ? SQK : SPV;
#pragma unroll
    for (int k = 0; k < nv; ++k)
      if (v + k < NV) sm.op(v + k);
    v += nv;
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int k = 0; k < NV; ++k)
    if (k >= v) sm.op(k);
  __builtin_amdgcn_sched_barrier(0);
}

// One pipelined iteration over full blocks (block b of the pipeline):
//   S^T(b+2) = K(b+2) Q^T from K operands already in registers (ka_cur),
//   K operands of block b+3 read from LDS into ka_next,
//   softmax(b+1) [s_in -> p_out], O^T += V^T(b) P^T(b) [p_in].
// The products need no LDS data of this iteration, the softmax needs scores
// computed an iteration ago, and V^T(b) is read first and used last, so no
// stream waits on another.  QK / SM / KR: which of the first three parts
// exist (the pipeline's last iterations run past the end of the sequence).
template <class C, bool QK, bool SM, bool KR>
__device__ __forceinline__ void pipe_iteration(const char* smem, int vblk, int kblk3, f16v (&s_in)[C::NQB],
                                               f16v (&s_out)[C::NQB], const h8 (&p_in)[C::NQB][2],
                                               h8 (&p_out)[C::NQB][2], const h8 (&ka_cur)[C::KST],
                                               h8 (&ka_next)[C::KST], WaveState<C>& ws, const LaneCtx& lc) {
  float alpha[C::NQB];
  bool resc;
  h8 va[C::NDW];
  load_vt<C>(smem, vblk, lc, ws.dt0, va);
  if (QK) qk_regs<C, !C::ONES>(ka_cur, ws, s_out);  // pipelined blocks are fast
  if (SM) softmax_block<C, false>(s_in, ws, lc, 32, false, p_out, alpha, resc);
  if (KR) load_k<C>(smem, kblk3, lc, ka_next);  // after the products read ka_cur
  pv_block<C>(va, p_in, ws);
  if (QK && SM && KR) sched_iteration<C>();
  __builtin_amdgcn_sched_barrier(0);  // iterations do not mix: each keeps its own interleave
}

// A full pipelined iteration: the fixed-order form (the compiler-scheduled one
// when PL_FIXED_ORDER is 0).
template <class C>
__device__ __forceinline__ void pipe_steady(const char* smem, int vblk, int kblk3, f16v (&s_in)[C::NQB],
                                            f16v (&s_out)[C::NQB], const h8 (&p_in)[C::NQB][2],
                                            h8 (&p_out)[C::NQB][2], const h8 (&ka_cur)[C::KST], h8 (&ka_next)[C::KST],
                                            WaveState<C>& ws, const LaneCtx& lc) {
#if PL_FIXED_ORDER
  pipe_iteration_fixed<C>(smem, vblk, kblk3, s_in, s_out, p_in, p_out, ka_cur, ka_next, ws, lc);
  return;
#endif
  pipe_iteration<C, true, true, true>(smem, vblk, kblk3, s_in, s_out, p_in, p_out, ka_cur, ka_next, ws, lc);
}

template <class C>
__global__ void __launch_bounds__(C::THREADS, C::MINB) refbank_attn_kernel(KParams p) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  int* const flags = reinterpret_cast<int*>(smem + C::FLAGS_AT);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  LaneCtx lc;
  lc.lane = tid & 63;
  lc.h = lc.lane >> 5;
  lc.c16 = lc.lane & 15;
  lc.g = lc.lane >> 4;
  const int c32 = lc.lane & 31;

  // XCD-aware remap of the workgroup id onto (head, frame, query tile, split).
  const int total = p.nqt * p.F * p.H * p.nsplit;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int split = lid % p.nsplit;
  lid /= p.nsplit;
  const int hd = lid / (p.F * p.nqt);
  const int rem = lid - hd * (p.F * p.nqt);
  const int f = rem / p.nqt;
  const int qt = rem - f * p.nqt;
  const int qrow0 = qt * C::QWG + (C::DSPLIT == 1 ? wave : wave % C::WQ) * 32 * C::NQB;

  WaveState<C> ws;
  ws.dt0 = C::DSPLIT == 1 ? 0 : (wave / C::WQ) * C::NDW;
  // Q^T operands: Q * scale * log2(e) rounded to fp16, zero beyond d and beyond Lq.
  {
    const _Float16* qb_ = p.q + (int64_t)f * p.q_fs + (int64_t)hd * C::D;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const int row = qrow0 + 32 * qb + c32;
#pragma unroll
      for (int st = 0; st < C::KST; ++st) {
        const int col = 16 * st + 8 * lc.h;
        h8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (row < p.Lq && col < C::D &&
            PL_BOUNDS(PL_IN((int64_t)f * p.q_fs + (int64_t)row * p.q_ld + (int64_t)hd * C::D + col, 8, p.q_ext),
                      kSiteQLoad)) {
          const h8 x = *reinterpret_cast<const h8*>(qb_ + (int64_t)row * p.q_ld + col);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (_Float16)((float)x[e] * p.c2);
        }
        ws.qf[qb][st] = v;
      }
    }
  }

  // The constant plane of every K and V tile (d = 40): chunk (1, 0, ..., 0)
  // for every key -- K's column D is ones (it meets the offset column of Q),
  // V^T's row D is ones (its products are the row sums).  The copies never
  // write this plane; the first barrier below publishes it.
  if constexpr (C::ONES) {
    for (int i = tid >> 6; i < 2 * C::NBUF; i += C::W) {
      h8 one = {0, 0, 0, 0, 0, 0, 0, 0};
      one[0] = (_Float16)1.0f;
      *reinterpret_cast<h8*>(smem + i * C::TILEB + C::CPR * C::PLB + 16 * lc.lane) = one;
    }
  }
  if constexpr (C::RSUM) {  // A of the row-sum products: row 0 (lanes with l % 16 == 0) all ones
    const _Float16 a1 = lc.c16 == 0 ? (_Float16)1.0f : (_Float16)0.0f;
    ws.onesA = (h8){a1, a1, a1, a1, a1, a1, a1, a1};
  }
  lane_offsets<C>(lc);
#ifdef PL_DEBUG_BOUNDS
  lc.lds_bytes = C::SMEM;
#endif

  // Tiles in the key sequence (this split's range of them) and this wave's
  // copy instructions per tile.
  int ntiles = 0;
  bool full = true;  // every tile holds BN real keys: no masking anywhere
  for (int s = 0; s < p.nseg; ++s) {
    ntiles += (int)((p.seg[s].len + C::BN - 1) / C::BN);
    full &= (p.seg[s].len % C::BN) == 0;
  }
  const int t_begin = min(split * p.tps, ntiles);
  ntiles = min(ntiles, t_begin + p.tps) - t_begin;
  int s0 = 0;  // segment and key offset of the split's first tile
  int64_t off0 = 0;
  for (int t = t_begin; s0 < p.nseg; ++s0) {
    const int nts = (int)((p.seg[s0].len + C::BN - 1) / C::BN);
    if (t < nts) {
      off0 = (int64_t)t * C::BN;
      break;
    }
    t -= nts;
  }
  Copier<C> cp;
#ifdef PL_DEBUG_BOUNDS
  cp.lds_end = lds_addr(smem) + (unsigned)C::SMEM;
#endif
  cp.ni = 0;
#pragma unroll
  for (int j = 0; j < C::NI; ++j) cp.ni += (wave + C::W * j < 2 * C::LI) ? 1 : 0;

  // Segment / offset of a tile -> its count of real keys; step to the next tile.
  auto tile_valid = [&](int s, int64_t off) -> int { return (int)min((int64_t)C::BN, p.seg[s].len - off); };
  auto tile_next = [&](int& s, int64_t& off) {
    off += C::BN;
    if (off >= p.seg[s].len) {
      s += 1;
      off = 0;
    }
  };

  // One pass over the whole key sequence.  The first pass freezes the offset
  // after tile 0 (fast tiles); if that overflowed anywhere in the workgroup, a
  // second pass recomputes everything with exact maxima on every tile.  The
  // two passes are separate instantiations (not one loop), so the rare exact
  // pass does not share register assignments with the fast one.  Returns
  // whether the pass must be redone.
  auto pass = [&](auto exact_tag) -> bool {
    constexpr bool exact_all = decltype(exact_tag)::value;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      ws.mrun[qb] = 0.f;
#pragma unroll
      for (int grp = 0; grp < 2; ++grp)
#pragma unroll
        for (int t = 0; t < C::NDW; ++t) ws.oacc[qb][grp][t] = (f4){0.f, 0.f, 0.f, 0.f};
      if constexpr (C::RSUM) ws.osum[qb][0] = ws.osum[qb][1] = (f4){0.f, 0.f, 0.f, 0.f};
      if constexpr (C::ONES) if (lc.h) ws.qf[qb][C::KST - 1][0] = (_Float16)0.0f;  // offset column: none yet
    }

    cp.s = s0;
    cp.off = off0;
    cp.issued = 0;
    while (cp.issued < C::NBUF - 1 && cp.issued < ntiles) issue_tile<C>(p, smem, cp, f, hd, wave, lc.lane);

    // ---- tile 0: exact ----
    int cs = s0;  // segment / offset of the tile being consumed
    int64_t coff = off0;
    wait_vm(cp.ni * (cp.issued - 1));  // tile 0 has landed
    __syncthreads();
    if (cp.issued < ntiles) issue_tile<C>(p, smem, cp, f, hd, wave, lc.lane);  // ring slot NBUF-1 is still unused
    tile_step<C, false>(smem, 0, tile_valid(cs, coff), true, ws, lc);
    tile_next(cs, coff);

    bool fast = false;
    if (!exact_all) {
      bool ok = true;
      if constexpr (C::ONES) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) ok &= fabsf(ws.mrun[qb]) <= kFastMaxOffset;
        // One decision for the whole workgroup: the waves share the copies of
        // every tile and its barriers, so they must all take the same path.
        const bool wave_ok = __all(ok);
        if (lc.lane == 0) flags[wave] = wave_ok ? 1 : 0;
        __syncthreads();
        int all_ok = 1;
#pragma unroll
        for (int w = 0; w < C::W; ++w) all_ok &= flags[w];
        ok = __builtin_amdgcn_readfirstlane(all_ok) != 0;
        if (ok && lc.h) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) ws.qf[qb][C::KST - 1][0] = (_Float16)(-ws.mrun[qb]);  // offset joins the product
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) ws.negm[qb][r] = -ws.mrun[qb];  // offset seeds the product
      }
      fast = ok;
    }

    if (C::PIPE && fast && full && ntiles > 1) {
      // ---- fast full tiles 1..ntiles-1, software pipelined over 32-key blocks ----
      // Pipeline block j (j = 0 .. nb-1) is half j%2 of tile 1 + j/2.  Iteration j
      // reads V of block j and K of block j+3 from LDS, so before an odd
      // iteration 2u+1 tile u+3 must have landed; tile u is then finished by
      // every wave and its slot is refilled.
      static_assert(!C::PIPE || C::NKB == 2, "the pipeline is written for two 32-key blocks per tile");
      static_assert(!C::PIPE || C::NBUF >= 4, "the pipeline reads from three tiles while the next one is copied");
      const int nb = 2 * (ntiles - 1);
      auto kblk = [&](int j) { return ((1 + (j >> 1)) % C::NBUF) * C::BUFB + (j & 1) * C::KBLK; };
      auto vblk = [&](int j) { return kblk(j) + C::TILEB; };
      FastCopier<C> fc;
      fast_seek<C>(p, fc, cp.s, cp.off, f, hd, lc.lane);
      // prologue: tiles 1 and 2 (if any) have landed; tile 0 is free
      wait_vm(cp.ni * (cp.issued - min(3, ntiles)));
      __syncthreads();
      if (cp.issued < ntiles && cp.issued < 1 + C::NBUF) fast_issue<C>(p, smem, fc, cp, f, hd, wave, lc.lane);
      f16v sA[C::NQB], sB[C::NQB];
      h8 pA[C::NQB][2], pB[C::NQB][2];
      h8 kaA[C::KST], kaB[C::KST];
      {
        float alpha[C::NQB];
        bool resc;
        qk_block<C, !C::ONES>(smem, kblk(0), ws, lc, sA);
        softmax_block<C, false>(sA, ws, lc, 32, false, pA, alpha, resc);
        qk_block<C, !C::ONES>(smem, kblk(1), ws, lc, sB);
        if (2 < nb) load_k<C>(smem, kblk(2), lc, kaA);
      }
      // steady state: the copies of the NBUF-4 tiles after u+3 may stay in
      // flight (this wave's own count: the waves issue 2 or 3 copies a tile)
      const int steady_wait = cp.ni * (C::NBUF - 4);
      // Even blocks read (sB -> pB, sA <- S^T, pA into PV, K into kaB), odd
      // blocks the mirror image, so no registers are copied.
      int u = 0;
      for (; 2 * u + 4 < nb; ++u) {
        pipe_steady<C>(smem, vblk(2 * u), kblk(2 * u + 3), sB, sA, pA, pB, kaA, kaB, ws, lc);
        if (cp.issued >= u + C::NBUF)
          wait_vm(steady_wait);  // tile u+3 has landed
        else
          wait_vm(0);
        __syncthreads();  // ... everywhere; tile u is finished
        if (cp.issued < ntiles && cp.issued < u + 1 + C::NBUF) fast_issue<C>(p, smem, fc, cp, f, hd, wave, lc.lane);
        pipe_steady<C>(smem, vblk(2 * u + 1), kblk(2 * u + 4), sA, sB, pB, pA, kaB, kaA, ws, lc);
      }
      __builtin_amdgcn_s_setprio(0);  // back to the default for the tail
      // Blocks 2u.. are left: four of them (every tile they need has landed
      // and no copy remains), or two when the sequence has only two tiles.
      if (nb - 2 * u == 4) {
        pipe_steady<C>(smem, vblk(2 * u), kblk(2 * u + 3), sB, sA, pA, pB, kaA, kaB, ws, lc);
        pipe_iteration<C, true, true, false>(smem, vblk(2 * u + 1), 0, sA, sB, pB, pA, kaB, kaA, ws, lc);
        u += 1;
      }
      pipe_iteration<C, false, true, false>(smem, vblk(2 * u), 0, sB, sA, pA, pB, kaA, kaB, ws, lc);
      pipe_iteration<C, false, false, false>(smem, vblk(2 * u + 1), 0, sA, sB, pB, pA, kaB, kaA, ws, lc);
    } else {
      // ---- remaining tiles one after another (exact unless fast) ----
      for (int t = 1; t < ntiles; ++t) {
        wait_vm(cp.ni * (cp.issued - (t + 1)));  // tile t has landed
        __syncthreads();                         // ... everywhere; tile t-1 is free
        if (cp.issued < ntiles) issue_tile<C>(p, smem, cp, f, hd, wave, lc.lane);
        const int kt = (t % C::NBUF) * C::BUFB;
        if (fast)
          tile_step<C, true>(smem, kt, tile_valid(cs, coff), false, ws, lc);
        else
          tile_step<C, false>(smem, kt, tile_valid(cs, coff), false, ws, lc);
        tile_next(cs, coff);
      }
    }

    // Tiles taken with exact maxima cannot overflow: only a pass that froze the
    // offset for a later tile needs the check (and its two barriers).
    if (exact_all || !fast || ntiles == 1) return false;
    // A frozen offset is only unsafe if some probability left the fp16 range:
    // then a row sum is inf or NaN.  Decide for the whole workgroup.
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      if constexpr (C::ONES) {
        constexpr int tl = C::D / 16, gl = (C::D % 16) / 4, rl = C::D % 4;
        if (lc.g == gl) {
#pragma unroll
          for (int grp = 0; grp < 2; ++grp) bad |= !(fabsf(ws.oacc[qb][grp][tl][rl]) <= 3.0e38f);
        }
      } else {
        if (lc.g == 0) bad |= !(fabsf(ws.osum[qb][0][0]) <= 3.0e38f) || !(fabsf(ws.osum[qb][1][0]) <= 3.0e38f);
      }
    }
    bad = __any(bad);
    __syncthreads();  // every wave is done with the ring before it may be refilled
    if (lc.lane == 0) flags[wave] = bad ? 1 : 0;
    __syncthreads();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < C::W; ++w) any_bad |= flags[w];
    return __builtin_amdgcn_readfirstlane(any_bad) != 0;
  };
  if (ntiles > 0 && pass(std::false_type{})) pass(std::true_type{});

  if (p.nsplit > 1) {
    // ---- this split's partials: unnormalised O^T, offset and row sum per query ----
    const int64_t pbase = ((int64_t)(f * p.H + hd) * p.nsplit + split) * p.Lq;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        float l;
        if constexpr (C::ONES) {
          constexpr int tl = C::D / 16, gl = (C::D % 16) / 4, rl = C::D % 4;
          l = __shfl(ws.oacc[qb][grp][tl][rl], 16 * gl + lc.c16, 64);
        } else {
          l = __shfl(ws.osum[qb][grp][0], lc.c16, 64);  // row 0: lanes 0..15
        }
        const float mo = __shfl(ws.mrun[qb], 16 * grp + lc.c16, 64);  // S layout: lane l%32 is query l%32
        const int row = qrow0 + 32 * qb + 16 * grp + lc.c16;
        if (row < p.Lq) {
          const bool empty = ntiles <= 0;
          float* po = p.part_o + (pbase + row) * C::D;
#pragma unroll
          for (int t = 0; t < C::NDW; ++t) {
            const int col = 16 * (ws.dt0 + t) + 4 * lc.g;
            if (col < C::D && PL_BOUNDS(PL_IN((pbase + row) * C::D + col, 4, p.part_ext), kSitePartO))
              *reinterpret_cast<f4*>(po + col) = empty ? (f4){0.f, 0.f, 0.f, 0.f} : ws.oacc[qb][grp][t];
          }
          if (lc.g == 0 && ws.dt0 == 0 &&
              PL_BOUNDS(PL_IN((pbase + row) * 2, 2, p.part_ext / C::D * 2), kSitePartMl)) {
            float* pm = p.part_ml + (pbase + row) * 2;
            pm[0] = empty ? -INFINITY : mo;
            pm[1] = empty ? 0.f : l;
          }
        }
      }
    }
    return;
  }

  // ---- normalise and write O (fp16, round to nearest even) ----
  _Float16* ob = p.o + (int64_t)f * p.o_fs + (int64_t)hd * C::D;
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      float l;
      if constexpr (C::ONES) {
        constexpr int tl = C::D / 16, gl = (C::D % 16) / 4, rl = C::D % 4;
        l = __shfl(ws.oacc[qb][grp][tl][rl], 16 * gl + lc.c16, 64);
      } else {
        l = __shfl(ws.osum[qb][grp][0], lc.c16, 64);  // row 0: lanes 0..15
      }
      const float inv = 1.0f / l;
      const int row = qrow0 + 32 * qb + 16 * grp + lc.c16;
      if (row < p.Lq) {
#pragma unroll
        for (int t = 0; t < C::NDW; ++t) {
          const int col = 16 * (ws.dt0 + t) + 4 * lc.g;
          if (col < C::D &&
              PL_BOUNDS(PL_IN((int64_t)f * p.o_fs + (int64_t)row * p.o_ld + (int64_t)hd * C::D + col, 4, p.o_ext),
                        kSiteOStore)) {
            h4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = (_Float16)(ws.oacc[qb][grp][t][r] * inv);
            *reinterpret_cast<h4*>(ob + (int64_t)row * p.o_ld + col) = out;
          }
        }
      }
    }
  }
}

// ---- short contexts: one segment of at most one tile -------------------------
//
// The expression cross-attention of the denoiser (PersonaLive, section
// 三条条件通路: the 512-d expression embedding becomes 32 tokens that the
// Spatial_Cross blocks attend to) and the CLIP one (a single 1x768 token)
// have a key sequence of at most one tile.  There the work is reading Q and
// writing O; each workgroup stages its (frame, head)'s keys once and its waves
// walk many 32-query blocks, loading the next block's Q while the current one
// is computed, so the memory latency overlaps the arithmetic.

template <class C>
__device__ __forceinline__ void load_q_block(const KParams& p, const _Float16* qb_, int row, const LaneCtx& lc,
                                             h8 (&qf)[C::KST]) {
#pragma unroll
  for (int st = 0; st < C::KST; ++st) {
    const int col = 16 * st + 8 * lc.h;
    h8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (row < p.Lq && col < C::D) v = *reinterpret_cast<const h8*>(qb_ + (int64_t)row * p.q_ld + col);
    qf[st] = v;
  }
}

#ifndef PL_SHORT_WGS
#define PL_SHORT_WGS 1024  // workgroups a short-context launch aims for (4 per CU)
#endif

// Q and O pass through LDS: each wave stages its 32-row block of Q (the head's
// d columns of 32 rows) with direct-to-LDS copies in which D/8 consecutive
// lanes read one row's 2d contiguous bytes, and writes O back the same way
// from LDS, so every memory instruction moves whole row slices instead of the
// 16- and 8-byte pieces of the matrix-core layouts.  Two such buffers per wave:
// the next block's Q lands while the current one is computed; O overwrites the
// Q it was computed from.
template <class C>
struct ShortStage {
  static constexpr int QB = 32 * C::D * 2;      // bytes of one 32-row block (row pitch 2d)
  static constexpr int CPRQ = C::D / 8;         // 16-byte chunks per row
  static constexpr int RPI = 64 / CPRQ;         // rows per wave-wide copy
  static constexpr int NQI = (32 + RPI - 1) / RPI;  // copies per block
  static constexpr int LDS = C::BUFB + C::W * 2 * QB;  // one K/V tile pair + the waves' buffers
  static_assert(NQI <= 24, "vmcnt wait table range");
};

template <class C>
__global__ void __launch_bounds__(C::THREADS, C::MINB) short_ctx_kernel(KParams p, int nsplit) {
  static_assert(C::NQB == 1 && C::DSPLIT == 1, "one 32-query block per step, all d tiles in each wave");
  using S = ShortStage<C>;
  __shared__ __attribute__((aligned(16))) char smem[S::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  LaneCtx lc;
  lc.lane = tid & 63;
  lc.h = lc.lane >> 5;
  lc.c16 = lc.lane & 15;
  lc.g = lc.lane >> 4;
  const int c32 = lc.lane & 31;

  // workgroup -> (frame, split, head), head fastest; ids dealt round-robin to
  // the 8 XCDs are remapped so that each XCD takes a contiguous range: all
  // heads of the same query rows then meet in one L2, which merges their
  // column slices of each Q and O line.
  const int total = p.H * p.F * nsplit;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int hd = lid % p.H;
  const int fs = lid / p.H;
  const int f = fs / nsplit;
  const int split = fs - f * nsplit;

  if constexpr (C::ONES) {  // the constant plane of the one K tile and the one V tile
    for (int i = tid >> 6; i < 2; i += C::W) {
      h8 one = {0, 0, 0, 0, 0, 0, 0, 0};
      one[0] = (_Float16)1.0f;
      *reinterpret_cast<h8*>(smem + i * C::TILEB + C::CPR * C::PLB + 16 * lc.lane) = one;
    }
  }
  lane_offsets<C>(lc);
#ifdef PL_DEBUG_BOUNDS
  lc.lds_bytes = S::LDS;
#endif

  // the whole key sequence is one (possibly ragged) tile
  Copier<C> cp;
#ifdef PL_DEBUG_BOUNDS
  cp.lds_end = lds_addr(smem) + (unsigned)S::LDS;
#endif
  cp.s = 0;
  cp.off = 0;
  cp.issued = 0;
  issue_tile<C>(p, smem, cp, f, hd, wave, lc.lane);
  const int valid = (int)min((int64_t)C::BN, p.seg[0].len);

  // this wave's query blocks: split s takes every nsplit-th group of W blocks
  const int nblk = (p.Lq + 31) / 32;
  const _Float16* qb_ = p.q + (int64_t)f * p.q_fs + (int64_t)hd * C::D;
  _Float16* ob = p.o + (int64_t)f * p.o_fs + (int64_t)hd * C::D;
  const int step = nsplit * C::W;
  char* qs = smem + C::BUFB + wave * 2 * S::QB;  // this wave's two block buffers
  const int qrow = lc.lane / S::CPRQ, qchunk = lc.lane % S::CPRQ;
  // copy Q rows 32 blk .. 32 blk + 31 into buffer b (rows past Lq re-read the
  // last row: their results are never stored)
  auto q_issue = [&](int blk, int b) {
    const char* src = reinterpret_cast<const char*>(qb_ + (int64_t)(32 * blk) * p.q_ld);
    const unsigned dst = lds_addr(qs + b * S::QB);
    const int last = p.Lq - 1 - 32 * blk;
#pragma unroll
    for (int j = 0; j < S::NQI; ++j) {
      const int r = j * S::RPI + qrow;
      const unsigned voff = (unsigned)(min(r, last) * p.q_ld * 2 + 16 * qchunk);
      const unsigned d = dst + j * S::RPI * S::CPRQ * 16;
      if (lc.lane < S::RPI * S::CPRQ && r < 32 &&
          PL_BOUNDS(PL_IN((int64_t)f * p.q_fs + (int64_t)hd * C::D + (int64_t)(32 * blk) * p.q_ld + voff / 2, 8, p.q_ext),
                    kSiteShortQSrc) &&
          PL_BOUNDS(d + 16u * (unsigned)(S::RPI * S::CPRQ) <= cp.lds_end, kSiteShortQDst))
        lds_dma16(d, voff, src);
    }
  };

  int blk = split * C::W + wave;
  if (blk < nblk) q_issue(blk, 0);
  wait_vm(0);
  __syncthreads();  // the K/V tile (and the constant plane) and the first Q block are in LDS

  WaveState<C> ws;
  ws.dt0 = 0;
  if constexpr (C::RSUM) {  // A of the row-sum products: row 0 (lanes with l % 16 == 0) all ones
    const _Float16 a1 = lc.c16 == 0 ? (_Float16)1.0f : (_Float16)0.0f;
    ws.onesA = (h8){a1, a1, a1, a1, a1, a1, a1, a1};
  }
  for (int b = 0; blk < nblk; blk += step, b ^= 1) {
    const bool next = blk + step < nblk;
    if (next) q_issue(blk + step, b ^ 1);  // that buffer's O was read out in the previous block
    // Q of this block has landed (loads complete in order; what may still be
    // outstanding is the previous block's stores and the copies just issued)
    if (next)
      wait_vm(S::NQI);
    else
      wait_vm(0);
    char* buf = qs + b * S::QB;
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      const int col = 16 * st + 8 * lc.h;
      h8 x = {0, 0, 0, 0, 0, 0, 0, 0};
      if (col < C::D && PL_BOUNDS(PL_IN((buf - smem) + c32 * (2 * C::D) + 2 * col, 16, S::LDS), kSiteShortBuf))
        x = *reinterpret_cast<const h8*>(buf + c32 * (2 * C::D) + 2 * col);
#pragma unroll
      for (int e = 0; e < 8; ++e) ws.qf[0][st][e] = (_Float16)((float)x[e] * p.c2);
    }
    ws.mrun[0] = 0.f;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
#pragma unroll
      for (int t = 0; t < C::NDW; ++t) ws.oacc[0][grp][t] = (f4){0.f, 0.f, 0.f, 0.f};
      if constexpr (C::RSUM) ws.osum[0][grp] = (f4){0.f, 0.f, 0.f, 0.f};
    }
    tile_step<C, false>(smem, 0, valid, true, ws, lc);

    // normalise, round to fp16 (nearest even) into the block buffer
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      float l;
      if constexpr (C::ONES) {
        constexpr int tl = C::D / 16, gl = (C::D % 16) / 4, rl = C::D % 4;
        l = __shfl(ws.oacc[0][grp][tl][rl], 16 * gl + lc.c16, 64);
      } else {
        l = __shfl(ws.osum[0][grp][0], lc.c16, 64);  // row 0: lanes 0..15
      }
      const float inv = 1.0f / l;
      const int row = 16 * grp + lc.c16;
#pragma unroll
      for (int t = 0; t < C::NDW; ++t) {
        const int col = 16 * t + 4 * lc.g;
        if (col < C::D && PL_BOUNDS(PL_IN((buf - smem) + row * (2 * C::D) + 2 * col, 8, S::LDS), kSiteShortBuf)) {
          h4 out;
#pragma unroll
          for (int r = 0; r < 4; ++r) out[r] = (_Float16)(ws.oacc[0][grp][t][r] * inv);
          *reinterpret_cast<h4*>(buf + row * (2 * C::D) + 2 * col) = out;
        }
      }
    }
    // O rows out, whole row slices per lane group
#pragma unroll
    for (int j = 0; j < S::NQI; ++j) {
      const int r = j * S::RPI + qrow;
      if (lc.lane < S::RPI * S::CPRQ && r < 32 && 32 * blk + r < p.Lq &&
          PL_BOUNDS(PL_IN((buf - smem) + r * (2 * C::D) + 16 * qchunk, 16, S::LDS), kSiteShortBuf) &&
          PL_BOUNDS(PL_IN((int64_t)f * p.o_fs + (int64_t)hd * C::D + (int64_t)(32 * blk + r) * p.o_ld + 8 * qchunk, 8,
                          p.o_ext),
                    kSiteShortO))
        *reinterpret_cast<h8*>(ob + (int64_t)(32 * blk + r) * p.o_ld + 8 * qchunk) =
            *reinterpret_cast<const h8*>(buf + r * (2 * C::D) + 16 * qchunk);
    }
  }
}

template <int D, int MINB>
hipError_t launch_short(const KParams& kp, hipStream_t stream) {
  using C = Cfg<D, 1, 2, 2, MINB, false, 4>;
  KParams p = kp;
  // 32-bit per-lane copy offsets: a key tile and a 32-row Q block
  if (p.seg[0].ld * 2 * C::BN > 0x7fffffffLL || p.q_ld * 2 * 32 > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t base = (int64_t)p.F * p.H;
  // about four workgroups per CU in total, each wave walking one or more blocks
  const int nblk = (p.Lq + 31) / 32;
  int nsplit = (int)std::max<int64_t>(1, (int64_t)PL_SHORT_WGS / std::max<int64_t>(base, 1));
  nsplit = std::min(nsplit, std::max(1, nblk / C::W));
  if (base * nsplit > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(short_ctx_kernel<C>, dim3((unsigned)(base * nsplit)), dim3(C::THREADS), 0, stream, p, nsplit);
  return hipGetLastError();
}

// Merge the key splits of every query row: with M the largest split offset,
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, rounded to fp16.  One
// thread per 4 output columns, columns fastest, so partial reads and output
// stores are contiguous.
template <int D>
__global__ void __launch_bounds__(256) split_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml, _Float16* o,
                                                            int64_t o_ld, int64_t o_fs, int F, int H, int Lq,
                                                            int nsplit, [[maybe_unused]] int64_t o_ext) {
  constexpr int Q = D / 4;
  const int64_t total = (int64_t)F * H * Lq * Q;
  [[maybe_unused]] const int64_t parts = (int64_t)F * H * nsplit * Lq;  // rows of partials
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int qd = (int)(i % Q);
    int64_t rest = i / Q;
    const int row = (int)(rest % Lq);
    rest /= Lq;
    const int hd = (int)(rest % H);
    const int f = (int)(rest / H);
    const int64_t pb = (int64_t)(f * H + hd) * nsplit * Lq + row;  // split s at pb + s * Lq
    if (!PL_BOUNDS(PL_IN(pb, 1, parts) && PL_IN(pb + (int64_t)(nsplit - 1) * Lq, 1, parts), kSiteCombineIn)) continue;
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, part_ml[(pb + (int64_t)sp * Lq) * 2]);
    float L = 0.f;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < nsplit; ++sp) {
      const int64_t r = pb + (int64_t)sp * Lq;
      const float w = __builtin_amdgcn_exp2f(part_ml[r * 2] - M);
      L = fmaf(w, part_ml[r * 2 + 1], L);
      const f4 x = *reinterpret_cast<const f4*>(part_o + r * D + 4 * qd);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(w, x[k], acc[k]);
    }
    const float inv = 1.0f / L;
    h4 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = (_Float16)(acc[k] * inv);
    if (PL_BOUNDS(PL_IN((int64_t)f * o_fs + (int64_t)row * o_ld + (int64_t)hd * D + 4 * qd, 4, o_ext), kSiteCombineOut))
      *reinterpret_cast<h4*>(o + (int64_t)f * o_fs + (int64_t)row * o_ld + (int64_t)hd * D + 4 * qd) = out;
  }
}

// Workgroups of one launch: query tiles x frames x heads (x key splits).
template <class C>
int64_t attn_workgroups(int F, int Lq, int H) {
  return (int64_t)((Lq + C::QWG - 1) / C::QWG) * F * H;
}

#ifndef PL_SPLIT_TARGET_WGS
#define PL_SPLIT_TARGET_WGS 256  // d = 160 workgroups the GPU holds at once (one per CU: LDS)
#endif

// How many key splits a launch takes (and the tiles per split): only for the
// head dim whose workgroups take a whole CU each (d = 160, the 16^2 and 8^2
// levels: a 127.5 KB copy ring, one wave per SIMD), and only as far as the
// launch leaves CUs idle -- more workgroups than CUs would run in a second
// generation and lose what the split gains.  Within that, the count follows a
// cost model fitted to one-frame and 16-frame launches of both levels: a
// workgroup spends about 1.3 us per key tile, and each split adds a round
// trip of F*H*Lq*(d+2)*4 bytes of partials (written, then merged) at about
// 1.5 TB/s, so n splits of T tiles take about 1.3 T/n + c n us, least at
// n = sqrt(1.3 T / c).  (Measured, d = 160 with the 4x bank: one frame at
// 16^2, 20 tiles: 5 splits 24.2 us, 10 splits 26.0, 2 splits 31.5, one pass
// 46.2; one frame at 8^2, 5 tiles: 5 splits 13.7 us, 2 splits 15.4, one pass
// 15.7; 16 frames at 8^2: 2 splits 21.5 us against 16.3 in one pass, where the
// model's optimum is 1.4, so no split.)
template <class C>
void split_plan(int F, int Lq, int H, const int64_t* seg_len, int nseg, int& nsplit, int& tps) {
  int ntiles = 0;
  for (int s = 0; s < nseg; ++s) ntiles += (int)((seg_len[s] + C::BN - 1) / C::BN);
  nsplit = 1;
  tps = 1 << 30;
  if (C::D != 160 || ntiles < 2) return;
  const int64_t wgs = attn_workgroups<C>(F, Lq, H);
  if (2 * wgs > PL_SPLIT_TARGET_WGS) return;
  const double tile_us = 1.3, partial_us = (double)F * H * Lq * (C::D + 2) * 4 / 1.5e6;
  int64_t want = std::llround(std::sqrt(tile_us * ntiles / partial_us));
  want = std::min<int64_t>(std::min<int64_t>(want, ntiles), PL_SPLIT_TARGET_WGS / wgs);
  if (want < 2) return;
  tps = (int)((ntiles + want - 1) / want);
  nsplit = (ntiles + tps - 1) / tps;
  if (nsplit < 2) {
    nsplit = 1;
    tps = 1 << 30;
  }
}

template <int D, int NQB, int NKB, int NBUF, int MINB, bool PIPE, int W, int DSPLIT = 1>
hipError_t launch_cfg(const KParams& kp, hipStream_t stream, float* workspace) {
  using C = Cfg<D, NQB, NKB, NBUF, MINB, PIPE, W, DSPLIT>;
  KParams p = kp;
  for (int i = 0; i < p.nseg; ++i)
    if (p.seg[i].ld * 2 * C::BN > 0x7fffffffLL) return hipErrorInvalidValue;  // 32-bit copy offsets
  p.nqt = (p.Lq + C::QWG - 1) / C::QWG;
  p.nsplit = 1;
  p.tps = 1 << 30;
  p.part_o = p.part_ml = nullptr;
  if (workspace) {
    int64_t lens[PL_MAX_SEGMENTS];
    for (int i = 0; i < p.nseg; ++i) lens[i] = p.seg[i].len;
    split_plan<C>(p.F, p.Lq, p.H, lens, p.nseg, p.nsplit, p.tps);
    if (p.nsplit > 1) {
      p.part_o = workspace;
      p.part_ml = workspace + (int64_t)p.F * p.H * p.nsplit * p.Lq * D;
#ifdef PL_DEBUG_BOUNDS
      p.part_ext = (int64_t)p.F * p.H * p.nsplit * p.Lq * D;
#endif
    }
  }
  const int64_t blocks = (int64_t)p.nqt * p.F * p.H * p.nsplit;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(refbank_attn_kernel<C>, dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, p);
  if (p.nsplit == 1) return hipGetLastError();
  if (hipError_t e = hipGetLastError()) return e;
  const int64_t items = (int64_t)p.F * p.H * p.Lq * (D / 4);
  const int64_t cblocks = std::min<int64_t>((items + 255) / 256, 4096);
#ifdef PL_DEBUG_BOUNDS
  const int64_t o_ext = p.o_ext;
#else
  const int64_t o_ext = 0;
#endif
  hipLaunchKernelGGL(split_combine_kernel<D>, dim3((unsigned)cblocks), dim3(256), 0, stream, p.part_o, p.part_ml,
                     p.o, p.o_ld, p.o_fs, p.F, p.H, p.Lq, p.nsplit, o_ext);
  return hipGetLastError();
}

// d = 80: query blocks per wave, key blocks per tile, ring buffers, workgroups
// per CU, pipelined fast tiles, waves per workgroup
#ifndef PL_D80_CFG
#define PL_D80_CFG 1, 2, 4, 1, true, 8
#endif

// d = 160 configurations: 4 waves of 32 query rows; for frames of at most 64
// rows, 2 query blocks with 2 waves each, each wave holding half of O^T's d
// tiles (one wave per SIMD either way: the split halves each wave's PV chain,
// 20.3 -> 16.4 us at the 8^2 level; at 16^2, where 8 such waves would share the
// SIMDs two by two, the repeated S^T work costs more: 54.5 -> 62.5 us)
using Cfg160 = Cfg<160, 1, 2, 3, 1, false, 4>;
using Cfg160s = Cfg<160, 1, 2, 3, 1, false, 4, 2>;

}  // namespace

size_t refbank_attn_workspace_bytes(int32_t F, int32_t Lq, int32_t H, int32_t d, const int64_t* seg_len,
                                    int32_t nseg) {
  if (d != 160 || (nseg == 1 && seg_len[0] <= 64)) return 0;  // no split for the other kernels
  int nsplit, tps;
  if (Lq <= 64)
    split_plan<Cfg160s>(F, Lq, H, seg_len, nseg, nsplit, tps);
  else
    split_plan<Cfg160>(F, Lq, H, seg_len, nseg, nsplit, tps);
  if (nsplit < 2) return 0;
  return (size_t)F * H * nsplit * Lq * (d + 2) * sizeof(float);
}

hipError_t debug_bounds_mask(unsigned long long* mask, bool reset) {
#ifdef PL_DEBUG_BOUNDS
  hipError_t e = hipMemcpyFromSymbol(mask, HIP_SYMBOL(g_bounds_mask), sizeof(*mask));
  if (e != hipSuccess || !reset) return e;
  const unsigned long long zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_bounds_mask), &zero, sizeof(zero));
#else
  (void)reset;
  *mask = 0;
  return hipErrorNotSupported;
#endif
}

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
  p.nsplit = 1;
  p.tps = 1 << 30;
  p.part_o = p.part_ml = nullptr;
#ifdef PL_DEBUG_BOUNDS
  {
    const int64_t width = (int64_t)a.H * a.d;
    p.q_ext = (int64_t)(a.F - 1) * a.q_frame_stride + (int64_t)(a.Lq - 1) * a.q_ld + width;
    p.o_ext = (int64_t)(a.F - 1) * a.o_frame_stride + (int64_t)(a.Lq - 1) * a.o_ld + width;
    for (int i = 0; i < PL_MAX_SEGMENTS; ++i)
      p.seg_ext[i] = i < a.nseg ? (int64_t)(a.F - 1) * a.seg[i].frame_stride + (a.seg[i].len - 1) * a.seg[i].ld + width
                                : 0;
    p.part_ext = 0;
  }
#endif
  float* ws = static_cast<float*>(a.workspace);
  // a single segment of at most one tile: the short-context kernel
  if (a.nseg == 1 && a.seg[0].len <= 64) {
    p.nqt = 0;
    switch (a.d) {
      case 32: return launch_short<32, 4>(p, stream);
      case 40: return launch_short<40, 3>(p, stream);
      case 80: return launch_short<80, 2>(p, stream);
      case 160: return launch_short<160, 1>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.d) {
    case 32: return launch_cfg<32, 2, 2, 4, 2, true, 4>(p, stream, nullptr);
    case 40: return launch_cfg<40, 2, 2, 4, 2, true, 4>(p, stream, nullptr);
    case 80: return launch_cfg<80, PL_D80_CFG>(p, stream, nullptr);
    case 160:
      if (a.Lq <= 64) return launch_cfg<160, 1, 2, 3, 1, false, 4, 2>(p, stream, ws);
      return launch_cfg<160, 1, 2, 3, 1, false, 4>(p, stream, ws);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pl
