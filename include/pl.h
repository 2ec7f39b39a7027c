/*
 * pl.h -- C ABI of the MI355X (gfx950) hot path of the PersonaLive streaming
 * pyramid denoiser: reference-bank spatial self-attention, the per-window
 * DDIM step of the latents pile, the motion-bank drift check, and the pile's
 * integer state machine.
 *
 * Sources are cited by page and section: "PersonaLive" is the PersonaLive
 * write-up on juhe.plus (sections 它解决什么 / specification, 流式金字塔去噪 /
 * streaming pyramid denoising, 首帧怎么办 / first frames, 抗身份漂移的补丁 /
 * anti identity-drift patch, 三条条件通路 / three conditioning paths,
 * TensorRT 融合 / TensorRT fusion).
 *
 * Conventions shared by every call
 *   - Device pointers are HIP device addresses on the current device; host
 *     pointers are ordinary process memory read before the call returns.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises device memory.
 *   - `stream` is a hipStream_t passed as `void*` (NULL = the default stream).
 *     Work is enqueued on it and the call returns without waiting.
 *   - Every argument is validated before anything is launched: a call that
 *     returns an error has written nothing.  Errors are status codes; the
 *     calling thread's pl_last_error() holds a one-line explanation.  No C++
 *     exception crosses the ABI.  All calls are reentrant.
 */
#ifndef PL_H_
#define PL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pl_status;
typedef struct pl_pile pl_pile;  /* the latents pile's state machine (defined below) */
#define PL_OK 0            /* success */
#define PL_EINVAL 1        /* invalid argument (null pointer, size or index out of range) */
#define PL_EUNSUPPORTED 2  /* valid in principle but not implemented (head dim, alignment) */
#define PL_EDEVICE 3       /* the HIP runtime reported an error at launch */

#define PL_ABI_VERSION 5
#define PL_MAX_SEGMENTS 8       /* key segments per attention call: self + reference + anchors (5 used) */
#define PL_MAX_WINDOWS 8        /* windows per pile (the pages use 4) */
#define PL_MAX_MOTION_BANK 4    /* reference embedding + at most 3 anchors */

/* ABI version of the loaded library (PL_ABI_VERSION at build time). */
int32_t pl_abi_version(void);

/* Static name of a status code ("PL_OK", ...); "PL_UNKNOWN" otherwise. */
const char* pl_status_string(pl_status s);

/* Thread-local text describing the calling thread's most recent failure, or
 * "" if its last call succeeded.  Valid until that thread's next pl_* call. */
const char* pl_last_error(void);

/* ------------------------------------------------------------------------ *
 * Reference-bank spatial self-attention (one transformer layer)
 *
 * PersonaLive, section 三条条件通路: the Reference UNet writes each layer's
 * features into a bank once per stream; the denoiser concatenates the layer's
 * bank features with its own keys/values and runs spatial self-attention.
 * Section 抗身份漂移的补丁: each drift anchor appends one more entry per
 * layer; section TensorRT 融合 bounds the bank at 4x the reference length.
 *
 * For every frame f < F and head h < H, with rows r < Lq:
 *   O[f, r, h*d:(h+1)*d] = softmax_j( scale * Q[f, r, h] . K_cat[f, j, h] ) V_cat[f, j, h]
 * where the key axis j runs over the segments in order (the result does not
 * depend on that order).  No mask, bias or dropout.
 *
 * Data: fp16 (IEEE binary16) everywhere; products are accumulated in fp32,
 * the softmax is evaluated in fp32 and O is rounded to nearest even.
 * Layout: token-major.  Row r of frame f of a tensor X starts at
 *   X + f * frame_stride + r * ld      (elements, not bytes)
 * and head h occupies that row's elements [h*d, (h+1)*d).  This is the
 * layout the q/k/v projections produce, so no transposes are needed.
 * ------------------------------------------------------------------------ */

/* One source of keys/values.  The segments of a call are a virtual
 * concatenation: nothing is copied. */
typedef struct pl_kv_segment {
  const void* k;         /* device fp16; row r of frame f at k + f*frame_stride + r*ld */
  const void* v;         /* device fp16; same indexing as k */
  int64_t len;           /* keys in this segment (>= 1) */
  int64_t ld;            /* row stride in elements (>= H*d, multiple of 8) */
  int64_t frame_stride;  /* elements between frames; 0 = shared by all frames (bank entries) */
} pl_kv_segment;

/* Bytes of device workspace pl_refbank_attn needs for these sizes.
 * The current kernels need none and return 0; callers should still query it. */
size_t pl_refbank_attn_workspace_size(int32_t F, int32_t Lq, int32_t H, int32_t d,
                                      const int64_t* seg_len, int32_t nseg);

/* Launch one reference-bank attention layer.
 *   q, o          device fp16 [F][Lq][ld]; o must not overlap q or any K/V
 *                 (checked: PL_EINVAL when o's address range meets that of q or
 *                 of a segment's k or v, unless the two share a row stride, the
 *                 frame strides are whole rows, and their column ranges within
 *                 a row are disjoint -- column slices of one fused buffer).
 *   q_ld, o_ld    row strides in elements (>= H*d, multiple of 8).
 *   *_frame_stride  elements between frames (>= Lq*ld is not required, but
 *                 rows of different frames must not overlap in o).
 *   F, Lq, H      frames (>= 1), query rows per frame (>= 1), heads (>= 1).
 *   d             head dimension: 32, 40, 80 or 160 (else PL_EUNSUPPORTED).
 *   segs, nseg    host array of 1..PL_MAX_SEGMENTS segments, total keys <= 2^24.
 *   scale         logit scale, > 0 (usually 1/sqrt(d)).
 *   workspace     device memory of workspace_bytes >= the size above (may be
 *                 NULL when that size is 0).
 * All device pointers must be 16-byte aligned (PL_EUNSUPPORTED otherwise). */
pl_status pl_refbank_attn(const void* q, int64_t q_ld, int64_t q_frame_stride,
                          void* o, int64_t o_ld, int64_t o_frame_stride,
                          int32_t F, int32_t Lq, int32_t H, int32_t d,
                          const pl_kv_segment* segs, int32_t nseg, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Block-causal attention over chunked sequences (several chunks' queries in
 * one call).  LPM write-up, section 6.3 分块因果注意力, and the deep-compression-
 * VAE write-up: a sequence is cut into non-overlapping chunks; a token attends
 * to its own chunk and to earlier chunks (a limited number of them), never to
 * a later one, and to the persistent reference tokens.
 * For each frame, query row r belongs to chunk r / chunk_len.  Segment
 * causal_seg holds the sequence's own keys and values, row j in chunk
 * j / chunk_len (its len must equal Lq); row r sees its row j only if
 * chunk(j) <= chunk(r) and chunk(r) - chunk(j) <= max_history (negative:
 * unlimited).  Every other segment (reference tokens, sinks) is visible to
 * every row.  Other arguments as pl_refbank_attn (single-pass kernels, no
 * workspace).  The call checks every chunk's views before launching, then
 * issues one launch per chunk over that chunk's rows and visible key range:
 * nothing is copied.  PL_EINVAL additionally for causal_seg out of range,
 * chunk_len < 1, a causal segment whose len is not Lq, or more than 65536
 * chunks. */
pl_status pl_refbank_attn_chunked(const void* q, int64_t q_ld, int64_t q_frame_stride,
                                  void* o, int64_t o_ld, int64_t o_frame_stride,
                                  int32_t F, int32_t Lq, int32_t H, int32_t d,
                                  const pl_kv_segment* segs, int32_t nseg, int32_t causal_seg,
                                  int32_t chunk_len, int32_t max_history, float scale, void* stream);

/* pl_refbank_attn without a caller workspace, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, layout, results and
 * errors as pl_refbank_attn, without workspace / workspace_bytes: the launches
 * that split the key axis put their partials in a scratch array the library
 * holds on each GPU (16 MiB, kept until the process ends; its address is
 * looked up once per device, with that device current, on the first call
 * there).  Nothing is allocated, freed or cleared by a call.
 * PL_EINVAL if the split of these sizes needs more than 16 MiB of scratch
 * (pl_refbank_attn_workspace_size reports what it needs); PL_EDEVICE if the
 * scratch's address cannot be obtained.  Every call on one GPU shares that
 * scratch and leaves its own partials there: calls that overlap in time on
 * one GPU (concurrent streams, or threads) race and must not be issued. */
pl_status pl_refbank_attn_noalloc(const void* q, int64_t q_ld, int64_t q_frame_stride,
                                  void* o, int64_t o_ld, int64_t o_frame_stride,
                                  int32_t F, int32_t Lq, int32_t H, int32_t d,
                                  const pl_kv_segment* segs, int32_t nseg, float scale, void* stream);

/* Bounds report of a checking build: for whoever changes the attention
 * kernels' indexing (no page defines it).  A library built with
 * PL_DEBUG_BOUNDS checks every global and LDS access of the attention kernels
 * (pl_refbank_attn and its variants, the short-context and key-split paths)
 * against the extent of the buffer it belongs to before making it; a failed
 * check sets one bit of a device-wide mask and the access is skipped.  Bits:
 * 0 K/V copy source, 1 K/V copy destination (LDS), 2 Q load, 3 O store,
 * 4 and 5 key-split partials, 6 and 7 K and V^T operand reads (LDS),
 * 8 to 11 short context (Q copy source and destination, O store, block
 * buffer), 12 and 13 key-split merge (partials read, O store).
 *   mask   out: the bits set since the last reset (0: every access stayed in
 *          its buffer).
 *   reset  non-zero: clear the mask after reading it.
 * Synchronises the current device (blocking copies of the mask).  Builds
 * without the checks write 0 and return PL_EUNSUPPORTED; PL_EINVAL if mask
 * is NULL; PL_EDEVICE on a HIP error. */
pl_status pl_debug_bounds(uint64_t* mask, int32_t reset);

/* ------------------------------------------------------------------------ *
 * Projections either side of the attention
 *
 * PersonaLive, section 三条条件通路: the bank stores each reference layer's
 * hidden states and the denoiser attends to them next to its own keys and
 * values, so the bank's keys and values are that layer's linear projections
 * of them (projecting each entry once, when it is written, gives the same
 * keys as projecting the joined sequence: a projection acts on each token
 * separately).  The denoiser's to_q / to_k / to_v / to_out are linear layers
 * of the same kind.
 *
 *   y[m][n] = sum_k x[m][k] * w[n][k] (+ bias[n]), fp16 in and out, fp32
 *   accumulation, output rounded to nearest even.
 *   x     device fp16 [M][x_ld], x_ld >= K, multiple of 8, 16-byte aligned.
 *   w     device fp16 [N][w_ld] (out features x in features, as linear layers
 *         store it), w_ld >= K, multiple of 8, 16-byte aligned.  A fused
 *         q/k/v weight [3C][C] gives y = [q | k | v], whose column slices are
 *         valid pl_refbank_attn operands (row stride 3C).
 *   bias  device fp32 [N], 16-byte aligned, or NULL.
 *   y     device fp16 [M][y_ld], y_ld >= N, multiple of 4, 8-byte aligned; must
 *         not overlap x or w.
 *   M in 1..2^31; N a multiple of 64; K a multiple of 16 (PL_EUNSUPPORTED
 *   otherwise).
 * ------------------------------------------------------------------------ */
pl_status pl_linear(const void* x, int64_t x_ld, const void* w, int64_t w_ld, const float* bias, void* y,
                    int64_t y_ld, int64_t M, int32_t N, int32_t K, void* stream);

/* ------------------------------------------------------------------------ *
 * Per-window DDIM step of the latents pile
 *
 * PersonaLive, section 它解决什么: DDIM, epsilon prediction, 4 steps.
 * Section 流式金字塔去噪: the pile holds W windows at their own timesteps
 * (999 / 666 / 333 / 0 with a step length of 333); one forward gives every
 * window its epsilon estimate and each window steps from t to t - step_len;
 * the window leaving the queue hands pred_original_sample (the x0 estimate)
 * to the VAE instead of its last sample.
 *
 * For window w with a = alpha_bar[t_w] and a' = alpha_bar[t_w - step_len]
 * (a' = final_alpha_cumprod when t_w - step_len < 0), eta = 0, no clipping:
 *   x0     = (x_t - sqrt(1 - a) * eps) / sqrt(a)
 *   x_prev = sqrt(a') * x0 + sqrt(1 - a') * eps
 * The host folds these into per-window coefficients in fp64; the kernel
 * applies them in fp32 in one pass over x_t and eps.
 *
 *   x_t, eps      device fp32 [W][elems_per_window], window-major.
 *   x_prev        device fp32, same shape; may alias x_t (in-place update).
 *   x0_out        device fp32 [elems_per_window]: x0 of window emit_window.
 *                 Required when emit_window >= 0, ignored when it is -1.
 *   W             1..PL_MAX_WINDOWS; elems_per_window >= 1.
 *   t_host        host int32 [W], each in [0, T).
 *   step_len      >= 1 (333 on the pages).
 *   alphas_cumprod_host  host fp64 [T] with values in (0, 1], or NULL for
 *                 Stable Diffusion's scaled_linear schedule (betas from
 *                 0.00085 to 0.012 in sqrt space, T must be 1000).
 *   final_alpha_cumprod  a' used when t - step_len < 0; pass a negative
 *                 value to use alpha_bar[0]; otherwise must lie in (0, 1].
 *   emit_window   -1 or the index of the window whose x0 is written.
 * No alignment requirement (16-byte aligned buffers take the vector path). */
pl_status pl_pyramid_ddim_step(const float* x_t, const float* eps, float* x_prev, float* x0_out,
                               int32_t W, int64_t elems_per_window,
                               const int32_t* t_host, int32_t step_len,
                               const double* alphas_cumprod_host, int32_t T,
                               double final_alpha_cumprod, int32_t emit_window, void* stream);

/* Same step, and the pile rolls on the device: when emit_window >= 0 the
 * leaving window's slot of x_prev receives the next round's new window --
 * pure N(0, 1) noise, pl_window_noise(seed, new_window_id) -- instead of its
 * own x_prev, which the pile discards anyway (that window is popped after
 * this step).  PersonaLive, section 流式金字塔去噪: each round a new window of
 * noise enters at the top timestep; the TensorRT section's bind() keeps the
 * rolling latents on the device between rounds, the new window arriving as
 * the new_noise input.  Writing it here costs no extra memory traffic: those
 * bytes are written by the step anyway.  With x_prev aliasing x_t the pile
 * is ready for the next round (pl_pile_begin_round returns that slot as the
 * new window's slot).  Other arguments and errors: as pl_pyramid_ddim_step. */
pl_status pl_pyramid_ddim_step_roll(const float* x_t, const float* eps, float* x_prev, float* x0_out,
                                    int32_t W, int64_t elems_per_window,
                                    const int32_t* t_host, int32_t step_len,
                                    const double* alphas_cumprod_host, int32_t T,
                                    double final_alpha_cumprod, int32_t emit_window,
                                    uint64_t seed, uint64_t new_window_id, void* stream);

/* ------------------------------------------------------------------------ *
 * The round with its state on the device (one captured graph per stream)
 *
 * PersonaLive, section TensorRT 融合: bind() keeps the rolling latents and
 * the pile's bookkeeping on the device so that a whole round is one host
 * call.  Here the pile's integer state (a pl_pile, initialised with
 * pl_pile_init and copied to device memory by the caller) is read and
 * advanced by the kernels themselves, so the launches of a round take the
 * same arguments every round and can be captured once in a HIP graph and
 * replayed.
 * ------------------------------------------------------------------------ */

/* Host: write Stable Diffusion's scaled_linear alpha_bar table (betas from
 * 0.00085 to 0.012 in sqrt space, fp64) into out[0..T-1]; T must be 1000.
 * (The caller copies it to the device for pl_pyramid_ddim_step_device.) */
pl_status pl_sd_alphas_cumprod(double* out, int32_t T);

/* One round of the pile's device-side roll, driven by the device state:
 *   1. the new window enters (as pl_pile_begin_round would place it: id
 *      next_id, slot (head + count) % W, t = t_top);
 *   2. the DDIM step of pl_pyramid_ddim_step_roll with each slot's timestep,
 *      the leaving slot (the window at t = 0, if any) and the next window's
 *      id (its noise, pl_window_noise(seed, id), fills the leaving slot of
 *      x_prev) all read from the state; the coefficients are computed in
 *      fp64 on the device from alphas_cumprod and rounded to fp32;
 *   3. the state advances as pl_pile_end_round would leave it.
 * Two kernel launches, no host synchronisation, no allocation and no memset.
 *   x_t, eps, x_prev  device fp32 [W][elems_per_window] (x_prev may alias x_t),
 *                 16-byte aligned; elems_per_window a multiple of 4.
 *   x0_out        device fp32 [elems_per_window], 16-byte aligned: written in
 *                 the rounds in which a window leaves.
 *   W             2..PL_MAX_WINDOWS, equal to the W of the state.
 *   pile          device pl_pile, 8-byte aligned, initialised by pl_pile_init
 *                 (no round open); values read from it are clamped into range,
 *                 so a corrupted state gives wrong results but no access out
 *                 of bounds.
 *   alphas_cumprod  device fp64 [T] (e.g. pl_sd_alphas_cumprod), 8-byte aligned.
 *   final_alpha_cumprod  as pl_pyramid_ddim_step (negative: alphas_cumprod[0]).
 * Errors: PL_EINVAL for null pointers or sizes out of range, PL_EUNSUPPORTED
 * for misaligned buffers; nothing is launched then. */
pl_status pl_pyramid_ddim_step_device(const float* x_t, const float* eps, float* x_prev, float* x0_out,
                                      int32_t W, int64_t elems_per_window, pl_pile* pile,
                                      const double* alphas_cumprod, int32_t T, double final_alpha_cumprod,
                                      uint64_t seed, void* stream);

/* ------------------------------------------------------------------------ *
 * Window noise, staircase prefill, first-frames interpolation
 *
 * PersonaLive, section 流式金字塔去噪: windows of pure noise enter the pile;
 * section 首帧怎么办: the queue starts with three windows (12 frames) of
 * staircase noise, and the first frames' pose / expression inputs are 12 + 1
 * linearly interpolated points from the reference's to the first driving
 * frame's, the last point dropped.  The pages do not say how noise is drawn;
 * here it is a pure function of (seed, window id, element):
 *
 *   Philox-4x64-10 (Salmon et al., "Parallel random numbers: as easy as 1,
 *   2, 3", SC 2011) with key (seed, window id) and counter (i / 4, 0, 0, 0)
 *   gives four 64-bit words for elements 4(i/4) .. 4(i/4)+3; word x maps to
 *   u = ((x >> 40) + 1) / 2^24 in (0, 1]; words (0, 1) and (2, 3) give two
 *   normals each, r cos(2 pi u_odd) and r sin(2 pi u_odd) with
 *   r = sqrt(-2 ln u_even) (Box-Muller), computed in fp32.
 * ------------------------------------------------------------------------ */

/* out: device fp32 [n], n in 1..2^40, any alignment. */
pl_status pl_window_noise(float* out, int64_t n, uint64_t seed, uint64_t window_id, void* stream);

/* Staircase prefill: slot w of the pile (w < n_windows) holds the window at
 * t = w * step_len: sqrt(a) * ref + sqrt(1 - a) * noise(seed, w), with
 * a = alpha_bar[t] from the table (NULL: SD scaled_linear, T = 1000) and
 * window ids 0 .. n_windows-1 (as pl_pile_init with prefill numbers them).
 * Reading: the pages say "staircase noise" and the reference image; what
 * exactly is noised is not stated -- here the reference latent.
 *   ref   device fp32 [elems_per_window] (e.g. the reference frame's latent
 *         tiled over the window's frames); must not overlap the pile.
 *   pile  device fp32 [n_windows][elems_per_window].
 *   n_windows in 1..PL_MAX_WINDOWS with (n_windows-1)*step_len < T. */
pl_status pl_pile_prefill(const float* ref, float* pile, int32_t n_windows, int64_t elems_per_window,
                          int32_t step_len, const double* alphas_cumprod_host, int32_t T, uint64_t seed,
                          void* stream);

/* out[k][i] = a[i] + (b[i] - a[i]) * k / n for k = 0 .. n-1 (n + 1 evenly
 * spaced points from a to b, the last one, b, dropped), fp32.
 *   a, b  device fp32 [D]; out device fp32 [n][D], not overlapping a or b.
 *   D in 1..2^40, n in 1..65535 (12 on the pages). */
pl_status pl_lerp_points(const float* a, const float* b, int64_t D, int32_t n, float* out, void* stream);

/* ------------------------------------------------------------------------ *
 * Motion-bank minimum-L2 drift check
 *
 * PersonaLive, section 抗身份漂移的补丁: the current frame's expression
 * embedding is compared with the motion bank; if its smallest L2 distance
 * exceeds the threshold (17 on the pages) the caller appends an anchor, at
 * most three times per stream.  Section 三条条件通路: the embedding is the
 * 512-dimensional MotEncoder output.
 *
 * For each query i, with the Euclidean distances d_j = ||query[i] - bank[j]||_2
 * accumulated in fp64 (each fp32 difference and its square are exact there;
 * the sum has a fixed reduction order): argmin[i] = the lowest j reaching
 * min_j d_j, exceeds[i] = (min_j d_j > threshold) ? 1 : 0 decided in fp64,
 * min_dist[i] = min_j d_j rounded to fp32.
 *
 *   query         device fp32 [nq][D]; bank device fp32 [n][D].
 *   nq >= 1; n in 1..PL_MAX_MOTION_BANK; D in 1..65536.
 *   min_dist      device fp32 [nq]; argmin device int32 [nq]; exceeds device u8 [nq].
 * The append decision and its cap belong to the caller. */
pl_status pl_motion_bank_min_l2(const float* query, int32_t nq, const float* bank, int32_t n,
                                int32_t D, float threshold, float* min_dist, int32_t* argmin,
                                uint8_t* exceeds, void* stream);

/* ------------------------------------------------------------------------ *
 * Latents-pile state machine (host only, no device work)
 *
 * PersonaLive, section 流式金字塔去噪: a deque of W windows, oldest at t = 0
 * and the newest, just enqueued, at the top timestep; each round appends a
 * window at the top, steps every window one level and pops the oldest after
 * its t = 0 evaluation, so the queue length is constant.  Section 首帧怎么办:
 * the queue is pre-filled with W-1 windows of staircase noise so the first
 * round already emits.
 *
 * The pile's device storage is W window slots used as a ring; this struct
 * tracks which slot holds which window at which t.  A window is evaluated at
 * t_top, t_top - step_len, ..., 0 in consecutive rounds and is popped after
 * its t = 0 evaluation (t_top must be a multiple of step_len).
 * ------------------------------------------------------------------------ */
struct pl_pile {
  int32_t W;                       /* slots = windows per forward */
  int32_t step_len;                /* timestep decrement per round */
  int32_t t_top;                   /* timestep of a newly enqueued window */
  int32_t count;                   /* windows currently held */
  int32_t head;                    /* slot of the oldest held window */
  int32_t in_round;                /* 1 between begin_round and end_round */
  int32_t t[PL_MAX_WINDOWS];       /* timestep per slot (valid for held slots) */
  int64_t id[PL_MAX_WINDOWS];      /* window id per slot, -1 = free */
  int64_t next_id;                 /* id of the next enqueued window */
};

/* Initialise.  W in 2..PL_MAX_WINDOWS, step_len >= 1, t_top = (W-1)*step_len.
 * prefill != 0 places W-1 windows at 0, step_len, ..., (W-2)*step_len in
 * slots 0..W-2 (ids 0..W-2, oldest first). */
pl_status pl_pile_init(pl_pile* p, int32_t W, int32_t step_len, int32_t t_top, int32_t prefill);

/* Start a round: enqueue a new window at t_top.
 *   new_slot  out: slot the new window occupies (the caller fills its latents).
 *   t_slot    out host int32 [W]: timestep per slot for this round's DDIM step
 *             (free slots, which exist only without prefill, report t_top and
 *             hold no window).
 *   emit_slot out: slot holding the window at t = 0, or -1 if none yet.
 * PL_EINVAL if a round is already open. */
pl_status pl_pile_begin_round(pl_pile* p, int32_t* new_slot, int32_t* t_slot, int32_t* emit_slot);

/* Finish the round: pop the window at t = 0 (if any) and step the others down
 * by step_len.  emitted_id out: the popped window's id or -1.
 * PL_EINVAL if no round is open. */
pl_status pl_pile_end_round(pl_pile* p, int64_t* emitted_id);

#ifdef __cplusplus
}
#endif

#endif /* PL_H_ */
