"""Thin ctypes binding of ``libpl.so`` (declared in ``include/pl.h``).

The raw entry points keep their C names (``pl_refbank_attn``, ...).  The
tensor helpers below only marshal arguments: they read pointers, strides and
the current HIP stream from PyTorch tensors and call the library; every step
of the computation runs in the library's HIP kernels.  There is no fallback:
if the library is missing or the call fails, an exception is raised.

PyTorch must be imported before the library is loaded so that ``libpl.so``
binds to the HIP runtime PyTorch already loaded (one runtime per process).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PL_LIBRARY names another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("PL_LIBRARY") or os.path.join(_HERE, "libpl.so")

PL_OK, PL_EINVAL, PL_EUNSUPPORTED, PL_EDEVICE = 0, 1, 2, 3
PL_MAX_SEGMENTS = 8
PL_MAX_WINDOWS = 8
PL_MAX_MOTION_BANK = 4

# every symbol include/pl.h declares
EXPORTED = (
    "pl_abi_version",
    "pl_status_string",
    "pl_last_error",
    "pl_refbank_attn_workspace_size",
    "pl_refbank_attn",
    "pl_refbank_attn_noalloc",
    "pl_refbank_attn_chunked",
    "pl_debug_bounds",
    "pl_pyramid_ddim_step",
    "pl_pyramid_ddim_step_roll",
    "pl_sd_alphas_cumprod",
    "pl_pyramid_ddim_step_device",
    "pl_window_noise",
    "pl_pile_prefill",
    "pl_lerp_points",
    "pl_linear",
    "pl_motion_bank_min_l2",
    "pl_pile_init",
    "pl_pile_begin_round",
    "pl_pile_end_round",
)


class PlError(RuntimeError):
    """A pl_* call returned a non-zero status."""

    def __init__(self, name, status, detail):
        self.status = status
        super().__init__(f"{name} failed with {status_name(status)}: {detail}")


class pl_kv_segment(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("len", ctypes.c_int64),
        ("ld", ctypes.c_int64),
        ("frame_stride", ctypes.c_int64),
    ]


class pl_pile(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.c_int32),
        ("step_len", ctypes.c_int32),
        ("t_top", ctypes.c_int32),
        ("count", ctypes.c_int32),
        ("head", ctypes.c_int32),
        ("in_round", ctypes.c_int32),
        ("t", ctypes.c_int32 * PL_MAX_WINDOWS),
        ("id", ctypes.c_int64 * PL_MAX_WINDOWS),
        ("next_id", ctypes.c_int64),
    ]


_lib = None


def load():
    """Load libpl.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m streaming_diffusion_portrait_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, f64, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                                  ctypes.c_void_p, ctypes.c_size_t)
    lib.pl_abi_version.restype = i32
    lib.pl_abi_version.argtypes = []
    lib.pl_status_string.restype = ctypes.c_char_p
    lib.pl_status_string.argtypes = [i32]
    lib.pl_last_error.restype = ctypes.c_char_p
    lib.pl_last_error.argtypes = []
    lib.pl_refbank_attn_workspace_size.restype = sz
    lib.pl_refbank_attn_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i64), i32]
    lib.pl_refbank_attn.restype = i32
    lib.pl_refbank_attn.argtypes = [vp, i64, i64, vp, i64, i64, i32, i32, i32, i32,
                                    ctypes.POINTER(pl_kv_segment), i32, f32, vp, sz, vp]
    lib.pl_refbank_attn_noalloc.restype = i32
    lib.pl_refbank_attn_noalloc.argtypes = [vp, i64, i64, vp, i64, i64, i32, i32, i32, i32,
                                            ctypes.POINTER(pl_kv_segment), i32, f32, vp]
    lib.pl_debug_bounds.restype = i32
    lib.pl_debug_bounds.argtypes = [ctypes.POINTER(ctypes.c_uint64), i32]
    lib.pl_refbank_attn_chunked.restype = i32
    lib.pl_refbank_attn_chunked.argtypes = [vp, i64, i64, vp, i64, i64, i32, i32, i32, i32,
                                            ctypes.POINTER(pl_kv_segment), i32, i32, i32, i32, f32, vp]
    lib.pl_pyramid_ddim_step.restype = i32
    lib.pl_pyramid_ddim_step.argtypes = [vp, vp, vp, vp, i32, i64, ctypes.POINTER(i32), i32,
                                         ctypes.POINTER(f64), i32, f64, i32, vp]
    u64 = ctypes.c_uint64
    lib.pl_pyramid_ddim_step_roll.restype = i32
    lib.pl_pyramid_ddim_step_roll.argtypes = [vp, vp, vp, vp, i32, i64, ctypes.POINTER(i32), i32,
                                              ctypes.POINTER(f64), i32, f64, i32, u64, u64, vp]
    lib.pl_sd_alphas_cumprod.restype = i32
    lib.pl_sd_alphas_cumprod.argtypes = [ctypes.POINTER(f64), i32]
    lib.pl_pyramid_ddim_step_device.restype = i32
    lib.pl_pyramid_ddim_step_device.argtypes = [vp, vp, vp, vp, i32, i64, vp, vp, i32, f64, u64, vp]
    lib.pl_window_noise.restype = i32
    lib.pl_window_noise.argtypes = [vp, i64, u64, u64, vp]
    lib.pl_pile_prefill.restype = i32
    lib.pl_pile_prefill.argtypes = [vp, vp, i32, i64, i32, ctypes.POINTER(f64), i32, u64, vp]
    lib.pl_lerp_points.restype = i32
    lib.pl_lerp_points.argtypes = [vp, vp, i64, i32, vp, vp]
    lib.pl_linear.restype = i32
    lib.pl_linear.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i32, i32, vp]
    lib.pl_motion_bank_min_l2.restype = i32
    lib.pl_motion_bank_min_l2.argtypes = [vp, i32, vp, i32, i32, f32, vp, vp, vp, vp]
    lib.pl_pile_init.restype = i32
    lib.pl_pile_init.argtypes = [ctypes.POINTER(pl_pile), i32, i32, i32, i32]
    lib.pl_pile_begin_round.restype = i32
    lib.pl_pile_begin_round.argtypes = [ctypes.POINTER(pl_pile), ctypes.POINTER(i32), ctypes.POINTER(i32),
                                        ctypes.POINTER(i32)]
    lib.pl_pile_end_round.restype = i32
    lib.pl_pile_end_round.argtypes = [ctypes.POINTER(pl_pile), ctypes.POINTER(i64)]
    _lib = lib
    return lib


def status_name(status):
    return load().pl_status_string(int(status)).decode()


def last_error():
    return load().pl_last_error().decode()


def _check(name, status):
    if status != PL_OK:
        raise PlError(name, status, last_error())


# ---- raw entry points, same names as the C ABI ----------------------------------
def pl_refbank_attn(*args):
    return load().pl_refbank_attn(*args)


def pl_refbank_attn_noalloc(*args):
    return load().pl_refbank_attn_noalloc(*args)


def pl_refbank_attn_chunked(*args):
    return load().pl_refbank_attn_chunked(*args)


def pl_refbank_attn_workspace_size(*args):
    return load().pl_refbank_attn_workspace_size(*args)


def pl_pyramid_ddim_step(*args):
    return load().pl_pyramid_ddim_step(*args)


def pl_pyramid_ddim_step_roll(*args):
    return load().pl_pyramid_ddim_step_roll(*args)


def pl_sd_alphas_cumprod(*args):
    return load().pl_sd_alphas_cumprod(*args)


def pl_pyramid_ddim_step_device(*args):
    return load().pl_pyramid_ddim_step_device(*args)


def pl_window_noise(*args):
    return load().pl_window_noise(*args)


def pl_pile_prefill(*args):
    return load().pl_pile_prefill(*args)


def pl_lerp_points(*args):
    return load().pl_lerp_points(*args)


def pl_linear(*args):
    return load().pl_linear(*args)


def pl_motion_bank_min_l2(*args):
    return load().pl_motion_bank_min_l2(*args)


def pl_pile_init(*args):
    return load().pl_pile_init(*args)


def pl_pile_begin_round(*args):
    return load().pl_pile_begin_round(*args)


def pl_pile_end_round(*args):
    return load().pl_pile_end_round(*args)


# ---- tensor helpers ---------------------------------------------------------------
def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _rows(t, name):
    """(row stride, frame stride) of a [F, L, C] or [L, C] tensor with unit column stride."""
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")
    if t.dim() == 3:
        return t.stride(1), t.stride(0)
    if t.dim() == 2:
        return t.stride(0), 0
    raise ValueError(f"{name} must be [F, L, C] or [L, C]")


def make_segments(segments, frames=None, channels=None):
    """Segment table for the key axis (the bank segment assembly).

    ``segments``: sequence of ``(k, v)`` fp16 device tensors, either
    ``[F, Ls, C]`` (per-frame: the frame's own tokens), ``[1, Ls, C]`` or
    ``[Ls, C]`` (shared by every frame: the reference entry and anchors).
    ``frames`` / ``channels``: the query's F and C; a 3-D segment must have
    F or 1 frames and every segment C columns (checked here, since the
    library never sees a segment's extent).  Nothing is copied; the table
    holds pointers and strides.  Returns ``(array, keepalive)``.
    """
    n = len(segments)
    if not 1 <= n <= PL_MAX_SEGMENTS:
        raise ValueError(f"1..{PL_MAX_SEGMENTS} segments required")
    arr = (pl_kv_segment * n)()
    for i, (k, v) in enumerate(segments):
        if k.shape != v.shape or k.stride() != v.stride():
            raise ValueError("k and v of a segment must share shape and strides")
        if channels is not None and k.shape[-1] != channels:
            raise ValueError(f"segment {i} has {k.shape[-1]} columns, q has {channels}")
        ld, fs = _rows(k, "k")
        if k.dim() == 3:
            if k.shape[0] == 1 and frames != 1:
                fs = 0  # one set of rows for every frame
            elif frames is not None and k.shape[0] != frames:
                raise ValueError(f"segment {i} has {k.shape[0]} frames, q has {frames} (or pass 1 to share)")
        _need(k, torch.float16, "k")
        _need(v, torch.float16, "v")
        arr[i] = pl_kv_segment(k.data_ptr(), v.data_ptr(), k.shape[-2], ld, fs)
    return arr, segments


def _workspace(F, L, heads, d, segs, device, workspace=None):
    """(pointer, bytes) of the key-split workspace the call needs: ``workspace``
    (a device tensor) if given, else a fresh allocation; (None, 0) when the
    launch splits nothing."""
    if workspace is False:  # run the single-pass kernels
        return None, 0, None
    lens = (ctypes.c_int64 * len(segs))(*[s.len for s in segs])
    need = load().pl_refbank_attn_workspace_size(F, L, heads, d, lens, len(segs))
    if workspace is None:
        if not need:
            return None, 0, None
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous device tensor")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), workspace


def debug_bounds(reset=True):
    """Mask of attention access sites that failed their bounds check (see
    ``pl_debug_bounds``); None when the loaded library has no checks."""
    mask = ctypes.c_uint64(0)
    st = load().pl_debug_bounds(ctypes.byref(mask), 1 if reset else 0)
    if st == PL_EUNSUPPORTED:
        return None
    _check("pl_debug_bounds", st)
    return int(mask.value)


def workspace_size(F, L, heads, d, seg_lens):
    """Bytes of workspace ``pl_refbank_attn`` needs for these sizes (0: none)."""
    lens = (ctypes.c_int64 * len(seg_lens))(*[int(x) for x in seg_lens])
    return int(load().pl_refbank_attn_workspace_size(F, L, heads, d, lens, len(seg_lens)))


def refbank_attn(q, segments, heads, out=None, scale=None, stream=None, workspace=None):
    """O = ref-bank attention of one layer (see ``pl_refbank_attn``).

    ``q``: fp16 device ``[F, L, C]``; ``segments`` as for :func:`make_segments`;
    ``heads``: H with d = C / H.  ``workspace``: a device tensor of at least
    :func:`workspace_size` bytes for the launches that split the key axis
    (allocated here when needed and not given; ``False`` runs the single-pass
    kernels instead).  Returns ``out`` (allocated if None).
    """
    _need(q, torch.float16, "q")
    if q.dim() != 3:
        raise ValueError("q must be [F, L, C]")
    F, L, C = q.shape
    if C % heads:
        raise ValueError("C must be divisible by heads")
    d = C // heads
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.float16, "out")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = d ** -0.5
    q_ld, q_fs = _rows(q, "q")
    o_ld, o_fs = _rows(out, "out")
    segs, _keep = make_segments(segments, F, C)
    ws, ws_bytes, _ws_keep = _workspace(F, L, heads, d, segs, q.device, workspace)
    st = pl_refbank_attn(ctypes.c_void_p(q.data_ptr()), q_ld, q_fs, ctypes.c_void_p(out.data_ptr()), o_ld, o_fs,
                         F, L, heads, d, segs, len(segments), float(scale), ws, ws_bytes, _stream_ptr(stream))
    _check("pl_refbank_attn", st)
    return out


def chunked_attn(q, self_kv, shared, heads, chunk_len, max_history=-1, out=None, scale=None, stream=None):
    """Block-causal attention over chunked sequences (see ``pl_refbank_attn_chunked``).

    ``q``: fp16 device ``[F, L, C]``; ``self_kv``: (k, v) ``[F, L, C]``, the
    sequence's own keys (row j in chunk j // chunk_len); ``shared``: list of
    (k, v) ``[Ls, C]`` visible to every row.  Returns ``out``.
    """
    _need(q, torch.float16, "q")
    if q.dim() != 3:
        raise ValueError("q must be [F, L, C]")
    F, L, C = q.shape
    if C % heads:
        raise ValueError("C must be divisible by heads")
    d = C // heads
    if self_kv[0].dim() != 3 or tuple(self_kv[0].shape) != (F, L, C):
        raise ValueError("the causal segment must be [F, L, C] like q")
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.float16, "out")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = d ** -0.5
    q_ld, q_fs = _rows(q, "q")
    o_ld, o_fs = _rows(out, "out")
    segs, _keep = make_segments([tuple(self_kv)] + [tuple(kv) for kv in shared], F, C)
    st = pl_refbank_attn_chunked(ctypes.c_void_p(q.data_ptr()), q_ld, q_fs, ctypes.c_void_p(out.data_ptr()), o_ld,
                                 o_fs, F, L, heads, d, segs, len(segs), 0, int(chunk_len), int(max_history),
                                 float(scale), _stream_ptr(stream))
    _check("pl_refbank_attn_chunked", st)
    return out


def _schedule(alphas_cumprod):
    if alphas_cumprod is None:
        return None, 1000
    ab = (ctypes.c_double * len(alphas_cumprod))(*[float(a) for a in alphas_cumprod])
    return ab, len(alphas_cumprod)


def pyramid_ddim_step(x_t, eps, t_windows, x_prev=None, x0_out=None, emit_window=-1, step_len=333,
                      alphas_cumprod=None, final_alpha_cumprod=-1.0, stream=None, roll=None):
    """Per-window DDIM step over a window-major fp32 pile (see ``pl_pyramid_ddim_step``).

    ``x_t``/``eps``: fp32 device tensors whose leading axis splits into
    ``W = len(t_windows)`` contiguous windows.  ``x_prev`` may be ``x_t``
    (in place).  ``roll=(seed, new_window_id)`` calls
    ``pl_pyramid_ddim_step_roll``: the emitted window's slot of ``x_prev``
    then holds the next window's noise.  Returns ``(x_prev, x0_out)``.
    """
    _need(x_t, torch.float32, "x_t")
    _need(eps, torch.float32, "eps")
    if not (x_t.is_contiguous() and eps.is_contiguous()) or x_t.shape != eps.shape:
        raise ValueError("x_t and eps must be contiguous with equal shapes")
    W = len(t_windows)
    if W < 1 or x_t.numel() % W:
        raise ValueError("the pile must split into W windows")
    per = x_t.numel() // W
    if x_prev is None:
        x_prev = torch.empty_like(x_t)
    _need(x_prev, torch.float32, "x_prev")
    if not x_prev.is_contiguous() or x_prev.numel() != x_t.numel():
        raise ValueError("x_prev must be contiguous with x_t's size")
    if emit_window >= 0 and x0_out is None:
        x0_out = torch.empty(per, dtype=torch.float32, device=x_t.device)
    if x0_out is not None:
        _need(x0_out, torch.float32, "x0_out")
        if not x0_out.is_contiguous() or x0_out.numel() != per:
            raise ValueError("x0_out must be contiguous with one window's size")
    ts = (ctypes.c_int32 * W)(*[int(t) for t in t_windows])
    ab_ptr, T = _schedule(alphas_cumprod)
    args = [ctypes.c_void_p(x_t.data_ptr()), ctypes.c_void_p(eps.data_ptr()), ctypes.c_void_p(x_prev.data_ptr()),
            ctypes.c_void_p(x0_out.data_ptr()) if x0_out is not None else None,
            W, per, ts, int(step_len), ab_ptr, T, float(final_alpha_cumprod), int(emit_window)]
    if roll is None:
        _check("pl_pyramid_ddim_step", pl_pyramid_ddim_step(*args, _stream_ptr(stream)))
    else:
        seed, new_id = roll
        _check("pl_pyramid_ddim_step_roll",
               pl_pyramid_ddim_step_roll(*args, int(seed), int(new_id), _stream_ptr(stream)))
    return x_prev, x0_out


def window_noise(n_or_out, seed, window_id, stream=None):
    """N(0, 1) noise of one window (see ``pl_window_noise``): fp32 device [n]."""
    if isinstance(n_or_out, torch.Tensor):
        out = n_or_out
        _need(out, torch.float32, "out")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    else:
        out = torch.empty(int(n_or_out), dtype=torch.float32, device="cuda")
    _check("pl_window_noise", pl_window_noise(ctypes.c_void_p(out.data_ptr()), out.numel(), int(seed),
                                              int(window_id), _stream_ptr(stream)))
    return out


def pile_prefill(ref, n_windows, seed, step_len=333, alphas_cumprod=None, out=None, stream=None):
    """Staircase prefill (see ``pl_pile_prefill``): fp32 [n_windows, ref.numel()]."""
    _need(ref, torch.float32, "ref")
    if not ref.is_contiguous():
        raise ValueError("ref must be contiguous")
    per = ref.numel()
    if out is None:
        out = torch.empty((n_windows, per), dtype=torch.float32, device=ref.device)
    _need(out, torch.float32, "out")
    if not out.is_contiguous() or out.numel() < n_windows * per:
        raise ValueError("out must be contiguous with n_windows windows")
    ab_ptr, T = _schedule(alphas_cumprod)
    _check("pl_pile_prefill", pl_pile_prefill(ctypes.c_void_p(ref.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                              int(n_windows), per, int(step_len), ab_ptr, T, int(seed),
                                              _stream_ptr(stream)))
    return out


def _as_rows(t, n, name):
    """``t`` [..., n] seen as a [rows, n] matrix with one row stride, without a copy."""
    if t.dim() == 2:
        return t
    try:
        return t.view(-1, n)
    except RuntimeError as e:
        raise ValueError(f"{name} cannot be seen as [rows, {n}] with one row stride "
                         f"(strides {t.stride()}); pass a 2-D view") from e


def linear(x, w, bias=None, out=None, stream=None):
    """y = x W^T (+ bias) (see ``pl_linear``).

    ``x``: fp16 device ``[M, K]`` (or ``[..., K]``, flattened over the leading
    axes; rows may be strided); ``w``: fp16 ``[N, K]``; ``bias``: fp32 ``[N]``
    or None.  Returns ``out`` ``[..., N]`` (allocated if None).
    """
    if x.stride(-1) != 1 or w.dim() != 2 or w.stride(-1) != 1:
        raise ValueError("x and w need unit stride in their last dimension; w must be [N, K]")
    lead = tuple(x.shape[:-1])
    K = x.shape[-1]
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K] with x's K")
    # views, never copies: rows that cannot be seen as one [M, K] / [M, N] matrix raise
    x2 = _as_rows(x, K, "x")
    M = x2.shape[0]
    if out is not None:
        if tuple(out.shape) != (*lead, N):
            raise ValueError(f"out must have shape {(*lead, N)}, got {tuple(out.shape)}")
        if out.stride(-1) != 1:
            raise ValueError("out needs unit stride in its last dimension")
        y2 = _as_rows(out, N, "out")
    if bias is not None and (not bias.is_contiguous() or bias.numel() != N):
        raise ValueError("bias must be contiguous [N]")
    _need(x, torch.float16, "x")
    _need(w, torch.float16, "w")
    if out is None:
        out = torch.empty((*lead, N), dtype=torch.float16, device=x.device)
        y2 = _as_rows(out, N, "out")
    _need(out, torch.float16, "out")
    if bias is not None:
        _need(bias, torch.float32, "bias")
    _check("pl_linear", pl_linear(ctypes.c_void_p(x2.data_ptr()), x2.stride(0), ctypes.c_void_p(w.data_ptr()),
                                  w.stride(0), ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
                                  ctypes.c_void_p(y2.data_ptr()), y2.stride(0), M, N, K, _stream_ptr(stream)))
    return out


def lerp_points(a, b, n, out=None, stream=None):
    """n evenly spaced points from a towards b, b excluded (see ``pl_lerp_points``): fp32 [n, D]."""
    _need(a, torch.float32, "a")
    _need(b, torch.float32, "b")
    if not (a.is_contiguous() and b.is_contiguous()) or a.numel() != b.numel():
        raise ValueError("a and b must be contiguous with equal sizes")
    D = a.numel()
    if out is None:
        out = torch.empty((int(n), D), dtype=torch.float32, device=a.device)
    _need(out, torch.float32, "out")
    if not out.is_contiguous() or out.numel() != int(n) * D:
        raise ValueError("out must be contiguous [n, D]")
    _check("pl_lerp_points", pl_lerp_points(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), D,
                                            int(n), ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
    return out


def motion_bank_min_l2(query, bank, threshold=17.0, out=None, stream=None):
    """Minimum L2 distance of each query to the motion bank (see ``pl_motion_bank_min_l2``).

    ``query``: fp32 device ``[nq, D]`` (or ``[D]``); ``bank``: fp32 ``[n, D]``.
    Returns ``(min_dist fp32 [nq], argmin int32 [nq], exceeds uint8 [nq])``.
    """
    _need(query, torch.float32, "query")
    _need(bank, torch.float32, "bank")
    if query.dim() == 1:
        query = query.unsqueeze(0)
    if not (query.is_contiguous() and bank.is_contiguous()) or query.shape[1] != bank.shape[1]:
        raise ValueError("query [nq, D] and bank [n, D] must be contiguous and share D")
    nq, D = query.shape
    n = bank.shape[0]
    if out is None:
        dev = query.device
        out = (torch.empty(nq, dtype=torch.float32, device=dev), torch.empty(nq, dtype=torch.int32, device=dev),
               torch.empty(nq, dtype=torch.uint8, device=dev))
    md, am, ex = out
    st = pl_motion_bank_min_l2(ctypes.c_void_p(query.data_ptr()), nq, ctypes.c_void_p(bank.data_ptr()), n, D,
                               float(threshold), ctypes.c_void_p(md.data_ptr()), ctypes.c_void_p(am.data_ptr()),
                               ctypes.c_void_p(ex.data_ptr()), _stream_ptr(stream))
    _check("pl_motion_bank_min_l2", st)
    return md, am, ex


class Pile:
    """Host-side latents-pile state machine backed by ``pl_pile_*``."""

    def __init__(self, W=4, step_len=333, t_top=None, prefill=True):
        self._p = pl_pile()
        if t_top is None:
            t_top = (W - 1) * step_len
        _check("pl_pile_init", pl_pile_init(ctypes.byref(self._p), W, step_len, t_top, 1 if prefill else 0))
        self.W = W

    def begin_round(self):
        """-> (new_slot, t_per_slot list, emit_slot or -1)."""
        ns, es = ctypes.c_int32(), ctypes.c_int32()
        ts = (ctypes.c_int32 * self.W)()
        _check("pl_pile_begin_round", pl_pile_begin_round(ctypes.byref(self._p), ctypes.byref(ns), ts, ctypes.byref(es)))
        return ns.value, list(ts), es.value

    def end_round(self):
        """-> id of the popped window or -1."""
        e = ctypes.c_int64()
        _check("pl_pile_end_round", pl_pile_end_round(ctypes.byref(self._p), ctypes.byref(e)))
        return e.value

    def slot_ids(self):
        return [self._p.id[s] for s in range(self.W)]


def sd_alphas_cumprod():
    """The library's built-in alpha_bar table (SD scaled_linear, T = 1000) as a host list."""
    ab = (ctypes.c_double * 1000)()
    _check("pl_sd_alphas_cumprod", pl_sd_alphas_cumprod(ab, 1000))
    return list(ab)


class DevicePile:
    """The pile's state machine held in device memory (see ``pl_pyramid_ddim_step_device``).

    The state starts as ``pl_pile_init`` leaves it and is read and advanced by
    the kernels, so ``step`` issues the same launches every round -- a round
    built from it can be captured once in a graph and replayed.  ``state()``
    copies the state back to the host (a synchronising read).
    """

    def __init__(self, W=4, step_len=333, prefill=True, device="cuda", alphas_cumprod=None):
        host = pl_pile()
        _check("pl_pile_init", pl_pile_init(ctypes.byref(host), W, step_len, (W - 1) * step_len,
                                            1 if prefill else 0))
        raw = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8)
        self.buf = raw.to(device)  # 8-byte aligned device allocation
        ab = sd_alphas_cumprod() if alphas_cumprod is None else [float(a) for a in alphas_cumprod]
        self.ab = torch.tensor(ab, dtype=torch.float64, device=device)
        self.W = W

    def step(self, x_t, eps, x_prev, x0_out, seed, final_alpha_cumprod=-1.0, stream=None):
        """One round: the new window enters, the rolling DDIM step, the state advances."""
        for t, name in ((x_t, "x_t"), (eps, "eps"), (x_prev, "x_prev"), (x0_out, "x0_out")):
            _need(t, torch.float32, name)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if x_t.numel() != eps.numel() or x_prev.numel() != x_t.numel() or x_t.numel() % self.W:
            raise ValueError("x_t, eps and x_prev must hold W equal windows")
        per = x_t.numel() // self.W
        if x0_out.numel() != per:
            raise ValueError("x0_out must hold one window")
        _check("pl_pyramid_ddim_step_device",
               pl_pyramid_ddim_step_device(ctypes.c_void_p(x_t.data_ptr()), ctypes.c_void_p(eps.data_ptr()),
                                           ctypes.c_void_p(x_prev.data_ptr()), ctypes.c_void_p(x0_out.data_ptr()),
                                           self.W, per, ctypes.c_void_p(self.buf.data_ptr()),
                                           ctypes.c_void_p(self.ab.data_ptr()), self.ab.numel(),
                                           float(final_alpha_cumprod), int(seed), _stream_ptr(stream)))

    def state(self):
        return pl_pile.from_buffer_copy(self.buf.cpu().numpy().tobytes())


class PreparedAttn:
    """A pl_refbank_attn call with its arguments marshalled once.

    For a streaming loop that attends the same buffers every round: calling
    the object only crosses into the library (one ctypes call), so per-launch
    host cost stays far below the small layers' GPU time.  The tensors must
    stay alive and unchanged in shape while the object is used; ``stream``
    is fixed at preparation (default: the current stream then).  A launch
    that splits the key axis keeps its workspace (``workspace``, or one
    allocated here) for the object's lifetime; calls on one workspace must
    not overlap in time.
    """

    def __init__(self, q, segments, heads, out, scale=None, stream=None, workspace=None):
        _need(q, torch.float16, "q")
        _need(out, torch.float16, "out")
        if q.dim() != 3 or out.shape != q.shape:
            raise ValueError("q and out must be [F, L, C] of the same shape")
        F, L, C = q.shape
        if C % heads:
            raise ValueError("C must be divisible by heads")
        d = C // heads
        if scale is None:
            scale = d ** -0.5
        q_ld, q_fs = _rows(q, "q")
        o_ld, o_fs = _rows(out, "out")
        self._segs, self._keep = make_segments(segments, F, C)
        ws, ws_bytes, self._ws = _workspace(F, L, heads, d, self._segs, q.device, workspace)
        self._tensors = (q, out)
        self.workspace_bytes = ws_bytes
        self.args = (ctypes.c_void_p(q.data_ptr()), q_ld, q_fs, ctypes.c_void_p(out.data_ptr()), o_ld, o_fs,
                     F, L, heads, d, self._segs, len(segments), float(scale), ws, ws_bytes, _stream_ptr(stream))
        self.flops = 4 * F * L * sum(s.len for s in self._segs) * C
        self._fn = load().pl_refbank_attn

    def __call__(self, stream=None):
        """Launch; ``stream`` (e.g. a graph's capture stream) overrides the prepared one."""
        args = self.args if stream is None else self.args[:-1] + (_stream_ptr(stream),)
        st = self._fn(*args)
        if st != PL_OK:
            raise PlError("pl_refbank_attn", st, last_error())
