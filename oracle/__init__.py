"""Plain, slow, fp64 CPU oracle for the streaming pyramid denoiser's hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP path in ``streaming_diffusion_portrait_amd``.

Sources (cited by page and section; the pages are the PersonaLive write-up on
juhe.plus, "PersonaLive" for short, and the hysenlabs repository review):

* ``attention``  -- reference-bank spatial self-attention
  (PersonaLive, section "三条条件通路" / three conditioning paths: the 16
  reference-layer features are concatenated with the denoiser's own K/V for
  spatial self-attention), and block-causal attention over a chunked
  sequence (LPM write-up, section 6.3 分块因果注意力; the deep-compression-VAE
  write-up: full attention inside a chunk, earlier chunks only across).
* ``ddim``       -- the per-window DDIM step of the streaming pyramid
  (PersonaLive, sections "它解决什么" / specification and
  "流式金字塔去噪" / streaming pyramid denoising).
* ``motion``     -- the motion-bank minimum-L2 drift check
  (PersonaLive, section "抗身份漂移的补丁" / anti identity-drift patch).
* ``pile``       -- the ``latents_pile`` queue state machine
  (PersonaLive, section "流式金字塔去噪").
* ``linear``     -- the projections either side of the attention
  (PersonaLive, section "三条条件通路": the bank holds hidden states that the
  layer projects into keys and values).
* ``noise``      -- the pile's device-side roll: counter-based window noise,
  the staircase prefill and the first frames' motion interpolation
  (PersonaLive, sections "流式金字塔去噪", "首帧怎么办" and the TensorRT
  section's ``new_noise`` input and ``bind()``).

Every floating-point computation here is float64.  Each function states the
passage it follows; readings of points the pages leave open are listed in the
repository's design notes.  Parity status: every function here is pinned by
``tests/test_oracle_*.py`` against brute force, closed forms, invariants or a
library routine.  The staircase prefill's recipe (the reference latent noised
to each level) is a reading of a passage that does not state it: the
arithmetic is pinned, the choice of content is "parity unpinned".
"""

from .attention import refbank_attention, attend_rows, concat_segments, chunk_causal_attention
from .ddim import (
    sd_scaled_linear_alphas_cumprod,
    ddim_coefficients,
    ddim_step,
    pyramid_ddim_step,
)
from .motion import motion_bank_min_l2
from .pile import PyramidPile
from .linear import linear
from .noise import philox4x64, uniform24, window_noise, noise_at, staircase_prefill, lerp_points

__all__ = [
    "refbank_attention",
    "attend_rows",
    "concat_segments",
    "chunk_causal_attention",
    "sd_scaled_linear_alphas_cumprod",
    "ddim_coefficients",
    "ddim_step",
    "pyramid_ddim_step",
    "motion_bank_min_l2",
    "PyramidPile",
    "linear",
    "philox4x64",
    "uniform24",
    "window_noise",
    "noise_at",
    "staircase_prefill",
    "lerp_points",
]
