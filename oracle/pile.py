"""Oracle: the ``latents_pile`` queue of the streaming pyramid.

Test infrastructure only (see the package docstring).

PersonaLive write-up, section "流式金字塔去噪": the pile is a deque of 4
windows of 4 frames, each window parked at its own noise level, oldest at
t = 0 and the newest, just enqueued, at t = 999.  Each round (1) the new
window is noised to t = 999 and appended, (2) the 16 frames go through one
UNet forward and the DDIM step moves every window one level, (3) the oldest
window has reached the end and is popped from the left and sent to the VAE.
The queue length is constant, so the stream has no clip boundary.  Section
"首帧怎么办": at start the queue is pre-filled with 12 frames of staircase
noise so that the first round already emits.

Reading: a window is evaluated at 999, 666, 333 and 0 in four consecutive
rounds and is popped after its t = 0 evaluation, emitting that evaluation's
x0 prediction (four evaluations = the four DDIM steps of the table).  Between
rounds the pile therefore holds three windows (12 frames) at 0 / 333 / 666.
"""

from collections import deque


class PyramidPile:
    """Integer state machine of the pile: window ids and their timesteps."""

    def __init__(self, timesteps=(999, 666, 333, 0), frames_per_window=4, prefill=True):
        self.timesteps = tuple(int(t) for t in timesteps)
        self.step_len = self.timesteps[0] - self.timesteps[1]
        self.frames_per_window = frames_per_window
        self.windows = deque()  # entries [window_id, t], oldest first
        self.next_id = 0
        if prefill:
            # staircase: the prefilled windows sit at the table's lower levels,
            # oldest at t = 0 (0 / 333 / 666 for the 4-level table)
            for t in reversed(self.timesteps[1:]):
                self.windows.append([self._new_id(), t])

    def _new_id(self):
        i = self.next_id
        self.next_id += 1
        return i

    def frames(self):
        return len(self.windows) * self.frames_per_window

    def round(self):
        """Run one round.

        Returns ``(evaluated, emitted_id)``: ``evaluated`` lists
        ``(window_id, t)`` oldest first as seen by the 16-frame forward;
        ``emitted_id`` is the window popped after this round (its x0 is the
        output), or None if no window has reached t = 0 yet.
        """
        self.windows.append([self._new_id(), self.timesteps[0]])
        evaluated = [(w, t) for w, t in self.windows]
        emitted = None
        if self.windows[0][1] == self.timesteps[-1]:
            emitted = self.windows.popleft()[0]
        for w in self.windows:
            w[1] -= self.step_len
        return evaluated, emitted
