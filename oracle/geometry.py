"""Joint token layout and 3D positions (test infrastructure only).

Row order of the joint sequence: video rows, then audio rows, then text rows. Video row
``(t*H + y)*W + x`` is latent frame t, row y, column x of a T x H x W grid. When the video
tokens are pair-merged (token reduction), merged row ``(t*H + y)*(W/2) + m`` stands for the
horizontal pair x = 2m, 2m+1 and sits at position x = 2m + 0.5, the mean of the pair.
Reading taken: the pages name a single token stream for video, audio and text (mobbang.com,
"MiniMax H3：视频与音轨一起生成的开源模型") but not its order or any position encoding.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Geometry:
    frames: int
    grid_h: int
    grid_w: int
    n_audio: int
    n_text: int
    merged: bool = False

    @property
    def n_video(self) -> int:
        n = self.frames * self.grid_h * self.grid_w
        return n // 2 if self.merged else n

    @property
    def n_tokens(self) -> int:
        return self.n_video + self.n_audio + self.n_text

    def as_merged(self) -> "Geometry":
        if self.grid_w % 2:
            raise ValueError("token pairing needs an even latent width")
        return dataclasses.replace(self, merged=True)

    def as_unmerged(self) -> "Geometry":
        return dataclasses.replace(self, merged=False)

    def positions(self):
        """(pos [N, 3] float64 of (t, y, x), rotated [N] bool): only video rows are rotated."""
        n = self.n_tokens
        pos = np.zeros((n, 3), dtype=np.float64)
        rot = np.zeros(n, dtype=bool)
        i = 0
        w_cols = self.grid_w // 2 if self.merged else self.grid_w
        for t in range(self.frames):
            for y in range(self.grid_h):
                for c in range(w_cols):
                    x = 2 * c + 0.5 if self.merged else float(c)
                    pos[i] = (t, y, x)
                    rot[i] = True
                    i += 1
        assert i == self.n_video
        return pos, rot
