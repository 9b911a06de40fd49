"""The 2-D RoPE positions of a DiT item as the pages' reading defines them,
written out plainly (an independent statement of the rule that both the library's
enc_positions and the oracle's inputs must follow):
  - the first G*G rows of an item's first range are the G x G image, row-major:
    row t at (column t % G, row t // G);
  - further rows of the first range pad the image to a multiple of 32 (zimage.rs,
    cortiq-engine 0.7.6, `prepare`: lengths padded to 32, the learned pad row of
    `ZDev`); the pages do not show their positions; reading: (0, 0), no rotation;
  - the rows of the second range are the captions, caption j at (G + j, G + j)
    (its own padding rows included: the caller's tables cover the padded length)."""
import numpy as np


def dit_positions(rows, items, grids):
    pos = np.zeros((rows, 2), np.int32)
    for (rr, g) in zip(items, grids):
        (r0, n0) = rr[0]
        for t in range(n0):
            if t < g * g:
                pos[r0 + t] = (t % g, t // g)
            else:
                pos[r0 + t] = (0, 0)
        if len(rr) > 1:
            (c0, nc) = rr[1]
            for j in range(nc):
                pos[c0 + j] = (g + j, g + j)
    return pos
