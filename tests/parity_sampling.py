"""Choice of the tokens compared with the oracle on large workloads (host logic)."""
import numpy as np

TILE_M, TILE_XT = 256, 32  # rows per M-tile of the large-M schedule, extra rows a tile may carry


def tile_aware_positions(counts, offsets, bm=TILE_M, xt=TILE_XT, block=32):
    """Sorted positions that touch every tile of the large-M schedule: the
    first and last row of every 32-row block of each expert's segment, and of
    every M-tile (an expert's c rows go to as few tiles as hold them at up to
    bm + xt rows; rows beyond n * bm ride as extra rows in the first tiles,
    xt each) its first and last row and all of its extra rows."""
    pos = set()
    for e, c in enumerate(counts):
        c, off = int(c), int(offsets[e])
        if c == 0:
            continue
        for b in range(0, c, block):
            pos.update((off + b, off + min(b + block, c) - 1))
        n = (c + bm + xt - 1) // (bm + xt)
        extra = max(c - n * bm, 0)
        for i in range(n):
            r0 = i * bm + min(extra, i * xt)
            rows = bm + min(max(extra - i * xt, 0), xt) if extra > 0 else (c - i * bm if i == n - 1 else bm)
            pos.update((off + r0, off + r0 + rows - 1))
            pos.update(off + r0 + r for r in range(bm, rows))
    return np.array(sorted(pos), dtype=np.int64)
