"""Host logic of the full-size parity sample (no GPU)."""
import numpy as np

from parity_sampling import tile_aware_positions


def test_tile_aware_sample_covers_every_tile():
    # host logic of the sample above: every tile's first, last and extra rows
    counts = np.array([557, 0, 288, 33, 256, 1, 16384], dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    pos = set(tile_aware_positions(counts, offsets).tolist())
    # 557 rows: tiles of 288 (rows 0..287, extra 256..287) and 269 (288..556, extra 544..556)
    assert {0, 287, 288, 556} <= pos and set(range(256, 288)) <= pos and set(range(544, 557)) <= pos
    assert 557 + 288 - 1 in pos and 557 + 256 in pos  # 288 rows: one tile with 32 extra rows
    assert all(0 <= p < offsets[-1] for p in pos)
