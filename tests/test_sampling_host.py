"""CPU check of the tile-complete sampler the full-size GPU tests use."""
import numpy as np

from tests.gpu_util import tile_complete_samples


def test_tile_complete_samples_hit_every_band():
    for n in (8, 100, 320, 4352, 16384):
        s = tile_complete_samples(n, 0)
        assert s[0] == 0 and s[-1] == n - 1 and np.all(np.diff(s) > 0)
        for b0 in range(0, n, 64):
            assert np.any((s >= b0) & (s < b0 + 64)), (n, b0)
