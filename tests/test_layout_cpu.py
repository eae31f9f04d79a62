"""CPU check of the documented pool index map used by the GPU tests."""

import numpy as np

from synth import draws
from tests.test_gpu_parity import layout_index


def test_layout_index_is_a_bijection():
    for args in ((5, 16, 2, 128, draws.BF16), (3, 4, 1, 64, draws.F32), (2, 2, 3, 32, draws.BF16),
                 (2, 6, 1, 64, draws.F32)):
        for which in "kv":
            idx = layout_index(*args, which)
            assert np.array_equal(np.sort(idx.ravel()), np.arange(idx.size))
