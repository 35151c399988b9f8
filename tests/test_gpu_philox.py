"""The in-kernel uniform stream equals the oracle's Philox4x64-10 stream bit for bit."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import spechead as sh
from oracle import philox

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,offset,purpose", [(0, 0, 0), (5001, 17, 1), (2 ** 63 + 12345, 2 ** 40, 6)])
def test_philox_stream_matches_oracle(seed, offset, purpose):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    rows, n = 5, 1031
    got = sh.philox_uniform(seed, offset, purpose, rows, n, "cuda").cpu().numpy().astype(np.float64)
    for r in range(rows):
        want = philox.uniforms(seed, offset, purpose, r, np.arange(n))
        np.testing.assert_array_equal(got[r], want)
