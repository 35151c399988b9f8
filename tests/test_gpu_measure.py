"""The read-bandwidth helper through the C ABI: it must read every word it is given (the XOR of
all 32-bit words of the buffer, checked against numpy's on the same words), at sizes below,
at and past one stride of its grid, and with a ragged tail."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import spechead as sh
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1024 * 256 * 16, 1024 * 256 * 16 * 4 + 48, 33 << 20])
def test_read_probe_folds_every_word(nbytes):
    P.log(f"read probe over {nbytes} bytes")
    words = np.random.default_rng(nbytes).integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    sh.read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
