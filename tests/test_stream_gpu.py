"""The calibration stream (anq_stream_rw) computes what its header states:
unit j of dst is the XOR of source units j, j + n_out, ... below n_in, started
from the unit index (64-bit little endian, then 8 zero bytes) where j >= n_in.
Checked for more reads than writes, more writes than reads, and equal counts,
with and without the non-temporal hint."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def expected(src: np.ndarray, n_in: int, n_out: int) -> np.ndarray:
    u = src[:n_in * 16].view(np.uint64).reshape(n_in, 2) if n_in else np.zeros((0, 2), np.uint64)
    out = np.zeros((n_out, 2), np.uint64)
    for j in range(n_out):
        if j < n_in:
            v = u[j].copy()
        else:
            v = np.array([j, 0], np.uint64)
        k = j + n_out
        while k < n_in:
            v ^= u[k]
            k += n_out
        out[j] = v
    return out.view(np.uint8).reshape(-1)


@pytest.mark.parametrize("n_in,n_out", [(0, 5), (1000, 1000), (2500, 1000), (1000, 2500),
                                        (4096, 257), (37, 37 * 3 + 1)])
@pytest.mark.parametrize("nt", [True, False])
def test_stream_matches_its_definition(n_in, n_out, nt):
    import nvfp4_quantization_place_amd as A
    rng = np.random.default_rng(n_in * 7 + n_out)
    src = rng.integers(0, 256, max(n_in, 1) * 16, dtype=np.uint8)
    dst = torch.full((n_out * 16 + 64,), 0xEE, dtype=torch.uint8, device="cuda")
    A.stream_rw(torch.from_numpy(src).cuda(), n_in * 16, dst, n_out * 16, nontemporal=nt)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    np.testing.assert_array_equal(got[:n_out * 16], expected(src, n_in, n_out))
    assert np.all(got[n_out * 16:] == 0xEE)          # nothing past the bytes asked for
