"""The device arithmetic behind the kernels' exact results, checked
exhaustively on the GPU at hand through anq_selfcheck_arith: the reciprocal
(hardware estimate plus one FMA correction) against IEEE 1/b over every normal
b below 2^120, the NVFP4 block-scale quotient against IEEE amax / 6 over every
non-negative binary32, the FP8 quotient's E4M3 codes against those of IEEE
a / s over every binary32 a at seven scales, and the E2M1 conversion's
saturation of every value at or beyond +-6."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def test_selfcheck_counts_are_zero():
    import nvfp4_quantization_place_amd as A
    print("anq_selfcheck_arith", flush=True)
    counts = A.selfcheck_arith()
    assert counts == [0, 0, 0, 0], counts


def test_selfcheck_on_a_side_stream_overwrites_counts():
    import nvfp4_quantization_place_amd as A
    st = torch.cuda.Stream()
    counts = torch.full((4,), 12345, dtype=torch.int64, device="cuda")
    with torch.cuda.stream(st):
        rc = A.lib().anq_selfcheck_arith(counts.data_ptr(), st.cuda_stream)
    assert rc == 0
    st.synchronize()
    assert counts.tolist() == [0, 0, 0, 0]
