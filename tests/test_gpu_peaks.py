"""The measurement probes on the GPU, through the C ABI (needs an MI355X).

The matrix-core probe's result has a closed form: lane l of a wave feeds
A[m][k] = ((m + k) mod 8) * 2^-10 and B[k][n] = ((n >> 3) mod 4) * 2^-10, so
every v_mfma_f32_32x32x16_bf16 adds 56 * ((n >> 3) mod 4) * 2^-20 to C[m][n]
(the sum of (m + k) mod 8 over 16 consecutive k is 56), and the stored sum of
two elements of four chains after `iters` rounds is
448 * ((l >> 3) mod 4) * iters * 2^-20, exact in float32 for small iters.
The copy probe must reproduce its source byte for byte."""
import pytest

torch = pytest.importorskip("torch")

from gpu_util import log  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


@pytest.mark.parametrize("iters", [0, 1, 37])
def test_mfma_probe_closed_form(gqe, iters):
    blocks = gqe.peak_blocks()
    log(f"[peaks] mfma probe blocks {blocks} iters {iters}")
    assert blocks >= 2
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    gqe.peak_mfma_bf16(out, blocks, iters)
    torch.cuda.synchronize()
    lane = torch.arange(blocks * 256, device="cuda") % 64
    want = 448.0 * ((lane >> 3) % 4).float() * iters * 2.0 ** -20
    assert torch.equal(out, want)


@pytest.mark.parametrize("n16", [0, 1, 255, 4097, 1 << 20])
def test_copy_probe_reproduces_source(gqe, n16):
    log(f"[peaks] copy probe {16 * n16} bytes")
    g = torch.Generator(device="cuda").manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (4 * n16,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    gqe.peak_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
