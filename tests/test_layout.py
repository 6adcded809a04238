"""Host-side checks of the tiled V^T workspace layout helpers used by the GPU tests."""
import numpy as np

from gpu_util import vt_decode, vt_encode


def test_vt_roundtrip_and_padding():
    rng = np.random.default_rng(5)
    for L in (1, 15, 16, 64, 65, 200):
        v = rng.standard_normal((2, 3, L, 8))
        vt = vt_encode(v)
        nt = (L + 63) // 64
        assert vt.shape == (2, 3, nt, 8, 64)
        assert np.array_equal(vt_decode(vt, L), v)
        # padding columns are zero
        assert np.count_nonzero(vt) == np.count_nonzero(v)


def test_vt_key_permutation():
    """Inside each 16-key group, key 8a+4u+r lands at column 8u+4a+r."""
    L = 64
    v = np.arange(L, dtype=np.float64)[None, None, :, None]  # value = key index
    vt = vt_encode(v)[0, 0, 0, 0]
    for key in range(L):
        g, p = divmod(key, 16)
        a, u, r = p >> 3, (p >> 2) & 1, p & 3
        assert vt[16 * g + 8 * u + 4 * a + r] == key
