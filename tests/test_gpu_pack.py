"""qlin_pack_weight against the packed layout's definition: for 16-row group
s, K block kb (nkb = ceil(K / 128)), half h and lane l, the 16 bytes at
1024 ((s nkb + kb) 2 + h) + 16 l are codes [16 s + l % 16][128 kb +
32 (l / 16) + 16 h + 0 .. 15], zeros past K.  The expected bytes are formed
here by numpy reshapes and transposes of the padded row-major codes (a plain
permutation, independent of the kernel's index arithmetic), for one and
several matrices, with ragged K; nothing is written outside the output."""
import numpy as np
import pytest
import torch

import skinny_bit_gemm_amd as q

pytestmark = pytest.mark.gpu

from _gpu import gpu_pack, to_dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def expected_packed(w):
    """[batch][N][K] uint8 -> [batch][packed bytes] by the layout's definition."""
    b, N, K = w.shape
    nkb = -(-K // 128)
    pad = np.zeros((b, N, nkb * 128), dtype=np.uint8)
    pad[:, :, :K] = w
    # row 16 s + r, byte 128 kb + 32 q + 16 h + j  ->  order (s, kb, h, q, r, j)
    a = pad.reshape(b, N // 16, 16, nkb, 4, 2, 16)          # b, s, r, kb, q, h, j
    return a.transpose(0, 1, 3, 5, 4, 2, 6).reshape(b, -1)


@pytest.mark.parametrize("batch,N,K", [(1, 16, 16), (1, 48, 1040), (1, 256, 512), (3, 64, 2064), (5, 32, 128)])
def test_pack_matches_the_layout_definition(batch, N, K):
    rng = np.random.default_rng(N * K + batch)
    w = rng.integers(0, 256, size=(batch, N, K), dtype=np.uint8)
    assert q.qlin_packed_weight_bytes(N, K) == N * (-(-K // 128)) * 128
    print(f"[pack] batch={batch} N={N} K={K}", flush=True)
    got = gpu_pack(to_dev(w), N, K, batch=batch).cpu().numpy().reshape(batch, -1)
    want = expected_packed(w)
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    # and the first bytes by hand: group 0, block 0, half 0, lane 0 holds row
    # 0, bytes 0..15; lane 16 holds row 0, bytes 32..47 (zeros past K)
    assert np.array_equal(got[0, :16], w[0, 0, :16])
    lane16 = np.zeros(16, dtype=np.uint8)
    lane16[:max(0, min(K, 48) - 32)] = w[0, 0, 32:48]
    assert np.array_equal(got[0, 16 * 16:16 * 17], lane16)
