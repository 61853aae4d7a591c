"""The MXFP4 pool re-indexing used by the GPU tests (tests/gpu_common.mx_pool_logical)
inverts the tile layout the cache description in include/paged_kv.h states.  Runs on
the CPU: tiles are packed element by element straight from that description, then
unpacked by the helper."""
import numpy as np

from tests.gpu_common import VPOS, mx_pool_logical


def pack_from_description(codes, scales, P, D):
    """Logical K/V rows (codes [2][P][D], scales [2][P][D/32]) -> one head's K and V
    tiles, placing every nibble where the header's MXFP4 paragraph puts it."""
    J, C = D // 32, P * D // 2
    tiles = np.zeros((2, C + P * J), np.uint8)
    for t in range(P):
        for d in range(D):
            j, c, e = d // 32, (d // 8) % 4, d % 8
            byte = t * (D // 2) + 4 * (c * J + j) + e // 2           # K: word c*J + j, nibble e
            tiles[0, byte] |= codes[0, t, d] << (4 * (e % 2))
            k = VPOS[t % 32]
            cc, ee, m, u = k // 8, k % 8, d % 16, d // 16
            byte = (t // 32) * 16 * D + 4 * ((4 * m + cc) * (D // 16) + u) + ee // 2
            tiles[1, byte] |= codes[1, t, d] << (4 * (ee % 2))
        for j in range(J):
            tiles[0, C + t * J + j] = scales[0, t, j]
            tiles[1, C + ((t // 32) * 32 + VPOS[t % 32]) * J + j] = scales[1, t, j]
    return tiles


def test_pool_logical_inverts_the_described_layout():
    rng = np.random.default_rng(0)
    for P, D in ((32, 64), (64, 128)):
        N, H = 2, 3
        J = D // 32
        codes = rng.integers(0, 16, size=(N, H, 2, P, D)).astype(np.uint8)
        scales = rng.integers(0, 256, size=(N, H, 2, P, J)).astype(np.uint8)
        bits = np.zeros((N, 2, H, P * D // 2 + P * J), np.uint8)
        for n in range(N):
            for h in range(H):
                bits[n, :, h] = pack_from_description(codes[n, h], scales[n, h], P, D)
        got = mx_pool_logical(bits, P, D)
        want = np.concatenate([codes, scales], axis=-1).transpose(0, 2, 1, 3, 4)
        assert np.array_equal(got, want), (P, D)
