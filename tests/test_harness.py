"""CPU checks of the parity bookkeeping in gpu_harness: the shortcut that counts
byte-identical code tiles without unpacking them must give the same counts as
unpacking every tile."""
import numpy as np
import pytest

from gpu_harness import Tally, unpack_fields


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_identical_tiles_shortcut_counts_like_a_full_unpack(orc, bits):
    rng = np.random.default_rng(bits)
    tb = orc.tile_bytes(bits, 128, 128)
    a = rng.integers(0, 256, (40, tb), dtype=np.uint8)
    b = a.copy()
    for i in range(0, 40, 6):  # flip a few bits in some tiles, several in one
        for _ in range(1 + (i == 12) * 5):
            b[i, rng.integers(tb)] ^= np.uint8(1 << int(rng.integers(8)))
    t = Tally()
    t.add_tiles(a, b, bits)
    d = np.abs(unpack_fields(a, bits).astype(int) - unpack_fields(b, bits).astype(int))
    assert t.tiles == 40
    assert t.codes == d.size
    assert t.code_mismatch == int((d != 0).sum()) > 0
    assert t.code_maxdiff == int(d.max())


def test_all_identical_tiles(orc):
    tb = orc.tile_bytes(6, 16, 16)
    a = np.random.default_rng(1).integers(0, 256, (5, tb), dtype=np.uint8)
    t = Tally()
    t.add_tiles(a, a.copy(), 6)
    assert (t.tiles, t.codes, t.code_mismatch, t.code_maxdiff) == (5, 5 * 256, 0, 0)
